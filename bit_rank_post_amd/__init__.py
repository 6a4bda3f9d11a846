"""Python binding of libtileq.so, the MI355X (gfx950) TileQ MoE forward.

Argument marshalling only: every step of the forward runs in the HIP kernels
behind the C ABI (include/tileq.h).  Device buffers and streams come from
PyTorch tensors (``tensor.data_ptr()``, ``torch.cuda.current_stream()``).
The library must be built first (``python -m bit_rank_post_amd.build``);
loading fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# TILEQ_LIB_PATH selects another build of the same library (the sanitizer build)
LIB_PATH = os.environ.get("TILEQ_LIB_PATH") or os.path.join(HERE, "libtileq.so")

TQ_F16, TQ_BF16, TQ_F32, TQ_F64 = 0, 1, 2, 3
TQ_SINGLE, TQ_SWIGLU = 0, 1
P_SINGLE, P_GATE, P_UP, P_DOWN = 0, 0, 1, 2
STATUS = {0: "TQ_OK", 1: "TQ_EINVAL", 2: "TQ_ESHAPE", 3: "TQ_ENOMEM", 4: "TQ_EHIP",
          5: "TQ_EUNSUPPORTED", 6: "TQ_ESTATE"}
EXPORTS = ["tq_layer_create", "tq_upload_proj", "tq_upload_shared_expert",
           "tq_workspace_size", "tq_forward", "tq_forward_from_logits", "tq_forward_noalloc", "tq_layer_destroy", "tq_last_error",
           "tq_abi_version", "tq_layer_set_path", "tq_forward_path", "tq_debug_route", "tq_debug_dequant", "tq_debug_row_bound", "tq_router_topk",
           "tq_profile_enable", "tq_profile_read", "tq_pack_workspace_size", "tq_pack_proj",
           "tq_calibrate_read"]
STAGES = ["route", "row_exponent", "column_stage_in", "gemm_in", "column_stage_down",
          "shared_expert", "gemm_down", "combine"]


class TileQError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {text}")
        self.status = status
        self.text = text


class ProjDesc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("group", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("tile_of_expert", ctypes.POINTER(ctypes.c_int32)),
                ("U", ctypes.c_void_p), ("sigma", ctypes.c_void_p),
                ("sigma_dtype", ctypes.c_int32), ("V", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p)]


class PackDesc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("group", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("sketch", ctypes.c_int32), ("power_iters", ctypes.c_int32),
                ("act", ctypes.c_int32),
                ("tile_of_expert", ctypes.POINTER(ctypes.c_int32)),
                ("W", ctypes.c_void_p), ("w_dtype", ctypes.c_int32),
                ("omega", ctypes.c_void_p),
                ("U", ctypes.c_void_p), ("sigma", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libtileq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: run python -m bit_rank_post_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.tq_layer_create.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(vp)]
        L.tq_upload_proj.argtypes = [vp, i32, ctypes.POINTER(ProjDesc), vp]
        L.tq_upload_shared_expert.argtypes = [vp, i32, vp, vp, vp, vp]
        L.tq_workspace_size.argtypes = [vp, i32, i32, ctypes.POINTER(sz)]
        L.tq_forward.argtypes = [vp, vp, i32, vp, vp, i32, vp, i32, vp, sz, vp]
        L.tq_forward_from_logits.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, i32, vp, sz, vp]
        L.tq_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, i32, vp, i32, vp]
        L.tq_layer_destroy.argtypes = [vp]
        L.tq_last_error.restype = ctypes.c_char_p
        L.tq_abi_version.restype = i32
        L.tq_layer_set_path.argtypes = [vp, i32]
        L.tq_forward_path.argtypes = [vp, i32, i32, ctypes.POINTER(i32)]
        L.tq_debug_route.argtypes = [vp, i32, vp, i32, i32, vp, sz] + [vp] * 7 + [vp]
        L.tq_debug_dequant.argtypes = [vp, i32, i32, vp, vp]
        L.tq_debug_row_bound.argtypes = [vp, i32, vp]
        L.tq_router_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.tq_profile_enable.argtypes = [vp, i32]
        L.tq_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float)]
        L.tq_calibrate_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.tq_pack_workspace_size.argtypes = [ctypes.POINTER(PackDesc), ctypes.POINTER(sz)]
        L.tq_pack_proj.argtypes = [ctypes.POINTER(PackDesc), vp, sz, vp]
        for name in EXPORTS:
            if name not in ("tq_last_error", "tq_abi_version"):
                getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise TileQError(fn, status, lib().tq_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)


def calibrate_read(buf, scratch, stream=None):
    """One plain streaming read of the device tensor buf (benchmark
    calibration); scratch is a device int32 tensor of at least one element."""
    _check("tq_calibrate_read", lib().tq_calibrate_read(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(scratch), _stream(stream)))


def router_topk(logits, k, ids, weights, stream=None):
    """Top-k router on the device: logits f32 [T][K] -> ids int32 [T][k],
    weights f32 [T][k] (caller-allocated device tensors)."""
    T, K = logits.shape
    _check("tq_router_topk", lib().tq_router_topk(_ptr(logits), T, K, k, _ptr(ids), _ptr(weights),
                                                  _stream(stream)))


def pack_proj(*, K, M, N, d_in, d_out, rank, group, bits, sketch, power_iters, act,
              tile_of_expert, W, w_dtype, omega, U, sigma, V, codes, scales, zeros, ws=None,
              stream=None):
    """Offline packer on the device (tq_pack_proj): W (device [K][d_out][d_in]
    of w_dtype) and omega (device f64 [N*d_in][sketch]) in; U, sigma, V,
    codes, scales, zeros (caller-allocated device tensors) out.  Synchronous."""
    tiles = (ctypes.c_int32 * len(tile_of_expert))(*[int(t) for t in tile_of_expert])
    d = PackDesc(K, M, N, d_in, d_out, rank, group, bits, sketch, power_iters, act,
                 ctypes.cast(tiles, ctypes.POINTER(ctypes.c_int32)), _ptr(W), w_dtype, _ptr(omega),
                 _ptr(U), _ptr(sigma), _ptr(V), _ptr(codes), _ptr(scales), _ptr(zeros))
    n = ctypes.c_size_t()
    _check("tq_pack_workspace_size", lib().tq_pack_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    if ws is None:
        import torch
        ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device="cuda")
    _check("tq_pack_proj", lib().tq_pack_proj(ctypes.byref(d), _ptr(ws), ws.numel() * ws.element_size(),
                                              _stream(stream)))


class Layer:
    """An uploaded MoE layer (owns its device weights)."""

    def __init__(self, kind: int, act: int, d_model: int, d_ff: int, K: int):
        h = ctypes.c_void_p()
        _check("tq_layer_create", lib().tq_layer_create(kind, act, d_model, d_ff, K,
                                                        ctypes.byref(h)))
        self.h = h
        self.kind, self.act, self.d_model, self.d_ff, self.K = kind, act, d_model, d_ff, K

    def upload_proj(self, which, *, K, M, N, d_in, d_out, rank, group, tile_of_expert,
                    U, sigma, V, codes, scales, zeros, bits=2, sigma_dtype=TQ_F32, stream=None):
        """tile_of_expert: host sequence of K ints; the rest device tensors
        (sigma f32 or, with sigma_dtype=TQ_F16, f16)."""
        tiles = (ctypes.c_int32 * len(tile_of_expert))(*[int(t) for t in tile_of_expert])
        d = ProjDesc(K, M, N, d_in, d_out, rank, group, bits,
                     ctypes.cast(tiles, ctypes.POINTER(ctypes.c_int32)),
                     _ptr(U), _ptr(sigma), sigma_dtype, _ptr(V), _ptr(codes), _ptr(scales),
                     _ptr(zeros))
        _check("tq_upload_proj", lib().tq_upload_proj(self.h, which, ctypes.byref(d),
                                                      _stream(stream)))

    def upload_shared_expert(self, d_ff_shared, wg, wu, wd, stream=None):
        _check("tq_upload_shared_expert", lib().tq_upload_shared_expert(
            self.h, d_ff_shared, _ptr(wg), _ptr(wu), _ptr(wd), _stream(stream)))

    def set_path(self, path: int):
        _check("tq_layer_set_path", lib().tq_layer_set_path(self.h, path))

    def forward_path(self, T: int, topk: int) -> int:
        """1 (decode kernels) or 2 (prefill kernels): the path tq_forward takes."""
        p = ctypes.c_int32()
        _check("tq_forward_path", lib().tq_forward_path(self.h, T, topk, ctypes.byref(p)))
        return p.value

    def workspace_size(self, T: int, topk: int) -> int:
        n = ctypes.c_size_t()
        _check("tq_workspace_size", lib().tq_workspace_size(self.h, T, topk, ctypes.byref(n)))
        return n.value

    def forward(self, x, T, ids, gates, topk, y, y_dtype, ws, stream=None):
        _check("tq_forward", lib().tq_forward(self.h, _ptr(x), T, _ptr(ids), _ptr(gates), topk,
                                              _ptr(y), y_dtype, _ptr(ws),
                                              ws.numel() * ws.element_size(), _stream(stream)))

    def forward_from_logits(self, x, T, logits, topk, ids_out, gates_out, y, y_dtype, ws,
                            stream=None):
        """Top-k router on the logits, then the forward; the routing lands in
        ids_out / gates_out."""
        _check("tq_forward_from_logits", lib().tq_forward_from_logits(
            self.h, _ptr(x), T, _ptr(logits), topk, _ptr(ids_out), _ptr(gates_out), _ptr(y),
            y_dtype, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))

    def forward_noalloc(self, x, T, ids, gates, topk, y, y_dtype, stream=None):
        """tq_forward on the library's static scratch array (no workspace)."""
        _check("tq_forward_noalloc", lib().tq_forward_noalloc(
            self.h, _ptr(x), T, _ptr(ids), _ptr(gates), topk, _ptr(y), y_dtype, _stream(stream)))

    def debug_route(self, which, ids, T, topk, ws, cnt, off, perm, inv, col_off, col_tok,
                    slot2col, stream=None):
        _check("tq_debug_route", lib().tq_debug_route(
            self.h, which, _ptr(ids), T, topk, _ptr(ws), ws.numel() * ws.element_size(),
            _ptr(cnt), _ptr(off), _ptr(perm), _ptr(inv), _ptr(col_off), _ptr(col_tok),
            _ptr(slot2col), _stream(stream)))

    def debug_dequant(self, which, expert, w_out, stream=None):
        _check("tq_debug_dequant", lib().tq_debug_dequant(self.h, which, expert, _ptr(w_out),
                                                          _stream(stream)))

    def debug_row_bound(self, which):
        """Per-expert bound on the effective weight's row sums of |W| (numpy f32 [K])."""
        out = np.zeros(self.K, np.float32)
        _check("tq_debug_row_bound", lib().tq_debug_row_bound(
            self.h, which, out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def profile_enable(self, on: bool = True):
        _check("tq_profile_enable", lib().tq_profile_enable(self.h, 1 if on else 0))

    def profile_read(self):
        """Stage durations (ms) of the last profiled forward, keyed by STAGES."""
        ms = (ctypes.c_float * 8)()
        _check("tq_profile_read", lib().tq_profile_read(self.h, ms))
        return dict(zip(STAGES, list(ms)))

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib().tq_layer_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass
