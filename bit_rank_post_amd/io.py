"""Marshalling helpers: host arrays (the stored format of a layer) to device
tensors and uploads through the C ABI.  No arithmetic of the method here."""
from __future__ import annotations

import numpy as np
import torch

from . import TQ_BF16, TQ_F16, TQ_F32, TQ_SINGLE, TQ_SWIGLU, Layer

ACT = {"f16": TQ_F16, "bf16": TQ_BF16}
PROJ_INDEX = {"single": 0, "gate": 0, "up": 1, "down": 2}


def to_device(a: np.ndarray, act: str | None = None, device="cuda"):
    """Copy a host array to the GPU.  bf16 data (uint16 bit patterns) becomes a
    torch.bfloat16 tensor; uint32/uint16 become int32/int16 views."""
    a = np.ascontiguousarray(a)
    if act == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def upload_proj(L: Layer, which: int, p: dict, stream=None):
    """sigma goes up as stored: float16 arrays as TQ_F16, anything else as f32."""
    act = p["act"]
    sig = np.asarray(p["sigma"])
    sig16 = sig.dtype == np.float16
    sig = sig if sig16 else sig.astype(np.float32)
    dev = dict(U=to_device(p["U"], act) if p["rank"] else None,
               V=to_device(p["V"], act) if p["rank"] else None,
               sigma=to_device(sig.view(np.uint16) if sig16 else sig) if p["rank"] else None,
               codes=to_device(p["codes"]),
               scales=to_device(p["scales"].view(np.uint16)),
               zeros=to_device(p["zeros"].view(np.uint16)))
    L.upload_proj(which, K=p["K"], M=p["M"], N=p["N"], d_in=p["d_in"], d_out=p["d_out"],
                  rank=p["rank"], group=p["group"], tile_of_expert=p["tile_of_expert"],
                  bits=p.get("bits", 2), sigma_dtype=TQ_F16 if sig16 else TQ_F32,
                  stream=stream, **dev)


def upload_layer(layer: dict, stream=None) -> Layer:
    """Upload a layer dict {kind, act, K, d_model, d_ff, proj: {...}, shared}."""
    kind = TQ_SINGLE if layer["kind"] == "single" else TQ_SWIGLU
    L = Layer(kind, ACT[layer["act"]], layer["d_model"], layer["d_ff"], layer["K"])
    for name, p in layer["proj"].items():
        upload_proj(L, PROJ_INDEX[name], p, stream)
    sh = layer.get("shared")
    if sh is not None:
        L.upload_shared_expert(sh["d_ff"], to_device(sh["wg"]), to_device(sh["wu"]),
                               to_device(sh["wd"]), stream)
    return L


def tokens_to_device(x, ids, gates, act):
    return (to_device(x, act), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(gates, np.float32)).cuda())


def workspace(L: Layer, T: int, topk: int):
    n = L.workspace_size(T, topk)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")


W_DTYPES = {np.dtype(np.float16): 0, np.dtype(np.float32): 2, np.dtype(np.float64): 3}


def pack_proj(W: np.ndarray, tiles, M: int, N: int, rank: int, group: int, bits: int,
              omega: np.ndarray, act: str = "f16", power_iters: int = 0, w_bf16: bool = False):
    """Pack dense expert weights W [K][d_out][d_in] (float16/32/64, or bf16 bit
    patterns as uint16 with w_bf16) on the device; returns the projection in
    the upload format (host arrays, as synth.make_proj lays them out)."""
    from . import TQ_F16, TQ_BF16, pack_proj as _pack
    K, d_out, d_in = W.shape
    wdt = 1 if w_bf16 else W_DTYPES[np.asarray(W).dtype]
    Wd = torch.from_numpy(np.ascontiguousarray(W).view(np.int16) if w_bf16 else np.ascontiguousarray(W)).cuda()
    od = torch.from_numpy(np.ascontiguousarray(omega, np.float64)).cuda()
    r = max(rank, 1)
    dev = dict(U=torch.zeros((M * d_out, r), dtype=torch.int16, device="cuda"),
               sigma=torch.zeros(r, dtype=torch.float32, device="cuda"),
               V=torch.zeros((N * d_in, r), dtype=torch.int16, device="cuda"),
               codes=torch.zeros((K, d_out, bits * d_in // 32), dtype=torch.int32, device="cuda"),
               scales=torch.zeros((K, d_out, d_in // group), dtype=torch.int16, device="cuda"),
               zeros=torch.zeros((K, d_out, d_in // group), dtype=torch.int16, device="cuda"))
    _pack(K=K, M=M, N=N, d_in=d_in, d_out=d_out, rank=rank, group=group, bits=bits,
          sketch=omega.shape[1], power_iters=power_iters, act=TQ_BF16 if act == "bf16" else TQ_F16,
          tile_of_expert=tiles, W=Wd, w_dtype=wdt, omega=od, **dev)
    h = {k: v.cpu().numpy() for k, v in dev.items()}
    U = h["U"][:, :rank].view(np.uint16)
    V = h["V"][:, :rank].view(np.uint16)
    if act == "f16":
        U, V = U.view(np.float16), V.view(np.float16)
    return dict(K=K, M=M, N=N, d_in=d_in, d_out=d_out, rank=rank, group=group, bits=bits, act=act,
                tile_of_expert=np.asarray(tiles, np.int32), U=np.ascontiguousarray(U),
                sigma=h["sigma"][:rank].copy(), V=np.ascontiguousarray(V),
                codes=h["codes"].view(np.uint32), scales=h["scales"].view(np.float16),
                zeros=h["zeros"].view(np.float16))
