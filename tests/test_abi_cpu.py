"""The C-ABI library on the CPU (no GPU needed): it loads, exports every entry
point declared in include/tileq.h, and rejects invalid requests on the host
before any device work (pointers passed here are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_rank_post_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tileq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tq.LIB_PATH):
        pytest.skip("libtileq.so not built")
    return tq.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tq.EXPORTS)
    assert L.tq_abi_version() == 2


def status(fn, *args):
    return fn(*args)


def test_layer_create_validation(L):
    h = ctypes.c_void_p()
    assert L.tq_layer_create(7, 0, 256, 512, 8, ctypes.byref(h)) == 1
    assert L.tq_layer_create(0, 2, 256, 512, 8, ctypes.byref(h)) == 1
    assert L.tq_layer_create(0, 0, 0, 512, 8, ctypes.byref(h)) == 2
    assert L.tq_layer_create(0, 0, 256, 512, 300, ctypes.byref(h)) == 2
    assert b"K = 300" in L.tq_last_error()
    assert L.tq_layer_create(0, 0, 256, 512, 8, None) == 1
    assert L.tq_layer_create(0, 0, 256, 512, 8, ctypes.byref(h)) == 0
    assert L.tq_layer_destroy(h) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def desc(**kw):
    base = dict(K=8, M=2, N=4, d_in=256, d_out=512, rank=16, group=64, bits=2, sigma_dtype=2)
    base.update(kw)
    tiles = kw.pop("tiles", list(range(8)))
    base.pop("tiles", None)
    arr = (ctypes.c_int32 * len(tiles))(*tiles)
    d = tq.ProjDesc(base["K"], base["M"], base["N"], base["d_in"], base["d_out"],
                    base["rank"], base["group"], base["bits"],
                    ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)),
                    FAKE, FAKE, base["sigma_dtype"], FAKE, FAKE, FAKE, FAKE)
    d._keep = arr
    return d


@pytest.mark.parametrize("kw,code,text", [
    (dict(tiles=[0, 1, 2, 3, 4, 5, 6, 6]), 1, b"share tile 6"),     # not injective
    (dict(tiles=[0, 1, 2, 3, 4, 5, 6, 8]), 1, b"outside"),          # out of range
    (dict(tiles=[-1, 1, 2, 3, 4, 5, 6, 7]), 1, b"outside"),
    (dict(K=9), 2, b"K = 9"),                                        # layer has 8
    (dict(M=1, N=4), 2, b"K = 8 > M*N"),
    (dict(d_in=128), 2, b"must be 256 -> 512"),
    (dict(group=48), 2, b"group = 48"),
    (dict(group=512), 2, b"group = 512"),
    (dict(rank=-1), 2, b"rank"),
    (dict(rank=129), 2, b"rank"),
    (dict(N=40, M=1), 2, b"N = 40"),
    (dict(bits=4), 5, b"bits = 4"),
    (dict(sigma_dtype=1), 1, b"sigma_dtype"),                       # bf16 sigma
])
def test_upload_validation(L, kw, code, text):
    h = ctypes.c_void_p()
    assert L.tq_layer_create(0, 0, 256, 512, 8, ctypes.byref(h)) == 0
    try:
        d = desc(**kw)
        st = L.tq_upload_proj(h, 0, ctypes.byref(d), None)
        assert st == code, (st, L.tq_last_error())
        assert text in L.tq_last_error(), L.tq_last_error()
    finally:
        L.tq_layer_destroy(h)


def test_state_and_token_checks(L):
    h = ctypes.c_void_p()
    assert L.tq_layer_create(1, 0, 256, 512, 8, ctypes.byref(h)) == 0
    n = ctypes.c_size_t()
    assert L.tq_workspace_size(h, 4, 2, ctypes.byref(n)) == 6          # nothing uploaded
    assert L.tq_forward(h, FAKE, 4, FAKE, FAKE, 2, FAKE, 0, FAKE, 1 << 20, None) == 6
    assert L.tq_upload_proj(h, 3, ctypes.byref(desc()), None) == 1      # no 4th projection
    assert L.tq_upload_shared_expert(h, 100, FAKE, FAKE, FAKE, None) == 2
    assert L.tq_layer_set_path(h, 5) == 1
    assert L.tq_debug_dequant(h, 0, 0, FAKE, None) == 6
    assert L.tq_layer_destroy(h) == 0
    assert L.tq_layer_destroy(None) == 0


def test_forward_variants_validate_on_host(L):
    h = ctypes.c_void_p()
    assert L.tq_layer_create(0, 0, 256, 512, 8, ctypes.byref(h)) == 0
    n = ctypes.c_size_t()
    # nothing uploaded: both variants refuse before any device work
    assert L.tq_forward_from_logits(h, FAKE, 4, FAKE, 2, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20,
                                    None) == 6
    assert L.tq_forward_noalloc(h, FAKE, 4, FAKE, FAKE, 2, FAKE, 0, None) == 6
    assert L.tq_forward_path(h, 4, 2, ctypes.byref(ctypes.c_int32())) == 6
    assert L.tq_workspace_size(h, 4, 2, ctypes.byref(n)) == 6
    assert L.tq_layer_destroy(h) == 0


def pack_desc(**kw):
    base = dict(K=2, M=1, N=2, d_in=128, d_out=64, rank=4, group=32, bits=2, sketch=8,
                power_iters=0, act=tq.TQ_F16, w_dtype=tq.TQ_F32)
    tiles = kw.pop("tiles", [0, 1])
    base.update(kw)
    arr = (ctypes.c_int32 * len(tiles))(*tiles)
    d = tq.PackDesc(base["K"], base["M"], base["N"], base["d_in"], base["d_out"], base["rank"],
                    base["group"], base["bits"], base["sketch"], base["power_iters"], base["act"],
                    ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), FAKE, base["w_dtype"],
                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    d._keep = arr
    return d


@pytest.mark.parametrize("kw,code,text", [
    (dict(sketch=3), 2, b"sketch"),                       # fewer columns than the rank
    (dict(sketch=137), 2, b"sketch"),
    (dict(tiles=[1, 1]), 1, b"share tile"),
    (dict(tiles=[0, 2]), 1, b"out of range"),
    (dict(bits=4), 5, b"bits = 4"),
    (dict(bits=3, group=96, d_in=384), 5, b"power-of-two"),
    (dict(w_dtype=7), 1, b"w_dtype"),
    (dict(act=tq.TQ_F32), 1, b"act"),
    (dict(rank=129, sketch=136), 2, b"rank"),
    (dict(power_iters=17), 2, b"power_iters"),
    (dict(d_in=96), 2, b"d_in"),
    (dict(K=3), 2, b"grid"),
])
def test_pack_validation(L, kw, code, text):
    n = ctypes.c_size_t()
    d = pack_desc(**kw)
    assert L.tq_pack_workspace_size(ctypes.byref(d), ctypes.byref(n)) == code, L.tq_last_error()
    assert text in L.tq_last_error(), L.tq_last_error()
    assert L.tq_pack_proj(ctypes.byref(d), FAKE, 1 << 30, None) == code


def test_pack_workspace_grows_with_sketch(L):
    n8, n64 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.tq_pack_workspace_size(ctypes.byref(pack_desc()), ctypes.byref(n8)) == 0
    assert L.tq_pack_workspace_size(ctypes.byref(pack_desc(sketch=64)), ctypes.byref(n64)) == 0
    assert 0 < n8.value < n64.value
    # a workspace smaller than the size asked for is refused before device work
    assert L.tq_pack_proj(ctypes.byref(pack_desc()), FAKE, n8.value - 1, None) == 2


@pytest.mark.parametrize("T,K,k,code", [(-1, 8, 2, 2), (4, 0, 1, 2), (4, 257, 2, 2),
                                        (4, 8, 0, 2), (4, 8, 9, 2), (4, 64, 33, 2),
                                        (0, 8, 2, 0)])
def test_router_validation(L, T, K, k, code):
    assert L.tq_router_topk(FAKE, T, K, k, FAKE, FAKE, None) == code, L.tq_last_error()


def test_calibrate_read_validation(L):
    scratch = ctypes.c_void_p(0x2000)
    assert L.tq_calibrate_read(None, 64, scratch, None) == 1
    assert L.tq_calibrate_read(FAKE, 64, None, None) == 1
    assert L.tq_calibrate_read(ctypes.c_void_p(0x1008), 64, scratch, None) == 1
    assert L.tq_calibrate_read(FAKE, 60, scratch, None) == 1
    assert b"multiples of 16" in L.tq_last_error()
