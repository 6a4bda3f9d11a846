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
