"""The packer oracle against its pins, and planted mistakes in copies of it
(on the CPU), each of which must fail at least one pin."""
import importlib
import importlib.util
import os
import sys

import numpy as np
import pytest

from oracle import pack_ref
from tests import pins_pack

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", pins_pack.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(pack_ref)


def fresh():
    spec = importlib.util.spec_from_file_location(
        "oracle.pack_ref_mutant", os.path.join(ROOT, "oracle", "pack_ref.py"),
        submodule_search_locations=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    return mod


def m_unrounded_factors(P):
    """residual against the fp64 factors, not the stored ones"""
    P.stored_factors = lambda U, S, V, act: (np.asarray(U), np.asarray(S), np.asarray(V),
                                             np.asarray(S, np.float32))


def m_tile_transposed(P):
    orig = P.assemble_wbig

    def assemble_wbig(W, tiles, M, N):
        t = [(int(v) % N) * M + int(v) // N if M == N else int(v) for v in tiles]
        return orig(W, t, M, N)
    P.assemble_wbig = assemble_wbig


def m_rtn_no_zero_point(P):
    orig = P.quantize_rtn

    def quantize_rtn(w, group, bits):
        q, s, z = orig(w, group, bits)
        return np.clip(q - np.repeat(z.astype(np.int64), group, axis=1), 0, (1 << bits) - 1), s, \
            np.zeros_like(z)
    P.quantize_rtn = quantize_rtn


def m_rtn_truncate(P):
    orig_rint = np.rint

    def quantize_rtn(w, group, bits):
        qmax = (1 << bits) - 1
        w = np.asarray(w, np.float64)
        rows, d_in = w.shape
        wg = w.reshape(rows, d_in // group, group)
        mn = np.minimum(wg.min(axis=2), 0.0)
        mx = np.maximum(wg.max(axis=2), 0.0)
        s16 = P.tileq_ref.rnd_act((mx - mn) / qmax, "f16")
        s16 = np.where(s16 == 0, 1.0, s16)
        z = np.clip(orig_rint(-mn / s16), 0, qmax)
        q = np.clip(np.floor(wg / s16[..., None]) + z[..., None], 0, qmax)
        return q.reshape(rows, d_in).astype(np.int64), s16.astype(np.float16), z.astype(np.float16)
    P.quantize_rtn = quantize_rtn


def m_sigma_ascending(P):
    orig = P.sketch_svd

    def sketch_svd(Wbig, omega, rank, power_iters=0):
        U, S, V = orig(Wbig, omega, rank, power_iters)
        return U[:, ::-1], S[::-1], V[:, ::-1]
    P.sketch_svd = sketch_svd


def m_no_power_iterations(P):
    orig = P.range_finder
    P.range_finder = lambda Wbig, omega, power_iters=0: orig(Wbig, omega, 0)


def m_bit_string_msb(P):
    orig = P.pack_codes

    def pack_codes(q, bits):
        q = np.asarray(q)
        if bits == 3:
            q = ((q & 1) << 2) | (q & 2) | (q >> 2)
        return orig(q, bits)
    P.pack_codes = pack_codes


MUTANTS = [m_unrounded_factors, m_tile_transposed, m_rtn_no_zero_point, m_rtn_truncate,
           m_sigma_ascending, m_no_power_iterations, m_bit_string_msb]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_caught(mutant):
    P = fresh()
    mutant(P)
    caught = []
    for pin in pins_pack.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(P)
        except Exception as exc:  # noqa: BLE001 - any failure counts
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"{mutant.__name__} passed every pin"
