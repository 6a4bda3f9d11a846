"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
that each one fails at least one pin from tests/pins.py.  This shows the pins
constrain every part of the oracle: unpacking, the residual, the factor
blocks, the tile map, gating, SwiGLU, rounding and the routing lists."""
import importlib.util
import os

import numpy as np
import pytest

from tests import pins

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "oracle", "tileq_ref.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("tileq_ref_mutant", ORACLE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_zero_sign(r):
    def residual(q, s, z, G):
        s = np.repeat(np.asarray(s, np.float16).astype(np.float64), G, axis=-1)
        z = np.repeat(np.asarray(z, np.float16).astype(np.float64), G, axis=-1)
        return s * (q + z)
    r.residual = residual


def m_group_index(r):
    def residual(q, s, z, G):
        ng = q.shape[-1] // G
        s = np.tile(np.asarray(s, np.float16).astype(np.float64), (1,) * (q.ndim - 1) + (G,))
        z = np.tile(np.asarray(z, np.float16).astype(np.float64), (1,) * (q.ndim - 1) + (G,))
        return s[..., :ng * G] * (q - z[..., :ng * G])
    r.residual = residual


def m_bit_order(r):
    def unpack_codes(codes, d_in):
        codes = np.asarray(codes, dtype=np.uint32)
        sh = (15 - np.arange(16, dtype=np.uint32)) * np.uint32(2)
        q = (codes[..., None] >> sh) & np.uint32(3)
        return q.reshape(codes.shape[:-1] + (d_in,)).astype(np.int64)
    r.unpack_codes = unpack_codes


def m_drop_sigma(r):
    orig = r.lowrank_block

    def lowrank_block(proj, m, n):
        p = dict(proj)
        p["sigma"] = np.ones_like(np.asarray(proj["sigma"]))
        return orig(p, m, n)
    r.lowrank_block = lowrank_block


def m_swap_mn(r):
    orig = r.lowrank_block
    r.lowrank_block = lambda proj, m, n: orig(proj, n % proj["M"], m % proj["N"])


def m_tile_stride(r):
    r.tile_coords = lambda tile, N: (int(tile) % N, int(tile) // N)


def m_wrong_expert_residual(r):
    orig = r.expert_residual
    r.expert_residual = lambda proj, e: orig(proj, (e + 1) % proj["K"])


def m_ignore_gates(r):
    orig = r.forward_single
    r.forward_single = lambda p, x, ids, g, tokens=None: orig(
        p, x, ids, np.ones_like(np.asarray(g, np.float64)), tokens)


def m_swiglu_swap(r):
    def swiglu_expert(layer, e, X, cache):
        pg, pu = layer["proj"]["gate"], layer["proj"]["up"]
        a = X @ cache.get("gate", pg, e).T
        b = X @ cache.get("up", pu, e).T
        return r.rnd_act(r.silu(b) * a, layer["act"])
    r.swiglu_expert = swiglu_expert


def m_silu_sign(r):
    r.silu = lambda v: np.asarray(v, np.float64) / (1.0 + np.exp(np.asarray(v, np.float64)))


def m_rnd_truncate(r):
    orig = r.rnd_act

    def rnd_act(v, act):
        if act == "f32":
            return orig(v, act)
        bits = 11 if act == "f16" else 8
        v = np.asarray(v, np.float64)
        m, e = np.frexp(v)
        return np.ldexp(np.trunc(np.ldexp(m, bits)), e - bits)
    r.rnd_act = rnd_act


def m_route_unstable(r):
    orig = r.route

    def route(ids, K, n_of=None):
        res = orig(ids, K, n_of)
        perm = res["perm"].copy()
        for e in range(K):
            a, b = res["off"][e], res["off"][e + 1]
            perm[a:b] = perm[a:b][::-1]
        res["perm"] = perm
        return res
    r.route = route


def m_transposed_down(r):
    orig = r.expert_weight

    def expert_weight(proj, e):
        W = orig(proj, e)
        return W.T if W.shape[0] == W.shape[1] else W
    r.expert_weight = expert_weight


def m_deq_double_round(r):
    def deq_canonical(q, s, z, G, out="f16"):
        s = np.repeat(np.asarray(s, np.float16), G, axis=-1)
        z = np.repeat(np.asarray(z, np.float16), G, axis=-1)
        w16 = ((q.astype(np.float16) - z) * s).astype(np.float16)
        return r.rnd_act(w16.astype(np.float64), out)
    r.deq_canonical = deq_canonical


def m_router_ties_high(r):
    orig = r.router_topk

    def router_topk(logits, k):
        L = np.asarray(logits, np.float64)
        flipped = L[:, ::-1]                       # ties now go to the higher id
        ids, w = orig(flipped, k)
        return (L.shape[1] - 1 - ids).astype(np.int32), w
    r.router_topk = router_topk


def m_router_softmax_all(r):
    orig = r.router_topk

    def router_topk(logits, k):
        ids, _ = orig(logits, k)
        L = np.asarray(logits, np.float64)
        ex = np.exp(L - L.max(axis=1, keepdims=True))
        w = ex / ex.sum(axis=1, keepdims=True)     # not renormalised over the k
        return ids, np.take_along_axis(w, ids, axis=1)
    r.router_topk = router_topk


def m_deq_round_zero(r):
    orig = r.deq_canonical
    r.deq_canonical = lambda q, s, z, G, out="f16": orig(q, s, np.rint(np.asarray(z, np.float16)), G, out)


def m_subset_sorted(r):
    """token subsets answered in ascending token order, not the order asked"""
    fs, fw = r.forward_single, r.forward_swiglu
    r.forward_single = lambda p, x, ids, g, tokens=None: fs(
        p, x, ids, g, None if tokens is None else np.sort(tokens))
    r.forward_swiglu = lambda layer, x, ids, g, tokens=None, keep_weights=True: fw(
        layer, x, ids, g, None if tokens is None else np.sort(tokens), keep_weights)


def m_bit_order3(r):
    """3-bit codes read most significant bit first"""
    orig = r.unpack_codes

    def unpack_codes(codes, d_in, bits=2):
        q = orig(codes, d_in, bits)
        if bits == 3:
            q = ((q & 1) << 2) | (q & 2) | (q >> 2)
        return q
    r.unpack_codes = unpack_codes


def m_bits_ignored(r):
    """every projection read as 2-bit codes"""
    orig = r.unpack_codes
    r.unpack_codes = lambda codes, d_in, bits=2: orig(np.asarray(codes)[..., :d_in // 16], d_in, 2)


MUTANTS = [m_zero_sign, m_group_index, m_bit_order, m_drop_sigma, m_swap_mn,
           m_tile_stride, m_wrong_expert_residual, m_ignore_gates, m_swiglu_swap,
           m_silu_sign, m_rnd_truncate, m_route_unstable, m_transposed_down,
           m_deq_double_round, m_router_ties_high, m_router_softmax_all, m_deq_round_zero,
           m_subset_sorted, m_bit_order3, m_bits_ignored]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_caught(mutant):
    r = fresh_oracle()
    mutant(r)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(r)
        except Exception as exc:  # noqa: BLE001 - any failure counts
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"{mutant.__name__} passed every pin"
