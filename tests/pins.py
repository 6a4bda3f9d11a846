"""Pins of the CPU oracle to facts outside itself.

Each pin takes the oracle module as an argument and raises AssertionError when
the oracle disagrees with a closed form, an invariant, a hand-derived fixture
(tests/golden/) or an independent implementation (numpy's own float16
conversion, torch's bfloat16 conversion, the pure-Python scalar oracle).
test_oracle_pins.py runs them on the real oracle; test_oracle_mutants.py runs
them on copies with planted mistakes and requires that each mistake fails at
least one pin.

Passages followed ("TileQ: Efficient Low-Rank Quantization of
Mixture-of-Experts with 2D Tiling", gist.science technical summary):
  section 2.1 step 4 (experts placed as tiles of W_big), step 5 (global
  low-rank U, Sigma, V plus per-expert quantized residual), "Key Technical
  Insight" (row -> left/output basis, column -> right/input basis), section 2.2
  (batch input, routing weights, in-place rank-space accumulation), section 4
  "Memory Efficiency" (8x fewer extra parameters for 64 experts).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# ----------------------------------------------------------------------------
# builders (test side, independent of the oracle)


def f64(a, act):
    return synth.act_as_f32(np.asarray(a), act).astype(np.float64)


def proj_from(q, s, z, U, sigma, V, tiles, M, N, G, act="f16", bits=2):
    K, d_out, d_in = q.shape
    return dict(K=K, M=M, N=N, d_in=d_in, d_out=d_out, rank=U.shape[1],
                group=G, bits=bits, act=act, tile_of_expert=np.asarray(tiles, np.int32),
                U=U, sigma=np.asarray(sigma, np.float32), V=V,
                codes=synth.pack_codes(q, bits), scales=np.asarray(s, np.float16),
                zeros=np.asarray(z, np.float16))


def random_struct(K, M, N, d_in, d_out, rank, G, seed, act="f16", zero_res=False, bits=2):
    """A projection with random codes, scales, zero points, factors and map.
    Returns (proj, q) where q are the codes before packing."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 1 << bits, (K, d_out, d_in))
    z = rng.integers(0, 1 << bits, (K, d_out, d_in // G)).astype(np.float16)
    s = rng.uniform(0.01, 0.1, (K, d_out, d_in // G)).astype(np.float16)
    if zero_res:
        q = np.repeat(z.astype(np.int64), G, axis=-1)
    U = synth.to_act((rng.standard_normal((M * d_out, rank)) / np.sqrt(d_out)).astype(np.float32), act)
    V = synth.to_act((rng.standard_normal((N * d_in, rank)) / np.sqrt(d_in)).astype(np.float32), act)
    sigma = np.sort(rng.uniform(0.1, 10.0, rank))[::-1].astype(np.float16).astype(np.float32)
    tiles = rng.permutation(M * N)[:K]
    return proj_from(q, s, z, U, sigma, V, tiles, M, N, G, act, bits), q


def residual_from_q(q, s, z, G):
    """Test-side residual from the codes *before* packing."""
    sf = np.repeat(np.asarray(s, np.float64), G, axis=-1)
    zf = np.repeat(np.asarray(z, np.float64), G, axis=-1)
    return sf * (q - zf)


def tokens(d, K, k, T, seed, act="f16"):
    x, ids, g = synth.make_custom_tokens(d, K, k, T, act, seed)
    return x, ids, g


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))

# ----------------------------------------------------------------------------
# formats


def pin_unpack_golden(ref):
    with open(os.path.join(GOLDEN, "unpack_codes.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            w, codes = line.split(":")
            want = [int(c) for c in codes.split()]
            got = ref.unpack_codes(np.array([int(w, 16)], np.uint32), 16)
            assert list(got) == want, (w, list(got), want)


def pin_unpack_bytes(ref):
    """Exhaustive over the 256 byte values: a word is 4 bytes (little endian),
    byte b of the word holds codes 4b..4b+3 at bits 2*(i % 4)."""
    for pos in range(4):
        b = np.arange(256, dtype=np.uint32)
        words = b << np.uint32(8 * pos)
        q = ref.unpack_codes(words[:, None], 16)
        for c in range(4):
            want = (np.arange(256) >> (2 * c)) & 3
            assert np.array_equal(q[:, 4 * pos + c], want)
        others = [i for i in range(16) if i // 4 != pos]
        assert not q[:, others].any()
    rng = np.random.default_rng(7)
    q0 = rng.integers(0, 4, (5, 96))
    assert np.array_equal(ref.unpack_codes(synth.pack_codes(q0), 96), q0)


def pin_unpack3_golden(ref):
    with open(os.path.join(GOLDEN, "unpack_codes3.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            words, codes = line.split(":")
            w = np.array([int(x, 16) for x in words.split()], np.uint32)
            want = [0] * 32
            for kv in codes.split():
                i, v = kv.split("=")
                want[int(i)] = int(v)
            got = ref.unpack_codes(w[None, :], 32, 3)[0]
            assert list(got) == want, (words, list(got), want)


def pin_unpack3_bytes(ref):
    """Every byte value at every byte position of a three-word group, against
    a scalar read of the bit string (code i = sum_j bit(3i + j) 2^j), and the
    generator's packing round trip."""
    for pos in range(12):
        b = np.arange(256, dtype=np.uint32)
        words = np.zeros((256, 3), np.uint32)
        words[:, pos // 4] = b << np.uint32(8 * (pos % 4))
        q = ref.unpack_codes(words, 32, 3)
        for v in range(256):
            w = [int(x) for x in words[v]]
            for i in range(32):
                want = sum(((w[(3 * i + j) // 32] >> ((3 * i + j) % 32)) & 1) << j for j in range(3))
                assert q[v, i] == want, (pos, v, i)
    rng = np.random.default_rng(8)
    q0 = rng.integers(0, 8, (5, 96))
    assert np.array_equal(ref.unpack_codes(synth.pack_codes(q0, 3), 96, 3), q0)


def pin_p2_zero_rank_3bit(ref):
    """3-bit residual, rank 0: y_t = sum_j g R_e x_t from the codes before
    packing; and the closed form x = ones, q = 7, z = 2 -> y_o = 5 sum_g s[o,g] G."""
    rng = np.random.default_rng(24)
    K, d_out, d_in, G = 4, 16, 64, 32
    q = rng.integers(0, 8, (K, d_out, d_in))
    s = rng.uniform(0.01, 0.1, (K, d_out, d_in // G)).astype(np.float16)
    z = rng.integers(0, 8, (K, d_out, d_in // G)).astype(np.float16)
    p = proj_from(q, s, z, np.zeros((2 * d_out, 0), np.float16), [], np.zeros((2 * d_in, 0), np.float16),
                  [0, 1, 2, 3], 2, 2, G, bits=3)
    x, ids, g = tokens(d_in, K, 2, 7, seed=25)
    y = ref.forward_single(p, x, ids, g)
    R = residual_from_q(q, s, z, G)
    want = np.zeros_like(y)
    for t in range(7):
        for j in range(2):
            want[t] += g[t, j] * (R[ids[t, j]] @ x[t].astype(np.float64))
    assert rel_err(y, want) < 1e-12
    p7 = proj_from(np.full(q.shape, 7), s, np.full(z.shape, 2, np.float16), p["U"], [], p["V"],
                   [0, 1, 2, 3], 2, 2, G, bits=3)
    y7 = ref.forward_single(p7, np.ones((1, d_in), np.float16), np.array([[1]]),
                            np.array([[1.0]], np.float32))
    assert rel_err(y7[0], 5.0 * s[1].astype(np.float64).sum(axis=1) * G) < 1e-12


def _golden_residual():
    d = {}
    deq = []
    with open(os.path.join(GOLDEN, "residual_dequant.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "deq":
                deq.append({kv.split("=")[0]: float(kv.split("=")[1]) for kv in parts[1:]})
            else:
                d[parts[0]] = [float(v) for v in parts[1:]]
    return d, deq


def pin_residual_golden(ref):
    d, _ = _golden_residual()
    G = int(d["group"][0])
    q = np.array([d["q"]], np.int64)
    s = np.array([d["s"]], np.float16)
    z = np.array([d["z"]], np.float16)
    got = ref.residual(q, s, z, G)
    assert np.array_equal(got[0], np.array(d["R"])), got


def pin_deq_golden(ref):
    _, deq = _golden_residual()
    for c in deq:
        q = np.array([[int(c["q"])]])
        s = np.array([[c["s"]]], np.float16)
        z = np.array([[c["z"]]], np.float16)
        assert float(ref.deq_canonical(q, s, z, 1, "f16")[0, 0]) == c["f16"], c
        assert float(ref.deq_canonical(q, s, z, 1, "bf16")[0, 0]) == c["bf16"], c


def pin_rnd_f16_vs_numpy(ref):
    """rnd_act(., f16) against numpy's own double->half conversion."""
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000),
        np.array([65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.0]),
    ])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).astype(np.float64)
    got = ref.rnd_act(v, "f16")
    assert np.array_equal(got, want), v[got != want][:5]


def pin_rnd_bf16(ref):
    """Hand cases (ties to even, overflow) and torch's float->bfloat16."""
    cases = {1.0 + 2.0 ** -8: 1.0, 1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,
             1.0 + 2.0 ** -8 + 2.0 ** -30: 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -8): -1.0,
             3.4e38: math.inf, 0.0: 0.0}
    for v, want in cases.items():
        assert float(ref.rnd_act(np.array([v]), "bf16")[0]) == want, v
    rng = np.random.default_rng(12)
    v32 = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)).astype(np.float32)
    want = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    got = ref.rnd_act(v32.astype(np.float64), "bf16")
    assert np.array_equal(got, want)


def pin_silu(ref):
    v = np.array([0.0, 1.0, -1.0, 2.0, 50.0, -800.0])
    got = ref.silu(v)
    want = [0.0, 0.7310585786300049, -0.2689414213699951, 1.7615941559557646,
            50.0, 0.0]
    assert np.allclose(got, want, rtol=1e-15, atol=0), got
    x = np.linspace(-20, 20, 101)
    assert np.allclose(ref.silu(x) - ref.silu(-x), x, rtol=0, atol=1e-13)

# ----------------------------------------------------------------------------
# weights and forward


def pin_p1_factored_block(ref):
    """Block (m, n) of W_big (explicit) = factored U_m Sigma (V_n^T x)."""
    for act in ("f16", "bf16"):
        p, _ = random_struct(6, 2, 3, 32, 48, 8, 16, seed=21, act=act)
        W = ref.wbig(p)
        assert W.shape == (2 * 48, 3 * 32)
        U, V, sig = f64(p["U"], act), f64(p["V"], act), p["sigma"].astype(np.float64)
        x = np.random.default_rng(3).standard_normal(32)
        for m in range(2):
            for n in range(3):
                Um, Vn = U[m * 48:(m + 1) * 48], V[n * 32:(n + 1) * 32]
                fact = Um @ (sig * (Vn.T @ x))
                blk = ref.lowrank_block(p, m, n)
                assert rel_err(blk @ x, fact) < 1e-12
                assert rel_err(W[m * 48:(m + 1) * 48, n * 32:(n + 1) * 32], blk) < 1e-12


def pin_p2_zero_rank(ref):
    """rank 0: y_t = sum_j g R_e x_t with R from the codes before packing."""
    p, q = random_struct(5, 2, 3, 64, 32, 0, 32, seed=22)
    x, ids, g = tokens(64, 5, 2, 9, seed=23)
    y = ref.forward_single(p, x, ids, g)
    R = residual_from_q(q, p["scales"], p["zeros"], 32)
    X = x.astype(np.float64)
    want = np.zeros_like(y)
    for t in range(9):
        for j in range(2):
            want[t] += g[t, j] * (R[ids[t, j]] @ X[t])
    assert rel_err(y, want) < 1e-12
    # closed form: x = ones, q = 2, z = 1 everywhere -> y_o = sum_g s[o,g] * G
    qq = np.full(q.shape, 2)
    zz = np.ones(p["zeros"].shape, np.float16)
    p1 = proj_from(qq, p["scales"], zz, p["U"], p["sigma"], p["V"],
                   p["tile_of_expert"], 2, 3, 32)
    ones = np.ones((1, 64), np.float16)
    y1 = ref.forward_single(p1, ones, np.array([[4]]), np.array([[1.0]], np.float32))
    want1 = p["scales"][4].astype(np.float64).sum(axis=1) * 32
    assert rel_err(y1[0], want1) < 1e-12


def pin_p3_zero_residual(ref):
    """q = z: pure low rank, y_t = sum_m U_m Sigma (sum_{j: m_j = m} g V_{n_j}^T x)
    -- the rank-space accumulation of section 2.2 against the explicit blocks."""
    for act in ("f16", "bf16"):
        p, _ = random_struct(7, 2, 4, 48, 32, 6, 16, seed=24, act=act, zero_res=True)
        x, ids, g = tokens(48, 7, 3, 11, seed=25, act=act)
        y = ref.forward_single(p, x, ids, g)
        U, V, sig = f64(p["U"], act), f64(p["V"], act), p["sigma"].astype(np.float64)
        X = f64(x, act)
        want = np.zeros_like(y)
        for t in range(11):
            S = np.zeros((2, 6))
            for j in range(3):
                m, n = divmod(int(p["tile_of_expert"][ids[t, j]]), 4)
                S[m] += g[t, j] * sig * (V[n * 48:(n + 1) * 48].T @ X[t])
            for m in range(2):
                want[t] += U[m * 32:(m + 1) * 32] @ S[m]
        assert rel_err(y, want) < 1e-12


def pin_p4_token_perm(ref):
    p, _ = random_struct(6, 2, 3, 32, 32, 4, 16, seed=26)
    x, ids, g = tokens(32, 6, 2, 13, seed=27)
    y = ref.forward_single(p, x, ids, g)
    pi = np.random.default_rng(5).permutation(13)
    y2 = ref.forward_single(p, x[pi], ids[pi], g[pi])
    assert rel_err(y2, y[pi]) < 1e-12


def pin_p5_slots(ref):
    """Slot order within a token does not matter; [e, e] with g1, g2 equals
    [e] with g1 + g2."""
    p, _ = random_struct(6, 2, 3, 32, 32, 4, 16, seed=28)
    x, ids, g = tokens(32, 6, 3, 7, seed=29)
    y = ref.forward_single(p, x, ids, g)
    y2 = ref.forward_single(p, x, ids[:, ::-1].copy(), g[:, ::-1].copy())
    assert rel_err(y2, y) < 1e-12
    dup = np.stack([ids[:, 0], ids[:, 0]], axis=1)
    gd = np.stack([g[:, 0], g[:, 1]], axis=1)
    y3 = ref.forward_single(p, x, dup, gd)
    g64 = g.astype(np.float64)
    y4 = ref.forward_single(p, x, ids[:, :1].copy(), (g64[:, 0] + g64[:, 1])[:, None])
    assert rel_err(y3, y4) < 1e-12


def pin_p6_textbook(ref):
    """K = M = N = 1, k = 1, g = 1: y = (U Sigma V^T + R) x."""
    p, q = random_struct(1, 1, 1, 64, 48, 5, 32, seed=30)
    x, _, _ = tokens(64, 1, 1, 4, seed=31)
    y = ref.forward_single(p, x, np.zeros((4, 1), np.int32), np.ones((4, 1), np.float32))
    U, V = f64(p["U"], "f16"), f64(p["V"], "f16")
    W = U @ np.diag(p["sigma"].astype(np.float64)) @ V.T
    W = W + residual_from_q(q, p["scales"], p["zeros"], 32)[0]
    assert rel_err(y, x.astype(np.float64) @ W.T) < 1e-12


def pin_p7_grid_relabel(ref):
    """Permuting grid rows (with the U blocks) and columns (with the V blocks)
    consistently with the map leaves y unchanged."""
    M, N, d_in, d_out = 3, 2, 32, 16
    p, _ = random_struct(5, M, N, d_in, d_out, 4, 16, seed=32)
    x, ids, g = tokens(d_in, 5, 2, 6, seed=33)
    y = ref.forward_single(p, x, ids, g)
    rp = np.array([2, 0, 1])
    cp = np.array([1, 0])
    q = p.copy()
    U = p["U"].reshape(M, d_out, -1)
    V = p["V"].reshape(N, d_in, -1)
    U2 = np.empty_like(U)
    V2 = np.empty_like(V)
    U2[rp] = U
    V2[cp] = V
    q["U"] = U2.reshape(M * d_out, -1)
    q["V"] = V2.reshape(N * d_in, -1)
    m, n = np.divmod(p["tile_of_expert"], N)
    q["tile_of_expert"] = (rp[m] * N + cp[n]).astype(np.int32)
    assert rel_err(ref.forward_single(q, x, ids, g), y) < 1e-12


def pin_p8_linearity(ref):
    p, _ = random_struct(6, 2, 3, 32, 32, 4, 16, seed=34)
    x, ids, g = tokens(32, 6, 3, 7, seed=35)
    y = ref.forward_single(p, x, ids, g)
    assert rel_err(ref.forward_single(p, x, ids, 2.5 * g.astype(np.float64)), 2.5 * y) < 1e-12
    parts = sum(ref.forward_single(p, x, ids[:, j:j + 1].copy(), g[:, j:j + 1].copy())
                for j in range(3))
    assert rel_err(parts, y) < 1e-12


def pin_dropped_ids(ref):
    """An id outside [0, K) contributes nothing."""
    p, _ = random_struct(6, 2, 3, 32, 32, 4, 16, seed=36)
    x, ids, g = tokens(32, 6, 2, 5, seed=37)
    bad = ids.copy()
    bad[1, 0] = 6
    bad[3, 1] = -1
    g0 = g.copy()
    g0[1, 0] = 0
    g0[3, 1] = 0
    assert rel_err(ref.forward_single(p, x, bad, g), ref.forward_single(p, x, ids, g0)) < 1e-12


def _tiny_lists(p, act):
    return dict(K=p["K"], M=p["M"], N=p["N"], d_in=p["d_in"], d_out=p["d_out"],
                rank=p["rank"], G=p["group"], bits=p.get("bits", 2),
                tile=[int(v) for v in p["tile_of_expert"]],
                U=f64(p["U"], act).tolist(), V=f64(p["V"], act).tolist(),
                sigma=[float(v) for v in p["sigma"]],
                codes=p["codes"].tolist(), s=p["scales"].astype(np.float64).tolist(),
                z=p["zeros"].astype(np.float64).tolist())


def pin_p11_two_oracles(ref):
    """numpy fp64 oracle vs the pure-Python scalar oracle (rel <= 1e-12)."""
    from oracle import tiny_ref
    for act in ("f16", "bf16"):
        p, _ = random_struct(4, 2, 2, 32, 16, 3, 16, seed=38, act=act)
        x, ids, g = tokens(32, 4, 2, 3, seed=39, act=act)
        y = ref.forward_single(p, x, ids, g)
        yt = tiny_ref.forward_single(_tiny_lists(p, act), f64(x, act).tolist(),
                                     ids.tolist(), g.astype(np.float64).tolist())
        assert rel_err(y, np.array(yt)) < 1e-12
    # 3-bit residual codes
    p, _ = random_struct(4, 2, 2, 64, 16, 3, 32, seed=46, bits=3)
    x, ids, g = tokens(64, 4, 2, 3, seed=47)
    y = ref.forward_single(p, x, ids, g)
    yt = tiny_ref.forward_single(_tiny_lists(p, "f16"), f64(x, "f16").tolist(),
                                 ids.tolist(), g.astype(np.float64).tolist())
    assert rel_err(y, np.array(yt)) < 1e-12
    # SwiGLU
    act = "f16"
    pg, _ = random_struct(4, 2, 2, 32, 16, 3, 16, seed=40)
    pu, _ = random_struct(4, 2, 2, 32, 16, 3, 16, seed=41)
    pd, _ = random_struct(4, 2, 2, 16, 32, 3, 16, seed=42)
    layer = dict(kind="swiglu", act=act, K=4, d_model=32, d_ff=16,
                 proj=dict(gate=pg, up=pu, down=pd), shared=None)
    x, ids, g = tokens(32, 4, 2, 3, seed=43)
    y = ref.forward_swiglu(layer, x, ids, g)
    rnd = lambda v: float(np.float16(v))
    yt = tiny_ref.forward_swiglu(_tiny_lists(pg, act), _tiny_lists(pu, act),
                                 _tiny_lists(pd, act), f64(x, act).tolist(),
                                 ids.tolist(), g.astype(np.float64).tolist(), rnd)
    assert rel_err(y, np.array(yt)) < 1e-12


def pin_p12_storage(ref):
    """Section 4 (memory efficiency): 64 experts on 8 x 8 with d_in = d_out
    need ~8x fewer low-rank parameters than per-expert factors."""
    p, _ = random_struct(64, 8, 8, 32, 32, 2, 16, seed=44)
    sh, pe = ref.storage_params(p)
    assert pe == 64 * 2 * (32 + 32)
    assert sh == 2 * (8 * 32 + 8 * 32) + 2
    assert abs(pe / sh - 8.0) < 0.02


def pin_token_subset(ref):
    """forward(tokens=t) equals rows t of the whole-batch forward (the sampled
    full-size checks rest on it): single projection and SwiGLU with a shared
    expert, subsets in any order, with repeats and dropped ids."""
    p, _ = random_struct(6, 2, 3, 32, 48, 4, 16, seed=61)
    x, ids, g = tokens(32, 6, 2, 17, seed=62)
    ids = ids.copy()
    ids[4, 1] = 9
    full = ref.forward_single(p, x, ids, g)
    for t in ([3], [16, 0, 7], [5, 5, 2], list(range(17))[::-1]):
        sub = ref.forward_single(p, x, ids, g, tokens=np.array(t))
        assert np.array_equal(sub, full[t]) or rel_err(sub, full[t]) < 1e-13, t
    pg, _ = random_struct(4, 2, 2, 32, 16, 3, 16, seed=63)
    pu, _ = random_struct(4, 2, 2, 32, 16, 3, 16, seed=64)
    pd, _ = random_struct(4, 2, 2, 16, 32, 3, 16, seed=65)
    layer = dict(kind="swiglu", act="f16", K=4, d_model=32, d_ff=16,
                 proj=dict(gate=pg, up=pu, down=pd),
                 shared=synth.make_shared(32, 16, np.random.SeedSequence(66)))
    x, ids, g = tokens(32, 4, 2, 11, seed=67)
    full = ref.forward_swiglu(layer, x, ids, g)
    for t in ([10], [2, 9, 4], [1, 1]):
        for keep in (True, False):
            sub = ref.forward_swiglu(layer, x, ids, g, tokens=np.array(t), keep_weights=keep)
            assert rel_err(sub, full[t]) < 1e-13, (t, keep)


def _identity_shift(d):
    """Codes, scales, zeros of W[o][i] = 1 iff i == (o + 1) % d (one group)."""
    q = np.zeros((1, d, d), np.int64)
    q[0, np.arange(d), (np.arange(d) + 1) % d] = 1
    return q, np.ones((1, d, 1), np.float16), np.zeros((1, d, 1), np.float16)


def pin_swiglu_closed_form(ref):
    """One expert, rank 0.  x = e_0; gate column 0 = 0.5*((o % 4) - 1),
    up column 0 = 1, down = shift permutation:  y_o = g * RND(silu(a_{o+1}))."""
    d = 32
    qg = np.zeros((1, d, d), np.int64)
    qg[0, :, 0] = np.arange(d) % 4
    pg = proj_from(qg, np.full((1, d, 1), 0.5, np.float16), np.ones((1, d, 1), np.float16),
                   np.zeros((d, 0), np.float16), [], np.zeros((d, 0), np.float16), [0], 1, 1, d)
    qu = np.zeros((1, d, d), np.int64)
    qu[0, :, 0] = 1
    pu = proj_from(qu, np.ones((1, d, 1), np.float16), np.zeros((1, d, 1), np.float16),
                   np.zeros((d, 0), np.float16), [], np.zeros((d, 0), np.float16), [0], 1, 1, d)
    qd, sd, zd = _identity_shift(d)
    pdn = proj_from(qd, sd, zd, np.zeros((d, 0), np.float16), [],
                    np.zeros((d, 0), np.float16), [0], 1, 1, d)
    layer = dict(kind="swiglu", act="f16", K=1, d_model=d, d_ff=d,
                 proj=dict(gate=pg, up=pu, down=pdn), shared=None)
    x = np.zeros((1, d), np.float16)
    x[0, 0] = 1
    y = ref.forward_swiglu(layer, x, np.array([[0]]), np.array([[0.75]], np.float32))
    a = 0.5 * ((np.arange(d) % 4) - 1)
    h = np.array([float(np.float16(v / (1 + math.exp(-v)))) for v in a])
    want = 0.75 * h[(np.arange(d) + 1) % d]
    assert np.allclose(y[0], want, rtol=1e-15, atol=0), (y[0][:6], want[:6])


def pin_shared_closed_form(ref):
    """Dense shared expert alone: y = W_d RND(silu(W_g x) * (W_u x))."""
    d = 16
    wg = np.zeros((d, d), np.float16)
    wg[:, 0] = (np.arange(d) - 8) / 4.0
    wu = np.zeros((d, d), np.float16)
    wu[:, 0] = 2.0
    wd = np.zeros((d, d), np.float16)
    wd[np.arange(d), (np.arange(d) + 3) % d] = 1
    x = np.zeros((2, d), np.float16)
    x[:, 0] = [1.0, -1.0]
    y = ref.shared_expert(dict(wg=wg, wu=wu, wd=wd), x.astype(np.float64), "f16")
    for t, sgn in enumerate([1.0, -1.0]):
        a = sgn * (np.arange(d) - 8) / 4.0
        b = sgn * 2.0
        h = np.array([float(np.float16(v / (1 + math.exp(-v)) * b)) for v in a])
        assert np.allclose(y[t], h[(np.arange(d) + 3) % d], rtol=1e-15, atol=0)


def check_route(r, ids, K, n_of=None):
    """Invariants that define the canonical lists uniquely."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < K))[0]
    perm = r["perm"]
    assert sorted(perm.tolist()) == valid.tolist()
    keys = flat[perm]
    assert np.all(np.diff(keys) >= 0)
    same = np.diff(keys) == 0
    assert np.all(np.diff(perm)[same] > 0)
    assert np.array_equal(r["cnt"], np.bincount(flat[valid], minlength=K)[:K])
    assert r["off"][0] == 0 and np.array_equal(np.diff(r["off"]), r["cnt"])
    for p_, s in enumerate(perm):
        assert r["inv"][s] == p_
    assert np.all(r["inv"][np.setdiff1d(np.arange(T * k), valid)] == -1)
    if n_of is not None:
        pairs = r["col_pairs"]
        want = sorted({(int(n_of[flat[s]]), int(s // k)) for s in valid})
        assert [tuple(p) for p in pairs.tolist()] == want
        for n in range(len(r["col_off"]) - 1):
            seg = pairs[r["col_off"][n]:r["col_off"][n + 1]]
            assert np.all(seg[:, 0] == n)
        for s in valid:
            assert tuple(pairs[r["slot2col"][s]]) == (n_of[flat[s]], s // k)


def pin_route(ref):
    rng = np.random.default_rng(45)
    cases = [rng.integers(0, 8, (33, 2)),                 # random
             np.full((20, 2), 3),                         # all slots on one expert
             np.array([[0, 0], [1, 1], [0, 1]]),          # duplicates
             np.array([[5, 2]]),                          # T = 1
             np.array([[9, -1], [2, 8], [7, 7]]),         # dropped ids
             rng.integers(0, 8, (500, 6))]
    n_of = np.array([3, 1, 2, 0, 1, 3, 2, 0])
    for ids in cases:
        r = ref.route(ids, 8, n_of)
        check_route(r, ids, 8, n_of)


def pin_router(ref):
    """Router top-k: ids against numpy's stable argsort of -logits (ties to the
    lower id); weights against scipy's softmax when k = K (then the selected
    logits are all of them) and, for k < K, the closed-form ratios
    w_i / w_j = exp(l_i - l_j) with sum 1; k = 1 gives weight 1; NaN logits
    are never chosen before finite ones; all -inf gives uniform weights."""
    from scipy.special import softmax
    rng = np.random.default_rng(71)
    for K, k in [(8, 2), (60, 4), (64, 6), (256, 8), (5, 5), (16, 1)]:
        L = rng.standard_normal((40, K))
        L[:10] = np.round(L[:10] * 2) / 2            # many ties
        ids, w = ref.router_topk(L, k)
        want = np.argsort(-L, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, want), (K, k)
        sel = np.take_along_axis(L, want, axis=1)
        assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert np.allclose(np.log(w[:, 1:] / w[:, :1]), sel[:, 1:] - sel[:, :1], atol=1e-9)
        if k == K:
            assert np.allclose(w, np.take_along_axis(softmax(L, axis=1), want, axis=1), atol=1e-12)
        if k == 1:
            assert np.all(w == 1.0)
    L = np.array([[np.nan, 1.0, np.nan, -2.0], [-np.inf] * 4])
    ids, w = ref.router_topk(L, 2)
    assert ids[0].tolist() == [1, 3] and ids[1].tolist() == [0, 1]
    assert np.allclose(w[1], 0.5)


ALL_PINS = [pin_unpack_golden, pin_unpack_bytes, pin_residual_golden, pin_deq_golden,
            pin_rnd_f16_vs_numpy, pin_rnd_bf16, pin_silu, pin_p1_factored_block,
            pin_p2_zero_rank, pin_p3_zero_residual, pin_p4_token_perm, pin_p5_slots,
            pin_p6_textbook, pin_p7_grid_relabel, pin_p8_linearity, pin_dropped_ids,
            pin_p11_two_oracles, pin_p12_storage, pin_swiglu_closed_form,
            pin_shared_closed_form, pin_route, pin_router, pin_token_subset, pin_unpack3_golden,
            pin_unpack3_bytes, pin_p2_zero_rank_3bit]
