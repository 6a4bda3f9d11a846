"""Pins of the packer oracle (oracle/pack_ref.py) to facts outside itself:
the truncated SVD from numpy.linalg.svd of the whole W_big (a different
routine), Eckart-Young's optimal error, an exactly low-rank matrix, hand-derived
quantization fixtures (tests/golden/rtn_group.txt), brute-force nearest codes,
the forward oracle's own unpacking of the packed codes, and the quantization
error bound of the packed projection read back by the forward oracle.

Passages followed ("TileQ: Efficient Low-Rank Quantization of
Mixture-of-Experts with 2D Tiling", gist.science technical summary): section
2.1 step 4 (experts as tiles of W_big), step 5 (global low-rank decomposition
of W_big approximated by Gaussian sketching; factors stored; each expert's
residual quantized).
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


def experts_of(Wbig, tiles, M, N, d_out, d_in):
    K = len(tiles)
    W = np.zeros((K, d_out, d_in))
    for e, t in enumerate(tiles):
        m, n = divmod(int(t), N)
        W[e] = Wbig[m * d_out:(m + 1) * d_out, n * d_in:(n + 1) * d_in]
    return W


def pin_pack_exact_rank(P):
    """An exactly rank-r W_big (all tiles filled) is recovered to 1e-10 and its
    sigma equals numpy's full SVD's leading values."""
    rng = np.random.default_rng(201)
    M, N, d_out, d_in, r = 2, 3, 32, 64, 6
    A = rng.standard_normal((M * d_out, r))
    B = rng.standard_normal((N * d_in, r))
    Wbig = A @ B.T
    tiles = rng.permutation(M * N)
    W = experts_of(Wbig, tiles, M, N, d_out, d_in)
    omega = rng.standard_normal((N * d_in, r + 4))
    U, S, V = P.sketch_svd(P.assemble_wbig(W, tiles, M, N), omega, r)
    assert rel((U * S) @ V.T, Wbig) < 1e-10
    ref = np.linalg.svd(Wbig, compute_uv=False)[:r]
    assert rel(S, ref) < 1e-10
    assert np.all(np.diff(S) <= 0)                                # descending
    assert rel(U.T @ U, np.eye(r)) < 1e-10 and rel(V.T @ V, np.eye(r)) < 1e-10


def pin_pack_truncated_svd(P):
    """With the sketch as wide as W_big, the rank-r result is the truncated
    SVD (unique for distinct singular values) of numpy.linalg.svd."""
    rng = np.random.default_rng(202)
    M, N, d_out, d_in, r = 2, 2, 16, 24, 5
    Wbig = rng.standard_normal((M * d_out, N * d_in))
    tiles = np.array([3, 0, 2, 1])
    W = experts_of(Wbig, tiles, M, N, d_out, d_in)
    omega = rng.standard_normal((N * d_in, N * d_in))
    U, S, V = P.sketch_svd(P.assemble_wbig(W, tiles, M, N), omega, r)
    Uf, Sf, Vft = np.linalg.svd(Wbig)
    best = (Uf[:, :r] * Sf[:r]) @ Vft[:r]
    assert rel((U * S) @ V.T, best) < 1e-10
    assert rel(S, Sf[:r]) < 1e-10


def pin_pack_power_iterations(P):
    """Eckart-Young: no rank-r result beats the truncated SVD's error
    sqrt(sum_{i > r} sigma_i^2); a narrow sketch of a slowly decaying spectrum
    misses it by far, two power iterations come within 1 %."""
    rng = np.random.default_rng(203)
    m, n, r = 64, 96, 8
    Uo, _ = np.linalg.qr(rng.standard_normal((m, m)))
    Vo, _ = np.linalg.qr(rng.standard_normal((n, m)))
    sv = 1.0 / (1.0 + np.arange(m))
    Wbig = (Uo * sv) @ Vo.T
    W = Wbig.reshape(1, m, n)
    opt = np.sqrt(np.sum(sv[r:] ** 2))
    omega = rng.standard_normal((n, r + 4))
    errs = []
    for q in (0, 2):
        U, S, V = P.sketch_svd(P.assemble_wbig(W, [0], 1, 1), omega, r, power_iters=q)
        errs.append(np.linalg.norm(Wbig - (U * S) @ V.T))
    assert errs[0] >= opt * (1 - 1e-12) and errs[1] >= opt * (1 - 1e-12)
    assert errs[1] <= 1.01 * opt and errs[0] > 1.2 * opt


def pin_pack_empty_tiles(P):
    """Tiles without an expert are zero blocks of W_big; the experts land at
    block (m, n) = divmod(tile, N)."""
    rng = np.random.default_rng(204)
    W = rng.standard_normal((3, 4, 8))
    big = P.assemble_wbig(W, [5, 0, 2], 2, 3)
    assert big.shape == (8, 24)
    assert np.array_equal(big[4:8, 16:24], W[0]) and np.array_equal(big[0:4, 0:8], W[1])
    assert np.array_equal(big[0:4, 16:24], W[2])
    for m, n in [(0, 1), (1, 0), (1, 1)]:
        assert not big[m * 4:(m + 1) * 4, n * 8:(n + 1) * 8].any()


def pin_rtn_golden(P):
    with open(os.path.join(GOLDEN, "rtn_group.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            kv = dict(item.split("=") for item in line.split())
            w = np.array([[float(v) for v in kv["w"].split(",")]])
            q, s, z = P.quantize_rtn(w, w.shape[1], int(kv["bits"]))
            assert float(s[0, 0]) == float(kv["s"]), (line, s)
            assert float(z[0, 0]) == float(kv["z"]), (line, z)
            assert q[0].tolist() == [int(v) for v in kv["q"].split(",")], (line, q)


def pin_rtn_nearest(P):
    """Brute force: every code is the nearest level of w/s + z in 0..Q
    (clamped at the ends), z is the nearest level of -mn/s, and quantizing
    the exact dequantized values s (q - z) gives back q."""
    rng = np.random.default_rng(205)
    for bits in (2, 3):
        qmax = (1 << bits) - 1
        w = rng.standard_normal((6, 64)) * 0.02
        w[0, :16] = np.abs(w[0, :16])                  # a group with mn = 0
        q, s, z = P.quantize_rtn(w, 16, bits)
        s64 = np.repeat(s.astype(np.float64), 16, axis=1)
        z64 = np.repeat(z.astype(np.float64), 16, axis=1)
        for (i, j), v in np.ndenumerate(w):
            t = v / s64[i, j] + z64[i, j]
            best = min(range(qmax + 1), key=lambda c: (abs(t - c), c % 2))
            assert q[i, j] == best, (bits, i, j, t, q[i, j])
        wr = s64 * (q - z64)
        q2, s2, z2 = P.quantize_rtn(wr, 16, bits)
        assert np.array_equal(z2, z)
        same_s = np.repeat(s2 == s, 16, axis=1)
        assert np.array_equal(q2[same_s], q[same_s])


def pin_pack_codes_unpack(P):
    """The packer's packing read back by the forward oracle's unpacking."""
    from oracle import tileq_ref
    rng = np.random.default_rng(206)
    for bits in (2, 3):
        q = rng.integers(0, 1 << bits, (3, 5, 128))
        assert np.array_equal(tileq_ref.unpack_codes(P.pack_codes(q, bits), 128, bits), q)


def pin_pack_error_bound(P):
    """End to end: the packed projection, read back by the forward oracle
    (explicit expert weights from the stored factors and codes), is within
    half a quantization step (plus the end clamp) of the dense weights; and
    the low-rank part alone leaves the residual the packer quantized."""
    from oracle import tileq_ref
    rng = np.random.default_rng(207)
    M, N, d_out, d_in, r = 2, 2, 32, 128, 8
    A = rng.standard_normal((M * d_out, r)) / np.sqrt(d_out)
    B = rng.standard_normal((N * d_in, r)) / np.sqrt(d_in)
    Wbig = (A * np.linspace(3, 0.5, r)) @ B.T + 0.02 * rng.standard_normal((M * d_out, N * d_in))
    tiles = np.array([2, 3, 1])
    W = experts_of(Wbig, tiles, M, N, d_out, d_in)
    for bits, act in ((2, "f16"), (3, "bf16")):
        omega = rng.standard_normal((N * d_in, r + 8))
        p = P.pack_proj(W, tiles, M, N, r, 32, bits, omega, act=act, power_iters=1)
        for e in range(3):
            We = tileq_ref.expert_weight(p, e)
            s = np.repeat(p["scales"][e].astype(np.float64), 32, axis=1)
            # half a step, plus the clamp at the ends (s may round down by
            # 2^-11 relative, moving the extreme level by up to Q 2^-11 steps)
            qmax = (1 << bits) - 1
            assert np.all(np.abs(We - W[e]) <= (0.5 + qmax * 2.0 ** -10) * s), (bits, e)
            m, n = divmod(int(tiles[e]), N)
            low = tileq_ref.lowrank_block(p, m, n)
            assert rel(W[e] - low, p["residual"][e]) < 1e-12


ALL_PINS = [pin_pack_exact_rank, pin_pack_truncated_svd, pin_pack_power_iterations,
            pin_pack_empty_tiles, pin_rtn_golden, pin_rtn_nearest, pin_pack_codes_unpack,
            pin_pack_error_bound]
