"""Plain fp64 CPU oracle of the offline TileQ packer: dense expert weights in,
the stored form of one projection out (the input format of the forward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

What it computes ("TileQ: Efficient Low-Rank Quantization of Mixture-of-Experts
with 2D Tiling", gist.science technical summary):

* Section 2.1 step 4 (2D-Tiling Placement): the K experts of a projection are
  placed as tiles of one block matrix W_big on an M x N grid (expert e at tile
  (m, n) = divmod(tile_of_expert[e], N)); a tile without an expert is a zero
  block (the map is injective, not necessarily onto).
* Section 2.1 step 5 (Quantization): W_big gets a global low-rank
  decomposition U Sigma V^T, approximated with a Gaussian sketch instead of a
  full SVD; the factors are stored and each expert's residual is quantized.

The Gaussian sketch is read as the randomized range finder with a small SVD
(Halko, Martinsson and Tropp, "Finding structure with randomness", 2011):
  Y = W_big Omega with Omega [N d_in][l] standard normal (l = rank +
  oversampling, the random numbers passed in), optionally refined by q power
  iterations Y <- W_big (W_big^T Q); Q an orthonormal basis of range(Y);
  B = Q^T W_big; the SVD of the small B = U~ S V~^T; U = Q U~_r, Sigma = S_r,
  V = V~_r (the r leading triplets).
The residual of expert e is its weight minus block (m, n) of the STORED
factors (U and V rounded to the activation format, sigma to fp32), so the
quantization also absorbs the factors' rounding.  The pages quantize it with
GPTQ/GPTVQ and rotations, which need calibration data; the reading here is
asymmetric round-to-nearest per group of G inputs (the residual quantizer of
the forward's input format):
  mn = min(min w, 0), mx = max(max w, 0), Q = 2^bits - 1,
  s = RND_f16((mx - mn) / Q), 1 where that is 0,
  z = clamp(rint(-mn / s), 0, Q), q = clamp(rint(w / s) + z, 0, Q),
  every step in fp64 with rint rounding half to even.
Library primitives serve as steps: numpy matmul, numpy.linalg.qr for the
orthonormal basis and numpy.linalg.svd for the small SVD.
"""
from __future__ import annotations

import numpy as np

from . import tileq_ref


def assemble_wbig(W, tiles, M, N):
    """W_big [M d_out][N d_in] (fp64) from expert weights W [K][d_out][d_in]
    placed at their tiles; empty tiles are zero blocks."""
    W = np.asarray(W, np.float64)
    K, d_out, d_in = W.shape
    big = np.zeros((M * d_out, N * d_in))
    for e in range(K):
        m, n = divmod(int(tiles[e]), N)
        big[m * d_out:(m + 1) * d_out, n * d_in:(n + 1) * d_in] = W[e]
    return big


def range_finder(Wbig, omega, power_iters=0):
    """Orthonormal basis Q of range(W_big Omega), refined by power iterations
    (each re-orthonormalised)."""
    Q, _ = np.linalg.qr(Wbig @ np.asarray(omega, np.float64))
    for _ in range(power_iters):
        Q, _ = np.linalg.qr(Wbig @ (Wbig.T @ Q))
    return Q


def sketch_svd(Wbig, omega, rank, power_iters=0):
    """The r leading singular triplets of W_big from the sketch: (U [m][r],
    sigma [r] descending, V [n][r]) in fp64."""
    Q = range_finder(Wbig, omega, power_iters)
    B = Q.T @ Wbig
    Ut, S, Vt = np.linalg.svd(B, full_matrices=False)
    r = min(rank, len(S))
    U = Q @ Ut[:, :r]
    V = Vt[:r].T
    if r < rank:                           # fewer directions than asked: zero padding
        U = np.concatenate([U, np.zeros((U.shape[0], rank - r))], axis=1)
        V = np.concatenate([V, np.zeros((V.shape[0], rank - r))], axis=1)
        S = np.concatenate([S[:r], np.zeros(rank - r)])
    return U, S[:rank], V


def quantize_rtn(w, group, bits):
    """Asymmetric round-to-nearest group quantization of w [rows][d_in] (fp64)
    along d_in, as in the module docstring.  Returns (q int64, s f16, z f16)."""
    qmax = (1 << bits) - 1
    w = np.asarray(w, np.float64)
    rows, d_in = w.shape
    wg = w.reshape(rows, d_in // group, group)
    mn = np.minimum(wg.min(axis=2), 0.0)
    mx = np.maximum(wg.max(axis=2), 0.0)
    s16 = tileq_ref.rnd_act((mx - mn) / qmax, "f16")
    s16 = np.where(s16 == 0, 1.0, s16)
    z = np.clip(np.rint(-mn / s16), 0, qmax)
    q = np.clip(np.rint(wg / s16[..., None]) + z[..., None], 0, qmax)
    return (q.reshape(rows, d_in).astype(np.int64), s16.astype(np.float16),
            z.astype(np.float16))


def pack_codes(q, bits):
    """Codes [..., d_in] into the forward's words: 2-bit 16 per word (code i
    at bits 2 (i % 16)); 3-bit as the row's little-endian bit string."""
    q = np.asarray(q, np.int64)
    d_in = q.shape[-1]
    if bits == 2:
        words = np.zeros(q.shape[:-1] + (d_in // 16,), np.uint64)
        for j in range(16):
            words |= (q[..., j::16].astype(np.uint64) & 3) << np.uint64(2 * j)
        return words.astype(np.uint32)
    nbits = 3 * d_in
    stream = np.zeros(q.shape[:-1] + (nbits,), np.uint8)
    for b in range(3):
        stream[..., b::3] = (q >> b) & 1
    stream = stream.reshape(q.shape[:-1] + (nbits // 32, 32)).astype(np.uint64)
    return (stream << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)


def stored_factors(U, S, V, act):
    """The factors as stored: U, V in the activation format (round to nearest
    even), sigma in fp32.  Returns (U_st, S_st, V_st) as fp64 values and the
    stored arrays (act storage, f32)."""
    # fp64 -> act directly (one rounding) through the oracle's own rounding
    Ur = tileq_ref.rnd_act(U, act)
    Vr = tileq_ref.rnd_act(V, act)
    Sr = np.asarray(S, np.float64).astype(np.float32)
    return Ur, Sr.astype(np.float64), Vr, Sr


def to_storage(v, act):
    """fp64 values that the activation format holds -> its storage array."""
    if act == "f16":
        return np.asarray(v).astype(np.float16)
    bits = np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)
    return bits.astype(np.uint16)


def pack_proj(W, tiles, M, N, rank, group, bits, omega, act="f16", power_iters=0):
    """The whole packer: expert weights W [K][d_out][d_in] -> the stored
    projection (dict in the forward's input format, plus the fp64 W_big and
    the exact residuals under 'wbig' / 'residual')."""
    W = np.asarray(W, np.float64)
    K, d_out, d_in = W.shape
    Wbig = assemble_wbig(W, tiles, M, N)
    U, S, V = sketch_svd(Wbig, omega, rank, power_iters)
    Ur, Sr, Vr, S32 = stored_factors(U, S, V, act)
    low = (Ur * Sr[None, :]) @ Vr.T
    res = np.zeros_like(W)
    codes, scales, zeros = [], [], []
    for e in range(K):
        m, n = divmod(int(tiles[e]), N)
        res[e] = W[e] - low[m * d_out:(m + 1) * d_out, n * d_in:(n + 1) * d_in]
        q, s, z = quantize_rtn(res[e], group, bits)
        codes.append(pack_codes(q, bits))
        scales.append(s)
        zeros.append(z)
    return dict(K=K, M=M, N=N, d_in=d_in, d_out=d_out, rank=rank, group=group, bits=bits,
                act=act, tile_of_expert=np.asarray(tiles, np.int32),
                U=to_storage(Ur, act), sigma=S32, V=to_storage(Vr, act),
                codes=np.stack(codes), scales=np.stack(scales), zeros=np.stack(zeros),
                wbig=Wbig, residual=res, factors64=(U, S, V))
