"""The offline packer on the GPU (tq_pack_proj) against the packer oracle.

Unique results are compared exactly or within their rounding: sigma (fp32),
the stored factors U and V (activation format, per column up to the sign
that the SVD leaves open), and -- on the device's own stored factors -- the
round-to-nearest codes, scales and zero points of every residual group
(a code may differ only where its value lies within 1e-9 of a rounding tie,
where both neighbours are correct).  The packed projection is then uploaded
and run through the forward against the forward oracle, and its weights are
checked to lie within half a quantization step of the dense weights."""
import numpy as np
import pytest
import torch

import bit_rank_post_amd as tq
from bit_rank_post_amd import io as tqio
from oracle import pack_ref as P
from oracle import tileq_ref as R
from tests.gpu_util import assert_parity, need_gpu, run_forward, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    need_gpu()


def dense_experts(K, M, N, d_out, d_in, rank, seed, noise=0.02, tiles=None, exact=False):
    """Expert weights drawn as blocks of a global low-rank matrix (sigma
    log-uniform over [0.1, 10]) plus N(0, noise) per expert; returns (W fp64
    [K][d_out][d_in], tiles)."""
    rng = np.random.default_rng(seed)
    if tiles is None:
        tiles = rng.permutation(M * N)[:K]
    A = rng.standard_normal((M * d_out, rank)) / np.sqrt(d_out)
    B = rng.standard_normal((N * d_in, rank)) / np.sqrt(d_in)
    sv = np.sort(np.exp(rng.uniform(np.log(0.1), np.log(10.0), rank)))[::-1]
    big = (A * sv) @ B.T
    W = np.zeros((K, d_out, d_in))
    for e, t in enumerate(tiles):
        m, n = divmod(int(t), N)
        W[e] = big[m * d_out:(m + 1) * d_out, n * d_in:(n + 1) * d_in]
        if not exact:
            W[e] += noise * rng.standard_normal((d_out, d_in))
    return W, np.asarray(tiles, np.int32)


def act_values(a, act):
    return R.to_f64(a, act)


def align_signs(Ud, Uo):
    s = np.sign(np.sum(Ud * Uo, axis=0))
    s[s == 0] = 1.0
    return s


def check_factors(dev, orc, act):
    """sigma within 2 fp32 ulps; U, V column by column (sign aligned) within
    one ulp of the activation format, mismatches rare."""
    sd, so = dev["sigma"].astype(np.float64), orc["sigma"].astype(np.float64)
    assert np.all(np.abs(sd - so) <= 2 * np.spacing(np.abs(so).astype(np.float32)).astype(np.float64)), \
        (sd[:4], so[:4])
    for key in ("U", "V"):
        d = act_values(dev[key], act)
        o = act_values(orc[key], act)
        sg = align_signs(d, o)
        d = d * sg
        ulp = np.maximum(np.spacing(np.abs(o).astype(np.float32)).astype(np.float64) *
                         (2 ** 13 if act == "f16" else 2 ** 16),
                         2.0 ** -24 if act == "f16" else 2.0 ** -133)
        diff = np.abs(d - o)
        assert np.all(diff <= 1.01 * ulp + 1e-30), (key, float(diff.max()))
        frac = float(np.mean(diff > 0))
        say(f"  {key}: {frac:.2e} of the stored entries one ulp apart (rounding of equal fp64 values)")
        assert frac < 1e-3, (key, frac)


def check_rtn(dev, W, act):
    """Codes, scales and zero points against the oracle's quantizer applied
    to the residual of the device's own stored factors."""
    K, d_out, d_in = W.shape
    G, bits, N = dev["group"], dev["bits"], dev["N"]
    U = act_values(dev["U"], act) * dev["sigma"].astype(np.float64)[None, :]
    V = act_values(dev["V"], act)
    for e in range(K):
        m, n = divmod(int(dev["tile_of_expert"][e]), N)
        res = W[e] - U[m * d_out:(m + 1) * d_out] @ V[n * d_in:(n + 1) * d_in].T
        q, s, z = P.quantize_rtn(res, G, bits)
        assert np.array_equal(dev["scales"][e].view(np.uint16), s.view(np.uint16)), e
        assert np.array_equal(dev["zeros"][e].view(np.uint16), z.view(np.uint16)), e
        qd = R.unpack_codes(dev["codes"][e], d_in, bits)
        bad = qd != q
        if bad.any():
            t = res / np.repeat(s.astype(np.float64), G, axis=1) + np.repeat(z.astype(np.float64), G, axis=1)
            gap = np.abs(t - np.floor(t) - 0.5)
            assert np.all(gap[bad] < 1e-9) and np.all(np.abs(qd - q)[bad] == 1), (e, int(bad.sum()))
            say(f"  expert {e}: {int(bad.sum())} codes at rounding ties")


@pytest.mark.parametrize("K,M,N,d_out,d_in,rank,sketch,G,bits,act,q,wdt", [
    (8, 2, 4, 512, 256, 16, 24, 64, 2, "f16", 0, "f32"),     # Mixtral-like grid, small
    (8, 2, 4, 512, 256, 16, 24, 64, 3, "bf16", 1, "f16"),    # 3-bit, bf16 factors, power iteration
    (60, 8, 8, 128, 256, 32, 40, 128, 2, "f16", 1, "f64"),   # Qwen-like: 4 empty tiles
    (4, 2, 2, 64, 384, 8, 8, 32, 2, "f16", 0, "bf16"),       # sketch = rank, 4-step tail
])
def test_pack_matches_oracle(K, M, N, d_out, d_in, rank, sketch, G, bits, act, q, wdt):
    W, tiles = dense_experts(K, M, N, d_out, d_in, rank, seed=K + d_out + bits)
    if wdt == "f16":
        Win = W.astype(np.float16)
    elif wdt == "bf16":
        import synth
        Win = synth.to_act(W.astype(np.float32), "bf16")
    else:
        Win = W.astype(np.float32 if wdt == "f32" else np.float64)
    Wx = R.to_f64(Win, wdt if wdt in ("f16", "bf16") else "f32") if wdt != "f64" else W
    omega = np.random.default_rng(7).standard_normal((N * d_in, sketch))
    dev = tqio.pack_proj(Win, tiles, M, N, rank, G, bits, omega, act=act, power_iters=q,
                         w_bf16=(wdt == "bf16"))
    orc = P.pack_proj(Wx, tiles, M, N, rank, G, bits, omega, act=act, power_iters=q)
    check_factors(dev, orc, act)
    check_rtn(dev, Wx, act)
    # the packed projection in the forward, and its weights against the dense ones
    layer = dict(kind="single", act=act, K=K, d_model=d_in, d_ff=d_out, proj=dict(single=dev),
                 shared=None)
    L = tqio.upload_layer(layer)
    import synth
    x, ids, g = synth.make_custom_tokens(d_in, K, 2, 40, act, seed=11)
    y, _ = run_forward(L, x, ids, g, act, "f32")
    assert_parity(y, R.forward(layer, x, ids, g), what=f"packed projection forward K={K} bits={bits}")
    # half a step, plus the clamp at the ends: s = RND_f16((mx - mn) / Q) may
    # round down by 2^-11 relative, moving the extreme level by up to Q 2^-11 steps
    qmax = (1 << bits) - 1
    for e in range(min(K, 6)):
        We = R.expert_weight(dev, e)
        s = np.repeat(dev["scales"][e].astype(np.float64), G, axis=1)
        assert np.all(np.abs(We - Wx[e]) <= (0.5 + qmax * 2.0 ** -10) * s), e


def test_pack_exact_rank_sigma():
    """An exactly rank-8 W_big (fp64 input): sigma equals numpy's full SVD of
    W_big to fp32 rounding."""
    K, M, N, d_out, d_in, r = 8, 2, 4, 64, 128, 8
    W, tiles = dense_experts(K, M, N, d_out, d_in, r, seed=5, exact=True)
    omega = np.random.default_rng(9).standard_normal((N * d_in, r + 4))
    dev = tqio.pack_proj(W, tiles, M, N, r, 32, 2, omega, act="f16")
    big = P.assemble_wbig(W, tiles, M, N)
    ref = np.linalg.svd(big, compute_uv=False)[:r].astype(np.float32)
    assert np.array_equal(dev["sigma"], ref) or np.max(np.abs(dev["sigma"] - ref) / ref) < 1.2e-7


def test_pack_rejects_bad_arguments():
    import ctypes
    omega = torch.zeros((512, 8), dtype=torch.float64, device="cuda")
    W = torch.zeros((2, 64, 128), dtype=torch.float32, device="cuda")
    out = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    base = dict(K=2, M=1, N=2, d_in=128, d_out=64, rank=4, group=32, bits=2, sketch=8,
                power_iters=0, act=tq.TQ_F16, tile_of_expert=[0, 1], W=W, w_dtype=tq.TQ_F32,
                omega=omega, U=out, sigma=out, V=out, codes=out, scales=out, zeros=out)
    for kw, text in [(dict(sketch=3), "sketch"), (dict(sketch=137), "sketch"),
                     (dict(tile_of_expert=[1, 1]), "share tile"), (dict(bits=4), "bits"),
                     (dict(w_dtype=7), "w_dtype"), (dict(act=tq.TQ_F32), "act")]:
        args = dict(base)
        args.update(kw)
        with pytest.raises(tq.TileQError, match=text):
            tq.pack_proj(**args)
    del ctypes


def test_pack_mixtral_gate_full_size():
    """The packer at the Mixtral-shaped gate projection's size (8 experts on
    2 x 4, d_out 14336, d_in 4096, rank 64, sketch 72, one power iteration,
    fp16 weights): factors against the oracle in full, the quantization on
    256 rows of every expert spread over the row range."""
    import synth
    K, M, N, d_out, d_in, r, l, G = 8, 2, 4, 14336, 4096, 64, 72, 128
    W16, tiles = synth.make_dense_experts(K, M, N, d_out, d_in, r, seed=31)
    omega = np.random.default_rng(32).standard_normal((N * d_in, l))
    say("  device packer (Mixtral-shaped gate)")
    dev = tqio.pack_proj(W16, tiles, M, N, r, G, 2, omega, act="f16", power_iters=1)
    say("  oracle sketch")
    W = W16.astype(np.float64)
    big = P.assemble_wbig(W, tiles, M, N)
    U, S, V = P.sketch_svd(big, omega, r, power_iters=1)
    del big
    Ur, Sr, Vr, S32 = P.stored_factors(U, S, V, "f16")
    orc = dict(sigma=S32, U=P.to_storage(Ur, "f16"), V=P.to_storage(Vr, "f16"))
    check_factors(dev, orc, "f16")
    rows = np.linspace(0, d_out - 1, 256).astype(int)
    Ud = act_values(dev["U"], "f16") * dev["sigma"].astype(np.float64)[None, :]
    Vd = act_values(dev["V"], "f16")
    for e in range(K):
        m, n = divmod(int(tiles[e]), N)
        res = W[e][rows] - Ud[m * d_out + rows] @ Vd[n * d_in:(n + 1) * d_in].T
        q, s, z = P.quantize_rtn(res, G, 2)
        assert np.array_equal(dev["scales"][e][rows].view(np.uint16), s.view(np.uint16)), e
        assert np.array_equal(dev["zeros"][e][rows].view(np.uint16), z.view(np.uint16)), e
        qd = R.unpack_codes(dev["codes"][e][rows], d_in, 2)
        bad = qd != q
        if bad.any():
            t = res / np.repeat(s.astype(np.float64), G, axis=1) + np.repeat(z.astype(np.float64), G, axis=1)
            gap = np.abs(t - np.floor(t) - 0.5)
            assert np.all(gap[bad] < 1e-9), (e, int(bad.sum()))
