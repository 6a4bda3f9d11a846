"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer work is compared bit for bit (routing lists; dequantized weights), the
forward output within max|dy| <= 2e-3 * ||y_oracle||_inf (fp16 in, fp32
accumulation; bf16 outputs additionally get half a bf16 ulp).  Full-size
configurations are checked on sampled tokens, whose outputs the oracle
computes from explicitly built expert weights."""
import numpy as np
import pytest
import torch

import bit_rank_post_amd as tq
import synth
from bit_rank_post_amd import io as tqio
from oracle import tileq_ref as R
from tests import pins
from tests.gpu_util import assert_parity, need_gpu, run_forward, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    need_gpu()


# ---------------------------------------------------------------------------
# integer work: dequantized weights and routing lists, bit-exact


def single_layer_from(p):
    return dict(kind="single", act=p["act"], K=p["K"], d_model=p["d_in"], d_ff=p["d_out"],
                proj=dict(single=p), shared=None)


def test_dequant_exhaustive_fp16_scales():
    """Every finite fp16 scale with |s| < 1024 (both signs) x every integer
    zero point x every code, through the forward's own unpack path."""
    sbits = np.concatenate([np.arange(0x0000, 0x6400), np.arange(0x8000, 0xE400)]).astype(np.uint16)
    rows, G, d_in = len(sbits), 32, 128
    s = np.repeat(sbits[:, None], 4, axis=1).view(np.float16)[None]
    z = np.tile(np.arange(4, dtype=np.float16), (rows, 1))[None]
    i = np.arange(d_in)[None, :]
    o = np.arange(rows)[:, None]
    q = ((i + o + i // 4) % 4)[None]
    p = pins.proj_from(q, s, z, np.zeros((rows, 0), np.float16), [],
                       np.zeros((d_in, 0), np.float16), [0], 1, 1, G)
    L = tqio.upload_layer(single_layer_from(p))
    w = torch.empty((rows, d_in), dtype=torch.float16, device="cuda")
    L.debug_dequant(0, 0, w)
    torch.cuda.synchronize()
    got = w.cpu().numpy().view(np.uint16)
    want = R.deq_canonical(q[0], s[0], z[0], G, "f16").astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5])


@pytest.mark.parametrize("G,d_in,d_out,K", [(64, 1408, 64, 3), (128, 4096, 32, 2), (32, 384, 48, 2)])
def test_dequant_random_groups(G, d_in, d_out, K):
    rng = np.random.default_rng(G + d_in)
    q = rng.integers(0, 4, (K, d_out, d_in))
    s = rng.uniform(1e-4, 0.5, (K, d_out, d_in // G)).astype(np.float16)
    z = rng.integers(0, 4, (K, d_out, d_in // G)).astype(np.float16)
    p = pins.proj_from(q, s, z, np.zeros((d_out, 0), np.float16), [],
                       np.zeros((d_in, 0), np.float16), list(range(K)), 1, K, G)
    L = tqio.upload_layer(single_layer_from(p))
    for e in range(K):
        w = torch.empty((d_out, d_in), dtype=torch.float16, device="cuda")
        L.debug_dequant(0, e, w)
        torch.cuda.synchronize()
        want = R.deq_canonical(q[e], s[e], z[e], G, "f16").astype(np.float16)
        assert np.array_equal(w.cpu().numpy().view(np.uint16), want.view(np.uint16)), e


# zero points for the table dequantization: fractional, negative, subnormal,
# signed zero, beyond the code range; each row of a layer carries one set
# (one per group), so every scale is tried against four of them
ZERO_SETS = [(0.5, -1.25, 2.75, 7.0), (2.0 ** -24, -0.0, 3.0, -3.5),
             (100.5, -1000.0, 0.25, 1.5), (1.5, 1.5, 1.5, 1.5)]


@pytest.mark.parametrize("zset", range(len(ZERO_SETS)))
def test_dequant_exhaustive_general(zset):
    """Every finite fp16 scale (both signs, any magnitude) against fractional
    and out-of-range zero points, wherever the dequantized weights stay
    finite (the others are rejected at upload, tested below): bit-exact with
    RND_f16(fl32(fl32(q - z) * s)), through the table dequantization."""
    zs = np.array(ZERO_SETS[zset], np.float16)
    sbits = np.concatenate([np.arange(0x0000, 0x7C00), np.arange(0x8000, 0xFC00)]).astype(np.uint16)
    sv = sbits.view(np.float16)
    G, d_in = 32, 128
    q4 = np.arange(4)[None, None, :]           # codes 0..3 inside each of the 4 groups
    deq = R.deq_canonical(np.broadcast_to(q4, (len(sv), 4, 4)).reshape(len(sv), 16),
                          np.repeat(sv[:, None], 4, axis=1),
                          np.tile(zs, (len(sv), 1)), 4)
    ok = np.all(np.isfinite(deq), axis=1)
    sv = sv[ok]
    rows = len(sv)
    rows -= rows % 16
    sv = sv[:rows]
    s = np.repeat(sv[:, None], 4, axis=1)[None]
    z = np.tile(zs, (rows, 1))[None]
    i = np.arange(d_in)[None, :]
    o = np.arange(rows)[:, None]
    q = ((i + o + i // 4) % 4)[None]
    p = pins.proj_from(q, s, z, np.zeros((rows, 0), np.float16), [],
                       np.zeros((d_in, 0), np.float16), [0], 1, 1, G)
    say(f"  zero points {ZERO_SETS[zset]}: {rows} scales")
    L = tqio.upload_layer(single_layer_from(p))
    w = torch.empty((rows, d_in), dtype=torch.float16, device="cuda")
    L.debug_dequant(0, 0, w)
    torch.cuda.synchronize()
    got = w.cpu().numpy().view(np.uint16)
    want = R.deq_canonical(q[0], s[0], z[0], G, "f16").astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5])


def test_upload_rejects_nonfinite_and_overflow():
    p, _ = pins.random_struct(2, 1, 2, 128, 16, 0, 32, seed=1)
    for field, val, text in [("zeros", np.inf, "not finite"), ("zeros", np.nan, "not finite"),
                             ("scales", np.inf, "not finite"), ("scales", np.nan, "not finite"),
                             ("scales", 60000.0, "overflows"), ("zeros", -30000.0, "overflows")]:
        p2 = dict(p)
        a = p[field].copy()
        a[1, 3, 2] = np.float16(val)
        if field == "zeros" and val == -30000.0:
            p2["scales"] = np.full_like(p["scales"], 4.0)     # 4 * 30003 > 65504
        p2[field] = a
        with pytest.raises(tq.TileQError, match=text):
            tqio.upload_layer(single_layer_from(p2))


def general_struct(K, M, N, d_in, d_out, rank, G, seed, big=40000.0):
    """A projection with fractional zero points (some outside the code range),
    signed scales and, on 1 % of the groups, scales `big` times larger (up to
    1200 by default): the table dequantization."""
    p, q = pins.random_struct(K, M, N, d_in, d_out, rank, G, seed)
    rng = np.random.default_rng(seed + 1000)
    z = rng.uniform(-2.0, 5.0, p["zeros"].shape).astype(np.float16)
    s = (rng.uniform(0.001, 0.03, p["scales"].shape) * rng.choice([-1, 1], p["scales"].shape))
    sel = rng.random(p["scales"].shape) < 0.01
    s = np.where(sel, s * big, s).astype(np.float16)
    return pins.proj_from(q, s, z, p["U"], p["sigma"], p["V"], p["tile_of_expert"], M, N, G)


@pytest.mark.parametrize("path", [1, 2])
def test_general_zero_points_and_scales(path):
    """Forward parity with fractional zero points and large scales (decode
    multiplies raw codes and corrects per group; prefill dequantizes through
    byte tables), single projection and SwiGLU, sigma uploaded as f16."""
    p = general_struct(8, 2, 4, 256, 64, 16, 64, seed=71)
    L = tqio.upload_layer(single_layer_from(p))
    L.set_path(path)
    for T in (5, 150):
        x, ids, g = pins.tokens(256, 8, 2, T, seed=T)
        y, _ = run_forward(L, x, ids, g, "f16")
        assert_parity(y, R.forward_single(p, x, ids, g), what=f"general z/s single T={T}")
    ss = [general_struct(8, 2, 4, di, do, 16, 64, seed=72 + i, big=10.0)
          for i, (di, do) in enumerate([(256, 384), (256, 384), (384, 256)])]
    for q in ss:
        q["sigma"] = q["sigma"].astype(np.float16)        # sigma_dtype = TQ_F16
    layer = dict(kind="swiglu", act="f16", K=8, d_model=256, d_ff=384,
                 proj=dict(gate=ss[0], up=ss[1], down=ss[2]), shared=None)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    T = 24 if path == 1 else 300
    x, ids, g = synth.make_custom_tokens(256, 8, 2, T, "f16", seed=73)
    y, _ = run_forward(L, x, ids, g, "f16", "f32")
    assert_parity(y, R.forward(layer, x, ids, g), what=f"general z/s swiglu path={path}")


def route_layer(K, M, N, seed):
    p, _ = pins.random_struct(K, M, N, 128, 16, 16, 32, seed=seed)
    return tqio.upload_layer(single_layer_from(p)), p


def check_route_device(L, p, ids):
    T, k = ids.shape
    S = T * k
    K, N = p["K"], p["N"]
    dev = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device="cuda")
    cnt, off, perm, inv = dev(K), dev(K + 1), dev(S), dev(S)
    col_off, col_tok, s2c = dev(N + 1), dev(S), dev(S)
    ws = tqio.workspace(L, T, k)
    idd = torch.from_numpy(ids.astype(np.int32)).cuda()
    L.debug_route(0, idd, T, k, ws, cnt, off, perm, inv, col_off, col_tok, s2c)
    torch.cuda.synchronize()
    n_of = p["tile_of_expert"] % N
    r = R.route(ids, K, n_of)
    h = lambda t: t.cpu().numpy().astype(np.int64)
    assert np.array_equal(h(cnt), r["cnt"])
    assert np.array_equal(h(off), r["off"])
    P = int(r["off"][-1])
    assert np.array_equal(h(perm)[:P], r["perm"])
    assert np.array_equal(h(inv), r["inv"])
    co = h(col_off)
    assert np.array_equal(co[:len(r["col_off"])], r["col_off"])
    npairs = len(r["col_pairs"])
    assert np.array_equal(h(col_tok)[:npairs], r["col_pairs"][:, 1])
    assert np.array_equal(h(s2c), r["slot2col"])


def test_route_bitexact_cases():
    rng = np.random.default_rng(5)
    L8, p8 = route_layer(8, 2, 4, 11)
    cases = [rng.integers(0, 8, (64, 2)), np.full((40, 2), 5), np.array([[3, 3]]),
             np.array([[1, 1], [1, 2], [2, 1]]), rng.integers(0, 3, (300, 4)),
             np.array([[9, -2], [4, 8], [7, 7], [0, 100]]),           # dropped ids
             rng.integers(0, 8, (16384, 2)),                          # T*k = 32768
             rng.integers(0, 8, (65, 2)),                             # smallest multi-workgroup case
             rng.integers(0, 8, (1025, 1)),                           # two slot workgroups, ragged
             np.where(rng.random((2000, 3)) < 0.05, -1,               # dropped ids, repeats
                      rng.integers(0, 9, (2000, 3)))]
    for ids in cases:
        say(f"  route case {ids.shape}")
        check_route_device(L8, p8, ids)
    L64, p64 = route_layer(64, 8, 8, 12)
    cfg = synth.CONFIG_BY_NAME["fine64_zipf_mixed4160"]
    _, ids, _ = synth.make_tokens(cfg, 4160)                           # Zipf(1.1) top-6
    check_route_device(L64, p64, ids)
    check_route_device(L64, p64, rng.integers(0, 64, (1, 6)))
    # one-workgroup lists at the largest token count it takes, and a
    # Qwen-shaped batch (60 experts on 8 x 8, top-4, 512 tokens)
    check_route_device(L8, p8, rng.integers(0, 8, (1024, 4)))
    L60, p60 = route_layer(60, 8, 8, 13)
    qcfg = synth.CONFIG_BY_NAME["qwen15_moe_prefill512"]
    _, qids, _ = synth.make_tokens(qcfg, 512)
    check_route_device(L60, p60, qids)


def test_dropped_ids_counted():
    p, _ = pins.random_struct(8, 2, 4, 128, 32, 8, 32, seed=3)
    L = tqio.upload_layer(single_layer_from(p))
    x, ids, g = pins.tokens(128, 8, 2, 10, seed=4)
    ids = ids.copy()
    ids[2, 1] = 8
    ids[7, 0] = -3
    y, dropped = run_forward(L, x, ids, g, "f16")
    assert dropped == 2
    assert_parity(y, R.forward_single(p, x, ids, g), what="dropped ids")

# ---------------------------------------------------------------------------
# forward parity


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("y_dtype", ["f32", "f16"])
def test_tiny_config(path, y_dtype):
    cfg = synth.CONFIG_BY_NAME["tiny"]
    layer = synth.make_layer(cfg)
    x, ids, g = synth.make_tokens(cfg, 64)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    y, dropped = run_forward(L, x, ids, g, cfg.act, y_dtype)
    assert dropped == 0
    assert_parity(y, R.forward(layer, x, ids, g), y_dtype, what=f"tiny path={path} y={y_dtype}")


@pytest.mark.parametrize("path", [1, 2])
def test_special_cases_single(path):
    """Zero rank (pure dequant GEMM), zero residual (pure low rank), the
    textbook K = M = N = 1 case, duplicates and ragged tails on the device."""
    cases = {
        "rank0": pins.random_struct(8, 2, 4, 256, 64, 0, 64, seed=31)[0],
        "zero_residual": pins.random_struct(8, 2, 4, 256, 64, 16, 64, seed=32, zero_res=True)[0],
        "textbook": pins.random_struct(1, 1, 1, 384, 48, 20, 128, seed=33)[0],
        "rank48_G32": pins.random_struct(6, 3, 3, 1408, 80, 48, 32, seed=34)[0],
        # 32 grid rows at rank 128: the combine's rank-space tile does not
        # fit LDS at once and is built one grid row at a time
        "tall_grid_r128": pins.random_struct(32, 32, 1, 256, 64, 128, 64, seed=35)[0],
    }
    for name, p in cases.items():
        L = tqio.upload_layer(single_layer_from(p))
        L.set_path(path)
        for T, k in [(1, 1), (37, p["K"] > 1 and 2 or 1), (200, 1)]:
            x, ids, g = pins.tokens(p["d_in"], p["K"], k, T, seed=T + k)
            if name == "textbook":
                g = np.ones_like(g)
            y, _ = run_forward(L, x, ids, g, "f16")
            assert_parity(y, R.forward_single(p, x, ids, g), what=f"{name} T={T} k={k}")
        # duplicates: the same expert twice in a token
        x, ids1, g1 = pins.tokens(p["d_in"], p["K"], 1, 9, seed=99)
        ids = np.ascontiguousarray(np.concatenate([ids1, ids1], axis=1))
        g = np.ascontiguousarray(np.concatenate([g1, 0.5 * g1], axis=1))
        y, _ = run_forward(L, x, ids, g, "f16")
        assert_parity(y, R.forward_single(p, x, ids, g), what=f"{name} duplicates")


@pytest.mark.parametrize("path", [1, 2])
def test_empty_and_largest_grid(path):
    """T = 0 is a no-op; the largest grid the library takes (K = 256 experts
    on 32 x 32 = 1024 tiles, rank 128, top-8) at both paths."""
    p, _ = pins.random_struct(256, 32, 32, 128, 32, 128, 64, seed=91)
    layer = single_layer_from(p)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    ws = tqio.workspace(L, 1, 8)
    y0 = torch.full((1, 32), 7.0, device="cuda")
    e32 = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    ef = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    L.forward(torch.empty((0, 128), dtype=torch.float16, device="cuda"), 0, e32, ef, 8, y0,
              tq.TQ_F32, ws)
    torch.cuda.synchronize()
    assert torch.all(y0 == 7.0)                 # nothing written
    T = 200
    x, ids, g = pins.tokens(128, 256, 8, T, seed=92)
    y, _ = run_forward(L, x, ids, g, "f16", "f32")
    assert_parity(y, R.forward_single(p, x, ids, g), what=f"K=256 on 32x32 path={path}")


def test_token_permutation_device():
    p, _ = pins.random_struct(8, 2, 4, 256, 64, 16, 64, seed=41)
    L = tqio.upload_layer(single_layer_from(p))
    x, ids, g = pins.tokens(256, 8, 2, 50, seed=42)
    y, _ = run_forward(L, x, ids, g, "f16")
    pi = np.random.default_rng(0).permutation(50)
    y2, _ = run_forward(L, x[pi], ids[pi], g[pi], "f16")
    assert_parity(y2, y[pi], what="token permutation")


def small_swiglu(act, seed, K=8, M=2, N=4, d_model=256, d_ff=384, r=16, G=64):
    ss = np.random.SeedSequence(seed).spawn(3)
    proj = {n: synth.make_proj(K, M, N, di, do, r, G, act, s)
            for (n, (di, do)), s in zip([("gate", (d_model, d_ff)), ("up", (d_model, d_ff)),
                                         ("down", (d_ff, d_model))], ss)}
    return dict(kind="swiglu", act=act, K=K, d_model=d_model, d_ff=d_ff, proj=proj, shared=None)


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("path", [1, 2])
def test_small_swiglu(act, path):
    layer = small_swiglu(act, 7)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    for T, k in [(1, 2), (45, 2), (300, 3)]:
        x, ids, g = synth.make_custom_tokens(256, 8, k, T, act, seed=T)
        y, _ = run_forward(L, x, ids, g, act, "f32")
        assert_parity(y, R.forward(layer, x, ids, g), what=f"swiglu {act} path={path} T={T}")


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_decode_two_column_tiles(act):
    """Decode gate/up with two 16-slot column tiles per workgroup (taken when
    the slots average 16 or more per active expert, 2-bit codes, group 128):
    skewed routings give experts with an empty second tile, with both tiles
    full, and with more than two tiles (the workgroup's second pass)."""
    layer = small_swiglu(act, 77, G=128)
    L = tqio.upload_layer(layer)
    L.set_path(1)
    for T, k, routing in [(64, 2, "zipf1.1"), (100, 3, "hot70"), (96, 2, "uniform")]:
        x, ids, g = synth.make_custom_tokens(256, 8, k, T, act, seed=T + k, routing=routing)
        counts = np.bincount(ids.reshape(-1), minlength=8)
        y, _ = run_forward(L, x, ids, g, act, "f32")
        assert_parity(y, R.forward(layer, x, ids, g),
                      what=f"two column tiles {act} T={T} k={k} {routing} slots/expert {counts.tolist()}")


@pytest.mark.parametrize("kind", ["single", "swiglu"])
def test_decode_two_fragments_per_wave(kind):
    """Decode residual of a down / single projection with two 16-row
    fragments per wave (taken at decode batch sizes when it allows more
    k-chunks in one round: here 136 or 131 fragments per expert, 8 experts):
    several k-chunks, the 4-step tail stage (d_in % 256 == 128) in the last
    chunk, and for the single layer an odd fragment count (the last wave's
    second fragment is computed but not stored)."""
    ss = np.random.SeedSequence(2024 if kind == "single" else 2025).spawn(3)
    if kind == "single":
        proj = synth.make_proj(8, 2, 4, 4224, 2096, 32, 128, "f16", ss[0])
        layer = dict(kind="single", act="f16", K=8, d_model=4224, d_ff=2096,
                     proj=dict(single=proj), shared=None)
        d_in = 4224
    else:
        proj = {n: synth.make_proj(8, 2, 4, di, do, 32, 128, "f16", q)
                for (n, (di, do)), q in zip([("gate", (2176, 4224)), ("up", (2176, 4224)),
                                             ("down", (4224, 2176))], ss)}
        layer = dict(kind="swiglu", act="f16", K=8, d_model=2176, d_ff=4224, proj=proj, shared=None)
        d_in = 2176
    L = tqio.upload_layer(layer)
    L.set_path(1)
    for T, routing in [(40, "uniform"), (64, "hot70"), (3, "uniform")]:
        x, ids, g = synth.make_custom_tokens(d_in, 8, 2, T, "f16", seed=T, routing=routing)
        y, _ = run_forward(L, x, ids, g, "f16", "f32")
        assert_parity(y, R.forward(layer, x, ids, g, keep_weights=False),
                      what=f"two fragments per wave {kind} T={T} {routing}")
    L.close()


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_decode_workspace_poisoned(act):
    """Decode batches (at most 16 slots per expert on average) on a workspace
    filled with NaN bytes beforehand: nothing the forward reads may be left
    over from earlier contents.  Routings: an expert with more than 32 slots
    (several column tiles), dropped ids (positions past the valid ones), a
    single token, and Zipf top-4."""
    layer = small_swiglu(act, 91, G=128)
    L = tqio.upload_layer(layer)
    L.set_path(1)
    rng = np.random.default_rng(5)
    cases = []
    x, ids, g = synth.make_custom_tokens(256, 8, 2, 64, act, seed=11, routing="hot70")
    cases.append(("hot70 T=64", x, ids, g))
    x, ids, g = synth.make_custom_tokens(256, 8, 2, 40, act, seed=12)
    ids = ids.copy()
    ids[rng.choice(40, 6, replace=False), rng.integers(0, 2, 6)] = rng.choice([-1, 8, 1000], 6)
    cases.append(("dropped T=40", x, ids, g))
    x, ids, g = synth.make_custom_tokens(256, 8, 2, 1, act, seed=13)
    cases.append(("T=1", x, ids, g))
    x, ids, g = synth.make_custom_tokens(256, 8, 4, 32, act, seed=14, routing="zipf1.1")
    cases.append(("zipf top-4 T=32", x, ids, g))
    for what, x, ids, g in cases:
        T, k = ids.shape
        assert T * k <= 16 * 8
        ws = tqio.workspace(L, T, k)
        ws.fill_(0xFF)
        counts = np.bincount(ids[(ids >= 0) & (ids < 8)], minlength=8)
        y, dropped = run_forward(L, x, ids, g, act, "f32", ws=ws)
        assert dropped == int(((ids < 0) | (ids >= 8)).sum())
        assert np.all(np.isfinite(y)), what
        assert_parity(y, R.forward(layer, x, ids, g),
                      what=f"poisoned workspace {act} {what} slots/expert {counts.tolist()}")
    L.close()


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_row_bound(act):
    """The per-expert bound on sum_i |W_e[o][i]| of the effective weight: the
    triangle-inequality sum recomputed here from the stored arrays, and not
    below the oracle's explicitly built weights' largest row sum."""
    layer = small_swiglu(act, 21)
    L = tqio.upload_layer(layer)
    for which, name in enumerate(("gate", "up", "down")):
        proj = layer["proj"][name]
        got = L.debug_row_bound(which).astype(np.float64)
        r, M, N = proj["rank"], proj["M"], proj["N"]
        d_out, d_in = proj["d_out"], proj["d_in"]
        U = R.to_f64(proj["U"], act).reshape(M, d_out, r)
        V = R.to_f64(proj["V"], act).reshape(N, d_in, r)
        sig = np.abs(np.asarray(proj["sigma"], np.float64))
        for e in range(proj["K"]):
            t = int(proj["tile_of_expert"][e])
            m, n = t // N, t % N
            res = np.abs(R.expert_residual(proj, e)).sum(axis=1)
            lr = (np.abs(U[m]) * sig) @ np.abs(V[n]).sum(axis=0)
            want = float((res + lr).max())
            true = float(np.abs(R.expert_weight(proj, e)).sum(axis=1).max())
            assert abs(got[e] - want) <= 1e-4 * want, (name, e, got[e], want)
            assert got[e] >= true * (1 - 1e-5), (name, e, got[e], true)


@pytest.mark.parametrize("path", [1, 2])
def test_bf16_swiglu_token_magnitudes(path):
    """bfloat16 tokens far outside the fp16 range (powers of two from 2^-40 to
    2^40 per token group): every group within the bar relative to its own
    outputs (the fp16 operands carry per-row power-of-two exponents)."""
    layer = small_swiglu("bf16", 23)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    T = 24 if path == 1 else 300
    x, ids, g = synth.make_custom_tokens(256, 8, 2, T, "bf16", seed=31)
    shifts = np.array([-40, -12, 0, 9, 40])
    grp = np.arange(T) % len(shifts)
    x32 = synth.act_as_f32(x, "bf16") * np.ldexp(1.0, shifts[grp])[:, None].astype(np.float32)
    xs = synth.to_act(x32, "bf16")
    y, _ = run_forward(L, xs, ids, g, "bf16", "f32")
    ref = R.forward(layer, xs, ids, g)
    for i, sh in enumerate(shifts):
        rows = grp == i
        assert_parity(y[rows], ref[rows], what=f"bf16 tokens x 2^{sh} path={path}")


@pytest.mark.parametrize("kind", ["swiglu", "single"])
def test_prefill_column_stage_k_split(kind):
    """Prefill with 2048-wide inputs to the projection whose rank vectors go to
    the combine: its column stage runs in k-range splits (fp32 slabs summed by
    the combine)."""
    if kind == "swiglu":
        layer = small_swiglu("f16", 41, d_model=256, d_ff=2048)
        d_in = 256
    else:
        layer = single_layer_from(synth.make_proj(8, 2, 4, 2048, 256, 32, 64, "f16",
                                                  np.random.SeedSequence(43)))
        d_in = 2048
    L = tqio.upload_layer(layer)
    L.set_path(2)
    x, ids, g = synth.make_custom_tokens(d_in, 8, 2, 300, "f16", seed=44)
    y, _ = run_forward(L, x, ids, g, "f16", "f32")
    assert_parity(y, R.forward(layer, x, ids, g), what=f"{kind} prefill, column stage k-split")


@pytest.mark.parametrize("scheme", ["per_expert", "shared_u", "shared_v", "rank0"])
@pytest.mark.parametrize("path", [1, 2])
def test_weight_schemes(scheme, path):
    """The comparison schemes of the low-rank part (per-expert factors, one
    factor shared by all experts, none) as tile maps through the same path."""
    from types import SimpleNamespace
    K = 8
    M, N, tiles = synth.scheme_grid(SimpleNamespace(K=K, M=2, N=4), scheme)
    r = 0 if scheme == "rank0" else 16
    ss = np.random.SeedSequence(51).spawn(3)
    proj = {n: synth.make_proj(K, M, N, di, do, r, 64, "f16", q, tiles=tiles)
            for (n, (di, do)), q in zip([("gate", (256, 384)), ("up", (256, 384)),
                                         ("down", (384, 256))], ss)}
    layer = dict(kind="swiglu", act="f16", K=K, d_model=256, d_ff=384, proj=proj, shared=None)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    T = 24 if path == 1 else 300
    x, ids, g = synth.make_custom_tokens(256, K, 2, T, "f16", seed=52)
    y, _ = run_forward(L, x, ids, g, "f16", "f32")
    assert_parity(y, R.forward(layer, x, ids, g), what=f"scheme {scheme} path={path}")


@pytest.mark.parametrize("K,k", [(8, 2), (60, 4), (64, 6), (256, 8), (5, 5), (128, 32), (16, 1)])
def test_router_topk(K, k):
    """Router: ids bit-exact with the oracle (ties from rounded logits, NaN and
    -inf rows included), weights within 1e-6; then its outputs drive a
    forward."""
    rng = np.random.default_rng(81 + K + k)
    T = 700
    L = rng.standard_normal((T, K)).astype(np.float32)
    L[:100] = np.round(L[:100] * 2) / 2
    L[100, :] = np.nan
    L[101, :] = -np.inf
    L[102, ::2] = np.nan
    ld = torch.from_numpy(L).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    tq.router_topk(ld, k, ids, w)
    torch.cuda.synchronize()
    want_ids, want_w = R.router_topk(L, k)
    assert np.array_equal(ids.cpu().numpy(), want_ids)
    err = float(np.max(np.abs(w.cpu().numpy().astype(np.float64) - want_w)))
    say(f"  router K={K} k={k}: ids exact, max|dw| = {err:.2e}")
    assert err <= 1e-6


def test_router_feeds_forward():
    layer = small_swiglu("f16", 61)
    L = tqio.upload_layer(layer)
    T, k = 300, 2
    x, _, _ = synth.make_custom_tokens(256, 8, k, T, "f16", seed=62)
    logits = np.random.default_rng(63).standard_normal((T, 8)).astype(np.float32)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    tq.router_topk(torch.from_numpy(logits).cuda(), k, ids, w)
    xd = tqio.to_device(x, "f16")
    y = torch.empty((T, 256), dtype=torch.float32, device="cuda")
    ws = tqio.workspace(L, T, k)
    L.forward(xd, T, ids, w, k, y, tq.TQ_F32, ws)
    torch.cuda.synchronize()
    rid, rw = R.router_topk(logits, k)
    assert_parity(y.cpu().numpy().astype(np.float64), R.forward(layer, x, rid, rw),
                  what="router -> forward")


@pytest.mark.parametrize("path,T,k", [(1, 1, 2), (1, 24, 2), (1, 64, 2), (2, 300, 2), (1, 16, 8),
                                      (2, 200, 8)])
def test_forward_from_logits(path, T, k):
    """The router fused into the forward (inside the first decode launch at
    decode batch sizes, one launch ahead otherwise): its ids and weights equal
    the standalone router's bit for bit, and y equals the two-call forward's
    bit for bit and the oracle's within the bar."""
    layer = small_swiglu("f16", 61)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    x, _, _ = synth.make_custom_tokens(256, 8, k, T, "f16", seed=64 + T)
    logits = np.random.default_rng(65 + T).standard_normal((T, 8)).astype(np.float32)
    logits[0, :4] = 0.25                     # ties go to the lower id
    ld = torch.from_numpy(logits).cuda()
    xd = tqio.to_device(x, "f16")
    ids_a = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w_a = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    y_a = torch.empty((T, 256), dtype=torch.float32, device="cuda")
    ws = tqio.workspace(L, T, k)
    L.forward_from_logits(xd, T, ld, k, ids_a, w_a, y_a, tq.TQ_F32, ws)
    ids_b = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_b = torch.empty((T, k), dtype=torch.float32, device="cuda")
    tq.router_topk(ld, k, ids_b, w_b)
    y_b = torch.empty((T, 256), dtype=torch.float32, device="cuda")
    L.forward(xd, T, ids_b, w_b, k, y_b, tq.TQ_F32, ws)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b)
    assert torch.equal(y_a, y_b)
    rid, rw = R.router_topk(logits, k)
    assert np.array_equal(ids_a.cpu().numpy(), rid)
    assert np.max(np.abs(w_a.cpu().numpy() - rw)) <= 1e-6
    assert_parity(y_a.cpu().numpy().astype(np.float64), R.forward(layer, x, rid, rw),
                  what=f"router fused into the forward, path={path} T={T} k={k}")


@pytest.mark.parametrize("path,T", [(1, 24), (2, 300)])
def test_small_swiglu_with_shared_expert(path, T):
    """The shared expert (on the layer's second stream) at decode and prefill."""
    layer = small_swiglu("f16", 9)
    layer["shared"] = synth.make_shared(256, 384, np.random.SeedSequence(12))
    L = tqio.upload_layer(layer)
    L.set_path(path)
    x, ids, g = synth.make_custom_tokens(256, 8, 2, T, "f16", seed=T + 1)
    y, _ = run_forward(L, x, ids, g, "f16", "f32")
    assert_parity(y, R.forward(layer, x, ids, g), what=f"swiglu + shared path={path} T={T}")


@pytest.mark.parametrize("path,T", [(1, 40), (2, 200)])
def test_shared_expert_partial_tiles(path, T):
    """Dense shared expert whose down projection ends in a partial 256-row
    weight tile (d_model 384), 5 dual weight tiles dealt over the 8 XCDs,
    and a ragged last 128-token tile."""
    layer = small_swiglu("f16", 21, d_model=384)
    layer["shared"] = synth.make_shared(384, 640, np.random.SeedSequence(22))
    L = tqio.upload_layer(layer)
    L.set_path(path)
    x, ids, g = synth.make_custom_tokens(384, 8, 2, T, "f16", seed=T + 3)
    y, _ = run_forward(L, x, ids, g, "f16", "f32")
    assert_parity(y, R.forward(layer, x, ids, g), what=f"shared partial tiles path={path} T={T}")


def test_qwen15_prefill512_with_shared_expert():
    cfg = synth.CONFIG_BY_NAME["qwen15_moe_prefill512"]
    layer = synth.make_layer(cfg)
    x, ids, g = synth.make_tokens(cfg, 512)
    L = tqio.upload_layer(layer)
    y, _ = run_forward(L, x, ids, g, cfg.act, "f16")
    say("  oracle (all 512 tokens)")
    assert_parity(y, R.forward(layer, x, ids, g), "f16", what="qwen15 prefill512")


def test_fine64_zipf_mixed4160_sampled():
    cfg = synth.CONFIG_BY_NAME["fine64_zipf_mixed4160"]
    layer = synth.make_layer(cfg)
    x, ids, g = synth.make_tokens(cfg, 4160)
    L = tqio.upload_layer(layer)
    y, _ = run_forward(L, x, ids, g, cfg.act, "f16")
    tok = np.concatenate([np.arange(0, 4096, 37), np.arange(4096, 4160)])
    say(f"  oracle on {len(tok)} sampled tokens")
    assert_parity(y[tok], R.forward(layer, x, ids, g, tokens=tok), "f16",
                  what="fine64 zipf 4160 (sampled)")


@pytest.fixture(scope="module")
def mixtral_f16():
    cfg = synth.CONFIG_BY_NAME["mixtral8x7b_decode"]
    layer = synth.make_layer(cfg)
    # the batches B = 1, 8, 32 are prefixes of the 64-token batch (the token
    # generator extends a smaller batch), so one oracle pass over 64 tokens
    # gives every token of every batch
    x, ids, g = synth.make_tokens(cfg, 64)
    say("  oracle (Mixtral-shaped layer, all 64 tokens)")
    ref = R.forward(layer, x, ids, g, keep_weights=False)
    return cfg, layer, tqio.upload_layer(layer), ref


@pytest.mark.parametrize("B", [1, 8, 32, 64])
def test_mixtral_decode(mixtral_f16, B):
    """Every token of the batch, at each decode batch size of the metric."""
    cfg, layer, L, ref = mixtral_f16
    x, ids, g = synth.make_tokens(cfg, B)
    x64, ids64, _ = synth.make_tokens(cfg, 64)
    assert np.array_equal(ids, ids64[:B]) and np.array_equal(x, x64[:B])
    y, _ = run_forward(L, x, ids, g, cfg.act, "f16")
    assert_parity(y, ref[:B], "f16", what=f"mixtral decode B={B} (all tokens)")


def tile_tokens(ids, K, tile=128):
    """For every expert: the tokens of the first slot of its first slot tile,
    of a slot in the middle of a full tile and of the last slot of its last
    (ragged) tile, with slots ordered by (expert, token, j) as the routing
    groups them."""
    flat = ids.reshape(-1)
    k = ids.shape[1]
    tok = set()
    for e in range(K):
        slots = np.nonzero(flat == e)[0]               # ascending slot id = (t, j) order
        if len(slots) == 0:
            continue
        last_tile = (len(slots) - 1) // tile
        picks = [0, len(slots) - 1, min(len(slots) - 1, tile // 2),
                 last_tile * tile, min(len(slots) - 1, max(0, last_tile - 1) * tile + 77)]
        tok.update(int(slots[i]) // k for i in picks)
    return np.array(sorted(tok))


def test_mixtral_prefill16k_bf16_every_expert_tile():
    cfg = synth.CONFIG_BY_NAME["mixtral8x7b_prefill16k_bf16"]
    layer = synth.make_layer(cfg)
    x, ids, g = synth.make_tokens(cfg, 16384)
    L = tqio.upload_layer(layer)
    ws = tqio.workspace(L, 16384, 2)
    y32, _ = run_forward(L, x, ids, g, cfg.act, "f32", ws=ws)
    yb, _ = run_forward(L, x, ids, g, cfg.act, "bf16", ws=ws)
    tok = tile_tokens(ids, cfg.K)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.K)
    covered = set(ids[tok].reshape(-1).tolist())
    assert covered == set(np.nonzero(counts)[0].tolist())
    say(f"  slots per expert {counts.tolist()}; oracle on {len(tok)} tokens covering the "
        f"first, a full and the last (ragged) 128-slot tile of every expert")
    ref = R.forward(layer, x, ids, g, tokens=tok, keep_weights=False)
    assert_parity(y32[tok], ref, "f32", what="mixtral prefill16k bf16 (y f32)")
    assert_parity(yb[tok], ref, "bf16", what="mixtral prefill16k bf16 (y bf16)")


# ---------------------------------------------------------------------------
# 3-bit residual codes (the pages' 3-bit setting, technical summary section 4)


def test_dequant3_exhaustive_fp16_scales():
    """3-bit codes: every finite fp16 scale with |s| < 1024 (both signs) x
    every integer zero point 0..7 x every code, through the forward's own
    unpack path (packed dequantization), bit-exact."""
    sbits = np.concatenate([np.arange(0x0000, 0x6400), np.arange(0x8000, 0xE400)]).astype(np.uint16)
    rows, G, d_in = len(sbits), 32, 256
    s = np.repeat(sbits[:, None], 8, axis=1).view(np.float16)[None]
    z = np.tile(np.arange(8, dtype=np.float16), (rows, 1))[None]
    i = np.arange(d_in)[None, :]
    o = np.arange(rows)[:, None]
    q = ((i + o + i // 8) % 8)[None]
    p = pins.proj_from(q, s, z, np.zeros((rows, 0), np.float16), [],
                       np.zeros((d_in, 0), np.float16), [0], 1, 1, G, bits=3)
    L = tqio.upload_layer(single_layer_from(p))
    w = torch.empty((rows, d_in), dtype=torch.float16, device="cuda")
    L.debug_dequant(0, 0, w)
    torch.cuda.synchronize()
    got = w.cpu().numpy().view(np.uint16)
    want = R.deq_canonical(q[0], s[0], z[0], G, "f16").astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5])


@pytest.mark.parametrize("zset", range(len(ZERO_SETS)))
def test_dequant3_exhaustive_general(zset):
    """3-bit codes through the table dequantization: every finite fp16 scale
    against fractional and out-of-range zero points wherever the weights stay
    finite, bit-exact; d_in = 384 has a 4-step tail group."""
    zs = np.array(ZERO_SETS[zset] + ZERO_SETS[(zset + 1) % len(ZERO_SETS)], np.float16)
    sbits = np.concatenate([np.arange(0x0000, 0x7C00), np.arange(0x8000, 0xFC00)]).astype(np.uint16)
    sv = sbits.view(np.float16)
    q8 = np.arange(8)[None, None, :]
    deq = R.deq_canonical(np.broadcast_to(q8, (len(sv), 8, 8)).reshape(len(sv), 64),
                          np.repeat(sv[:, None], 8, axis=1), np.tile(zs, (len(sv), 1)), 8)
    sv = sv[np.all(np.isfinite(deq), axis=1)]
    rows = len(sv) - len(sv) % 16
    sv = sv[:rows]
    G, d_in = 32, 384
    ng = d_in // G
    s = np.repeat(sv[:, None], ng, axis=1)[None]
    z = np.tile(np.resize(zs, ng), (rows, 1))[None]
    i = np.arange(d_in)[None, :]
    o = np.arange(rows)[:, None]
    q = ((3 * i + o + i // 8) % 8)[None]
    p = pins.proj_from(q, s, z, np.zeros((rows, 0), np.float16), [],
                       np.zeros((d_in, 0), np.float16), [0], 1, 1, G, bits=3)
    say(f"  3-bit, zero points {tuple(float(v) for v in zs)}: {rows} scales")
    L = tqio.upload_layer(single_layer_from(p))
    w = torch.empty((rows, d_in), dtype=torch.float16, device="cuda")
    L.debug_dequant(0, 0, w)
    torch.cuda.synchronize()
    got = w.cpu().numpy().view(np.uint16)
    want = R.deq_canonical(q[0], s[0], z[0], G, "f16").astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5])


@pytest.mark.parametrize("path", [1, 2])
def test_special_cases_single_3bit(path):
    """3-bit residuals: zero rank, zero residual, a 4-step tail group
    (d_in = 384), group sizes 32 and 128, ragged slot tiles, duplicates,
    fractional zero points (table dequantization)."""
    cases = {
        "rank0": pins.random_struct(8, 2, 4, 256, 64, 0, 64, seed=131, bits=3)[0],
        "zero_residual": pins.random_struct(8, 2, 4, 256, 64, 16, 64, seed=132, zero_res=True,
                                            bits=3)[0],
        "tail_G128": pins.random_struct(4, 2, 2, 384, 48, 20, 128, seed=133, bits=3)[0],
        "r48_G32": pins.random_struct(6, 3, 3, 1408, 80, 48, 32, seed=134, bits=3)[0],
    }
    p = dict(cases["r48_G32"])
    rng = np.random.default_rng(135)
    p["zeros"] = rng.uniform(-2.0, 9.0, p["zeros"].shape).astype(np.float16)
    cases["fractional_z"] = p
    for name, p in cases.items():
        L = tqio.upload_layer(single_layer_from(p))
        L.set_path(path)
        for T, k in [(1, 1), (37, 2), (200, 1)]:
            x, ids, g = pins.tokens(p["d_in"], p["K"], k, T, seed=T + k)
            y, _ = run_forward(L, x, ids, g, "f16")
            assert_parity(y, R.forward_single(p, x, ids, g), what=f"3-bit {name} T={T} k={k}")
        x, ids1, g1 = pins.tokens(p["d_in"], p["K"], 1, 9, seed=99)
        ids = np.ascontiguousarray(np.concatenate([ids1, ids1], axis=1))
        g = np.ascontiguousarray(np.concatenate([g1, 0.5 * g1], axis=1))
        y, _ = run_forward(L, x, ids, g, "f16")
        assert_parity(y, R.forward_single(p, x, ids, g), what=f"3-bit {name} duplicates")


def small_swiglu_bits(act, seed, bits, K=8, M=2, N=4, d_model=256, d_ff=384, r=16, G=64):
    ss = np.random.SeedSequence(seed).spawn(3)
    proj = {n: synth.make_proj(K, M, N, di, do, r, G, act, s, bits=b)
            for (n, (di, do)), s, b in zip([("gate", (d_model, d_ff)), ("up", (d_model, d_ff)),
                                            ("down", (d_ff, d_model))], ss, bits)}
    return dict(kind="swiglu", act=act, K=K, d_model=d_model, d_ff=d_ff, proj=proj, shared=None)


@pytest.mark.parametrize("bits", [(3, 3, 3), (3, 3, 2), (2, 2, 3)])
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("path", [1, 2])
def test_small_swiglu_3bit(bits, act, path):
    """SwiGLU with 3-bit residuals, alone and with the down projection at
    the other width (gate and up share one fused kernel and one width)."""
    layer = small_swiglu_bits(act, 171, bits)
    L = tqio.upload_layer(layer)
    L.set_path(path)
    for T, k in [(1, 2), (45, 2), (300, 3)]:
        x, ids, g = synth.make_custom_tokens(256, 8, k, T, act, seed=T + 5)
        y, _ = run_forward(L, x, ids, g, act, "f32")
        assert_parity(y, R.forward(layer, x, ids, g),
                      what=f"swiglu bits={bits} {act} path={path} T={T}")


def test_gate_up_widths_must_match():
    layer = small_swiglu_bits("f16", 172, (2, 3, 3))
    L = tqio.upload_layer(layer)
    x, ids, g = synth.make_custom_tokens(256, 8, 2, 4, "f16", seed=3)
    with pytest.raises(tq.TileQError, match="one width"):
        run_forward(L, x, ids, g, "f16", "f32", ws=torch.empty(1 << 20, dtype=torch.uint8,
                                                               device="cuda"))


@pytest.fixture(scope="module")
def mixtral_3bit():
    cfg = synth.CONFIG_BY_NAME["mixtral8x7b_decode"]
    layer = synth.make_layer(cfg, bits=3)
    x, ids, g = synth.make_tokens(cfg, 64)
    say("  oracle (Mixtral-shaped layer, 3-bit residuals, all 64 tokens)")
    ref = R.forward(layer, x, ids, g, keep_weights=False)
    return cfg, layer, tqio.upload_layer(layer), ref


@pytest.mark.parametrize("B", [1, 32, 64])
def test_mixtral_decode_3bit(mixtral_3bit, B):
    cfg, layer, L, ref = mixtral_3bit
    x, ids, g = synth.make_tokens(cfg, B)
    y, _ = run_forward(L, x, ids, g, cfg.act, "f16")
    assert_parity(y, ref[:B], "f16", what=f"mixtral decode 3-bit B={B} (all tokens)")


def test_mixtral_prefill16k_bf16_3bit_every_expert_tile():
    cfg = synth.CONFIG_BY_NAME["mixtral8x7b_prefill16k_bf16"]
    layer = synth.make_layer(cfg, bits=3)
    x, ids, g = synth.make_tokens(cfg, 16384)
    L = tqio.upload_layer(layer)
    y32, _ = run_forward(L, x, ids, g, cfg.act, "f32")
    tok = tile_tokens(ids, cfg.K)
    say(f"  3-bit 16k prefill: oracle on {len(tok)} tokens (every expert's first, full and last tile)")
    ref = R.forward(layer, x, ids, g, tokens=tok, keep_weights=False)
    assert_parity(y32[tok], ref, "f32", what="mixtral prefill16k bf16 3-bit (y f32)")
