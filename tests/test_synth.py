"""The seeded generators: determinism, storage format and the prefix
property (more tokens extend fewer)."""
import numpy as np

import synth
from oracle import tileq_ref


def test_tiny_layer_deterministic_and_well_formed():
    cfg = synth.CONFIG_BY_NAME["tiny"]
    a = synth.make_layer(cfg)
    b = synth.make_layer(cfg)
    p, q = a["proj"]["single"], b["proj"]["single"]
    for key in ("tile_of_expert", "U", "sigma", "V", "codes", "scales", "zeros"):
        assert np.array_equal(p[key], q[key]), key
    assert p["U"].shape == (2 * 512, 16) and p["V"].shape == (4 * 256, 16)
    assert p["codes"].shape == (8, 512, 256 // 16) and p["codes"].dtype == np.uint32
    assert p["scales"].shape == (8, 512, 256 // 64)
    assert len(set(p["tile_of_expert"].tolist())) == 8
    assert p["tile_of_expert"].min() >= 0 and p["tile_of_expert"].max() < 8
    z = p["zeros"].astype(np.float64)
    assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= 3
    assert np.all(np.diff(p["sigma"]) <= 0)
    assert 0.1 <= p["sigma"].min() and p["sigma"].max() <= 10.01


def test_residual_quantizer_error_bound():
    """RTN with an integer zero point: |w - s(q - z)| <= s/2 except where the
    zero point's rounding clips the range (then <= s)."""
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    q, s, z = synth.quantize_rtn_2bit(w, 64)
    deq = tileq_ref.residual(q.astype(np.int64), s, z, 64)
    sf = np.repeat(s.astype(np.float64), 64, axis=-1)
    assert np.all(np.abs(w - deq) <= sf * 1.0 + 1e-12)
    assert np.mean(np.abs(w - deq) <= sf * 0.5 + 1e-12) > 0.9


def test_tokens_prefix_and_routing():
    cfg = synth.CONFIG_BY_NAME["mixtral8x7b_decode"]
    x8, ids8, g8 = synth.make_tokens(cfg, 8)
    x32, ids32, g32 = synth.make_tokens(cfg, 32)
    assert np.array_equal(x8, x32[:8])
    assert np.array_equal(ids8, ids32[:8]) and np.array_equal(g8, g32[:8])
    assert ids32.shape == (32, 2) and np.all(ids32[:, 0] != ids32[:, 1])
    assert np.allclose(g32.sum(axis=1), 1.0, atol=1e-6)


def test_skewed_routing_shapes():
    cfg = synth.CONFIG_BY_NAME["fine64_zipf_mixed4160"]
    _, ids, _ = synth.make_tokens(cfg, 4160)
    cnt = np.bincount(ids.reshape(-1), minlength=64)
    assert cnt.sum() == 4160 * 6
    assert cnt.max() / np.median(cnt) > 8          # heavy skew
    cfg = synth.CONFIG_BY_NAME["mixtral8x7b_prefill16k_bf16"]
    x, ids, _ = synth.make_tokens(cfg, 2048)
    assert x.dtype == np.uint16
    cnt = np.bincount(ids.reshape(-1), minlength=8)
    hot = np.sort(cnt)[-4:].sum() / cnt.sum()
    assert 0.6 < hot < 0.8


def test_weight_scheme_maps():
    """Each comparison scheme is an injective tile map on its grid: per-expert
    factors put expert e alone in grid row e and column e; shared_u puts every
    expert in grid row 0 (one U), shared_v in grid column 0 (one V)."""
    cfg = synth.CONFIG_BY_NAME["mixtral8x7b_decode"]
    K = cfg.K
    for scheme in synth.SCHEMES:
        M, N, tiles = synth.scheme_grid(cfg, scheme)
        if tiles is None:
            assert (M, N) == (cfg.M, cfg.N)
            continue
        assert len(set(tiles.tolist())) == K and tiles.min() >= 0 and tiles.max() < M * N
        rows, cols = tiles // N, tiles % N
        if scheme == "per_expert":
            assert (M, N) == (K, K) and list(rows) == list(range(K)) and list(cols) == list(range(K))
        elif scheme == "shared_u":
            assert M == 1 and set(rows.tolist()) == {0} and sorted(cols.tolist()) == list(range(K))
        else:
            assert N == 1 and set(cols.tolist()) == {0} and sorted(rows.tolist()) == list(range(K))
