"""Seeded synthetic inputs for the TileQ MoE-layer forward.

Source: "TileQ: Efficient Low-Rank Quantization of Mixture-of-Experts with 2D
Tiling" (gist.science technical summary, section 2.1 steps 3-5 and the "Key
Technical Insight" paragraph): K experts sit on an M x N tile grid, experts of a
grid row share a left (output-space) factor, experts of a grid column share a
right (input-space) factor, one global Sigma, and each expert stores a
quantized residual.

This module only draws random numbers and lays them out in the storage format
that the forward consumes.  It holds none of the forward's arithmetic, so both
the CPU oracle tests and the GPU path can take their inputs from it.

Storage format produced here (the format the C ABI accepts):
  tile_of_expert  int32 [K]              tile = m*N + n, injective, need not be onto
  U               act   [M*d_out][r]     block m = rows m*d_out ... (m+1)*d_out-1
  sigma           f32   [r]              descending, values representable in fp16
  V               act   [N*d_in][r]      block n = rows n*d_in ... (n+1)*d_in-1
  codes           u32   [K][d_out][d_in/16]  code of input i at bits 2*(i%16)
                  (3-bit variant: [K][d_out][3*d_in/32], code i at bits 3i..3i+2
                  of the row's little-endian bit string)
  scales, zeros   f16   [K][d_out][d_in/G]   zeros are integers 0..3 (0..7)
  x               act   [T][d_model]
  ids             int32 [T][k],  gates f32 [T][k]
"act" is float16, or bfloat16 carried as its uint16 bit pattern.

Seeding: numpy PCG64 seeded from SeedSequence(20260512 + config index), with
independent spawned streams for every projection's map, U, sigma, V and
residual (one stream per expert), for the activations and for the routing, so
that the token count never changes the weights, and a larger token count
extends a smaller one (row prefixes agree).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BASE_SEED = 20260512

# ----------------------------------------------------------------------------
# configurations


@dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int
    kind: str            # "single" (one projection) or "swiglu" (gate, up, down)
    K: int
    M: int
    N: int
    d_model: int         # single: d_in;  swiglu: hidden size
    d_ff: int            # single: d_out; swiglu: expert FFN width
    rank: int
    group: int
    act: str             # "f16" or "bf16"
    topk: int
    tokens: tuple        # token counts the configuration is run at
    routing: str         # "uniform", "zipf1.1" or "hot70"
    shared_ff: int = 0   # dense fp16 shared expert width (0: none)

    def proj_shapes(self):
        """Return {name: (d_in, d_out)} for the projections of the layer."""
        if self.kind == "single":
            return {"single": (self.d_model, self.d_ff)}
        return {"gate": (self.d_model, self.d_ff),
                "up": (self.d_model, self.d_ff),
                "down": (self.d_ff, self.d_model)}


CONFIGS = [
    LayerConfig("tiny", 0, "single", K=8, M=2, N=4, d_model=256, d_ff=512,
                rank=16, group=64, act="f16", topk=2, tokens=(64,),
                routing="uniform"),
    LayerConfig("mixtral8x7b_decode", 1, "swiglu", K=8, M=2, N=4,
                d_model=4096, d_ff=14336, rank=64, group=128, act="f16",
                topk=2, tokens=(1, 8, 32), routing="uniform"),
    LayerConfig("qwen15_moe_prefill512", 2, "swiglu", K=60, M=8, N=8,
                d_model=2048, d_ff=1408, rank=32, group=128, act="f16",
                topk=4, tokens=(512,), routing="uniform", shared_ff=5632),
    LayerConfig("fine64_zipf_mixed4160", 3, "swiglu", K=64, M=8, N=8,
                d_model=2048, d_ff=1408, rank=48, group=64, act="f16",
                topk=6, tokens=(4096 + 64,), routing="zipf1.1"),
    LayerConfig("mixtral8x7b_prefill16k_bf16", 4, "swiglu", K=8, M=2, N=4,
                d_model=4096, d_ff=14336, rank=128, group=128, act="bf16",
                topk=2, tokens=(16384,), routing="hot70"),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}

# ----------------------------------------------------------------------------
# dtype helpers (storage only)


def to_act(a32: np.ndarray, act: str) -> np.ndarray:
    """Store float32 values in the activation format (RNE)."""
    if act == "f16":
        return a32.astype(np.float16)
    if act == "bf16":
        u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32)
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(act)


def act_as_f32(a: np.ndarray, act: str) -> np.ndarray:
    """Read the activation format back as float32 (exact)."""
    if act == "f16":
        return a.astype(np.float32)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_codes(q: np.ndarray, bits: int = 2) -> np.ndarray:
    """Pack residual codes [..., d_in] into uint32 words.  bits = 2 (values
    0..3): [..., d_in/16], code i at bits 2*(i % 16) of word i // 16.
    bits = 3 (values 0..7): [..., 3*d_in/32], the row as a little-endian bit
    string with code i at bits 3i .. 3i+2 (bit n = bit n % 32 of word n // 32)."""
    d_in = q.shape[-1]
    if bits == 2:
        assert d_in % 16 == 0
        q4 = q.reshape(q.shape[:-1] + (d_in // 16, 16)).astype(np.uint32)
        shifts = (2 * np.arange(16, dtype=np.uint32))
        return np.bitwise_or.reduce(q4 << shifts, axis=-1).astype(np.uint32)
    assert bits == 3 and d_in % 32 == 0
    qb = np.asarray(q, np.uint32)
    stream = np.stack([(qb >> np.uint32(j)) & np.uint32(1) for j in range(3)], axis=-1)
    stream = stream.reshape(q.shape[:-1] + (3 * d_in // 32, 32))
    return np.bitwise_or.reduce(stream << np.arange(32, dtype=np.uint32), axis=-1).astype(np.uint32)


def _threads():
    return max(1, min(16, os.cpu_count() or 1))

# ----------------------------------------------------------------------------
# projection weights


def quantize_rtn(w: np.ndarray, group: int, bits: int = 2):
    """Round-to-nearest asymmetric group quantization of w [rows][d_in] along
    d_in to codes 0..Q, Q = 2^bits - 1 (the synthetic residuals' generator).
    Per group: mn = min(min w, 0), mx = max(max w, 0), s = fp16((mx - mn) / Q)
    (1 where it would be 0), z = clamp(rint(-mn/s), 0, Q),
    q = clamp(rint(w/s) + z, 0, Q).  Returns (q uint8, s f16, z f16)."""
    qmax = (1 << bits) - 1
    rows, d_in = w.shape
    wg = w.reshape(rows, d_in // group, group)
    mn = np.minimum(wg.min(axis=2), 0.0)
    mx = np.maximum(wg.max(axis=2), 0.0)
    s16 = ((mx - mn) / np.float32(qmax)).astype(np.float16)
    s16[s16 == 0] = np.float16(1.0)
    s32 = s16.astype(np.float32)
    z = np.clip(np.rint(-mn / s32), 0, qmax)
    q = np.clip(np.rint(wg / s32[..., None]) + z[..., None], 0, qmax)
    return q.reshape(rows, d_in).astype(np.uint8), s16, z.astype(np.float16)


def quantize_rtn_2bit(w: np.ndarray, group: int):
    """quantize_rtn with 2-bit codes."""
    return quantize_rtn(w, group, 2)


def _residual_expert(ss, d_out, d_in, group, std, bits=2):
    rng = np.random.default_rng(ss)
    codes = np.empty((d_out, bits * d_in // 32), np.uint32)
    scales = np.empty((d_out, d_in // group), np.float16)
    zeros = np.empty((d_out, d_in // group), np.float16)
    step = max(1, (1 << 22) // d_in)           # bounded temporaries
    for r0 in range(0, d_out, step):
        r1 = min(d_out, r0 + step)
        w = rng.standard_normal((r1 - r0, d_in), dtype=np.float32) * np.float32(std)
        q, s, z = quantize_rtn(w, group, bits)
        codes[r0:r1] = pack_codes(q, bits)
        scales[r0:r1] = s
        zeros[r0:r1] = z
    return codes, scales, zeros


def make_proj(K, M, N, d_in, d_out, rank, group, act, seedseq,
              residual_std=0.02, threads=None, tiles=None, bits=2):
    """One projection's uploaded arrays (see module docstring).  tiles: the
    expert -> tile map (default: a random injective map); bits: residual code
    width (2, or 3 for the pages' 3-bit setting)."""
    assert K <= M * N and d_in % group == 0 and d_in % 16 == 0
    ss_map, ss_u, ss_sig, ss_v, ss_res = seedseq.spawn(5)
    if tiles is None:
        tiles = np.random.default_rng(ss_map).permutation(M * N)[:K].astype(np.int32)
    else:
        tiles = np.asarray(tiles, np.int32)
    U = np.random.default_rng(ss_u).standard_normal(
        (M * d_out, rank), dtype=np.float32) / np.float32(np.sqrt(d_out))
    V = np.random.default_rng(ss_v).standard_normal(
        (N * d_in, rank), dtype=np.float32) / np.float32(np.sqrt(d_in))
    lo, hi = np.log(0.1), np.log(10.0)
    sig = np.exp(np.random.default_rng(ss_sig).uniform(lo, hi, size=rank))
    sig = np.sort(sig)[::-1].astype(np.float16).astype(np.float32)
    res_ss = ss_res.spawn(K)
    with ThreadPoolExecutor(threads or _threads()) as ex:
        parts = list(ex.map(lambda s: _residual_expert(s, d_out, d_in, group,
                                                       residual_std, bits), res_ss))
    return dict(K=K, M=M, N=N, d_in=d_in, d_out=d_out, rank=rank, group=group,
                bits=bits, act=act, tile_of_expert=tiles,
                U=to_act(U, act), sigma=np.ascontiguousarray(sig),
                V=to_act(V, act),
                codes=np.stack([p[0] for p in parts]),
                scales=np.stack([p[1] for p in parts]),
                zeros=np.stack([p[2] for p in parts]))


def _streams(cfg: LayerConfig):
    root = np.random.SeedSequence(BASE_SEED + cfg.index)
    names = ["single_or_gate", "up", "down", "shared", "x", "routing"]
    return dict(zip(names, root.spawn(len(names))))


# Weight-sharing schemes of the low-rank part, all expressed as tile maps
# (the same kernels and routing serve every one):
#   tileq       the configuration's M x N grid, random injective map
#   rank0       no low-rank part (pure 2-bit residual MoE)
#   per_expert  every expert its own U and V: K x K grid, expert e at (e, e)
#   shared_u    one U for all experts, V per expert: 1 x K grid, e at (0, e)
#   shared_v    one V for all experts, U per expert: K x 1 grid, e at (e, 0)
SCHEMES = ("tileq", "rank0", "per_expert", "shared_u", "shared_v")


def scheme_grid(cfg: LayerConfig, scheme: str):
    """(M, N, tiles or None) of a weight-sharing scheme."""
    K = cfg.K
    e = np.arange(K, dtype=np.int32)
    if scheme in ("tileq", "rank0"):
        return cfg.M, cfg.N, None
    if scheme == "per_expert":
        return K, K, e * K + e
    if scheme == "shared_u":
        return 1, K, e
    if scheme == "shared_v":
        return K, 1, e
    raise ValueError(scheme)


def make_layer(cfg: LayerConfig, threads=None, rank=None, scheme="tileq", bits=2):
    """All weights of a configuration: {"proj": {name: proj}, "shared": ...}.
    bits = 3 gives the 3-bit-residual variant of the configuration (same
    seeds, codes 0..7)."""
    st = _streams(cfg)
    r = cfg.rank if rank is None else rank
    if scheme == "rank0":
        r = 0
    M, N, tiles = scheme_grid(cfg, scheme)
    proj = {}
    for name, (d_in, d_out) in cfg.proj_shapes().items():
        key = "single_or_gate" if name in ("single", "gate") else name
        proj[name] = make_proj(cfg.K, M, N, d_in, d_out, r, cfg.group,
                               cfg.act, st[key], threads=threads, tiles=tiles, bits=bits)
    layer = dict(kind=cfg.kind, act=cfg.act, K=cfg.K, d_model=cfg.d_model,
                 d_ff=cfg.d_ff, proj=proj, shared=None)
    if cfg.shared_ff:
        layer["shared"] = make_shared(cfg.d_model, cfg.shared_ff, st["shared"])
    return layer


def make_shared(d_model, d_ff, seedseq, std=0.02):
    """Dense fp16 shared expert: wg, wu [d_ff][d_model], wd [d_model][d_ff]."""
    a, b, c = seedseq.spawn(3)
    g = lambda s, shp: (np.random.default_rng(s).standard_normal(
        shp, dtype=np.float32) * np.float32(std)).astype(np.float16)
    return dict(d_ff=d_ff, wg=g(a, (d_ff, d_model)), wu=g(b, (d_ff, d_model)),
                wd=g(c, (d_model, d_ff)))

# ----------------------------------------------------------------------------
# tokens and routing


def popularity(K: int, routing: str, seedseq) -> np.ndarray:
    """Expert selection probabilities p[K]."""
    rng = np.random.default_rng(seedseq)
    if routing == "uniform":
        return np.full(K, 1.0 / K)
    if routing == "zipf1.1":
        order = rng.permutation(K)
        p = np.empty(K)
        p[order] = (np.arange(1, K + 1, dtype=np.float64)) ** -1.1
        return p / p.sum()
    if routing == "hot70":
        hot = rng.choice(K, size=min(4, K), replace=False)
        nh = len(hot)
        p = np.full(K, 0.3 / max(1, K - nh))
        p[hot] = 0.7 / nh
        return p / p.sum()
    raise ValueError(routing)


def make_routing(K: int, topk: int, T: int, routing: str, seedseq):
    """Top-k routing: scores = log p + Gumbel noise (Gumbel-top-k draws k
    distinct experts with probabilities p); ids are the k best scores (ties to
    the lower id), gates are the softmax over the k selected scores."""
    ss_pop, ss_noise = seedseq.spawn(2)
    p = popularity(K, routing, ss_pop)
    u = np.random.default_rng(ss_noise).random((T, K))
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    score = np.log(p)[None, :] - np.log(-np.log(u))
    order = np.argsort(-score, axis=1, kind="stable")[:, :topk]
    ids = order.astype(np.int32)
    sel = np.take_along_axis(score, order, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    gates = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(gates)


def make_tokens(cfg: LayerConfig, T: int):
    """(x [T][d_model] act, ids int32 [T][k], gates f32 [T][k])."""
    st = _streams(cfg)
    x = np.random.default_rng(st["x"]).standard_normal(
        (T, cfg.d_model), dtype=np.float32)
    ids, gates = make_routing(cfg.K, cfg.topk, T, cfg.routing, st["routing"])
    return to_act(x, cfg.act), ids, gates


def make_custom_tokens(d_model, K, topk, T, act, seed, routing="uniform"):
    """Tokens for hand-built test layers."""
    a, b = np.random.SeedSequence(seed).spawn(2)
    x = np.random.default_rng(a).standard_normal((T, d_model), dtype=np.float32)
    ids, gates = make_routing(K, topk, T, routing, b)
    return to_act(x, act), ids, gates


# ----------------------------------------------------------------------------
# dense expert weights (input of the offline packer)


def make_dense_experts(K, M, N, d_out, d_in, rank, seed, noise=0.02, tiles=None,
                       dtype=np.float16):
    """Dense expert weights W [K][d_out][d_in]: the expert's block of a
    random global low-rank matrix (columns N(0, 1/d) in std, singular values
    log-uniform over [0.1, 10], descending) plus N(0, noise) per element, and
    the expert -> tile map (random injective by default).  Random numbers and
    storage only."""
    rng = np.random.default_rng(seed)
    if tiles is None:
        tiles = rng.permutation(M * N)[:K].astype(np.int32)
    A = (rng.standard_normal((M * d_out, rank), dtype=np.float32) / np.float32(np.sqrt(d_out)))
    B = (rng.standard_normal((N * d_in, rank), dtype=np.float32) / np.float32(np.sqrt(d_in)))
    sv = np.sort(np.exp(rng.uniform(np.log(0.1), np.log(10.0), rank)))[::-1].astype(np.float32)
    W = np.empty((K, d_out, d_in), dtype)
    for e, t in enumerate(tiles):
        m, n = divmod(int(t), N)
        blk = (A[m * d_out:(m + 1) * d_out] * sv) @ B[n * d_in:(n + 1) * d_in].T
        blk += np.float32(noise) * rng.standard_normal((d_out, d_in), dtype=np.float32)
        W[e] = blk.astype(dtype)
    return W, np.asarray(tiles, np.int32)
