"""Plain fp64 CPU oracle for the TileQ fused MoE expert forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

What it computes, following "TileQ: Efficient Low-Rank Quantization of
Mixture-of-Experts with 2D Tiling" (gist.science technical summary):

* Section 2.1, step 4 ("2D-Tiling Placement"): every expert sits at one tile
  (m, n) of an M x N grid inside a large block matrix W_big.
* Section 2.1, step 5 ("Quantization") and "Key Technical Insight": W_big is
  decomposed globally into shared factors U, Sigma, V; grid row m shares the
  left (output-space) block U_m, grid column n shares the right (input-space)
  block V_n; each expert keeps a quantized residual.  Hence the expert weight
  is the (m, n) block of U Sigma V^T plus the dequantized residual.
* Section 2.2 ("Efficient Fused Sparse Low-Rank Inference"): the forward takes
  the whole token batch and the routing weights of the active experts.

The oracle does none of the fusion of section 2.2: it builds each used expert
weight W_e explicitly in fp64 and applies it per routed slot, which is the
plain definition the fused forward must reproduce up to rounding order.

Readings where the pages are silent:
  * residual R_e[o, i] = s_e[o, i//G] * (q_e[o, i] - z_e[o, i//G]), 2-bit
    codes q packed 16 per uint32 (code i at bits 2*(i % 16)) or 3-bit codes
    (the pages' other residual width, section 4 "Experimental Results") as a
    little-endian bit string (code i at bits 3i..3i+2), group G along d_in,
    fp16 scale s and fp16 zero point z;
  * a slot (t, j) whose expert id is outside [0, K) contributes nothing;
  * SwiGLU expert: h = RND_act(silu(W_gate x) * (W_up x)), y = sum_j g W_down h,
    silu(v) = v / (1 + exp(-v)); h is stored in the activation dtype;
  * shared expert (dense fp16): added to every token with weight 1, its
    intermediate also stored in the activation dtype.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# number formats


def to_f64(a: np.ndarray, act: str) -> np.ndarray:
    """Exact fp64 value of an activation-format array (float16, or bfloat16
    carried as uint16 bits)."""
    if act == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if act == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if act == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(act)


_FMT = {"f16": (11, -14, 65504.0), "bf16": (8, -126, 3.3895313892515355e38)}


def rnd_act(v: np.ndarray, act: str) -> np.ndarray:
    """Round fp64 values once, to nearest with ties to even, onto the grid of
    the activation format (fp16: 11 significant bits, normal exponent >= -14,
    subnormal quantum 2^-24; bf16: 8 significant bits, exponent >= -126).
    Overflow goes to +-inf.  Returns fp64 values that the format holds."""
    if act == "f32":
        return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)
    bits, emin, vmax = _FMT[act]
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    m, e = np.frexp(v[nz])                  # v = m * 2^e, 0.5 <= |m| < 1
    # exponent of the leading bit is e-1; quantum = 2^(max(e-1, emin) - (bits-1))
    qexp = np.maximum(e - 1, emin) - (bits - 1)
    r = np.ldexp(np.rint(np.ldexp(v[nz], -qexp)), qexp)   # rint: ties to even
    # the rounding halfway point of vmax: values at or above it overflow
    limit = vmax + np.ldexp(1.0, int(np.floor(np.log2(vmax))) - bits)
    r = np.where(np.abs(v[nz]) >= limit, np.copysign(np.inf, v[nz]), r)
    out[nz] = r
    out[~nz] = v[~nz]
    return out


def silu(v: np.ndarray) -> np.ndarray:
    """silu(v) = v * sigmoid(v) = v / (1 + exp(-v)), fp64."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))

# ----------------------------------------------------------------------------
# stored format -> fp64 weights


def unpack_codes(codes: np.ndarray, d_in: int, bits: int = 2) -> np.ndarray:
    """Residual codes from uint32 words.

    bits = 2: words [..., d_in/16]; code i is bits 2*(i % 16) .. 2*(i % 16)+1
    of word i // 16.
    bits = 3: words [..., 3*d_in/32] holding the row as one little-endian
    bit string; code i is bits 3i, 3i+1, 3i+2 of that string (bit n is bit
    n % 32 of word n // 32), so 32 codes fill 3 words and some codes span
    two words."""
    codes = np.asarray(codes, dtype=np.uint32)
    if bits == 2:
        sh = np.arange(16, dtype=np.uint32) * np.uint32(2)
        q = (codes[..., None] >> sh) & np.uint32(3)
        return q.reshape(codes.shape[:-1] + (d_in,)).astype(np.int64)
    if bits == 3:
        # the bit string, bit n of the row at index n
        bitpos = np.arange(32, dtype=np.uint32)
        stream = ((codes[..., None] >> bitpos) & np.uint32(1)).reshape(codes.shape[:-1] + (-1,))
        b = stream[..., :3 * d_in].reshape(codes.shape[:-1] + (d_in, 3)).astype(np.int64)
        return b[..., 0] + 2 * b[..., 1] + 4 * b[..., 2]
    raise ValueError(bits)


def residual(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
             group: int) -> np.ndarray:
    """R[o, i] = s[o, i // G] * (q[o, i] - z[o, i // G]) in fp64 (exact)."""
    s = np.repeat(np.asarray(scales, np.float16).astype(np.float64), group, axis=-1)
    z = np.repeat(np.asarray(zeros, np.float16).astype(np.float64), group, axis=-1)
    return s * (q.astype(np.float64) - z)


def tile_coords(tile: int, N: int):
    """tile = m * N + n  ->  (m, n)."""
    return int(tile) // N, int(tile) % N


def wbig(proj) -> np.ndarray:
    """Explicit W_big = U diag(sigma) V^T, shape (M*d_out, N*d_in) (small
    grids only)."""
    U = to_f64(proj["U"], proj["act"])
    V = to_f64(proj["V"], proj["act"])
    sig = np.asarray(proj["sigma"], np.float64)
    return (U * sig[None, :]) @ V.T


def lowrank_block(proj, m: int, n: int) -> np.ndarray:
    """Block (m, n) of W_big built directly: U_m diag(sigma) V_n^T."""
    d_in, d_out = proj["d_in"], proj["d_out"]
    U = to_f64(proj["U"][m * d_out:(m + 1) * d_out], proj["act"])
    V = to_f64(proj["V"][n * d_in:(n + 1) * d_in], proj["act"])
    sig = np.asarray(proj["sigma"], np.float64)
    return (U * sig[None, :]) @ V.T


def expert_residual(proj, e: int) -> np.ndarray:
    q = unpack_codes(proj["codes"][e], proj["d_in"], proj.get("bits", 2))
    return residual(q, proj["scales"][e], proj["zeros"][e], proj["group"])


def expert_weight(proj, e: int) -> np.ndarray:
    """W_e = (block (m_e, n_e) of U Sigma V^T) + R_e, fp64 [d_out][d_in]."""
    m, n = tile_coords(proj["tile_of_expert"][e], proj["N"])
    return lowrank_block(proj, m, n) + expert_residual(proj, e)


def deq_canonical(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                  group: int, out: str = "f16") -> np.ndarray:
    """Canonical dequantized residual weight in a storage format:
    RND_out(fl32(fl32(q - z) * fl32(s))), evaluated with float32 operations
    and then rounded once to `out`.  Returns fp64 values."""
    s = np.repeat(np.asarray(scales, np.float16).astype(np.float32), group, axis=-1)
    z = np.repeat(np.asarray(zeros, np.float16).astype(np.float32), group, axis=-1)
    w32 = (q.astype(np.float32) - z) * s
    return rnd_act(w32.astype(np.float64), out)

# ----------------------------------------------------------------------------
# router (upstream of section 2.2, which takes the routing weights as given)


def router_topk(logits: np.ndarray, k: int):
    """Top-k routing of each row of router logits [T][K]: the k largest
    logits in descending order, ties to the lower expert id, NaN read as
    -inf; the weights are the softmax over the k selected logits (uniform
    when the largest selected logit is -inf).  Returns (ids int32 [T][k],
    weights fp64 [T][k]).  The pages name no router; this is the plain top-k
    router a fused forward is fed by."""
    L = np.asarray(logits, np.float64)
    L = np.where(np.isnan(L), -np.inf, L)
    T, K = L.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        order = sorted(range(K), key=lambda e: (-L[t, e], e))[:k]
        ids[t] = order
        v = L[t, order]
        if v[0] == -np.inf:
            w[t] = 1.0 / k
        else:
            ex = np.exp(v - v[0])
            w[t] = ex / ex.sum()
    return ids, w


# ----------------------------------------------------------------------------
# routing lists (the unique grouping the fused forward must build)


def route(ids: np.ndarray, K: int, n_of=None):
    """Canonical grouping of the T*k slots s = t*k + j.

    Returns dict with
      cnt[K]        slots per expert (ids outside [0, K) are dropped)
      off[K+1]      exclusive prefix of cnt
      perm[P]       valid slots ordered by (expert, s)
      inv[T*k]      position of slot s in perm, -1 for a dropped slot
    and, when n_of (expert -> grid column) is given, the column work list:
      col_pairs     unique (n, t) pairs of valid slots, sorted by (n, t)
      col_off[N+1]  start of column n's pairs (N = max(n_of)+1 if not given)
      slot2col[T*k] index of (n_of[e_s], t) in col_pairs, -1 if dropped."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = [int(v) for v in ids.reshape(-1)]
    valid = [s for s in range(T * k) if 0 <= flat[s] < K]
    perm = sorted(valid, key=lambda s: (flat[s], s))
    cnt = [0] * K
    for s in valid:
        cnt[flat[s]] += 1
    off = [0]
    for c in cnt:
        off.append(off[-1] + c)
    inv = [-1] * (T * k)
    for p, s in enumerate(perm):
        inv[s] = p
    res = dict(cnt=np.array(cnt, np.int64), off=np.array(off, np.int64),
               perm=np.array(perm, np.int64), inv=np.array(inv, np.int64))
    if n_of is not None:
        n_of = [int(v) for v in n_of]
        pairs = sorted({(n_of[flat[s]], s // k) for s in valid})
        index = {p: i for i, p in enumerate(pairs)}
        Ncols = max(n_of) + 1 if n_of else 0
        col_off = [0] * (Ncols + 1)
        for (n, _t) in pairs:
            col_off[n + 1] += 1
        for n in range(Ncols):
            col_off[n + 1] += col_off[n]
        slot2col = [-1] * (T * k)
        for s in valid:
            slot2col[s] = index[(n_of[flat[s]], s // k)]
        res.update(col_pairs=np.array(pairs, np.int64).reshape(-1, 2),
                   col_off=np.array(col_off, np.int64),
                   slot2col=np.array(slot2col, np.int64))
    return res

# ----------------------------------------------------------------------------
# forward


class _WeightCache:
    """Builds W_e once per (projection, expert) and keeps it while needed."""

    def __init__(self):
        self._c = {}

    def get(self, name, proj, e):
        key = (name, e)
        if key not in self._c:
            self._c[key] = expert_weight(proj, e)
        return self._c[key]

    def drop(self, name, e):
        self._c.pop((name, e), None)


def forward_single(proj, x, ids, gates, tokens=None):
    """Single projection: y_t = sum_j g_{t,j} W_{e_{t,j}} x_t (fp64).

    tokens: optional list of token indices to evaluate (rows of the result
    follow that list)."""
    act = proj["act"]
    K = proj["K"]
    ids = np.asarray(ids)
    gates = np.asarray(gates, np.float64)
    tok = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    X = to_f64(x, act)[tok]
    I, G = ids[tok], gates[tok]
    y = np.zeros((len(tok), proj["d_out"]))
    for e in range(K):
        rows, js = np.nonzero(I == e)
        if len(rows) == 0:
            continue
        D = X[rows] @ expert_weight(proj, e).T
        np.add.at(y, rows, G[rows, js][:, None] * D)
    return y


def swiglu_expert(layer, e, X, cache):
    """h = RND_act(silu(W_gate,e X^T) * (W_up,e X^T)) for token rows X."""
    act = layer["act"]
    pg, pu = layer["proj"]["gate"], layer["proj"]["up"]
    a = X @ cache.get("gate", pg, e).T
    b = X @ cache.get("up", pu, e).T
    return rnd_act(silu(a) * b, act)


def shared_expert(shared, X, act):
    """Dense shared expert: W_d (RND_act(silu(W_g x) * (W_u x)))."""
    wg = shared["wg"].astype(np.float64)
    wu = shared["wu"].astype(np.float64)
    wd = shared["wd"].astype(np.float64)
    h = rnd_act(silu(X @ wg.T) * (X @ wu.T), act)
    return h @ wd.T


def forward_swiglu(layer, x, ids, gates, tokens=None, keep_weights=True):
    """SwiGLU MoE layer: y_t = sum_j g_{t,j} W_down,e (h_{t,j}) (+ shared(x_t)),
    fp64.  tokens: optional subset of token indices (sampled outputs)."""
    act = layer["act"]
    K = layer["K"]
    ids = np.asarray(ids)
    gates = np.asarray(gates, np.float64)
    tok = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    X = to_f64(x, act)[tok]
    I, G = ids[tok], gates[tok]
    y = np.zeros((len(tok), layer["d_model"]))
    cache = _WeightCache()
    pd = layer["proj"]["down"]
    contrib = np.zeros((len(tok), I.shape[1], layer["d_model"]))
    for e in range(K):
        rows, js = np.nonzero(I == e)
        if len(rows) == 0:
            continue
        h = swiglu_expert(layer, e, X[rows], cache)
        d = h @ cache.get("down", pd, e).T
        contrib[rows, js] = G[rows, js][:, None] * d
        if not keep_weights:
            for n in ("gate", "up", "down"):
                cache.drop(n, e)
    y += contrib.sum(axis=1)
    if layer.get("shared") is not None:
        y += shared_expert(layer["shared"], X, act)
    return y


def forward(layer, x, ids, gates, tokens=None, keep_weights=True):
    if layer["kind"] == "single":
        return forward_single(layer["proj"]["single"], x, ids, gates, tokens)
    return forward_swiglu(layer, x, ids, gates, tokens, keep_weights)


def storage_params(proj):
    """Parameter counts of the low-rank factors (section 4, memory
    efficiency): shared 2D-tiled factors r*(M*d_out + N*d_in) + r versus
    per-expert factors K*r*(d_in + d_out)."""
    r, K, M, N = proj["rank"], proj["K"], proj["M"], proj["N"]
    shared = r * (M * proj["d_out"] + N * proj["d_in"]) + r
    per_expert = K * r * (proj["d_in"] + proj["d_out"])
    return shared, per_expert
