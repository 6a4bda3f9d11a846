// Host runtime of the TileQ MoE forward: the C ABI of include/tileq.h.
//
// Validation happens on the host before any device work; forward only
// enqueues kernels on the caller's stream (no allocation, no sync, no read
// back) and picks the decode or prefill kernels from (T, topk, K) alone.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tileq.h"
#include "tq_internal.h"

using namespace tq;

namespace {

thread_local std::string g_err;

tq_status fail(tq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIPCHK(expr)                                                          \
  do {                                                                        \
    hipError_t e_ = (expr);                                                   \
    if (e_ != hipSuccess)                                                     \
      return fail(TQ_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));    \
  } while (0)

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct ProjHost {
  bool uploaded = false;
  ProjDev dev{};
  std::vector<int> tile;
};

void free_proj(ProjHost& p) {
  if (!p.uploaded) return;
  (void)hipFree(p.dev.codes);
  (void)hipFree(p.dev.sz);
  (void)hipFree(p.dev.U);
  (void)hipFree(p.dev.Vt);
  (void)hipFree(p.dev.sigma);
  (void)hipFree(p.dev.m_of);
  (void)hipFree(p.dev.n_of);
  (void)hipFree(p.dev.l1max);
  p = ProjHost{};
}

}  // namespace

struct tq_layer {
  tq_kind kind;
  tq_dtype act;
  int d_model, d_ff, K;
  ProjHost proj[3];
  SharedDev shared{};
  // the shared expert runs on a second stream of the layer's device, forked
  // from and joined back into the forward's stream by events
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  int path_override = 0;
  // stage timing (benchmark hook)
  bool prof = false;
  mutable bool prof_recorded = false;
  hipEvent_t ev[9] = {};
};

namespace tq {
// Compute units of the current device (cached per device id; concurrent
// first calls store the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace tq

namespace {

int nproj(const tq_layer* L) { return L->kind == TQ_SINGLE ? 1 : 3; }

void proj_dims(const tq_layer* L, int which, int* d_in, int* d_out) {
  if (L->kind == TQ_SINGLE || which != TQ_P_DOWN) {
    *d_in = L->d_model;
    *d_out = L->d_ff;
  } else {
    *d_in = L->d_ff;
    *d_out = L->d_model;
  }
}

// ---- workspace plan --------------------------------------------------------
struct Plan {
  int T, k, S, path, bm_gemm, rt_col, max_tiles_gemm, max_col_tiles;
  int nks;                       // k-chunks (fp32 slabs) of the last projection's residual
  bool pair;                     // decode: two 16-row fragments per wave in that residual
  int ap_T;                      // decode: column stage over all (column, token) pairs
  int col_tiles_x, col_tiles_down;   // decode column-stage tiles
  size_t flags, cnt, off, perm, inv, etab, arec, tile_gemm, tile_colx, colmask, cntw, rank, wgcnt, dropw;
  size_t col_off[2], col_tok[2], slot2col[2], tile_col[2];
  size_t P[3];
  int nsplit[3];
  int rows_cap;
  size_t zero_base;              // region zeroed by the route kernel (unused: 0 words)
  int zero_n;
  size_t ex, h, dres, hs, ys;
  int nys;                       // k-split slabs of the shared expert's down output
  size_t x16, ex_h16, h16;       // prefill, bfloat16 activations
  size_t xp, sums_x, ex_x, hp, sums_h, ex_h;   // decode activation preparation
  size_t total;
};

// The decode kernel covers groups that do not straddle its 256-input stages
// and needs one group size for the projections that share an input.
bool decode_ok(const tq_layer* L) {
  for (int q = 0; q < nproj(L); ++q) {
    const int g = L->proj[q].dev.group;
    if (g > 256 || (g & (g - 1)) != 0) return false;   // 32, 64, 128 or 256
  }
  // gate and up read one prepared copy of x: one group size and one class
  // pattern (code width)
  if (L->kind == TQ_SWIGLU && (L->proj[0].dev.group != L->proj[1].dev.group ||
                               L->proj[0].dev.bits != L->proj[1].dev.bits))
    return false;
  return true;
}

int choose_path(const tq_layer* L, int T, int k) {
  int path;
  if (L->path_override == 1 || L->path_override == 2) path = L->path_override;
  else path = ((long)T * k <= 16L * L->K) ? 1 : 2;
  if (path == 1 && !decode_ok(L)) path = 2;
  // the decode kernel addresses its activation rows with 32-bit buffer
  // offsets below 2^31
  if (path == 1 && (long)T * k * std::max(L->d_model, L->d_ff) * 2 >= 0x7FFFFFF0L) path = 2;
  return path;
}

// Column-stage k-splits.  Decode: see decode_col_splits.  Prefill: only the
// projection whose rank vectors go to the combine as fp32 (down, or the
// single projection) is split, when its row tiles (about rows / 128 + K)
// would run one workgroup per CU: n splits of the k-range run in
// ceil(tiles n / (2 CUs)) rounds of 1/n the length; each extra slab costs the
// combine a read, charged as 3 % of the unsplit time.  Each split keeps at
// least 32 k-steps.
int choose_nsplit(const tq_layer* L, int q, int path, long rows, int d_in) {
  if (path == 1) return decode_col_splits(d_in);
  const bool to_combine = (L->kind == TQ_SWIGLU) ? (q == 2) : (q == 0);
  if (!to_combine) return 1;
  const long tiles = (rows + 127) / 128 + L->K;
  const long slots = 2L * device_cus();
  const int nst = d_in >> 5;
  int best = 1;
  double best_cost = 1e30;
  for (int n = 1; n <= 8; ++n) {
    if (n > 1 && nst / n < 32) break;
    const long rounds = (tiles * n + slots - 1) / slots;
    const double cost = (double)rounds / n + 0.03 * (n - 1);
    if (cost < best_cost) {
      best_cost = cost;
      best = n;
    }
  }
  return best;
}

// k-chunks of the decode kernel for a down / single projection: the most
// (up to 8, each chunk keeping at least 4 stages) for which the active
// experts' 16-row fragments times the chunks still fit one round of the grid
// (16 fragments per CU: two 8-wave workgroups or one of 16 waves; with two
// fragments per wave, 32).  A second round costs more than longer chunks:
// every workgroup pays a fixed start (routing reads, first batch) and
// epilogue.  Each chunk writes its own fp32 slab of per-slot outputs.
int choose_nks(const tq_layer* L, int q, int S, bool pair) {
  const ProjDev& d = L->proj[q].dev;
  const long active = std::min<long>(L->K, S);
  const long cus = device_cus();
  const int nfull = (d.d_in >> 5) >> 3;
  const long per_cu = pair ? 32 : 16;
  int nks = 1;
  while (nks < 8 && active * d.nrb * (2L * nks) <= per_cu * cus && nfull / (2 * nks) >= 4) nks *= 2;
  return nks;
}

// Two 16-row fragments per wave for a down / single projection at decode
// batch sizes (2-bit codes, where such 8-wave workgroups run two per CU):
// taken when it allows more k-chunks in one round than one fragment per
// wave.  Each stage then streams twice the code bytes for the same fixed
// costs, in shorter chunks.
bool choose_pair(const tq_layer* L, int q, int S) {
  const ProjDev& d = L->proj[q].dev;
  if (d.bits != 2 || !decode_dual(2, d.group, d.bits) || (long)S > 16L * L->K) return false;
  return choose_nks(L, q, S, true) > choose_nks(L, q, S, false);
}

// Waves per decode workgroup and how many of them own a 16-row fragment.
// The grid runs in ceil(wgs / (CUs x workgroups per CU)) rounds and a round
// lasts about as long as one workgroup streams its rows.  Cost of a choice =
// rounds x (bytes of one stage of the workgroup, in KB: rows x NP KB of codes
// + 8 KB of activations, plus a fixed per-workgroup cost of about 12
// KB-equivalents per stage for ring fill, routing reads and epilogue).
// 8-wave workgroups run two per CU when their ring fits half the LDS; then
// the fixed cost of one is hidden behind the other's streaming, and leaving
// one wave without rows can make the rounds come out even.  The input
// projections may use 8, 12, 14 or 16 waves; single-projection launches 8 or
// 16.
void choose_waves(const tq_layer* L, int q, int S, int nks, int np, int* waves, int* rows_per) {
  const long active = std::min<long>(L->K, S);
  const int nrb = L->proj[q].dev.nrb;
  const long cus = device_cus();
  const int bits = L->proj[q].dev.bits;
  const bool dual = decode_dual(np, L->proj[q].dev.group, bits);
  static const int cand2[] = {16, 14, 12, 8};
  static const int cand1[] = {16, 8};
  const int* cand = (np == 2) ? cand2 : cand1;
  const int nc = (np == 2) ? 4 : 2;
  *waves = 16;
  *rows_per = 16;
  long best_cost = -1;
  for (int i = 0; i < nc; ++i) {
    const int w = cand[i];
    const long per_cu = (w == 8 && dual) ? 2 : 1;
    for (int r = w; r >= (per_cu == 2 ? w - 1 : w); --r) {
      const long wgs = active * ((nrb + r - 1) / r) * nks;
      const long rounds = (wgs + cus * per_cu - 1) / (cus * per_cu);
      const long cost = rounds * (r * np * bits + 16 + (per_cu == 2 ? 0 : 24));
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        *waves = w;
        *rows_per = r;
      }
    }
  }
}

Plan make_plan(const tq_layer* L, int T, int k, int path) {
  Plan p{};
  p.T = T;
  p.k = k;
  p.S = T * k;
  p.path = path;
  p.bm_gemm = (path == 1) ? 16 : 128;
  p.rt_col = (path == 1) ? 16 : 128;
  p.max_tiles_gemm = (p.S + p.bm_gemm - 1) / p.bm_gemm + L->K;
  p.max_col_tiles = (p.S + p.rt_col - 1) / p.rt_col + 32 + L->K;
  // decode: the column stage of the input projection(s) covers every
  // (column, token) pair, so it does not wait for the routing lists
  int nmax = 1;
  for (int c = 0; c < ((L->kind == TQ_SINGLE) ? 1 : 2); ++c)
    if (L->proj[c].uploaded) nmax = std::max(nmax, L->proj[c].dev.N);
  p.ap_T = (path == 1) ? T : 0;
  if (path == 1) p.max_col_tiles = std::max(p.max_col_tiles, nmax * ((T + p.rt_col - 1) / p.rt_col));
  // decode column-stage tiles (16 rows): every (column, token) pair for the
  // input projection(s); per-expert slot tiles for down
  p.col_tiles_x = nmax * ((T + 15) / 16);
  p.col_tiles_down = (p.S + 15) / 16 + L->K;
  const int S = p.S, K = L->K;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  p.flags = take(256);
  p.cnt = take(sizeof(int) * K);
  p.off = take(sizeof(int) * (K + 1));
  p.perm = take(sizeof(int) * S);
  p.inv = take(sizeof(int) * S);
  p.etab = take(sizeof(int) * ((size_t)K * S + 16));   // + 16: whole 16-entry reads
  p.arec = take(sizeof(int) * ((size_t)K * ROUTE_AREC + 1));
  p.tile_gemm = take(sizeof(int) * (K + 1));
  p.tile_colx = take(sizeof(int) * (K + 1));
  p.colmask = take(sizeof(int) * 2 * std::max(T, 1));
  p.wgcnt = take(sizeof(int) * 2 * 32 * ((S + 1023) / 1024 + 1));
  p.dropw = take(sizeof(int) * ((S + 1023) / 1024 + 1));
  p.cntw = take(sizeof(int) * (size_t)((S + 63) / 64) * K);
  p.rank = take(sizeof(int) * S);
  const int ncol = (L->kind == TQ_SINGLE) ? 1 : 2;
  for (int c = 0; c < 2; ++c) {
    const int N = (c < ncol && L->proj[c].uploaded) ? L->proj[c].dev.N : 1;
    p.col_off[c] = take(sizeof(int) * (N + 1));
    p.col_tok[c] = take(sizeof(int) * S);
    p.slot2col[c] = take(sizeof(int) * S);
    p.tile_col[c] = take(sizeof(int) * (N + 1));
  }
  p.rows_cap = (path == 1) ? std::max(S, nmax * T) : S;
  for (int q = 0; q < 3; ++q) {
    p.nsplit[q] = 1;
    p.P[q] = 0;
    if (q >= nproj(L)) continue;
    const ProjDev& d = L->proj[q].dev;
    p.nsplit[q] = choose_nsplit(L, q, path, S, d.d_in);
    if (d.r_pad > 0) p.P[q] = take((size_t)p.nsplit[q] * p.rows_cap * d.r_pad * sizeof(float));
  }
  const bool bf = (L->act == TQ_BF16);
  p.zero_n = 0;
  p.zero_base = take(sizeof(unsigned));
  // prefill with bfloat16 activations: exact fp16 copies of x and h scaled by
  // per-row powers of two (the MFMA kernels read fp16)
  const bool bfpre = bf && path == 2;
  p.ex = take(sizeof(int) * (bfpre ? std::max(T, 1) : 1));
  p.x16 = take(bfpre ? (size_t)T * L->d_model * 2 : 0);
  p.ex_h16 = take(sizeof(int) * ((bfpre && L->kind == TQ_SWIGLU) ? std::max(S, 1) : 1));
  p.h16 = take((bfpre && L->kind == TQ_SWIGLU) ? (size_t)S * L->d_ff * 2 : 0);
  p.h = take(L->kind == TQ_SWIGLU ? (size_t)S * L->d_ff * 2 : 0);
  int d_in_last, d_out_last;
  proj_dims(L, nproj(L) - 1, &d_in_last, &d_out_last);
  p.pair = path == 1 && choose_pair(L, nproj(L) - 1, S);
  p.nks = (path == 1) ? choose_nks(L, nproj(L) - 1, S, p.pair) : 1;
  p.dres = take((size_t)p.nks * S * d_out_last * sizeof(float));
  p.nys = 1;
  if (L->shared.d_ff > 0) {
    // shared down projection (256 output rows x 128 tokens per workgroup):
    // k-splits until the grid has about one workgroup per CU, at most 4
    // (each adds a T x d_model fp32 slab for the combine; more measured no
    // faster), each split keeping at least 8 stages of 64 inputs
    const long tiles = (long)((L->d_model + 255) / 256) * ((T + 127) / 128);
    const int nst = L->shared.d_ff / 64;
    while (p.nys < 4 && tiles * p.nys * 2 <= device_cus() && nst / (2 * p.nys) >= 8) p.nys *= 2;
    p.hs = take((size_t)T * L->shared.d_ff * 2);
    p.ys = take((size_t)p.nys * T * L->d_model * sizeof(float));
  }
  if (path == 1) {
    const ProjDev& d0 = L->proj[0].dev;
    p.xp = take((size_t)T * L->d_model * 2);
    p.sums_x = take((size_t)T * (L->d_model / d0.group) * 2 * sizeof(float));
    p.ex_x = take(sizeof(int) * T);
    if (L->kind == TQ_SWIGLU) {
      const ProjDev& dd = L->proj[2].dev;
      p.hp = take((size_t)S * L->d_ff * 2);
      p.sums_h = take((size_t)S * (L->d_ff / dd.group) * 2 * sizeof(float));
      p.ex_h = take(sizeof(int) * S);
    }
  }
  p.total = o;
  return p;
}

tq_status check_ready(const tq_layer* L) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  for (int q = 0; q < nproj(L); ++q)
    if (!L->proj[q].uploaded)
      return fail(TQ_ESTATE, "projection %d has not been uploaded", q);
  // gate and up are one fused kernel (the SwiGLU epilogue needs both)
  if (L->kind == TQ_SWIGLU && L->proj[0].dev.bits != L->proj[1].dev.bits)
    return fail(TQ_EUNSUPPORTED, "gate (%d-bit) and up (%d-bit) codes must have one width",
                L->proj[0].dev.bits, L->proj[1].dev.bits);
  return TQ_OK;
}

tq_status check_tokens(int T, int topk) {
  if (T < 0) return fail(TQ_ESHAPE, "T = %d < 0", T);
  if (topk < 1 || topk > 32) return fail(TQ_ESHAPE, "topk = %d outside [1, 32]", topk);
  if ((long)T * topk > (1L << 20)) return fail(TQ_ESHAPE, "T*topk = %ld > 2^20", (long)T * topk);
  return TQ_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

void fill_route(const tq_layer* L, const Plan& p, const int* ids, void* ws, RouteArgs& r) {
  r = RouteArgs{};
  r.ids = ids;
  r.T = p.T;
  r.k = p.k;
  r.S = p.S;
  r.K = L->K;
  r.ncol = (L->kind == TQ_SINGLE) ? 1 : 2;
  for (int c = 0; c < r.ncol; ++c) {
    r.n_of[c] = L->proj[c].dev.n_of;
    r.N[c] = L->proj[c].dev.N;
    r.col_off[c] = at<int>(ws, p.col_off[c]);
    r.col_tok[c] = at<int>(ws, p.col_tok[c]);
    r.slot2col[c] = at<int>(ws, p.slot2col[c]);
    r.tile_col[c] = at<int>(ws, p.tile_col[c]);
  }
  r.bm_gemm = p.bm_gemm;
  r.rt_col = p.rt_col;
  r.flags = at<int>(ws, p.flags);
  r.cnt = at<int>(ws, p.cnt);
  r.off = at<int>(ws, p.off);
  r.perm = at<int>(ws, p.perm);
  r.inv = at<int>(ws, p.inv);
  r.etab = (p.path == 1) ? at<int>(ws, p.etab) : nullptr;
  r.arec = (p.path == 1) ? at<int>(ws, p.arec) : nullptr;
  r.tile_gemm = at<int>(ws, p.tile_gemm);
  r.tile_colx = at<int>(ws, p.tile_colx);
  r.cntw = at<int>(ws, p.cntw);
  r.rank = at<int>(ws, p.rank);
  r.colmask = at<int>(ws, p.colmask);
  r.wgcnt = at<int>(ws, p.wgcnt);
  r.dropw = at<int>(ws, p.dropw);
  r.zero_init = at<unsigned>(ws, p.zero_base);
  r.zero_n = p.zero_n;
}

// column stage over the unique (column, token) pairs of projection c (input x)
ColArgs col_args_x(const tq_layer* L, const Plan& p, int c, const void* x, void* ws) {
  const ProjDev& d = L->proj[c].dev;
  ColArgs a{};
  a.A = x;
  a.lda = d.d_in;
  a.seg_off = at<int>(ws, p.col_off[c]);
  a.tile_off = at<int>(ws, p.tile_col[c]);
  a.row_src = at<int>(ws, p.col_tok[c]);
  a.seg_vblk = nullptr;
  a.nseg = d.N;
  a.Vt = d.Vt;
  a.r_pad = d.r_pad;
  a.d_in = d.d_in;
  a.nsplit = p.nsplit[c];
  a.steps_per_split = ((d.d_in >> 5) + p.nsplit[c] - 1) / p.nsplit[c];
  a.sigma = d.sigma;
  a.P = at<float>(ws, p.P[c]);
  a.rows_cap = p.rows_cap;
  a.ap_T = p.ap_T;
  // prefill SwiGLU: the gate/up GEMM reads Sigma p as its MFMA operand
  // (split-K is decode-only, so the one slab is final)
  a.hilo = (p.path != 1 && L->kind == TQ_SWIGLU && p.nsplit[c] == 1) ? 1 : 0;
  return a;
}

// column stage of the down projection: one row per slot position (h)
ColArgs col_args_down(const tq_layer* L, const Plan& p, const void* h, void* ws) {
  const ProjDev& d = L->proj[2].dev;
  ColArgs a{};
  a.A = h;
  a.lda = d.d_in;
  a.seg_off = at<int>(ws, p.off);
  a.tile_off = at<int>(ws, p.tile_colx);
  a.row_src = nullptr;
  a.seg_vblk = d.n_of;
  a.nseg = L->K;
  a.Vt = d.Vt;
  a.r_pad = d.r_pad;
  a.d_in = d.d_in;
  a.nsplit = p.nsplit[2];
  a.steps_per_split = ((d.d_in >> 5) + p.nsplit[2] - 1) / p.nsplit[2];
  a.sigma = d.sigma;
  a.P = at<float>(ws, p.P[2]);
  a.rows_cap = p.rows_cap;
  return a;
}

}  // namespace

// ============================================================================
// Scratch of tq_forward_noalloc: a file-scope device array, one copy per GPU
// the library runs on (held until the process ends).  In host code `scratch`
// only names the array; its device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_addr[64];          // per device id

tq_status scratch_address(void** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(TQ_EUNSUPPORTED, "device id %d >= 64", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255))
      return fail(TQ_EHIP, "scratch array address %p not 256-byte aligned", p);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return TQ_OK;
}

tq_status forward_impl(const tq_layer* L, const void* x, int32_t T, const int32_t* topk_ids,
                       const float* topk_w, int32_t topk, void* y, tq_dtype y_dtype, void* ws,
                       size_t ws_bytes, void* stream, const float* logits = nullptr);

}  // namespace

extern "C" {

const char* tq_last_error(void) { return g_err.c_str(); }

int32_t tq_abi_version(void) { return 2; }

tq_status tq_layer_create(tq_kind kind, tq_dtype act, int32_t d_model, int32_t d_ff, int32_t K,
                          tq_layer** out) {
  if (!out) return fail(TQ_EINVAL, "out is NULL");
  *out = nullptr;
  if (kind != TQ_SINGLE && kind != TQ_SWIGLU) return fail(TQ_EINVAL, "unknown kind %d", (int)kind);
  if (act != TQ_F16 && act != TQ_BF16) return fail(TQ_EINVAL, "act must be TQ_F16 or TQ_BF16");
  if (d_model <= 0 || d_ff <= 0 || K <= 0)
    return fail(TQ_ESHAPE, "d_model, d_ff and K must be positive");
  if (K > 256) return fail(TQ_ESHAPE, "K = %d > 256", K);
  tq_layer* L = new (std::nothrow) tq_layer();
  if (!L) return fail(TQ_ENOMEM, "host allocation failed");
  L->kind = kind;
  L->act = act;
  L->d_model = d_model;
  L->d_ff = d_ff;
  L->K = K;
  *out = L;
  return TQ_OK;
}

tq_status tq_layer_set_path(tq_layer* L, int32_t path) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (path < 0 || path > 2) return fail(TQ_EINVAL, "path must be 0, 1 or 2");
  L->path_override = path;
  return TQ_OK;
}

tq_status tq_forward_path(const tq_layer* L, int32_t T, int32_t topk, int32_t* path) {
  tq_status st = check_ready(L);
  if (st != TQ_OK) return st;
  if (!path) return fail(TQ_EINVAL, "path is NULL");
  st = check_tokens(T, topk);
  if (st != TQ_OK) return st;
  *path = choose_path(L, T, topk);
  return TQ_OK;
}

tq_status tq_upload_proj(tq_layer* L, int32_t which, const tq_proj_desc* d, void* stream) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (!d) return fail(TQ_EINVAL, "descriptor is NULL");
  if (which < 0 || which >= nproj(L)) return fail(TQ_EINVAL, "projection %d not in this layer", which);
  int d_in, d_out;
  proj_dims(L, which, &d_in, &d_out);
  if (d->K != L->K) return fail(TQ_ESHAPE, "K = %d, layer has %d experts", d->K, L->K);
  if (d->d_in != d_in || d->d_out != d_out)
    return fail(TQ_ESHAPE, "projection %d must be %d -> %d, got %d -> %d", which, d_in, d_out,
                d->d_in, d->d_out);
  if (d->M <= 0 || d->N <= 0) return fail(TQ_ESHAPE, "grid %d x %d", d->M, d->N);
  if ((long)d->M * d->N > 1024) return fail(TQ_ESHAPE, "M*N = %ld > 1024", (long)d->M * d->N);
  if (d->K > d->M * d->N) return fail(TQ_ESHAPE, "K = %d > M*N = %d", d->K, d->M * d->N);
  if (d->N > 32) return fail(TQ_ESHAPE, "N = %d > 32", d->N);
  if (d_in % 128) return fail(TQ_ESHAPE, "d_in = %d not a multiple of 128", d_in);
  if (d_out % 16) return fail(TQ_ESHAPE, "d_out = %d not a multiple of 16", d_out);
  if (d->group <= 0 || d->group % 32 || d_in % d->group)
    return fail(TQ_ESHAPE, "group = %d must be a multiple of 32 dividing d_in", d->group);
  if (d->rank < 0 || d->rank > 128) return fail(TQ_ESHAPE, "rank = %d outside [0, 128]", d->rank);
  if (d->bits != 2 && d->bits != 3)
    return fail(TQ_EUNSUPPORTED, "bits = %d: residual codes of 2 or 3 bits only", d->bits);
  if (d->bits == 3 && (d->group > 256 || (d->group & (d->group - 1)) != 0))
    return fail(TQ_EUNSUPPORTED, "group = %d: 3-bit codes need a power-of-two group of 32 to 256",
                d->group);
  if (d->rank > 0 && d->sigma_dtype != TQ_F16 && d->sigma_dtype != TQ_F32)
    return fail(TQ_EINVAL, "sigma_dtype must be TQ_F16 or TQ_F32");
  if (!d->tile_of_expert) return fail(TQ_EINVAL, "tile_of_expert is NULL");
  if (!d->codes || !d->scales || !d->zeros) return fail(TQ_EINVAL, "codes/scales/zeros NULL");
  if (d->rank > 0 && (!d->U || !d->V || !d->sigma)) return fail(TQ_EINVAL, "U/V/sigma NULL");
  std::vector<int> seen(d->M * d->N, -1);
  for (int e = 0; e < d->K; ++e) {
    const int t = d->tile_of_expert[e];
    if (t < 0 || t >= d->M * d->N)
      return fail(TQ_EINVAL, "expert %d: tile %d outside [0, %d)", e, t, d->M * d->N);
    if (seen[t] >= 0)
      return fail(TQ_EINVAL, "experts %d and %d share tile %d (the map must be injective)",
                  seen[t], e, t);
    seen[t] = e;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ProjHost np;
  ProjDev& v = np.dev;
  v.K = d->K;
  v.M = d->M;
  v.N = d->N;
  v.d_in = d_in;
  v.d_out = d_out;
  v.rank = d->rank;
  v.r_pad = (d->rank + 31) / 32 * 32;
  v.group = d->group;
  v.ng = d_in / d->group;
  v.nrb = d_out / 16;
  v.nsteps = d_in / 32;
  v.bits = d->bits;
  np.tile.assign(d->tile_of_expert, d->tile_of_expert + d->K);
  std::vector<int> m_of(d->K), n_of(d->K);
  for (int e = 0; e < d->K; ++e) {
    m_of[e] = np.tile[e] / d->N;
    n_of[e] = np.tile[e] % d->N;
  }
  const size_t ncode = (size_t)d->K * d_out * d->bits * (d_in / 32);
  const size_t nsz = (size_t)d->K * d_out * v.ng;
  int* bad = nullptr;
  float* vn = nullptr;
  auto cleanup = [&]() {
    (void)hipFree(v.codes);
    (void)hipFree(v.sz);
    (void)hipFree(v.U);
    (void)hipFree(v.Vt);
    (void)hipFree(v.sigma);
    (void)hipFree(v.m_of);
    (void)hipFree(v.n_of);
    (void)hipFree(v.l1max);
    (void)hipFree(bad);
    (void)hipFree(vn);
  };
#define UPCHK(expr)                                                            \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess) {                                                    \
      cleanup();                                                               \
      return fail(e_ == hipErrorOutOfMemory ? TQ_ENOMEM : TQ_EHIP, "%s failed: %s", #expr, \
                  hipGetErrorString(e_));                                      \
    }                                                                          \
  } while (0)
  UPCHK(hipMalloc(&v.codes, ncode * 4));
  UPCHK(hipMalloc(&v.sz, nsz * 4));
  UPCHK(hipMalloc(&v.m_of, sizeof(int) * d->K));
  UPCHK(hipMalloc(&v.n_of, sizeof(int) * d->K));
  UPCHK(hipMalloc(&bad, sizeof(int)));
  UPCHK(hipMalloc(&v.l1max, sizeof(float) * d->K));
  if (d->rank > 0) UPCHK(hipMalloc(&vn, sizeof(float) * d->N * d->rank));
  if (v.r_pad > 0) {
    UPCHK(hipMalloc(&v.U, (size_t)d->M * d_out * v.r_pad * 2));
    UPCHK(hipMalloc(&v.Vt, (size_t)d->N * v.r_pad * d_in * 2));
    UPCHK(hipMalloc(&v.sigma, (size_t)v.r_pad * 4));
  }
  UPCHK(hipMemsetAsync(bad, 0, sizeof(int), s));
  launch_repack_codes(d->codes, v.codes, d->K, d_out, d_in, d->bits, s);
  launch_pack_sz(d->scales, d->zeros, v.sz, d->K, d_out, v.ng, d->bits, bad, s);
  UPCHK(hipGetLastError());
  if (v.r_pad > 0) {
    launch_pad_u(d->U, v.U, d->M * d_out, d->rank, v.r_pad, s);
    launch_transpose_v(d->V, v.Vt, d->N, d_in, d->rank, v.r_pad, s);
    UPCHK(hipGetLastError());
    launch_sigma_to_f32(d->sigma, d->sigma_dtype == TQ_F16 ? 1 : 0, v.sigma, d->rank, v.r_pad, s);
    UPCHK(hipGetLastError());
  }
  UPCHK(hipMemcpyAsync(v.m_of, m_of.data(), sizeof(int) * d->K, hipMemcpyHostToDevice, s));
  UPCHK(hipMemcpyAsync(v.n_of, n_of.data(), sizeof(int) * d->K, hipMemcpyHostToDevice, s));
  {
    RowBoundArgs rb{};
    rb.codes = d->codes;
    rb.scales = d->scales;
    rb.zeros = d->zeros;
    rb.U = d->U;
    rb.sigma = v.sigma;
    rb.V = d->V;
    rb.m_of = v.m_of;
    rb.n_of = v.n_of;
    rb.K = d->K;
    rb.N = d->N;
    rb.d_out = d_out;
    rb.d_in = d_in;
    rb.G = d->group;
    rb.r = d->rank;
    rb.bf = L->act == TQ_BF16 ? 1 : 0;
    rb.bits = d->bits;
    rb.vn = vn;
    rb.l1max = v.l1max;
    UPCHK(hipMemsetAsync(v.l1max, 0, sizeof(float) * d->K, s));
    launch_row_bound(rb, s);
    UPCHK(hipGetLastError());
  }
  int hbad = 0;
  UPCHK(hipMemcpyAsync(&hbad, bad, sizeof(int), hipMemcpyDeviceToHost, s));
  UPCHK(hipStreamSynchronize(s));
  (void)hipFree(bad);
  bad = nullptr;
  (void)hipFree(vn);
  vn = nullptr;
  if (hbad & 3) {
    cleanup();
    return fail(TQ_EINVAL, "%s%s", (hbad & 1) ? "scale or zero point not finite; " : "",
                (hbad & 2) ? "a dequantized weight s (q - z) overflows fp16" : "");
  }
  v.deq_lut = (hbad & 4) ? 1 : 0;
#undef UPCHK
  free_proj(L->proj[which]);
  np.uploaded = true;
  L->proj[which] = np;
  return TQ_OK;
}

tq_status tq_upload_shared_expert(tq_layer* L, int32_t d_ff_shared, const void* wg, const void* wu,
                                  const void* wd, void* stream) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (L->kind != TQ_SWIGLU) return fail(TQ_EINVAL, "shared expert needs a SWIGLU layer");
  if (L->act != TQ_F16) return fail(TQ_EUNSUPPORTED, "shared expert supported for f16 layers only");
  if (!wg || !wu || !wd) return fail(TQ_EINVAL, "weights NULL");
  if (d_ff_shared <= 0 || d_ff_shared % 128)
    return fail(TQ_ESHAPE, "d_ff_shared = %d must be a positive multiple of 128", d_ff_shared);
  if (L->d_model % 128) return fail(TQ_ESHAPE, "d_model must be a multiple of 128");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t n = (size_t)d_ff_shared * L->d_model * 2;
  SharedDev sd{};
  sd.d_ff = d_ff_shared;
  auto drop = [&]() {
    (void)hipFree(sd.wg);
    (void)hipFree(sd.wu);
    (void)hipFree(sd.wd);
  };
#define SHCHK(expr)                                                            \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess) {                                                    \
      drop();                                                                  \
      return fail(e_ == hipErrorOutOfMemory ? TQ_ENOMEM : TQ_EHIP, "%s failed: %s", #expr, \
                  hipGetErrorString(e_));                                      \
    }                                                                          \
  } while (0)
  SHCHK(hipMalloc(&sd.wg, n));
  SHCHK(hipMalloc(&sd.wu, n));
  SHCHK(hipMalloc(&sd.wd, n));
  // k-step-blocked copies (contiguous fragment loads in the dense GEMM)
  launch_block_rows(wg, sd.wg, d_ff_shared, L->d_model, s);
  launch_block_rows(wu, sd.wu, d_ff_shared, L->d_model, s);
  launch_block_rows(wd, sd.wd, L->d_model, d_ff_shared, s);
  SHCHK(hipGetLastError());
  SHCHK(hipStreamSynchronize(s));
  if (!L->side) SHCHK(hipStreamCreateWithFlags(&L->side, hipStreamNonBlocking));
  if (!L->fork_ev) SHCHK(hipEventCreateWithFlags(&L->fork_ev, hipEventDisableTiming));
  if (!L->join_ev) SHCHK(hipEventCreateWithFlags(&L->join_ev, hipEventDisableTiming));
#undef SHCHK
  if (L->shared.d_ff) {
    (void)hipFree(L->shared.wg);
    (void)hipFree(L->shared.wu);
    (void)hipFree(L->shared.wd);
  }
  L->shared = sd;
  return TQ_OK;
}

tq_status tq_workspace_size(const tq_layer* L, int32_t T, int32_t topk, size_t* bytes) {
  tq_status st = check_ready(L);
  if (st != TQ_OK) return st;
  if (!bytes) return fail(TQ_EINVAL, "bytes is NULL");
  st = check_tokens(T, topk);
  if (st != TQ_OK) return st;
  *bytes = std::max(make_plan(L, T, topk, 1).total, make_plan(L, T, topk, 2).total);
  return TQ_OK;
}

tq_status tq_forward(const tq_layer* L, const void* x, int32_t T, const int32_t* topk_ids,
                     const float* topk_w, int32_t topk, void* y, tq_dtype y_dtype, void* ws,
                     size_t ws_bytes, void* stream) {
  return forward_impl(L, x, T, topk_ids, topk_w, topk, y, y_dtype, ws, ws_bytes, stream);
}

tq_status tq_forward_from_logits(const tq_layer* L, const void* x, int32_t T, const float* logits,
                                 int32_t topk, int32_t* topk_ids, float* topk_w, void* y,
                                 tq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  tq_status st = check_ready(L);
  if (st != TQ_OK) return st;
  if (topk < 1 || topk > std::min(L->K, 32))
    return fail(TQ_ESHAPE, "topk = %d outside [1, min(K, 32)] (the router picks distinct experts)",
                topk);
  if (T > 0 && !logits) return fail(TQ_EINVAL, "logits is NULL");
  return forward_impl(L, x, T, topk_ids, topk_w, topk, y, y_dtype, ws, ws_bytes, stream, logits);
}

tq_status tq_forward_noalloc(const tq_layer* L, const void* x, int32_t T, const int32_t* topk_ids,
                             const float* topk_w, int32_t topk, void* y, tq_dtype y_dtype,
                             void* stream) {
  tq_status st = check_ready(L);
  if (st != TQ_OK) return st;
  st = check_tokens(T, topk);
  if (st != TQ_OK) return st;
  if (T == 0) return TQ_OK;
  size_t need = 0;
  st = tq_workspace_size(L, T, topk, &need);
  if (st != TQ_OK) return st;
  if (need > TQ_NOALLOC_SCRATCH_BYTES)
    return fail(TQ_ESHAPE,
                "tq_forward_noalloc: T = %d, topk = %d needs %zu bytes of scratch, more than the "
                "%zu bytes of the library's static scratch array (use tq_forward with a workspace)",
                T, topk, need, (size_t)TQ_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != TQ_OK) return st;
  return forward_impl(L, x, T, topk_ids, topk_w, topk, y, y_dtype, ws, TQ_NOALLOC_SCRATCH_BYTES,
                      stream);
}

}  // extern "C"

namespace {

tq_status forward_impl(const tq_layer* L, const void* x, int32_t T, const int32_t* topk_ids,
                       const float* topk_w, int32_t topk, void* y, tq_dtype y_dtype, void* ws,
                       size_t ws_bytes, void* stream, const float* logits) {
  tq_status st = check_ready(L);
  if (st != TQ_OK) return st;
  st = check_tokens(T, topk);
  if (st != TQ_OK) return st;
  if (y_dtype != TQ_F16 && y_dtype != TQ_BF16 && y_dtype != TQ_F32)
    return fail(TQ_EINVAL, "unknown y_dtype %d", (int)y_dtype);
  if (T == 0) return TQ_OK;
  if (!x || !topk_ids || !topk_w || !y || !ws) return fail(TQ_EINVAL, "NULL buffer");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(TQ_EINVAL, "ws not 256-byte aligned");
  const int path = choose_path(L, T, topk);
  const Plan p = make_plan(L, T, topk, path);
  size_t need = 0;
  tq_workspace_size(L, T, topk, &need);
  if (ws_bytes < need) return fail(TQ_ESHAPE, "ws_bytes = %zu < %zu", ws_bytes, need);
  // activation rows are addressed with 32-bit byte offsets below 2^31
  if ((long)T * L->d_model * 2 >= 0x7FFFFFF0L)
    return fail(TQ_EUNSUPPORTED, "T * d_model * 2 = %ld bytes of activations >= 2^31",
                (long)T * L->d_model * 2);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Act act = (L->act == TQ_F16) ? ACT_F16 : ACT_BF16;
  const bool bf = (act == ACT_BF16);
  const bool dec = (path == 1);
  const bool swiglu = (L->kind == TQ_SWIGLU);
  const int K = L->K;
  auto mark = [&](int i) {
    if (L->prof) (void)hipEventRecord(L->ev[i], s);
  };
  // (a6) dense shared expert on the layer's side stream: it reads only x
  // and writes only its own buffers, so it overlaps the routed path; the
  // combine waits for it
  float* ys = nullptr;
  if (L->shared.d_ff > 0) {
    HIPCHK(hipEventRecord(L->fork_ev, s));
    HIPCHK(hipStreamWaitEvent(L->side, L->fork_ev, 0));
    DenseArgs da{};
    da.T = T;
    da.d_in = L->d_model;
    da.d_out = L->shared.d_ff;
    da.X = x;
    da.W0 = L->shared.wg;
    da.W1 = L->shared.wu;
    da.out_h = at<void>(ws, p.hs);
    launch_dense(da, 1, 1, L->side);
    DenseArgs db{};
    db.T = T;
    db.d_in = L->shared.d_ff;
    db.d_out = L->d_model;
    db.X = at<void>(ws, p.hs);
    db.W0 = L->shared.wd;
    db.out_f = at<float>(ws, p.ys);
    launch_dense(db, 0, p.nys, L->side);
    HIPCHK(hipEventRecord(L->join_ev, L->side));
    ys = at<float>(ws, p.ys);
  }
  // (a1) routing / grouping
  mark(0);
  RouteArgs ra;
  fill_route(L, p, topk_ids, ws, ra);
  if (p.ap_T > 0) ra.ncol = 0;     // decode: no column lists (every pair is computed)
  // decode with a small batch: the routing runs as one workgroup of the
  // activation-preparation / column-stage launch (neither reads the other);
  // with router logits given, that workgroup runs the top-k router first
  const bool fuse_route = dec && prep_col_can_route(ra);
  if (logits && fuse_route) {
    ra.logits = logits;
    ra.gates_out = const_cast<float*>(topk_w);
  } else if (logits) {
    launch_router_topk(logits, T, K, topk, const_cast<int*>(topk_ids), const_cast<float*>(topk_w), s);
  }
  if (!fuse_route) launch_route(ra, s);
  mark(1);
  // activation preparation (decode: class-scaled fp16 copy + group sums;
  // prefill bf16: exact fp16 copy) and (a2) the column stage of the
  // projection(s) reading x
  int* ex = nullptr;
  {
    ColArgs ca[2];
    int n = 0;
    const int ncol = swiglu ? 2 : 1;
    for (int c = 0; c < ncol; ++c)
      if (L->proj[c].dev.r_pad > 0) ca[n++] = col_args_x(L, p, c, x, ws);
    if (dec) {
      PrepArgs pa{};
      pa.X = x;
      pa.d = L->d_model;
      pa.G = L->proj[0].dev.group;
      pa.bits = L->proj[0].dev.bits;
      pa.Xp = at<void>(ws, p.xp);
      pa.sums = at<float>(ws, p.sums_x);
      pa.ex = at<int>(ws, p.ex_x);
      // one launch; the residual kernels add the column-stage slabs
      // themselves
      launch_prep_col(&pa, T, ca, n, p.col_tiles_x, fuse_route ? &ra : nullptr, act, s);
      mark(2);
    } else {
      if (bf) {
        ex = at<int>(ws, p.ex);
        launch_rows_to_f16(x, T, L->d_model, nullptr, ex, at<void>(ws, p.x16), s);
      }
      mark(2);
      if (n) launch_colproj(ca, n, p.rt_col, p.max_col_tiles, act, s);
    }
  }
  mark(3);
  float* dres = at<float>(ws, p.dres);
  void* h = swiglu ? at<void>(ws, p.h) : nullptr;
  // (a3 + a4 + a5) residual GEMM of the input projection(s)
  if (dec) {
    DecArgs da{};
    da.K = K;
    da.d_in = L->d_model;
    da.d_out = L->proj[0].dev.d_out;
    da.topk = topk;
    da.etab = at<int>(ws, p.etab);
    da.spec = p.S >= 2 * K;  // nearly every expert is routed to
    da.arec = da.spec ? nullptr : at<int>(ws, p.arec);  // else: active experts first
    da.off = at<int>(ws, p.off);
    da.cnt = at<int>(ws, p.cnt);
    da.gather = 1;
    da.rows = T;
    da.Xp = at<void>(ws, p.xp);
    da.sums = at<float>(ws, p.sums_x);
    da.ex = at<int>(ws, p.ex_x);
    da.p[0] = L->proj[0].dev;
    if (swiglu) {
      da.p[1] = L->proj[1].dev;
      for (int c = 0; c < 2; ++c) {
        da.P[c] = L->proj[c].dev.r_pad ? at<float>(ws, p.P[c]) : nullptr;
        da.slot2col[c] = at<int>(ws, p.slot2col[c]);
      }
      da.h = h;
      da.nks = 1;
      da.S = p.S;
      da.ap_T = p.ap_T;
      da.p_nsplit = p.nsplit[0];
      da.p_rows_cap = p.rows_cap;
      choose_waves(L, 0, p.S, 1, 2, &da.waves, &da.rows_per);
      // at 16 or more slots per active expert on average, most experts
      // fill a second 16-slot column tile: take both tiles in one pass over
      // the codes (two groups of 8 waves)
      const ProjDev& g0 = L->proj[0].dev;
      if (p.S >= 16L * std::min(K, p.S) && g0.group == L->proj[1].dev.group &&
          decode_two_tiles_ok(2, g0.group, g0.bits, g0.d_in)) {
        // two 8-wave workgroups per CU, each two groups of 4 waves; row
        // fragments per group by whole rounds, cost as in choose_waves
        da.nct = 2;
        da.waves = 8;
        const long active = std::min(K, p.S), cus = device_cus();
        long best = -1;
        for (int r = 4; r >= 3; --r) {
          const long wgs = active * ((g0.nrb + r - 1) / r);
          const long cost = ((wgs + 2 * cus - 1) / (2 * cus)) * (r * 2 * g0.bits + 16);
          if (best < 0 || cost < best) {
            best = cost;
            da.rows_per = r;
          }
        }
      }
      launch_gemm_decode(da, MODE_GATEUP, act, s);
    } else {
      da.dres = dres;
      da.gates = topk_w;
      da.nks = p.nks;
      da.S = p.S;
      // row stage in the first k-chunk's workgroups
      da.P[0] = L->proj[0].dev.r_pad ? at<float>(ws, p.P[0]) : nullptr;
      da.ap_T = p.ap_T;
      da.p_nsplit = p.nsplit[0];
      da.p_rows_cap = p.rows_cap;
      if (p.pair) {
        da.pair = 1;
        da.waves = 8;
        da.rows_per = 8;
      } else {
        choose_waves(L, 0, p.S, p.nks, 1, &da.waves, &da.rows_per);
      }
      launch_gemm_decode(da, MODE_RES, act, s);
    }
  } else {
    GemmArgs ga{};
    ga.K = K;
    ga.d_in = L->d_model;
    ga.d_out = L->proj[0].dev.d_out;
    ga.topk = topk;
    ga.S = p.S;
    ga.A = bf ? at<void>(ws, p.x16) : x;
    ga.rows = T;
    ga.gather = 1;
    ga.perm = at<int>(ws, p.perm);
    ga.off = at<int>(ws, p.off);
    ga.cnt = at<int>(ws, p.cnt);
    ga.tile_off = at<int>(ws, p.tile_gemm);
    ga.ex = ex;
    // fewer than 64 slots per expert on average: 64-slot tiles
    ga.narrow = (long)p.S < 64L * K ? 1 : 0;
    ga.p[0] = L->proj[0].dev;
    if (swiglu) {
      ga.p[1] = L->proj[1].dev;
      for (int c = 0; c < 2; ++c) {
        ga.P[c] = L->proj[c].dev.r_pad ? at<float>(ws, p.P[c]) : nullptr;
        if (ga.P[c] && p.nsplit[c] != 1) return fail(TQ_EUNSUPPORTED, "prefill column stage must be one slab");
        ga.slot2col[c] = at<int>(ws, p.slot2col[c]);
      }
      ga.p_rows = p.rows_cap;
      ga.h = h;
      if (bf) {
        // fp16 copy of h for down, scaled by a bound known before h is
        ga.h16 = at<void>(ws, p.h16);
        ga.exh = at<int>(ws, p.ex_h16);
      }
      launch_gemm_prefill(ga, MODE_GATEUP, act, p.max_tiles_gemm, s);
    } else {
      ga.dres = dres;
      ga.gates = topk_w;
      launch_gemm_prefill(ga, MODE_RES, act, p.max_tiles_gemm, s);
    }
  }
  mark(4);
  if (swiglu) {
    const ProjDev& dd = L->proj[2].dev;
    // (a2) column stage of down: one row per slot (decode: one launch with
    // the activation preparation of h)
    ColArgs ca = col_args_down(L, p, h, ws);
    const int ncd = dd.r_pad > 0 ? 1 : 0;
    if (dec) {
      PrepArgs pa{};
      pa.X = h;
      pa.d = L->d_ff;
      pa.G = dd.group;
      pa.bits = dd.bits;
      pa.Xp = at<void>(ws, p.hp);
      pa.sums = at<float>(ws, p.sums_h);
      pa.ex = at<int>(ws, p.ex_h);
      launch_prep_col(&pa, p.S, &ca, ncd, p.col_tiles_down, nullptr, act, s);
    } else if (ncd) {
      launch_colproj(&ca, 1, p.rt_col, p.max_col_tiles, act, s);
    }
    mark(5);
    // (a6) dense shared expert: launched on the side stream at the start of
    // the forward (below); the combine waits for it
    mark(6);
    // (a4) residual GEMM of down
    if (dec) {
      DecArgs da{};
      da.K = K;
      da.d_in = dd.d_in;
      da.d_out = dd.d_out;
      da.topk = topk;
      da.etab = at<int>(ws, p.etab);
      da.spec = p.S >= 2 * K;  // nearly every expert is routed to
      da.arec = da.spec ? nullptr : at<int>(ws, p.arec);  // else: active experts first
      da.off = at<int>(ws, p.off);
      da.cnt = at<int>(ws, p.cnt);
      da.gather = 0;
      da.rows = p.S;
      da.Xp = at<void>(ws, p.hp);
      da.sums = at<float>(ws, p.sums_h);
      da.ex = at<int>(ws, p.ex_h);
      da.p[0] = dd;
      da.dres = dres;
      da.gates = topk_w;
      da.nks = p.nks;
      da.S = p.S;
      // row stage (P rows = slot positions) in the first k-chunk's workgroups
      da.P[0] = dd.r_pad ? at<float>(ws, p.P[2]) : nullptr;
      da.ap_T = 0;
      da.p_nsplit = p.nsplit[2];
      da.p_rows_cap = p.rows_cap;
      if (p.pair) {
        da.pair = 1;
        da.waves = 8;
        da.rows_per = 8;
      } else {
        choose_waves(L, 2, p.S, p.nks, 1, &da.waves, &da.rows_per);
      }
      launch_gemm_decode(da, MODE_RES, act, s);
    } else {
      GemmArgs ga{};
      ga.K = K;
      ga.d_in = dd.d_in;
      ga.d_out = dd.d_out;
      ga.topk = topk;
      ga.S = p.S;
      ga.gather = 0;
      ga.rows = p.S;
      if (bf) {
        // the fp16 copy of h the gate/up kernel wrote beside it
        ga.A = at<void>(ws, p.h16);
        ga.ex = at<int>(ws, p.ex_h16);
      } else {
        ga.A = h;
      }
      ga.perm = at<int>(ws, p.perm);
      ga.off = at<int>(ws, p.off);
      ga.cnt = at<int>(ws, p.cnt);
      ga.tile_off = at<int>(ws, p.tile_gemm);
      ga.p[0] = dd;
      ga.dres = dres;
      ga.gates = topk_w;
      ga.narrow = (long)p.S < 64L * K ? 1 : 0;
      launch_gemm_prefill(ga, MODE_RES, act, p.max_tiles_gemm, s);
    }
  } else {
    mark(5);
    mark(6);
  }
  mark(7);
  // (a3 rank-space part + a5) combine
  if (L->shared.d_ff > 0) HIPCHK(hipStreamWaitEvent(s, L->join_ev, 0));
  {
    const int q = swiglu ? 2 : 0;
    const ProjDev& d = L->proj[q].dev;
    CombineArgs cb{};
    cb.T = T;
    cb.topk = topk;
    cb.K = K;
    cb.d_out = d.d_out;
    cb.M = d.M;
    cb.r_pad = dec ? 0 : d.r_pad;     // decode: the residual kernel added the row stage
    cb.ids = topk_ids;
    cb.gates = topk_w;
    cb.inv = at<int>(ws, p.inv);
    cb.prow = swiglu ? at<int>(ws, p.inv) : at<int>(ws, p.slot2col[0]);
    cb.ap_T = swiglu ? 0 : p.ap_T;
    cb.n_of = d.n_of;
    cb.m_of = d.m_of;
    cb.P = d.r_pad ? at<float>(ws, p.P[q]) : nullptr;
    cb.nsplit = dec ? 1 : p.nsplit[q];   // decode: the residual kernel summed P's slabs
    cb.rows_cap = p.rows_cap;
    cb.U = d.U;
    cb.dres = dres;
    cb.nks = p.nks;
    cb.S = p.S;
    cb.ys = ys;
    cb.nys = p.nys;
    cb.y = y;
    cb.y_dtype = (int)y_dtype;
    launch_combine(cb, act, s);
  }
  mark(8);
  if (L->prof) L->prof_recorded = true;
  HIPCHK(hipGetLastError());
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_profile_enable(tq_layer* L, int32_t on) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (on && !L->prof) {
    for (int i = 0; i < 9; ++i) HIPCHK(hipEventCreate(&L->ev[i]));
    L->prof = true;
  } else if (!on && L->prof) {
    for (int i = 0; i < 9; ++i) (void)hipEventDestroy(L->ev[i]);
    L->prof = false;
  }
  L->prof_recorded = false;
  return TQ_OK;
}

tq_status tq_profile_read(const tq_layer* L, float* stage_ms) {
  if (!L || !stage_ms) return fail(TQ_EINVAL, "NULL argument");
  if (!L->prof || !L->prof_recorded) return fail(TQ_ESTATE, "no profiled forward recorded");
  HIPCHK(hipEventSynchronize(L->ev[8]));
  for (int i = 0; i < 8; ++i) HIPCHK(hipEventElapsedTime(&stage_ms[i], L->ev[i], L->ev[i + 1]));
  return TQ_OK;
}

tq_status tq_calibrate_read(const void* buf, size_t bytes, uint32_t* scratch, void* stream) {
  if (!buf || !scratch) return fail(TQ_EINVAL, "NULL argument");
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15))
    return fail(TQ_EINVAL, "buf and bytes must be multiples of 16");
  launch_stream_read(buf, bytes, scratch, reinterpret_cast<hipStream_t>(stream));
  HIPCHK(hipGetLastError());
  return TQ_OK;
}

tq_status tq_layer_destroy(tq_layer* L) {
  if (!L) return TQ_OK;
  (void)hipDeviceSynchronize();
  if (L->prof)
    for (int i = 0; i < 9; ++i) (void)hipEventDestroy(L->ev[i]);
  for (int q = 0; q < 3; ++q) free_proj(L->proj[q]);
  if (L->shared.d_ff) {
    (void)hipFree(L->shared.wg);
    (void)hipFree(L->shared.wu);
    (void)hipFree(L->shared.wd);
  }
  if (L->side) (void)hipStreamDestroy(L->side);
  if (L->fork_ev) (void)hipEventDestroy(L->fork_ev);
  if (L->join_ev) (void)hipEventDestroy(L->join_ev);
  delete L;
  return TQ_OK;
}

tq_status tq_debug_route(const tq_layer* L, int32_t which, const int32_t* topk_ids, int32_t T,
                         int32_t topk, void* ws, size_t ws_bytes, int32_t* cnt, int32_t* off,
                         int32_t* perm, int32_t* inv, int32_t* col_off, int32_t* col_tok,
                         int32_t* slot2col, void* stream) {
  tq_status st = check_ready(L);
  if (st != TQ_OK) return st;
  st = check_tokens(T, topk);
  if (st != TQ_OK) return st;
  if (T == 0) return fail(TQ_ESHAPE, "T = 0");
  const int ncol = (L->kind == TQ_SINGLE) ? 1 : 2;
  if (which < 0 || which >= ncol) return fail(TQ_EINVAL, "which = %d has no column list", which);
  if (!topk_ids || !ws || !cnt || !off || !perm || !inv || !col_off || !col_tok || !slot2col)
    return fail(TQ_EINVAL, "NULL buffer");
  size_t need = 0;
  tq_workspace_size(L, T, topk, &need);
  if (ws_bytes < need) return fail(TQ_ESHAPE, "ws_bytes = %zu < %zu", ws_bytes, need);
  // activation rows are addressed with 32-bit byte offsets below 2^31
  if ((long)T * L->d_model * 2 >= 0x7FFFFFF0L)
    return fail(TQ_EUNSUPPORTED, "T * d_model * 2 = %ld bytes of activations >= 2^31",
                (long)T * L->d_model * 2);
  const Plan p = make_plan(L, T, topk, choose_path(L, T, topk));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  RouteArgs ra;
  fill_route(L, p, topk_ids, ws, ra);     // always with the column lists
  launch_route(ra, s);
  HIPCHK(hipGetLastError());
  const size_t S = (size_t)p.S;
  const int N = L->proj[which].dev.N;
  HIPCHK(hipMemcpyAsync(cnt, at<int>(ws, p.cnt), sizeof(int) * L->K, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(off, at<int>(ws, p.off), sizeof(int) * (L->K + 1), hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(perm, at<int>(ws, p.perm), sizeof(int) * S, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(inv, at<int>(ws, p.inv), sizeof(int) * S, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(col_off, at<int>(ws, p.col_off[which]), sizeof(int) * (N + 1),
                        hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(col_tok, at<int>(ws, p.col_tok[which]), sizeof(int) * S,
                        hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(slot2col, at<int>(ws, p.slot2col[which]), sizeof(int) * S,
                        hipMemcpyDeviceToDevice, s));
  return TQ_OK;
}

tq_status tq_debug_dequant(const tq_layer* L, int32_t which, int32_t expert, void* w_out,
                           void* stream) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (which < 0 || which >= nproj(L)) return fail(TQ_EINVAL, "projection %d not in layer", which);
  if (!L->proj[which].uploaded) return fail(TQ_ESTATE, "projection %d not uploaded", which);
  if (expert < 0 || expert >= L->K) return fail(TQ_EINVAL, "expert %d outside [0, %d)", expert, L->K);
  if (!w_out) return fail(TQ_EINVAL, "w_out is NULL");
  launch_debug_dequant(L->proj[which].dev, expert, w_out, reinterpret_cast<hipStream_t>(stream));
  HIPCHK(hipGetLastError());
  return TQ_OK;
}

tq_status tq_router_topk(const float* logits, int32_t T, int32_t K, int32_t k, int32_t* ids,
                         float* weights, void* stream) {
  if (T < 0) return fail(TQ_ESHAPE, "T = %d < 0", T);
  if (K < 1 || K > 256) return fail(TQ_ESHAPE, "K = %d outside [1, 256]", K);
  if (k < 1 || k > K || k > 32) return fail(TQ_ESHAPE, "k = %d outside [1, min(K, 32)]", k);
  if (T == 0) return TQ_OK;
  if (!logits || !ids || !weights) return fail(TQ_EINVAL, "NULL pointer");
  launch_router_topk(logits, T, K, k, ids, weights, reinterpret_cast<hipStream_t>(stream));
  HIPCHK(hipGetLastError());
  return TQ_OK;
}

}  // extern "C"

namespace {

tq_status pack_check(const tq_pack_desc* d) {
  if (!d) return fail(TQ_EINVAL, "descriptor is NULL");
  if (d->K <= 0 || d->M <= 0 || d->N <= 0 || d->d_in <= 0 || d->d_out <= 0)
    return fail(TQ_ESHAPE, "sizes must be positive");
  if ((long)d->M * d->N > 1024 || d->K > d->M * d->N || d->K > 256 || d->N > 32)
    return fail(TQ_ESHAPE, "K = %d experts on a %d x %d grid not supported", d->K, d->M, d->N);
  if (d->d_in % 128 || d->d_out % 16) return fail(TQ_ESHAPE, "d_in %% 128 and d_out %% 16 must be 0");
  if (d->group <= 0 || d->group % 32 || d->d_in % d->group)
    return fail(TQ_ESHAPE, "group = %d must be a multiple of 32 dividing d_in", d->group);
  if (d->bits != 2 && d->bits != 3) return fail(TQ_EUNSUPPORTED, "bits = %d", d->bits);
  if (d->bits == 3 && (d->group > 256 || (d->group & (d->group - 1)) != 0))
    return fail(TQ_EUNSUPPORTED, "group = %d: 3-bit codes need a power-of-two group of 32 to 256",
                d->group);
  if (d->rank < 0 || d->rank > 128) return fail(TQ_ESHAPE, "rank = %d outside [0, 128]", d->rank);
  if (d->sketch < std::max(d->rank, 1) || d->sketch > PACK_SKETCH_MAX)
    return fail(TQ_ESHAPE, "sketch = %d outside [max(rank, 1), %d]", d->sketch, PACK_SKETCH_MAX);
  if (d->power_iters < 0 || d->power_iters > 16) return fail(TQ_ESHAPE, "power_iters = %d", d->power_iters);
  if (d->act != TQ_F16 && d->act != TQ_BF16) return fail(TQ_EINVAL, "act must be TQ_F16 or TQ_BF16");
  if (d->w_dtype != TQ_F16 && d->w_dtype != TQ_BF16 && d->w_dtype != TQ_F32 && d->w_dtype != TQ_F64)
    return fail(TQ_EINVAL, "w_dtype must be TQ_F16, TQ_BF16, TQ_F32 or TQ_F64");
  if ((long)d->M * d->d_out * d->sketch * 8 >= (1L << 40)) return fail(TQ_ESHAPE, "sketch too large");
  if (!d->tile_of_expert || !d->W || !d->omega || !d->codes || !d->scales || !d->zeros)
    return fail(TQ_EINVAL, "NULL pointer");
  if (d->rank > 0 && (!d->U || !d->V || !d->sigma)) return fail(TQ_EINVAL, "U/V/sigma NULL");
  std::vector<int> seen(d->M * d->N, -1);
  for (int e = 0; e < d->K; ++e) {
    const int t = d->tile_of_expert[e];
    if (t < 0 || t >= d->M * d->N) return fail(TQ_EINVAL, "expert %d: tile %d out of range", e, t);
    if (seen[t] >= 0) return fail(TQ_EINVAL, "experts %d and %d share tile %d", seen[t], e, t);
    seen[t] = e;
  }
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_pack_workspace_size(const tq_pack_desc* d, size_t* bytes) {
  tq_status st = pack_check(d);
  if (st != TQ_OK) return st;
  if (!bytes) return fail(TQ_EINVAL, "bytes is NULL");
  *bytes = pack_workspace_bytes(d->M, d->N, d->d_in, d->d_out, d->rank, d->sketch);
  return TQ_OK;
}

tq_status tq_pack_proj(const tq_pack_desc* d, void* ws, size_t ws_bytes, void* stream) {
  tq_status st = pack_check(d);
  if (st != TQ_OK) return st;
  const size_t need = pack_workspace_bytes(d->M, d->N, d->d_in, d->d_out, d->rank, d->sketch);
  if (!ws) return fail(TQ_EINVAL, "ws is NULL");
  if (ws_bytes < need) return fail(TQ_ESHAPE, "ws_bytes = %zu < %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(TQ_EINVAL, "ws not 256-byte aligned");
  std::vector<int> emap(d->M * d->N, -1);
  for (int e = 0; e < d->K; ++e) emap[d->tile_of_expert[e]] = e;
  PackArgs a{};
  a.K = d->K;
  a.M = d->M;
  a.N = d->N;
  a.d_in = d->d_in;
  a.d_out = d->d_out;
  a.rank = d->rank;
  a.group = d->group;
  a.bits = d->bits;
  a.l = d->sketch;
  a.power_iters = d->power_iters;
  a.act_bf16 = d->act == TQ_BF16 ? 1 : 0;
  a.W = d->W;
  a.wdt = (int)d->w_dtype;
  a.tile_host = d->tile_of_expert;
  a.emap_host = emap.data();
  a.omega = d->omega;
  a.U = d->U;
  a.sigma = d->sigma;
  a.V = d->V;
  a.codes = d->codes;
  a.scales = d->scales;
  a.zeros = d->zeros;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  run_pack(a, ws, s);
  HIPCHK(hipGetLastError());
  HIPCHK(hipStreamSynchronize(s));
  return TQ_OK;
}

}  // extern "C"

extern "C" {

tq_status tq_debug_row_bound(const tq_layer* L, int32_t which, float* l1_out) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (which < 0 || which >= nproj(L)) return fail(TQ_EINVAL, "projection %d not in layer", which);
  if (!L->proj[which].uploaded) return fail(TQ_ESTATE, "projection %d not uploaded", which);
  if (!l1_out) return fail(TQ_EINVAL, "l1_out is NULL");
  HIPCHK(hipMemcpy(l1_out, L->proj[which].dev.l1max, sizeof(float) * L->K, hipMemcpyDeviceToHost));
  return TQ_OK;
}

}  // extern "C"
