// Routing / grouping step of the fused forward.
//
// "TileQ" technical summary, section 2.2: the fused inference replaces
// irregular per-token sparse dispatch with dense work over the whole batch.
// This kernel builds the grouping that the dense stages consume:
//   * slots s = t*k + j grouped by expert, ascending s inside an expert
//     (a stable counting sort), with inverse positions;
//   * per projection whose column stage reads the token activations, the
//     unique (grid column n, token t) pairs sorted by (n, t): V_n^T x_t is
//     computed once per pair, shared by every expert of column n the token
//     routes to;
//   * tile prefixes telling each GEMM / column-stage workgroup its segment.
// One workgroup of 1024 threads; every list is unique and the kernel is
// deterministic (ranks come from wave ballots, not atomics).
#include "tq_device.h"

namespace tq {

__global__ __launch_bounds__(1024) void route_kernel(RouteArgs a) {
  __shared__ int s_seg[1024];
  __shared__ int s_tot[257];
  __shared__ int s_off[257];
  __shared__ int s_w[17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, K = a.K, k = a.k, T = a.T;
  const int W = (S + 63) >> 6;

  for (int i = tid; i < W * K; i += 1024) a.cntw[i] = 0;
  for (int i = tid; i < a.zero_n; i += 1024) a.zero_init[i] = 0u;
  if (tid == 0) a.flags[0] = 0;
  __syncthreads();

  // (A) rank of each slot among the slots of its 64-slot chunk with the same
  //     expert: match mask from one ballot per key bit.
  const int nbits = 32 - __clz(K);
  int dropped = 0;
  for (int w = wave; w < W; w += 16) {
    const int s = (w << 6) + lane;
    const int e = (s < S) ? a.ids[s] : -1;
    const bool valid = (s < S) && e >= 0 && e < K;
    if (s < S && !valid) dropped++;
    const int key = valid ? e : K;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const int bit = (key >> b) & 1;
      const uint64_t bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int r = __popcll(match & lt);
    if (valid) {
      a.rank[s] = r;
      if (r == 0) a.cntw[w * K + e] = __popcll(match);
    }
  }
  if (dropped) atomicAdd(a.flags, dropped);
  __syncthreads();

  // (B) per expert, exclusive prefix of the chunk counts over chunks.
  {
    const int tpe = 1024 / K;
    const int e = tid / tpe, i = tid - e * tpe;
    const int seglen = (W + tpe - 1) / tpe;
    const int w0 = i * seglen, w1 = min(W, w0 + seglen);
    int sum = 0;
    if (e < K)
      for (int w = w0; w < w1; ++w) sum += a.cntw[w * K + e];
    s_seg[tid] = sum;
    __syncthreads();
    if (e < K && i == 0) {
      int run = 0;
      for (int j = 0; j < tpe; ++j) {
        const int v = s_seg[e * tpe + j];
        s_seg[e * tpe + j] = run;
        run += v;
      }
      s_tot[e] = run;
    }
    __syncthreads();
    if (e < K) {
      int run = s_seg[tid];
      for (int w = w0; w < w1; ++w) {
        const int v = a.cntw[w * K + e];
        a.cntw[w * K + e] = run;
        run += v;
      }
    }
  }
  if (tid == 0) {
    int run = 0, tg = 0, tc = 0;
    for (int e = 0; e < K; ++e) {
      const int c = s_tot[e];
      a.cnt[e] = c;
      a.off[e] = run;
      s_off[e] = run;
      a.tile_gemm[e] = tg;
      a.tile_colx[e] = tc;
      run += c;
      tg += (c + a.bm_gemm - 1) / a.bm_gemm;
      tc += (c + a.rt_col - 1) / a.rt_col;
    }
    a.off[K] = run;
    s_off[K] = run;
    a.tile_gemm[K] = tg;
    a.tile_colx[K] = tc;
  }
  __syncthreads();

  // (C) positions
  for (int s = tid; s < S; s += 1024) {
    const int e = a.ids[s];
    if (e >= 0 && e < K) {
      const int p = s_off[e] + a.cntw[(s >> 6) * K + e] + a.rank[s];
      a.perm[p] = s;
      a.inv[s] = p;
    } else {
      a.inv[s] = -1;
    }
  }

  // (D) column work lists: unique (n, t) pairs sorted by (n, t)
  const int tpt = (T + 1023) / 1024;
  const int t0 = tid * tpt, t1 = min(T, t0 + tpt);
  for (int c = 0; c < a.ncol; ++c) {
    const int* n_of = a.n_of[c];
    const int N = a.N[c];
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      unsigned m = 0u;
      for (int j = 0; j < k; ++j) {
        const int e = a.ids[t * k + j];
        if (e >= 0 && e < K) m |= 1u << n_of[e];
      }
      a.colmask[t] = (int)m;
    }
    for (int s = tid; s < S; s += 1024) {
      const int e = a.ids[s];
      if (!(e >= 0 && e < K)) a.slot2col[c][s] = -1;
    }
    int run_total = 0, run_tiles = 0;
    for (int n = 0; n < N; ++n) {
      int cl = 0;
      for (int t = t0; t < t1; ++t) cl += (a.colmask[t] >> n) & 1;
      int total;
      const int base = block_excl_scan(cl, s_w, &total);
      int idx = run_total + base;
      for (int t = t0; t < t1; ++t) {
        if ((a.colmask[t] >> n) & 1) {
          a.col_tok[c][idx] = t;
          for (int j = 0; j < k; ++j) {
            const int e = a.ids[t * k + j];
            if (e >= 0 && e < K && n_of[e] == n) a.slot2col[c][t * k + j] = idx;
          }
          ++idx;
        }
      }
      if (tid == 0) {
        a.col_off[c][n] = run_total;
        a.tile_col[c][n] = run_tiles;
      }
      run_total += total;
      run_tiles += (total + a.rt_col - 1) / a.rt_col;
    }
    if (tid == 0) {
      a.col_off[c][N] = run_total;
      a.tile_col[c][N] = run_tiles;
    }
  }
}

void launch_route(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, s, a);
}

}  // namespace tq
