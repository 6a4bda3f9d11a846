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
// Up to 1024 tokens (when S, T and the chunk-count table fit 4096 entries):
// one workgroup of 1024 threads; more: three launches over 1024-slot
// workgroups.  Every list is unique and the result deterministic
// (ranks come from wave ballots, counts are integer sums).
#include "route_body.h"

namespace tq {

constexpr int SMALL_S = 4096;

template <int SMAX>
__global__ __launch_bounds__(1024) void route_kernel(RouteArgs a) {
  __shared__ int lds[route_lds_ints(SMAX)];
  route_block<SMAX, 1024>(a, lds);
}

// ---- multi-workgroup path (more than 64 tokens) -----------------------------
// Workgroup b of 1024 threads owns the slots [1024 b, 1024 b + 1024) (16
// chunks of 64, one per wave) and the tokens [1024 b, 1024 b + 1024) (one
// per thread; S >= T, so the slot workgroups cover every token).  Three
// launches: counts (chunk ranks and per-chunk expert counts, token column
// masks and per-workgroup column counts), scans (one workgroup: prefixes
// over chunks and workgroups, offsets, tile prefixes), placement (positions
// and column entries).  The lists are the same as the one-workgroup path's.
constexpr int RM_NT = 1024;
constexpr int RM_KMAX = 256;
constexpr int RM_KTOK = 8;       // slots per token held in registers

__global__ __launch_bounds__(RM_NT) void route_count_kernel(RouteArgs a) {
  __shared__ int s_cnt[RM_NT / 64][RM_KMAX];
  __shared__ int s_col[2][32];
  __shared__ int s_drop;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, nb = gridDim.x;
  const int S = a.S, K = a.K, k = a.k, T = a.T;
  const int W = (S + 63) >> 6;
  for (int i = lane; i < K; i += 64) s_cnt[wave][i] = 0;
  if (tid < 64) s_col[tid >> 5][tid & 31] = 0;
  if (tid == 0) s_drop = 0;
  for (int i = b * RM_NT + tid; i < a.zero_n; i += nb * RM_NT) a.zero_init[i] = 0u;
  __syncthreads();

  // (A) rank of each slot among the slots of its chunk with the same expert
  const int w = b * (RM_NT / 64) + wave;
  const int s = (w << 6) + lane;
  const int e = (s < S) ? a.ids[s] : -1;
  const bool valid = (s < S) && e >= 0 && e < K;
  const int nbits = 32 - __clz(K);
  const int key = valid ? e : K;
  uint64_t match = __ballot(valid);
  for (int bt = 0; bt < nbits; ++bt) {
    const int bit = (key >> bt) & 1;
    const uint64_t bb = __ballot(bit);
    match &= bit ? bb : ~bb;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (valid) {
    const int r = __popcll(match & lt);
    a.rank[s] = r;
    if (r == 0) s_cnt[wave][e] = __popcll(match);
  }
  const uint64_t bad = __ballot(s < S && !valid);
  if (lane == 0 && bad) atomicAdd(&s_drop, __popcll(bad));

  // (D0) grid-column mask of each token, column counts of the workgroup
  const int t = b * RM_NT + tid;
  int ej[RM_KTOK];                 // the token's expert ids (k <= RM_KTOK: all loads in flight)
#pragma unroll
  for (int j = 0; j < RM_KTOK; ++j) ej[j] = (t < T && j < k) ? a.ids[t * k + j] : -1;
  for (int c = 0; c < a.ncol; ++c) {
    const int* n_of = c ? a.n_of[1] : a.n_of[0];
    const int N = c ? a.N[1] : a.N[0];
    unsigned m = 0u;
    if (t < T) {
      if (k <= RM_KTOK) {
#pragma unroll
        for (int j = 0; j < RM_KTOK; ++j)
          if (ej[j] >= 0 && ej[j] < K) m |= 1u << n_of[ej[j]];
      } else {
        for (int j = 0; j < k; ++j) {
          const int e2 = a.ids[t * k + j];
          if (e2 >= 0 && e2 < K) m |= 1u << n_of[e2];
        }
      }
      a.colmask[c * T + t] = (int)m;
    }
    for (int n = 0; n < N; ++n) {
      const uint64_t bb = __ballot((m >> n) & 1u);
      if (lane == 0 && bb) atomicAdd(&s_col[c][n], __popcll(bb));
    }
  }
  __syncthreads();
  // chunk counts expert-major ([K][W]): the scan reads each expert's run
  // of chunk counts with consecutive lanes on consecutive chunks
  if (w < W)
    for (int i = lane; i < K; i += 64) a.cntw[(size_t)i * W + w] = s_cnt[wave][i];
  if (tid < a.ncol * 32) {
    const int c = tid >> 5, n = tid & 31;
    a.wgcnt[(c * nb + b) * 32 + n] = s_col[c][n];
  }
  if (tid == 0) a.dropw[b] = s_drop;
}

__global__ __launch_bounds__(RM_NT) void route_scan_kernel(RouteArgs a, int nb) {
  __shared__ int s_tot[RM_KMAX];
  __shared__ int s_ctot[2][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = RM_NT / 64;
  const int S = a.S, K = a.K;
  const int W = (S + 63) >> 6;
  if (wave == 0) {
    int d = 0;
    for (int i = lane; i < nb; i += 64) d += a.dropw[i];
    d = wave_sum_i(d);
    if (lane == 0) a.flags[0] = d;
  }
  // (B) per expert, exclusive prefix of the chunk counts over chunks (table
  //     [K][W], chunk-minor): a wave per expert, lane l owning chunks
  //     64 u + l, so every load and store is coalesced; the prefix is a wave
  //     scan per group of 64 chunks plus the running total of the groups.  A
  //     wave takes its experts EB at a time with every load of the batch in
  //     flight at once (up to CH groups, W <= 64 CH; longer tables loop).
  constexpr int EB = 4, CH = 8;
  const int ngrp = (W + 63) >> 6;
  if (ngrp <= CH) {
    for (int e0 = wave * EB; e0 < K; e0 += NW * EB) {
      int v[EB][CH];
#pragma unroll
      for (int q = 0; q < EB; ++q)
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const int w = 64 * u + lane;
          v[q][u] = (e0 + q < K && w < W) ? a.cntw[(size_t)(e0 + q) * W + w] : 0;
        }
#pragma unroll
      for (int q = 0; q < EB; ++q) {
        int run = 0;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const int w = 64 * u + lane;
          const int inc = wave_incl_scan_i(v[q][u], lane);
          if (e0 + q < K && w < W) a.cntw[(size_t)(e0 + q) * W + w] = run + inc - v[q][u];
          run += __shfl(inc, 63, 64);
        }
        if (lane == 0 && e0 + q < K) s_tot[e0 + q] = run;
      }
    }
  } else {
    for (int e = wave; e < K; e += NW) {
      int run = 0;
      for (int w0 = 0; w0 < W; w0 += 64) {
        const int w = w0 + lane;
        const int v = (w < W) ? a.cntw[(size_t)e * W + w] : 0;
        const int inc = wave_incl_scan_i(v, lane);
        if (w < W) a.cntw[(size_t)e * W + w] = run + inc - v;
        run += __shfl(inc, 63, 64);
      }
      if (lane == 0) s_tot[e] = run;
    }
  }
  // per (projection, grid column): exclusive prefix of the workgroup counts,
  // in place; a wave takes its pairs PB at a time (nb <= 64: one load per
  // lane and pair, all in flight at once)
  constexpr int PB = 4;
  if (nb <= 64) {
    for (int q0 = wave * PB; q0 < a.ncol * 32; q0 += NW * PB) {
      int v[PB];
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int c = (q0 + q) >> 5, n = (q0 + q) & 31;
        const bool ok = q0 + q < a.ncol * 32 && n < (c ? a.N[1] : a.N[0]) && lane < nb;
        v[q] = ok ? a.wgcnt[(c * nb + lane) * 32 + n] : 0;
      }
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int c = (q0 + q) >> 5, n = (q0 + q) & 31;
        if (!(q0 + q < a.ncol * 32 && n < (c ? a.N[1] : a.N[0]))) continue;
        const int inc = wave_incl_scan_i(v[q], lane);
        if (lane < nb) a.wgcnt[(c * nb + lane) * 32 + n] = inc - v[q];
        if (lane == 63) s_ctot[c][n] = inc;
      }
    }
  } else {
    for (int q = wave; q < a.ncol * 32; q += NW) {
      const int c = q >> 5, n = q & 31;
      if (n >= (c ? a.N[1] : a.N[0])) continue;
      int run = 0;
      for (int b0 = 0; b0 < nb; b0 += 64) {
        const int bb = b0 + lane;
        const int v = (bb < nb) ? a.wgcnt[(c * nb + bb) * 32 + n] : 0;
        const int inc = wave_incl_scan_i(v, lane);
        if (bb < nb) a.wgcnt[(c * nb + bb) * 32 + n] = run + inc - v;
        run += __shfl(inc, 63, 64);
      }
      if (lane == 0) s_ctot[c][n] = run;
    }
  }
  __syncthreads();
  if (wave == 0) route_expert_offsets(a, s_tot, nullptr, nullptr, lane);
  if (wave == 1) {
    // column offsets and tile prefixes (lane = grid column, N <= 32)
    for (int c = 0; c < a.ncol; ++c) {
      const int N = c ? a.N[1] : a.N[0];
      int* col_off = c ? a.col_off[1] : a.col_off[0];
      int* tile_col = c ? a.tile_col[1] : a.tile_col[0];
      const int tot = (lane < N) ? s_ctot[c][lane] : 0;
      const int tl = (tot + a.rt_col - 1) / a.rt_col;
      const int ic = wave_incl_scan_i(tot, lane), it = wave_incl_scan_i(tl, lane);
      if (lane < N) {
        col_off[lane] = ic - tot;
        tile_col[lane] = it - tl;
      }
      if (lane == N - 1) {
        col_off[N] = ic;
        tile_col[N] = it;
      }
    }
  }
}

__global__ __launch_bounds__(RM_NT) void route_place_kernel(RouteArgs a) {
  __shared__ int s_wc[2][RM_NT / 64][32];   // tokens with bit n in each wave -> wave prefix
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, nb = gridDim.x;
  const int S = a.S, K = a.K, k = a.k, T = a.T;
  // (C) positions of the workgroup's slots
  const int s = b * RM_NT + tid;
  if (s < S) {
    const int e = a.ids[s];
    if (e >= 0 && e < K) {
      const int o = a.off[e];
      const int c = a.cntw[(size_t)e * ((S + 63) >> 6) + (s >> 6)] + a.rank[s];
      const int p = o + c;
      a.perm[p] = s;
      a.inv[s] = p;
      if (a.etab) a.etab[e * S + c] = s;
    } else {
      a.inv[s] = -1;
      for (int q = 0; q < a.ncol; ++q) (q ? a.slot2col[1] : a.slot2col[0])[s] = -1;
    }
  }
  // (D) column entries of the workgroup's tokens
  const int t = b * RM_NT + tid;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  unsigned m[2] = {0u, 0u};
  for (int c = 0; c < a.ncol; ++c) {
    const int N = c ? a.N[1] : a.N[0];
    m[c] = (t < T) ? (unsigned)a.colmask[c * T + t] : 0u;
    for (int n = 0; n < N; ++n) {
      const uint64_t bb = __ballot((m[c] >> n) & 1u);
      if (lane == 0) s_wc[c][wave][n] = __popcll(bb);
    }
  }
  __syncthreads();
  if (tid < a.ncol * 32) {
    const int c = tid >> 5, n = tid & 31;
    int run = 0;
    for (int wv = 0; wv < RM_NT / 64; ++wv) {
      const int v = s_wc[c][wv][n];
      s_wc[c][wv][n] = run;
      run += v;
    }
  }
  __syncthreads();
  const bool kreg = k <= RM_KTOK;
  int ej[RM_KTOK];
#pragma unroll
  for (int j = 0; j < RM_KTOK; ++j) ej[j] = (kreg && t < T && j < k) ? a.ids[t * k + j] : -1;
  for (int c = 0; c < a.ncol; ++c) {
    const int N = c ? a.N[1] : a.N[0];
    const int* n_of = c ? a.n_of[1] : a.n_of[0];
    const int* col_off = c ? a.col_off[1] : a.col_off[0];
    int* col_tok = c ? a.col_tok[1] : a.col_tok[0];
    int* slot2col = c ? a.slot2col[1] : a.slot2col[0];
    int nj[RM_KTOK];               // grid column of each slot's expert (-1: none)
#pragma unroll
    for (int j = 0; j < RM_KTOK; ++j) nj[j] = (ej[j] >= 0 && ej[j] < K) ? n_of[ej[j]] : -1;
    for (int n = 0; n < N; ++n) {
      const bool f = (m[c] >> n) & 1u;
      const uint64_t bb = __ballot(f);
      if (!f) continue;
      const int idx = col_off[n] + a.wgcnt[(c * nb + b) * 32 + n] + s_wc[c][wave][n] +
                      __popcll(bb & lt);
      col_tok[idx] = t;
      if (kreg) {
#pragma unroll
        for (int j = 0; j < RM_KTOK; ++j)
          if (nj[j] == n) slot2col[t * k + j] = idx;
      } else {
        for (int j = 0; j < k; ++j) {
          const int e2 = a.ids[t * k + j];
          if (e2 >= 0 && e2 < K && n_of[e2] == n) slot2col[t * k + j] = idx;
        }
      }
    }
  }
}

bool route_fits(const RouteArgs& a, int smax) {
  return a.S <= smax && a.T <= smax && ((a.S + 63) / 64) * a.K <= smax;
}

void launch_route(const RouteArgs& a, hipStream_t s) {
  // one workgroup while every list fits its LDS and a thread holds at most
  // one token (no global round trips between the phases, one launch);
  // otherwise the three-launch path
  if (a.T <= 1024 && route_fits(a, SMALL_S)) {
    hipLaunchKernelGGL(route_kernel<SMALL_S>, dim3(1), dim3(1024), 0, s, a);
  } else if (a.K <= RM_KMAX && !a.arec) {
    const int nb = (a.S + RM_NT - 1) / RM_NT;
    hipLaunchKernelGGL(route_count_kernel, dim3(nb), dim3(RM_NT), 0, s, a);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(RM_NT), 0, s, a, nb);
    hipLaunchKernelGGL(route_place_kernel, dim3(nb), dim3(RM_NT), 0, s, a);
  } else if (route_fits(a, SMALL_S)) {
    hipLaunchKernelGGL(route_kernel<SMALL_S>, dim3(1), dim3(1024), 0, s, a);
  } else {
    hipLaunchKernelGGL(route_kernel<0>, dim3(1), dim3(1024), 0, s, a);
  }
}

}  // namespace tq
