// Routing / grouping body shared by the routing kernel and the decode
// companion launch (see route.hip for what it builds).
#pragma once
#include "router_body.h"

namespace tq {

// SMAX > 0: S, T and (S/64) * K at most SMAX -- every scratch array lives in
// LDS (ids copied in), so the phases cost barriers, not global round trips.
// The body runs on one workgroup of NT threads (a multiple of 64, at most
// 1024) and takes its LDS from the caller: route_lds_ints(SMAX) ints.
__host__ __device__ constexpr int route_lds_ints(int smax) { return 1024 + 257 + 257 + 17 + 4 * smax; }

// Expert offsets, tile prefixes and active-expert records from the slot
// counts s_tot[K], on one wave (4 experts per lane, K <= 256).  s_off[K+1]
// and s_arank[K] (LDS copies for a later phase) may be nullptr.
__device__ __forceinline__ void route_expert_offsets(const RouteArgs& a, const int* s_tot,
                                                     int* s_off, int* s_arank, int lane) {
  const int K = a.K;
  int c[4], g[4], x[4], sc = 0, sg = 0, sx = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    c[q] = (e < K) ? s_tot[e] : 0;
    g[q] = (c[q] + a.bm_gemm - 1) / a.bm_gemm;
    x[q] = (c[q] + a.rt_col - 1) / a.rt_col;
    sc += c[q];
    sg += g[q];
    sx += x[q];
  }
  int na = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) na += (c[q] > 0);
  const int ic = wave_incl_scan_i(sc, lane), ig = wave_incl_scan_i(sg, lane),
            ix = wave_incl_scan_i(sx, lane), ia = wave_incl_scan_i(na, lane);
  int rc = ic - sc, rg = ig - sg, rx = ix - sx, ra = ia - na;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    if (e < K) {
      a.cnt[e] = c[q];
      a.off[e] = rc;
      if (s_off) s_off[e] = rc;
      a.tile_gemm[e] = rg;
      a.tile_colx[e] = rx;
      if (s_arank) s_arank[e] = (c[q] > 0) ? ra : -1;
      if (a.arec && c[q] > 0) {
        int* r = a.arec + ra * ROUTE_AREC;
        r[0] = e;
        r[1] = c[q];
        r[2] = rc;
      }
    }
    rc += c[q];
    rg += g[q];
    rx += x[q];
    ra += (c[q] > 0);
  }
  if (a.arec && lane == 63) a.arec[K * ROUTE_AREC] = ia;   // number of active experts
  const int tc = __shfl(ic, 63, 64), tgl = __shfl(ig, 63, 64), tx = __shfl(ix, 63, 64);
  if (lane == 0) {
    a.off[K] = tc;
    if (s_off) s_off[K] = tc;
    a.tile_gemm[K] = tgl;
    a.tile_colx[K] = tx;
  }
}

template <int SMAX, int NT>
__device__ void route_block(const RouteArgs& a, int* lds) {
  constexpr int NW = NT / 64;
  constexpr bool SMALL = SMAX > 0;
  int* s_seg = lds;                  // [1024]
  int* s_arank = s_seg + 512;        // [K]: rank of expert e among the active ones (-1: none)
  int* s_tot = s_seg + 1024;         // [257]
  int* s_off = s_tot + 257;          // [257]
  int* s_w = s_off + 257;            // [17]
  int* s_ids = s_w + 17;             // [SMAX] each
  int* s_rank = s_ids + SMAX;
  int* s_cntw = s_rank + SMAX;
  int* s_mask = s_cntw + SMAX;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, K = a.K, k = a.k, T = a.T;
  const int W = (S + 63) >> 6;
  const int* ids = a.ids;
  int* rank = a.rank;
  int* cntw = a.cntw;
  int* colmask = a.colmask;
  if constexpr (SMALL) {
    if (a.logits) {
      // the router first (decode companion launch): the picks go straight
      // into the LDS copy of the ids and out to the caller's id and weight
      // buffers
      router_rows(a.logits, T, K, k, wave, NW, const_cast<int*>(a.ids), a.gates_out, s_ids);
    } else {
      for (int i = tid; i < S; i += NT) s_ids[i] = a.ids[i];
    }
    ids = s_ids;
    rank = s_rank;
    cntw = s_cntw;
    colmask = s_mask;
  }

  for (int i = tid; i < W * K; i += NT) cntw[i] = 0;
  for (int i = tid; i < a.zero_n; i += NT) a.zero_init[i] = 0u;
  if (tid == 0) a.flags[0] = 0;
  __syncthreads();

  // (A) rank of each slot among the slots of its 64-slot chunk with the same
  //     expert: match mask from one ballot per key bit.
  const int nbits = 32 - __clz(K);
  int dropped = 0;
  for (int w = wave; w < W; w += NW) {
    const int s = (w << 6) + lane;
    const int e = (s < S) ? ids[s] : -1;
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
      rank[s] = r;
      if (r == 0) cntw[w * K + e] = __popcll(match);
    }
  }
  if (dropped) atomicAdd(a.flags, dropped);
  __syncthreads();

  // (B) per expert, exclusive prefix of the chunk counts over chunks: one
  //     wave per expert, lanes own contiguous chunk ranges.
  {
    const int seglen = (W + 63) >> 6;
    for (int e = wave; e < K; e += NW) {
      const int w0 = lane * seglen, w1 = min(W, w0 + seglen);
      int sum = 0;
      for (int w = w0; w < w1; ++w) sum += cntw[w * K + e];
      const int inc = wave_incl_scan_i(sum, lane);
      int run = inc - sum;
      for (int w = w0; w < w1; ++w) {
        const int v = cntw[w * K + e];
        cntw[w * K + e] = run;
        run += v;
      }
      if (lane == 63) s_tot[e] = inc;
    }
  }
  __syncthreads();
  // expert offsets and tile prefixes: wave 0, 4 experts per lane
  if (wave == 0) route_expert_offsets(a, s_tot, s_off, s_arank, lane);
  __syncthreads();

  // (C) positions
  for (int s = tid; s < S; s += NT) {
    const int e = ids[s];
    if (e >= 0 && e < K) {
      const int p = s_off[e] + cntw[(s >> 6) * K + e] + rank[s];
      a.perm[p] = s;
      a.inv[s] = p;
      if (a.etab) a.etab[e * S + (p - s_off[e])] = s;
      if (a.arec && p - s_off[e] < 16) a.arec[s_arank[e] * ROUTE_AREC + 4 + (p - s_off[e])] = s;
    } else {
      a.inv[s] = -1;
    }
  }

  // (D) column work lists: unique (n, t) pairs sorted by (n, t)
  if (T <= 64) {
    // one wave: a lane per token, ranks from ballots
    if (wave != 0) return;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c = 0; c < a.ncol; ++c) {
      const int* n_of = a.n_of[c];
      const int N = a.N[c];
      unsigned m = 0u;
      if (lane < T)
        for (int j = 0; j < k; ++j) {
          const int e = ids[lane * k + j];
          if (e >= 0 && e < K) m |= 1u << n_of[e];
        }
      for (int s = lane; s < S; s += 64) {
        const int e = ids[s];
        if (!(e >= 0 && e < K)) a.slot2col[c][s] = -1;
      }
      int run = 0, tiles = 0;
      for (int n = 0; n < N; ++n) {
        const bool f = (m >> n) & 1u;
        const uint64_t bb = __ballot(f);
        if (f) {
          const int idx = run + __popcll(bb & lt);
          a.col_tok[c][idx] = lane;
          for (int j = 0; j < k; ++j) {
            const int e = ids[lane * k + j];
            if (e >= 0 && e < K && n_of[e] == n) a.slot2col[c][lane * k + j] = idx;
          }
        }
        if (lane == 0) {
          a.col_off[c][n] = run;
          a.tile_col[c][n] = tiles;
        }
        const int cn = __popcll(bb);
        run += cn;
        tiles += (cn + a.rt_col - 1) / a.rt_col;
      }
      if (lane == 0) {
        a.col_off[c][N] = run;
        a.tile_col[c][N] = tiles;
      }
    }
    return;
  }
  if (SMALL && T <= NT) {
    // one token per thread: per wave and grid column the number of the
    // wave's tokens that reach the column (one ballot each), a prefix over
    // (column, wave) in LDS, then every entry's index in one pass -- two
    // barriers per projection instead of a block scan per column.  The
    // chunk-count table is done with (phase C read it before the barrier).
    static_assert(!SMALL || SMAX >= NW * 32 + 33, "LDS of the column lists");
    int* s_wc = s_cntw;              // [NW][32] per-wave counts -> prefixes
    int* s_cb = s_cntw + NW * 32;    // [33] column offsets
    const int t = tid;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // grid column of every expert, both projections (s_seg: free after phase C)
    int* s_nof = s_seg;              // [2][256]
    __syncthreads();
    for (int i = tid; i < a.ncol * 256; i += NT)
      if ((i & 255) < K) s_nof[i] = a.n_of[i >> 8][i & 255];
    for (int c = 0; c < a.ncol; ++c) {
      const int N = a.N[c];
      const int* n_of = s_nof + 256 * c;
      __syncthreads();               // the tables, phase C's reads, or the last projection's
      // grid column of each of the token's slots (-1: dropped id); the
      // first 8 in registers, further ones re-read
      unsigned m = 0u;
      int nj[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        nj[j] = -1;
        if (t < T && j < k) {
          const int e = ids[t * k + j];
          if (e >= 0 && e < K) nj[j] = n_of[e];
        }
        if (nj[j] >= 0) m |= 1u << nj[j];
      }
      for (int j = 8; t < T && j < k; ++j) {
        const int e = ids[t * k + j];
        if (e >= 0 && e < K) m |= 1u << n_of[e];
      }
      for (int n = 0; n < N; ++n) {
        const uint64_t bb = __ballot((m >> n) & 1u);
        if (lane == 0) s_wc[wave * 32 + n] = __popcll(bb);
      }
      __syncthreads();
      if (wave == 0) {
        // lane n < N: prefix of column n over the waves; then the column
        // offsets and tile prefixes over the columns
        int tot = 0;
        if (lane < N)
          for (int w = 0; w < NW; ++w) {
            const int v = s_wc[w * 32 + lane];
            s_wc[w * 32 + lane] = tot;
            tot += v;
          }
        const int tl = (tot + a.rt_col - 1) / a.rt_col;
        const int ic = wave_incl_scan_i(tot, lane), it = wave_incl_scan_i(tl, lane);
        if (lane < N) {
          s_cb[lane] = ic - tot;
          a.col_off[c][lane] = ic - tot;
          a.tile_col[c][lane] = it - tl;
        }
        if (lane == N - 1) {
          a.col_off[c][N] = ic;
          a.tile_col[c][N] = it;
        }
      }
      __syncthreads();
      for (int n = 0; n < N; ++n) {
        const bool f = (m >> n) & 1u;
        const uint64_t bb = __ballot(f);
        if (!f) continue;
        const int idx = s_cb[n] + s_wc[wave * 32 + n] + __popcll(bb & lt);
        a.col_tok[c][idx] = t;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (nj[j] == n) a.slot2col[c][t * k + j] = idx;
        for (int j = 8; j < k; ++j) {
          const int e = ids[t * k + j];
          if (e >= 0 && e < K && n_of[e] == n) a.slot2col[c][t * k + j] = idx;
        }
      }
      // slots routed nowhere have no column entry
      for (int q = tid; q < S; q += NT) {
        const int e = ids[q];
        if (!(e >= 0 && e < K)) a.slot2col[c][q] = -1;
      }
    }
    return;
  }
  const int tpt = (T + NT - 1) / NT;
  const int t0 = tid * tpt, t1 = min(T, t0 + tpt);
  for (int c = 0; c < a.ncol; ++c) {
    const int N = a.N[c];
    __syncthreads();
    if (tid < K) s_seg[tid] = a.n_of[c][tid];       // expert -> grid column
    __syncthreads();
    const int* n_of = s_seg;
    for (int t = t0; t < t1; ++t) {
      unsigned m = 0u;
      for (int j = 0; j < k; ++j) {
        const int e = ids[t * k + j];
        if (e >= 0 && e < K) m |= 1u << n_of[e];
      }
      colmask[t] = (int)m;
    }
    for (int s = tid; s < S; s += NT) {
      const int e = ids[s];
      if (!(e >= 0 && e < K)) a.slot2col[c][s] = -1;
    }
    int run_total = 0, run_tiles = 0;
    for (int n = 0; n < N; ++n) {
      int cl = 0;
      for (int t = t0; t < t1; ++t) cl += (colmask[t] >> n) & 1;
      int total;
      const int base = block_excl_scan(cl, s_w, &total);
      int idx = run_total + base;
      for (int t = t0; t < t1; ++t) {
        if ((colmask[t] >> n) & 1) {
          a.col_tok[c][idx] = t;
          for (int j = 0; j < k; ++j) {
            const int e = ids[t * k + j];
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

}  // namespace tq
