// Top-k router body shared by the router kernel (router.hip) and the decode
// companion launch, where one workgroup runs it just before the routing.
//
// The "TileQ" technical summary (section 2.2) takes the routing weights of the
// active experts as given; this produces them from router logits: per row,
// the k largest logits in descending order (ties to the lower expert id, NaN
// read as -inf) and their softmax renormalised over the k (uniform when the
// largest selected logit is -inf).
//
// A row is handled by an aligned segment of LPR lanes of one wave (LPR a
// power of two with 4 LPR >= K and LPR >= k, so a wave takes 64 / LPR rows at
// once): lane l of the segment holds logits l, l + LPR, l + 2 LPR, l + 3 LPR;
// k rounds of a segment-wide (value, id) argmax, each round's winner removed;
// lane j of the segment keeps the j-th pick.  Exact in the ids; the weights
// in fp32.
#pragma once
#include "tq_device.h"

namespace tq {

// Lanes per row for K experts and top-k (K <= 256, k <= 32).
__host__ __device__ inline int router_lpr(int K, int k) {
  int l = 1;
  while (l < k || 4 * l < K) l <<= 1;
  return l;
}

// Row t of logits [T][K] on the calling segment of LPR lanes (sub = lane
// within the segment; rows past the end pass valid = false, and every lane of
// the wave must call); lane sub < k returns pick sub in *id and *w.
template <int LPR>
__device__ __forceinline__ void router_row(const float* __restrict__ logits, int t, bool valid,
                                           int K, int k, int sub, int* id, float* w) {
  float v[4];
  bool live[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = sub + LPR * i;
    live[i] = valid && e < K;
    const float x = live[i] ? logits[(size_t)t * K + e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
  }
  float my_v = -INFINITY;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    // this lane's best remaining candidate (larger value, then lower id)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = sub + LPR * i;
      if (live[i] && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bi == sub + LPR * i) live[i] = false;
    if (sub == j) {
      my_v = bv;
      my_id = bi;
    }
  }
  const int seg0 = (threadIdx.x & 63) - sub;
  const float m = __shfl(my_v, seg0, 64);        // the largest selected logit
  float ex = 0.f;
  if (sub < k) ex = (m == -INFINITY) ? 1.f : expf(my_v - m);
  float sum = ex;
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  *id = my_id;
  *w = ex / sum;
}

// Rows [0, T) of logits by the waves w0, w0 + nw, ... (wave index w0 of nw),
// 64 / LPR rows per wave at a time; pick j of row t goes to ids[t k + j] and
// w[t k + j], and to lds_ids[t k + j] when given.
template <int LPR>
__device__ __forceinline__ void router_rows_lpr(const float* __restrict__ logits, int T, int K, int k,
                                                int w0, int nw, int* ids, float* w, int* lds_ids) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, sub = lane % LPR;
  for (int tb = w0 * RPW; tb < T; tb += nw * RPW) {
    const int t = tb + lane / LPR;
    int id;
    float wt;
    router_row<LPR>(logits, t, t < T, K, k, sub, &id, &wt);
    if (t < T && sub < k) {
      ids[(size_t)t * k + sub] = id;
      w[(size_t)t * k + sub] = wt;
      if (lds_ids) lds_ids[t * k + sub] = id;
    }
  }
}

__device__ inline void router_rows(const float* __restrict__ logits, int T, int K, int k, int w0,
                                   int nw, int* ids, float* w, int* lds_ids) {
  switch (router_lpr(K, k)) {
    case 1: router_rows_lpr<1>(logits, T, K, k, w0, nw, ids, w, lds_ids); break;
    case 2: router_rows_lpr<2>(logits, T, K, k, w0, nw, ids, w, lds_ids); break;
    case 4: router_rows_lpr<4>(logits, T, K, k, w0, nw, ids, w, lds_ids); break;
    case 8: router_rows_lpr<8>(logits, T, K, k, w0, nw, ids, w, lds_ids); break;
    case 16: router_rows_lpr<16>(logits, T, K, k, w0, nw, ids, w, lds_ids); break;
    case 32: router_rows_lpr<32>(logits, T, K, k, w0, nw, ids, w, lds_ids); break;
    default: router_rows_lpr<64>(logits, T, K, k, w0, nw, ids, w, lds_ids); break;
  }
}

}  // namespace tq
