// Top-k router upstream of the fused forward.  The "TileQ" technical summary
// (section 2.2) takes the routing weights of the active experts as given;
// this kernel produces them from router logits: per row, the k largest
// logits in descending order (ties to the lower expert id, NaN read as
// -inf) and their softmax renormalised over the k (uniform when the largest
// selected logit is -inf).  Output ids and weights feed the forward directly.
//
// One wave per row: lane l holds logits l, l + 64, l + 128, l + 192 (K <=
// 256); k rounds of a wave-wide (value, id) argmax, each round's winner
// removed; lane j keeps the j-th pick.  Exact in the ids; the weights in fp32.
#include "tq_device.h"

namespace tq {

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int K, int k, int* __restrict__ ids,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
  bool live[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    live[i] = e < K;
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
      const int e = lane + 64 * i;
      if (live[i] && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bi == lane + 64 * i) live[i] = false;
    if (lane == j) {
      my_v = bv;
      my_id = bi;
    }
  }
  const float m = __shfl(my_v, 0, 64);           // the largest selected logit
  float ex = 0.f;
  if (lane < k) ex = (m == -INFINITY) ? 1.f : expf(my_v - m);
  float sum = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

void launch_router_topk(const float* logits, int T, int K, int k, int* ids, float* w,
                        hipStream_t s) {
  if (T <= 0) return;
  hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, K, k,
                     ids, w);
}

}  // namespace tq
