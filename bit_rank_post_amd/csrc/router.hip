// Top-k router kernel upstream of the fused forward (see router_body.h):
// each wave takes 64 / LPR rows of logits at a time.
#include "router_body.h"

namespace tq {

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int K, int k, int* __restrict__ ids,
                                                          float* __restrict__ w) {
  router_rows(logits, T, K, k, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4, ids, w, nullptr);
}

void launch_router_topk(const float* logits, int T, int K, int k, int* ids, float* w,
                        hipStream_t s) {
  if (T <= 0) return;
  const int rpw = 64 / router_lpr(K, k);
  const int waves = (T + rpw - 1) / rpw;
  hipLaunchKernelGGL(router_topk_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, logits, T, K, k,
                     ids, w);
}

}  // namespace tq
