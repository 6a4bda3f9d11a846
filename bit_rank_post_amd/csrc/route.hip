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
#include "route_body.h"

namespace tq {

constexpr int SMALL_S = 4096;

template <int SMAX>
__global__ __launch_bounds__(1024) void route_kernel(RouteArgs a) {
  __shared__ int lds[route_lds_ints(SMAX)];
  route_block<SMAX, 1024>(a, lds);
}

bool route_fits(const RouteArgs& a, int smax) {
  return a.S <= smax && a.T <= smax && ((a.S + 63) / 64) * a.K <= smax;
}

void launch_route(const RouteArgs& a, hipStream_t s) {
  if (route_fits(a, SMALL_S))
    hipLaunchKernelGGL(route_kernel<SMALL_S>, dim3(1), dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL(route_kernel<0>, dim3(1), dim3(1024), 0, s, a);
}

}  // namespace tq
