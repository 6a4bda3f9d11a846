// Combine stage of the fused forward for down / single projections.
//
// "TileQ" technical summary, section 2.2: routing weights are applied to the
// rank-space projections of the active tiles and accumulated in place
// ("in-place accumulation buffer", no large 3D intermediate), then one
// batched product with the other shared factor gives the low-rank output.
// Here, per token t and grid row m,
//     S[t][m][:] = sum_{j : row(e_tj) = m} g_tj * Sigma * p_tj
// (p from the column stage), and the low-rank output is
//     l_t = sum_m U_m S[t][m]           (one GEMM with K = M * r),
// to which the gated residual outputs of the token's slots are added:
//     y_t = sum_j dres[pos(t, j)] + l_t (+ shared expert).
// S is built in LDS per 16-token tile and grid row (split into a high and a
// low part in the activation dtype for the MFMA), never in HBM.
#include "tq_device.h"

namespace tq {

template <typename T, typename YT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  typedef typename Vec8<T>::type V8;
  constexpr int SLD = 128 + 8;
  constexpr int KMAX = 32;
  __shared__ __attribute__((aligned(16))) T s_hi[16 * SLD];
  __shared__ __attribute__((aligned(16))) T s_lo[16 * SLD];
  __shared__ int s_m[16 * KMAX];        // grid row of each slot's expert (-1: none)
  __shared__ int s_row[16 * KMAX];      // row of P of each slot
  __shared__ float s_g[16 * KMAX];      // routing weight of each slot
  __shared__ int s_active;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int o_w = blockIdx.y * 64 + wave * 16;
  const bool ovalid = o_w < a.d_out;
  const int k = a.topk;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};

  if (a.r_pad > 0) {
    const int rp = a.r_pad;
    // per-slot data of the tile, once
    for (int i = tid; i < 16 * k; i += 256) {
      const int tt = i / k, j = i - tt * k;
      const int t = t0 + tt;
      int m = -1, row = 0;
      float g = 0.f;
      if (t < a.T) {
        const int s = t * k + j;
        const int e = a.ids[s];
        if (e >= 0 && e < a.K) {
          m = a.m_of[e];
          row = (a.ap_T > 0) ? a.n_of[e] * a.ap_T + t : a.prow[s];
          g = a.gates[s];
        }
      }
      s_m[tt * KMAX + j] = m;
      s_row[tt * KMAX + j] = row;
      s_g[tt * KMAX + j] = g;
    }
    for (int m = 0; m < a.M; ++m) {
      __syncthreads();
      if (tid == 0) {
        int any = 0;
        for (int i = 0; i < 16 * k && !any; ++i) any = (s_m[(i / k) * KMAX + i % k] == m);
        s_active = any;
      }
      __syncthreads();
      if (!s_active) continue;
      // S[t][m][:] = sum_{j : row(e_tj) = m} g_tj (Sigma p_tj), split hi + lo
      for (int i = tid; i < 16 * rp; i += 256) {
        const int tt = i / rp, c = i - tt * rp;
        float v = 0.f;
        for (int j = 0; j < k; ++j)
          if (s_m[tt * KMAX + j] == m)
            v += s_g[tt * KMAX + j] * a.P[(size_t)s_row[tt * KMAX + j] * rp + c];
        const T hi = from_f32<T>(v);
        s_hi[tt * SLD + c] = hi;
        s_lo[tt * SLD + c] = from_f32<T>(v - to_f32(hi));
      }
      __syncthreads();
      if (ovalid) {
        const T* up = reinterpret_cast<const T*>(a.U) +
                      ((size_t)m * a.d_out + o_w + l16) * rp + 8 * lg;
        for (int s2 = 0; s2 < rp; s2 += 32) {
          const V8 av = *reinterpret_cast<const V8*>(up + s2);
          const V8 bh = *reinterpret_cast<const V8*>(&s_hi[l16 * SLD + s2 + 8 * lg]);
          const V8 bl = *reinterpret_cast<const V8*>(&s_lo[l16 * SLD + s2 + 8 * lg]);
          acc = mfma16(av, bh, acc);
          acc = mfma16(av, bl, acc);
        }
      }
    }
  }
  if (!ovalid) return;
  const int t = t0 + l16;
  if (t >= a.T) return;
  const int o = o_w + 4 * lg;
  f32x4 v = acc;
  for (int j = 0; j < k; ++j) {
    const int pos = a.inv[t * k + j];
    if (pos < 0) continue;
    for (int c = 0; c < a.nks; ++c)
      v += *reinterpret_cast<const f32x4*>(a.dres + ((size_t)c * a.S + pos) * a.d_out + o);
  }
  if (a.ys)
    for (int c = 0; c < a.nys; ++c)
      v += *reinterpret_cast<const f32x4*>(a.ys + ((size_t)c * a.T + t) * a.d_out + o);
  YT* y = reinterpret_cast<YT*>(a.y) + (size_t)t * a.d_out + o;
  if constexpr (__is_same(YT, float)) {
    *reinterpret_cast<f32x4*>(y) = v;
  } else {
    YT r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = from_f32<YT>(v[q]);
    *reinterpret_cast<u32x2*>(y) = __builtin_bit_cast(u32x2, r);
  }
}

void launch_combine(const CombineArgs& a, Act act, hipStream_t s) {
  const dim3 grid((a.T + 15) / 16, (a.d_out + 63) / 64);
  if (act == ACT_F16) {
    if (a.y_dtype == 0) hipLaunchKernelGGL((combine_kernel<half_t, half_t>), grid, dim3(256), 0, s, a);
    else if (a.y_dtype == 1) hipLaunchKernelGGL((combine_kernel<half_t, __bf16>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<half_t, float>), grid, dim3(256), 0, s, a);
  } else {
    if (a.y_dtype == 0) hipLaunchKernelGGL((combine_kernel<__bf16, half_t>), grid, dim3(256), 0, s, a);
    else if (a.y_dtype == 1) hipLaunchKernelGGL((combine_kernel<__bf16, __bf16>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<__bf16, float>), grid, dim3(256), 0, s, a);
  }
}

}  // namespace tq
