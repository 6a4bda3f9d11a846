// Activation preparation for the decode (streaming) residual kernel.
//
// The decode kernel feeds the 2-bit codes to the MFMA without dequantizing
// them: each packed fp16 half holds 1 + q*c (c = 1/64, 1/16 or 1/4 depending
// on where the code sits, see unpack16()).  With the activation entering as
// x'_k = x~_k / c_k, a group sum of products is
//     sum_k (1 + q_k c_k) x'_k = X'_g + sum_k q_k x~_k,
// so the residual term of a group is s * (C_g - X'_g - z * X~_g), applied to
// the fp32 MFMA partial once per group.  This kernel writes, per activation
// row: x'_k (fp16), the group sums X~_g and X'_g (fp32), and the exponent E
// of the exact power-of-two row scaling x~ = x * 2^-E that keeps 64 * |x~|
// inside the fp16 range (max|x~| in [2^8, 2^9)).
#include "tq_device.h"

namespace tq {

// 1/c of input k: step parity b = (k/32) % 2, pair v = (k % 8) / 2.
__device__ __forceinline__ float class_inv(int k) {
  const int b = (k >> 5) & 1, v = (k & 7) >> 1;
  // b = 0: {64, 16, 4, 64};  b = 1: {64, 16, 4, 16}
  return (v == 0) ? 64.f : (v == 1) ? 16.f : (v == 2) ? 4.f : (b ? 16.f : 64.f);
}

// One workgroup (256 threads) per row; thread tid owns the 8-element chunks
// tid + 256 i.  The row is read once (up to 8 chunks per thread stay in
// registers between the maximum and the conversion; longer rows re-read the
// rest).
template <typename T>
__global__ __launch_bounds__(256) void act_prep_kernel(PrepArgs a) {
  typedef typename Vec8<T>::type V8;
  constexpr int KEEP = 8;
  __shared__ float s_red[4];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int src = a.row_src ? a.row_src[row] : row;
  if (src < 0) return;
  const T* xr = reinterpret_cast<const T*>(a.X) + (size_t)src * a.d;
  const int nch = a.d >> 3;
  V8 kept[KEEP];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < KEEP; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) {
      kept[i] = *reinterpret_cast<const V8*>(xr + 8 * c);
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)kept[i][j]));
    }
  }
  for (int c = tid + 256 * KEEP; c < nch; c += 256) {
    const V8 v = *reinterpret_cast<const V8*>(xr + 8 * c);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)v[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  int e2 = 0;
  if (m > 0.f) frexpf(m, &e2);
  const int E = (m > 0.f) ? e2 - 9 : 0;
  if (tid == 0) a.ex[row] = E;
  // scaled, class-scaled copy and group sums; a group is G/8 consecutive
  // chunks, i.e. G/8 consecutive threads of one wave (G <= 256)
  const int cpg = a.G >> 3;
  half_t* xo = reinterpret_cast<half_t*>(a.Xp) + (size_t)row * a.d;
  float* sums = a.sums + (size_t)row * (a.d / a.G) * 2;
  auto emit = [&](int c, const V8& v) {
    float st = 0.f, sp = 0.f;
    if (c < nch) {
      half8v o;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half_t xt = (half_t)ldexpf((float)v[j], -E);
        const half_t xp = (half_t)((float)xt * class_inv(8 * c + j));
        o[j] = xp;
        st += (float)xt;
        sp += (float)xp;
      }
      *reinterpret_cast<half8v*>(xo + 8 * c) = o;
    }
    for (int o2 = 1; o2 < cpg; o2 <<= 1) {
      st += __shfl_xor(st, o2, 64);
      sp += __shfl_xor(sp, o2, 64);
    }
    if (c < nch && (c % cpg) == 0) {
      sums[2 * (c / cpg)] = st;
      sums[2 * (c / cpg) + 1] = sp;
    }
  };
#pragma unroll
  for (int i = 0; i < KEEP; ++i) {
    const int c = tid + 256 * i;
    if (256 * i < nch) emit(c, kept[i]);      // whole-block condition: shuffles stay uniform
  }
  for (int base = 256 * KEEP; base < nch; base += 256) {
    const int c = base + tid;
    V8 v{};
    if (c < nch) v = *reinterpret_cast<const V8*>(xr + 8 * c);
    emit(c, v);
  }
}

void launch_act_prep(const PrepArgs& a, int rows, Act act, hipStream_t s) {
  if (rows <= 0) return;
  if (act == ACT_F16)
    hipLaunchKernelGGL(act_prep_kernel<half_t>, dim3(rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(act_prep_kernel<__bf16>, dim3(rows), dim3(256), 0, s, a);
}

}  // namespace tq
