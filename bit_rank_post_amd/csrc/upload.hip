// Upload-time kernels: re-lay the stored projection (section 2.1 step 5 of the
// "TileQ" technical summary: shared factors U, Sigma, V and the quantized
// per-expert residual) into the layouts the forward kernels read.
#include "tq_device.h"

namespace tq {

// Bit position inside a dword of input j = 2v + h of step b (see unpack16).
__device__ __forceinline__ int code_bit(int b, int v, int h) {
  const int pos0[4] = {4, 6, 8, 0};
  const int pos1[4] = {10, 12, 14, 2};
  return 16 * h + (b ? pos1[v] : pos0[v]);
}

// One thread per output dword of the repacked layout.
__global__ void repack_codes_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                    int K, int d_out, int d_in) {
  const int nsteps = d_in >> 5;
  const size_t words_per_expert = (size_t)d_out * (d_in >> 4);
  const size_t total = words_per_expert * K;
  const size_t words_per_rb = (size_t)nsteps * 32;     // 64 lanes * nsteps * 2 B / 4 B
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(idx / words_per_expert);
    const size_t rem = idx - (size_t)e * words_per_expert;
    const int rb = (int)(rem / words_per_rb);
    const int w = (int)(rem - (size_t)rb * words_per_rb);     // dword within row block
    const int sg = w >> 8;                                    // 256 dwords per full group
    const int gs = min(8, nsteps - (sg << 3));
    const int wi = w - (sg << 8);
    const int dpl = gs >> 1;                                  // dwords per lane
    const int lane = wi / dpl, d = wi - lane * dpl;
    const int row = rb * 16 + (lane & 15);
    const uint32_t* srow = src + (size_t)e * words_per_expert + (size_t)row * (d_in >> 4);
    uint32_t out = 0u;
    for (int b = 0; b < 2; ++b) {
      const int step = (sg << 3) + 2 * d + b;
      for (int j = 0; j < 8; ++j) {
        const int k = step * 32 + 8 * (lane >> 4) + j;
        const uint32_t q = (srow[k >> 4] >> (2 * (k & 15))) & 3u;
        out |= q << code_bit(b, j >> 1, j & 1);
      }
    }
    dst[idx] = out;
  }
}

// 3-bit code of input k from a row of the stored bit string (bits 3k .. 3k+2)
__device__ __forceinline__ uint32_t code3_at(const uint32_t* row, int k) {
  const int n = 3 * k, w = n >> 5, b = n & 31;
  uint64_t v = row[w];
  if (b > 29) v |= (uint64_t)row[w + 1] << 32;
  return (uint32_t)(v >> b) & 7u;
}

// 3-bit repacked layout, per row block of 16 rows: for each group of 8 MFMA
// k-steps, 1536 bytes: [64 lanes][dwords 0..3] (16 B per lane), then dword 4
// of the 64 lanes, then dword 5; a trailing group of 4 k-steps is three
// planes [dword j][64 lanes].  Dwords 0..2 are the unit of steps 0..3 of the
// group, dwords 3..5 the unit of steps 4..7 (see raw3_pair for the bits).
// One thread per output dword.
__global__ void repack_codes3_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                     int K, int d_out, int d_in) {
  const int nsteps = d_in >> 5;
  const size_t words_in_row = (size_t)3 * d_in / 32;
  const size_t words_per_rb = (size_t)nsteps * 48;      // 16 rows x 32 inputs x 3 bits / 32 per step
  const size_t total = (size_t)K * (d_out >> 4) * words_per_rb;
  const int nfull = nsteps >> 3;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t erb = idx / words_per_rb;               // expert * nrb + rb
    const int w = (int)(idx - erb * words_per_rb);
    const int e = (int)(erb / (d_out >> 4)), rb = (int)(erb % (d_out >> 4));
    const int sg = w / 384;                              // 384 dwords per full group
    const int wi = w - sg * 384;
    int lane, m;
    if (sg < nfull) {
      if (wi < 256) {
        lane = wi >> 2;
        m = wi & 3;
      } else {
        lane = (wi - 256) & 63;
        m = 4 + ((wi - 256) >> 6);
      }
    } else {                                             // 4-step tail: three planes
      lane = wi & 63;
      m = wi >> 6;
    }
    const int u = m / 3, j = m - 3 * u;                  // unit, dword within unit
    const int row = rb * 16 + (lane & 15), lg = lane >> 4;
    const uint32_t* srow = src + ((size_t)e * d_out + row) * words_in_row;
    uint32_t out = 0u;
    for (int f = 0; f < 5; ++f) {
      const int n = 5 * j + f, st = sg * 8 + 4 * u + (n >> 2), v = n & 3;
      const int k = st * 32 + 8 * lg + 2 * v;
      out |= code3_at(srow, k) << (3 * f);
      out |= code3_at(srow, k + 1) << (16 + 3 * f);
    }
    {
      const int st = sg * 8 + 4 * u + 3;                 // pair 15: step 3, inputs 6 and 7
      const int k = st * 32 + 8 * lg + 6;
      out |= ((code3_at(srow, k) >> j) & 1u) << 15;
      out |= ((code3_at(srow, k + 1) >> j) & 1u) << 31;
    }
    dst[idx] = out;
  }
}

void launch_repack_codes(const uint32_t* src, uint32_t* dst, int K, int d_out, int d_in, int bits,
                         hipStream_t s) {
  const size_t total = (size_t)K * d_out * bits * (d_in >> 5);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  if (bits == 3)
    hipLaunchKernelGGL(repack_codes3_kernel, dim3(blocks), dim3(256), 0, s, src, dst, K, d_out, d_in);
  else
    hipLaunchKernelGGL(repack_codes_kernel, dim3(blocks), dim3(256), 0, s, src, dst, K, d_out, d_in);
}

// scales/zeros [K][d_out][ng] -> [K][nrb][ng][16] (s | z << 16).  Flags in
// *bad: 1 a scale or zero point that is not finite, 2 a dequantized weight
// RND_f16((q - z) s) that overflows fp16 for some code q (the prefill kernels
// multiply fp16 weights), 4 a group outside the packed dequantization's range
// (zero point not an integer in 0..qmax, or |s| >= 1024): the projection then
// dequantizes through byte tables.  qmax = 3 (2-bit) or 7 (3-bit codes).
__global__ void pack_sz_kernel(const uint16_t* __restrict__ sc, const uint16_t* __restrict__ zr,
                               uint32_t* __restrict__ dst, int K, int d_out, int ng, int qmax,
                               int* bad) {
  const size_t total = (size_t)K * d_out * ng;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int g = (int)(idx % ng);
    const size_t eo = idx / ng;
    const int o = (int)(eo % d_out), e = (int)(eo / d_out);
    const uint16_t sb = sc[idx], zb = zr[idx];
    const float s = (float)__builtin_bit_cast(half_t, sb);
    const float z = (float)__builtin_bit_cast(half_t, zb);
    int flag = 0;
    if (!(fabsf(s) <= 65504.0f) || !(fabsf(z) <= 65504.0f)) flag |= 1;   // inf or nan
    if (!(fabsf(s) < 1024.0f) || !(z == rintf(z) && z >= 0.0f && z <= (float)qmax)) flag |= 4;
    if (!(flag & 1)) {
      // an fp16 infinity has all exponent bits set and a zero mantissa
      for (int q = 0; q <= qmax; ++q)
        if ((deq_bits((float)q, z, s) & 0x7FFFu) == 0x7C00u) flag |= 2;
    }
    if (flag) atomicOr(bad, flag);
    const size_t out = (((size_t)e * (d_out >> 4) + (o >> 4)) * ng + g) * 16 + (o & 15);
    dst[out] = (uint32_t)sb | ((uint32_t)zb << 16);
  }
}

void launch_pack_sz(const uint16_t* scales, const uint16_t* zeros, uint32_t* dst, int K,
                    int d_out, int ng, int bits, int* bad, hipStream_t s) {
  const size_t total = (size_t)K * d_out * ng;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_sz_kernel, dim3(blocks), dim3(256), 0, s, scales, zeros, dst, K,
                     d_out, ng, (1 << bits) - 1, bad);
}

// U [rows][r] -> [rows][r_pad] zero padded (2-byte elements)
__global__ void pad_u_kernel(const uint16_t* __restrict__ U, uint16_t* __restrict__ dst,
                             int rows, int r, int r_pad) {
  const size_t total = (size_t)rows * r_pad;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % r_pad);
    const size_t row = i / r_pad;
    dst[i] = (c < r) ? U[row * r + c] : (uint16_t)0;
  }
}

void launch_pad_u(const void* U, void* dst, int rows, int r, int r_pad, hipStream_t s) {
  const size_t total = (size_t)rows * r_pad;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pad_u_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(U), reinterpret_cast<uint16_t*>(dst),
                     rows, r, r_pad);
}

// sigma [r] (f16 or f32) -> [r_pad] f32, zero padded (f16 -> f32 is exact)
__global__ void sigma_to_f32_kernel(const void* __restrict__ src, int f16, float* __restrict__ dst,
                                    int r, int r_pad) {
  for (int c = threadIdx.x; c < r_pad; c += blockDim.x) {
    float v = 0.f;
    if (c < r)
      v = f16 ? (float)reinterpret_cast<const half_t*>(src)[c] : reinterpret_cast<const float*>(src)[c];
    dst[c] = v;
  }
}

void launch_sigma_to_f32(const void* src, int f16, float* dst, int r, int r_pad, hipStream_t s) {
  hipLaunchKernelGGL(sigma_to_f32_kernel, dim3(1), dim3(256), 0, s, src, f16, dst, r, r_pad);
}

// V [N*d_in][r] -> Vt [N][d_in/32][r_pad][32]: for each 32-input k-step, the
// k-step's inputs of every rank contiguous (one 1 KB block per 16 ranks)
__global__ void transpose_v_kernel(const uint16_t* __restrict__ V, uint16_t* __restrict__ dst,
                                   int N, int d_in, int r, int r_pad) {
  const size_t total = (size_t)N * r_pad * d_in;
  const int nsteps = d_in >> 5;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int kk = (int)(i & 31);
    const size_t q = i >> 5;
    const int c = (int)(q % r_pad);
    const size_t ns = q / r_pad;
    const int st = (int)(ns % nsteps), n = (int)(ns / nsteps);
    const int k = st * 32 + kk;
    dst[i] = (c < r) ? V[((size_t)n * d_in + k) * r + c] : (uint16_t)0;
  }
}

void launch_transpose_v(const void* V, void* dst, int N, int d_in, int r, int r_pad,
                        hipStream_t s) {
  const size_t total = (size_t)N * r_pad * d_in;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(transpose_v_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(V), reinterpret_cast<uint16_t*>(dst), N,
                     d_in, r, r_pad);
}

// Dense weight rows re-laid-out in k-step blocks: block s holds inputs
// 32 s .. 32 s + 31 of every row, 64 contiguous bytes per row, so that a
// 16-row MFMA fragment of one k-step is one contiguous 1 KB load and a tile
// of consecutive rows reads one contiguous range per k-step (a row-major
// matrix would give 64-byte pieces 2 d_in bytes apart).  One thread per
// 16-byte chunk of the output.
__global__ void block_rows_kernel(const uint4* __restrict__ W, uint4* __restrict__ dst, int rows,
                                  int d_in) {
  const size_t total = (size_t)rows * (d_in >> 3);
  const int cpr = d_in >> 3;                     // 16-byte chunks per row
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(o & 3);
    const size_t q = o >> 2;
    const int m = (int)(q % rows);
    const int st = (int)(q / rows);
    dst[o] = W[(size_t)m * cpr + st * 4 + c];
  }
}

void launch_block_rows(const void* W, void* dst, int rows, int d_in, hipStream_t s) {
  const size_t total = (size_t)rows * (d_in >> 3);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(block_rows_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(W), reinterpret_cast<uint4*>(dst), rows, d_in);
}

// Bound on the effective weight's rows, W_e = U_m Sigma V_n^T + R_e (the
// tiled decomposition of section 2.1): for every expert, an upper bound on
// max_o sum_i |W_e[o][i]| by the triangle inequality,
//   sum_i |R_e[o][i]| + sum_r |U_m[o][r]| |sigma_r| sum_i |V_n[i][r]|.
// Used to pick a power-of-two scale for intermediates before they are known.
__device__ __forceinline__ float act_bits_to_f32(uint16_t b, int bf) {
  return bf ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(half_t, (uint16_t)(b));
}

// vn[n][c] = sum_i |V[n*d_in + i][c]|; one workgroup per n, 8 input phases x
// 128 ranks, the phases summed in a fixed order.
__global__ __launch_bounds__(1024) void vnorm_kernel(const uint16_t* __restrict__ V, int d_in, int r,
                                                     int bf, float* __restrict__ vn) {
  __shared__ float s_part[8][128];
  const int n = blockIdx.x, c = threadIdx.x & 127, ph = threadIdx.x >> 7;
  float acc = 0.f;
  if (c < r)
    for (int i = ph; i < d_in; i += 8)
      acc += fabsf(act_bits_to_f32(V[((size_t)n * d_in + i) * r + c], bf));
  s_part[ph][c] = acc;
  __syncthreads();
  if (ph == 0 && c < r) {
    float t = 0.f;
    for (int q = 0; q < 8; ++q) t += s_part[q][c];
    vn[(size_t)n * r + c] = t;
  }
}

// One wave per (expert, output row); the row sums meet in l1max[e] by an
// integer max over the (non-negative) float bit patterns.
__global__ __launch_bounds__(256) void row_l1_kernel(const uint32_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint16_t* __restrict__ zeros,
                                                     const uint16_t* __restrict__ U,
                                                     const float* __restrict__ sigma,
                                                     const float* __restrict__ vn,
                                                     const int* __restrict__ m_of,
                                                     const int* __restrict__ n_of, int K, int d_out,
                                                     int d_in, int G, int r, int bf, int bits,
                                                     uint32_t* __restrict__ l1max) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)K * d_out) return;
  const int e = (int)(row / d_out), o = (int)(row % d_out);
  const int ng = d_in / G;
  float acc = 0.f;
  if (bits == 3) {
    const uint32_t* crow = codes + row * (size_t)(3 * d_in / 32);
    for (int c = lane; c < (d_in >> 4); c += 64) {       // 16 inputs per lane step
      const int g = (c << 4) / G;
      const float sa = fabsf((float)__builtin_bit_cast(half_t, (uint16_t)(scales[row * ng + g])));
      const float z = (float)__builtin_bit_cast(half_t, (uint16_t)(zeros[row * ng + g]));
      float cnt = 0.f;
      for (int j = 0; j < 16; ++j) cnt += fabsf((float)code3_at(crow, 16 * c + j) - z);
      acc += sa * cnt;
    }
  } else {
    const int nw = d_in >> 4;
    for (int w = lane; w < nw; w += 64) {
      const uint32_t word = codes[row * nw + w];
      const int g = (w << 4) / G;                   // G % 16 == 0: one group per word
      const float sa = fabsf((float)__builtin_bit_cast(half_t, (uint16_t)(scales[row * ng + g])));
      const float z = (float)__builtin_bit_cast(half_t, (uint16_t)(zeros[row * ng + g]));
      float cnt = 0.f;
      for (int j = 0; j < 16; ++j) cnt += fabsf((float)((word >> (2 * j)) & 3u) - z);
      acc += sa * cnt;
    }
  }
  if (r > 0) {
    const size_t urow = (size_t)m_of[e] * d_out + o;
    const int n = n_of[e];
    for (int c = lane; c < r; c += 64)
      acc += fabsf(act_bits_to_f32(U[urow * r + c], bf)) * fabsf(sigma[c]) * vn[(size_t)n * r + c];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    if (!(acc <= 3.0e38f)) acc = 3.0e38f;        // overflow or NaN: the largest finite bound
    atomicMax(l1max + e, __float_as_uint(acc));
  }
}

void launch_row_bound(const RowBoundArgs& b, hipStream_t s) {
  if (b.r > 0)
    hipLaunchKernelGGL(vnorm_kernel, dim3(b.N), dim3(1024), 0, s,
                       reinterpret_cast<const uint16_t*>(b.V), b.d_in, b.r, b.bf, b.vn);
  const size_t rows = (size_t)b.K * b.d_out;
  hipLaunchKernelGGL(row_l1_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, b.codes,
                     b.scales, b.zeros, reinterpret_cast<const uint16_t*>(b.U), b.sigma, b.vn,
                     b.m_of, b.n_of, b.K, b.d_out, b.d_in, b.G, b.r, b.bf, b.bits,
                     reinterpret_cast<uint32_t*>(b.l1max));
}

// Dequantized weights of one expert through the forward's own unpack path:
// one wave per (row block, step group); lane l writes its 8 inputs per step.
__global__ void debug_dequant_kernel(ProjDev p, int e, half_t* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int nsg = (p.nsteps + 7) >> 3;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.nrb * nsg) return;
  const int rb = item / nsg, sg = item - rb * nsg;
  const int gs = min(8, p.nsteps - (sg << 3));
  const int row = rb * 16 + (lane & 15);
  const int gsteps = p.group >> 5;
  const size_t zb = (((size_t)e * p.nrb + rb) * p.ng) * 16 + (lane & 15);
  half_t* orow = w + (size_t)row * p.d_in + 8 * (lane >> 4);
  if (p.bits == 3) {
    const uint32_t* gbase = p.codes + (size_t)e * p.d_out * (3 * p.d_in / 32) +
                            (size_t)rb * p.nsteps * 48 + (size_t)sg * 384;
    for (int u = 0; u < (gs >> 2); ++u) {
      uint32_t D[3];
      for (int j = 0; j < 3; ++j) {
        const int m = 3 * u + j;
        D[j] = (gs == 4) ? gbase[j * 64 + lane] : (m < 4 ? gbase[lane * 4 + m] : gbase[256 + (m - 4) * 64 + lane]);
      }
      const int s0 = (sg << 3) + 4 * u;
      half8v a[4];
      if (p.deq_lut) {
        a[0] = lut3_step<0>(D[0], D[1], D[2], deq_lut3(p.sz[zb + (size_t)((s0 + 0) / gsteps) * 16]));
        a[1] = lut3_step<1>(D[0], D[1], D[2], deq_lut3(p.sz[zb + (size_t)((s0 + 1) / gsteps) * 16]));
        a[2] = lut3_step<2>(D[0], D[1], D[2], deq_lut3(p.sz[zb + (size_t)((s0 + 2) / gsteps) * 16]));
        a[3] = lut3_step<3>(D[0], D[1], D[2], deq_lut3(p.sz[zb + (size_t)((s0 + 3) / gsteps) * 16]));
      } else {
        a[0] = deq3_step<0>(D[0], D[1], D[2], deq_const3(p.sz[zb + (size_t)((s0 + 0) / gsteps) * 16]));
        a[1] = deq3_step<1>(D[0], D[1], D[2], deq_const3(p.sz[zb + (size_t)((s0 + 1) / gsteps) * 16]));
        a[2] = deq3_step<2>(D[0], D[1], D[2], deq_const3(p.sz[zb + (size_t)((s0 + 2) / gsteps) * 16]));
        a[3] = deq3_step<3>(D[0], D[1], D[2], deq_const3(p.sz[zb + (size_t)((s0 + 3) / gsteps) * 16]));
      }
      for (int st = 0; st < 4; ++st)
        *reinterpret_cast<half8v*>(orow + (s0 + st) * 32) = a[st];
    }
    return;
  }
  const size_t codes_per_expert = (size_t)p.d_out * (p.d_in >> 4);
  const uint32_t* base = p.codes + (size_t)e * codes_per_expert +
                         (((size_t)rb * p.nsteps + (sg << 3)) * 64 + lane * gs) / 2;
  for (int d = 0; d < (gs >> 1); ++d) {
    const int s0 = (sg << 3) + 2 * d;
    const uint32_t w0 = p.sz[zb + (size_t)(s0 / gsteps) * 16];
    const uint32_t w1 = p.sz[zb + (size_t)((s0 + 1) / gsteps) * 16];
    half8v a0, a1;
    if (p.deq_lut) {
      deq_dword_lut(base[d], deq_lut(w0), deq_lut(w1), a0, a1);
    } else {
      deq_dword(base[d], deq_const(w0), deq_const(w1), a0, a1);
    }
    *reinterpret_cast<half8v*>(orow + s0 * 32) = a0;
    *reinterpret_cast<half8v*>(orow + s0 * 32 + 32) = a1;
  }
}

void launch_debug_dequant(const ProjDev& p, int expert, void* w_out, hipStream_t s) {
  const int nsg = (p.nsteps + 7) >> 3;
  const int items = p.nrb * nsg;
  hipLaunchKernelGGL(debug_dequant_kernel, dim3((items + 3) / 4), dim3(256), 0, s, p, expert,
                     reinterpret_cast<half_t*>(w_out));
}

// bfloat16 row -> fp16 row scaled by 2^-E with max|x| * 2^-E in [2^14, 2^15):
// exact for every element down to 2^-24 of the scaled range (8 significant
// bits fit in 11).  One workgroup (256 threads) per row, d % 8 == 0.
__global__ __launch_bounds__(256) void rows_to_f16_kernel(const uint16_t* __restrict__ X, int d,
                                                          const int* __restrict__ row_src,
                                                          int* __restrict__ ex, half_t* __restrict__ Y) {
  __shared__ float s_red[4];
  const int row = blockIdx.x;
  const int src = row_src ? row_src[row] : row;
  const int tid = threadIdx.x;
  const uint16_t* xr = X + (size_t)src * d;
  float m = 0.f;
  for (int c = tid; c < (d >> 3); c += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = fmaxf(m, fabsf(__uint_as_float(v[q] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(v[q] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  int e2 = 0;
  if (m > 0.f) frexpf(m, &e2);
  const int E = (m > 0.f) ? e2 - 15 : 0;
  if (tid == 0) ex[row] = E;
  half_t* yr = Y + (size_t)row * d;
  for (int c = tid; c < (d >> 3); c += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * c);
    half8v o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = (half_t)ldexpf(__uint_as_float(v[q] << 16), -E);
      o[2 * q + 1] = (half_t)ldexpf(__uint_as_float(v[q] & 0xFFFF0000u), -E);
    }
    *reinterpret_cast<half8v*>(yr + 8 * c) = o;
  }
}

void launch_rows_to_f16(const void* X, int rows, int d, const int* row_src, int* ex, void* Y,
                        hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(rows_to_f16_kernel, dim3(rows), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(X), d, row_src, ex,
                     reinterpret_cast<half_t*>(Y));
}

}  // namespace tq
