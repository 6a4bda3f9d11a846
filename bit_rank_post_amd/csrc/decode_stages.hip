// Decode-path companion stages of the residual kernels, fused per dependency
// level into one launch of 1024-thread workgroups:
//   before gate/up:  activation preparation of x   + column stage of gate/up
//   before down:     activation preparation of h   + column stage of down
// (the two halves of a launch are independent of each other).
//
// Activation preparation.  The decode residual kernel feeds the 2-bit codes
// to the MFMA without dequantizing them: each packed fp16 half holds 1 + q*c
// (c = 1/64, 1/16 or 1/4 depending on where the code sits, see unpack16()).
// With the activation entering as x'_k = x~_k / c_k, a group sum of products
// is  sum_k (1 + q_k c_k) x'_k = X'_g + sum_k q_k x~_k,  so the residual term
// of a group is s * (C_g - X'_g - z * X~_g).  Per activation row this writes
// x'_k (fp16), the group sums X~_g and X'_g (fp32) and the exponent E of the
// exact power-of-two scaling x~ = x * 2^-E that keeps 64 |x~| inside the fp16
// range (max|x~| in [2^8, 2^9)).
//
// Column stage ("TileQ" technical summary, section 2.2: the batch is
// projected onto a shared factor once): P[slab][row][:] = Sigma (V_n^T a_row)
// over the slab's 1024 inputs, for the rows of a 16-row tile.  A workgroup's
// 16 waves are 4 rank-fragment groups x 4 k-groups; the k-groups meet in LDS.
// Consumers add the slabs (deterministic, no atomics).
#include "tq_device.h"

namespace tq {

constexpr int DS_THREADS = 1024;
constexpr int DS_SLAB_STEPS = 32;        // 32 k-steps = 1024 inputs per slab

// 1/c of input k: step parity b = (k/32) % 2, pair v = (k % 8) / 2.
__device__ __forceinline__ float class_inv(int k) {
  const int b = (k >> 5) & 1, v = (k & 7) >> 1;
  // b = 0: {64, 16, 4, 64};  b = 1: {64, 16, 4, 16}
  return (v == 0) ? 64.f : (v == 1) ? 16.f : (v == 2) ? 4.f : (b ? 16.f : 64.f);
}

// Four rows per workgroup, 256 threads per row; thread t of a row owns the
// 8-element chunks t + 256 i.  The row is read once (up to 8 chunks per
// thread stay in registers; longer rows re-read the rest).
template <typename T>
__device__ void prep_rows(const PrepArgs& a, int rows, int blk, float* s_red /*[16]*/) {
  typedef typename Vec8<T>::type V8;
  constexpr int KEEP = 8;
  const int sub = threadIdx.x >> 8, tid = threadIdx.x & 255;
  const int lane = tid & 63, wv = tid >> 6;
  const int row = blk * 4 + sub;
  int src = -1;
  if (row < rows) src = a.row_src ? a.row_src[row] : row;
  const bool ok = src >= 0;
  const T* xr = reinterpret_cast<const T*>(a.X) + (size_t)(ok ? src : 0) * a.d;
  const int nch = ok ? (a.d >> 3) : 0;
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
  if (lane == 0) s_red[sub * 4 + wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[sub * 4], s_red[sub * 4 + 1]), fmaxf(s_red[sub * 4 + 2], s_red[sub * 4 + 3]));
  if (!ok) return;                       // no barrier follows
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
  for (int i = 0; i < KEEP; ++i)
    if (256 * i < nch) emit(tid + 256 * i, kept[i]);   // uniform per row: shuffles stay whole
  for (int base = 256 * KEEP; base < nch; base += 256) {
    const int c = base + tid;
    V8 v{};
    if (c < nch) v = *reinterpret_cast<const V8*>(xr + 8 * c);
    emit(c, v);
  }
}

// Column stage for one (16-row tile, 1024-input slab).  Waves: rank-fragment
// group fg = w & 3 (fragments fg, fg + 4 of r_pad / 16), k-group kg = w >> 2
// (k-steps kg + 4 i of the slab).  All loads of a wave are issued before its
// MFMAs; steps outside the slab and rows outside the tile read zeros through
// out-of-range offsets.
template <typename T>
__device__ void col_tile(const ColArgs& a, int blk, int* s_res, float* s_red /*[4][16][128]*/) {
  typedef typename Vec8<T>::type V8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fg = w & 3, kg = w >> 2;
  const int split = blk % a.nsplit;
  const int tile = blk / a.nsplit;
  int seg, row0, row_end;
  if (a.ap_T > 0) {
    const int tpc = (a.ap_T + 15) >> 4;
    seg = tile / tpc;
    if (seg >= a.nseg) return;
    row0 = seg * a.ap_T + (tile - seg * tpc) * 16;
    row_end = (seg + 1) * a.ap_T;
  } else {
    seg = find_segment(a.tile_off, a.nseg, tile, s_res);
    if (seg < 0) return;
    row0 = a.seg_off[seg] + (tile - a.tile_off[seg]) * 16;
    row_end = a.seg_off[seg + 1];
  }
  const int vblk = a.seg_vblk ? a.seg_vblk[seg] : seg;
  const int nfrag = a.r_pad >> 4;
  const int nsteps = a.d_in >> 5;
  const int st0 = split * DS_SLAB_STEPS;
  const int st1 = min(nsteps, st0 + DS_SLAB_STEPS);

  const int myrow = row0 + (lane & 15);
  const bool rvalid = myrow < row_end;
  int src = 0;
  if (rvalid) src = (a.ap_T > 0) ? myrow - seg * a.ap_T : (a.row_src ? a.row_src[myrow] : myrow);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, OOB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.Vt, OOB);
  const uint32_t avo = rvalid ? ((uint32_t)src * a.lda + 8 * (lane >> 4)) * 2u : OOB;
  // Vt [N][steps][r_pad][32]: fragment f of step st is 1 KB at (st r_pad + 16 f) * 64
  const uint32_t vvo = ((uint32_t)vblk * a.r_pad * a.d_in + (lane & 15) * 32 + 8 * (lane >> 4)) * 2u;
  constexpr int NI = DS_SLAB_STEPS / 4;
  u32x4 av[NI], bv[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int st = st0 + kg + 4 * i;
    const bool ok = st < st1;
    av[i] = bload128(ra, ok ? avo : OOB, ok ? st * 64u : 0u);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int f = fg + 4 * q;
      const bool fok = ok && f < nfrag;
      bv[i][q] = bload128(rv, fok ? vvo + 1024u * f : OOB, fok ? st * a.r_pad * 64u : 0u);
    }
  }
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (fg + 4 * q < nfrag)
        acc[q] = mfma16(__builtin_bit_cast(V8, av[i]), __builtin_bit_cast(V8, bv[i][q]), acc[q]);
  // k-groups meet in LDS: s_red[kg][row][rank]
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int f = fg + 4 * q;
    if (f < nfrag) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        s_red[(kg * 16 + 4 * (lane >> 4) + v) * 128 + 16 * f + (lane & 15)] = acc[q][v];
    }
  }
  __syncthreads();
  float* P = a.P + (size_t)split * a.rows_cap * a.r_pad;
  for (int i = tid; i < 16 * a.r_pad; i += DS_THREADS) {
    const int r = i / a.r_pad, c = i - r * a.r_pad;
    const int row = row0 + r;
    if (row < row_end) {
      const float v = s_red[r * 128 + c] + s_red[(16 + r) * 128 + c] +
                      s_red[(32 + r) * 128 + c] + s_red[(48 + r) * 128 + c];
      P[(size_t)row * a.r_pad + c] = v * a.sigma[c];
    }
  }
}

struct PrepColArgs {
  PrepArgs prep;
  int prep_rows, prep_blocks;
  ColArgs col[2];
  int ncol, col_blocks;          // column-stage blocks per projection (tiles x slabs)
};

template <typename T>
__global__ __launch_bounds__(DS_THREADS) void prep_col_kernel(PrepColArgs a) {
  __shared__ float s_red[4 * 16 * 128];
  __shared__ int s_res;
  const int b = blockIdx.x;
  if (b < a.prep_blocks) {
    prep_rows<T>(a.prep, a.prep_rows, b, s_red);
  } else {
    const int c = b - a.prep_blocks;
    const int z = c / a.col_blocks;
    col_tile<T>(a.col[z], c - z * a.col_blocks, &s_res, s_red);
  }
}

int decode_col_splits(int d_in) { return ((d_in >> 5) + DS_SLAB_STEPS - 1) / DS_SLAB_STEPS; }

void launch_prep_col(const PrepArgs* prep, int prep_rows, const ColArgs* col, int ncol,
                     int col_tiles, Act act, hipStream_t s) {
  PrepColArgs a{};
  if (prep) {
    a.prep = *prep;
    a.prep_rows = prep_rows;
    a.prep_blocks = (prep_rows + 3) / 4;
  }
  a.ncol = ncol;
  for (int z = 0; z < ncol; ++z) a.col[z] = col[z];
  a.col_blocks = ncol ? col_tiles * col[0].nsplit : 0;
  const int blocks = a.prep_blocks + ncol * a.col_blocks;
  if (blocks == 0) return;
  if (act == ACT_F16)
    hipLaunchKernelGGL(prep_col_kernel<half_t>, dim3(blocks), dim3(DS_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(prep_col_kernel<__bf16>, dim3(blocks), dim3(DS_THREADS), 0, s, a);
}

}  // namespace tq
