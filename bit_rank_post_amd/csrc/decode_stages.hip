// Decode-path companion stages of the residual kernels, fused per dependency
// level into one launch of 256-thread workgroups:
//   before gate/up:  routing (one workgroup, small batches), activation
//                    preparation of x, column stage of gate/up
//   before down:     activation preparation of h + column stage of down
// (the parts of a launch do not read each other's results).  Many small
// workgroups spread the few hundred KB each part reads over the CUs: one
// CU's load path, not HBM, bounds a workgroup that reads a lot.
//
// Activation preparation.  The decode residual kernel feeds the codes to the
// MFMA without dequantizing them: each packed fp16 half holds 1 + q*c (c =
// 1/64, 1/16 or 1/4 for 2-bit codes, see unpack16(), and 1/64, 1/16 or 1/8
// for 3-bit codes, see raw3_pair(), depending on where the code sits).
// With the activation entering as x'_k = x~_k / c_k, a group sum of products
// is  sum_k (1 + q_k c_k) x'_k = X'_g + sum_k q_k x~_k,  so the residual term
// of a group is s * (C_g - X'_g - z * X~_g).  Per activation row this writes
// x'_k (fp16), the group sums X~_g and X'_g (fp32) and the exponent E of the
// exact power-of-two scaling x~ = x * 2^-E that keeps 64 |x~| inside the fp16
// range (max|x~| in [2^8, 2^9)).
//
// Column stage ("TileQ" technical summary, section 2.2: the batch is
// projected onto a shared factor once): P[slab][row][:] = Sigma (V_n^T a_row)
// over the slab's 1024 inputs, for the rows of a 16-row tile.  A workgroup
// takes one rank-fragment group of a (tile, slab); its 4 waves are k-groups
// that meet in LDS.  Consumers add the slabs (deterministic, no atomics).
#include "route_body.h"

namespace tq {

constexpr int DS_THREADS = 256;
constexpr int DS_SLAB_STEPS = 32;        // 32 k-steps = 1024 inputs per slab

// 1/c of input 8 c + j is 2^e with e the class exponent of its code's
// mantissa position in the decode kernel's operand, a function of the step
// within a period of 4 k-steps (s = (c / 4) % 4) and of the pair v = j / 2:
// e = (prep_class_exponents(bits) >> 3 (4 s + v)) & 7.
//   2-bit (unpack16): 1/c = 64, 16, 4 for v = 0, 1, 2 and, for v = 3, 64 at
//   even steps, 16 at odd steps.
//   3-bit (raw3_pair): pair n = 4 s + v of a 4-step unit has 1/c =
//   2^(10 - cls3(n)).
__host__ __device__ constexpr uint64_t prep_class_exponents(int bits) {
  uint64_t t = 0;
  for (int n = 0; n < 16; ++n) {
    const int s = n >> 2, v = n & 3;
    const int e = (bits == 3) ? 10 - cls3(n) : (v == 0 ? 6 : v == 1 ? 4 : v == 2 ? 2 : ((s & 1) ? 4 : 6));
    t |= (uint64_t)e << (3 * n);
  }
  return t;
}

// One row per workgroup; thread t owns the 8-element chunks t + 256 i.  The
// row is read once (up to 8 chunks per thread stay in registers; longer rows
// re-read the rest).
template <typename T, int CPG>
__device__ void prep_row(const PrepArgs& a, int rows, int blk, float* s_red /*[4]*/) {
  typedef typename Vec8<T>::type V8;
  constexpr int KEEP = 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int row = blk;
  int src = -1;
  if (row < rows) src = a.row_src ? a.row_src[row] : row;
  if (src < 0) return;                   // uniform over the workgroup
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
  if (lane == 0) s_red[wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  int e2 = 0;
  if (m > 0.f) frexpf(m, &e2);
  const int E = (m > 0.f) ? e2 - 9 : 0;
  if (tid == 0) a.ex[row] = E;
  // scaled, class-scaled copy and group sums; a group is CPG = G/8
  // consecutive chunks, i.e. CPG consecutive lanes of one wave (G <= 256)
  half_t* xo = reinterpret_cast<half_t*>(a.Xp) + (size_t)row * a.d;
  float* sums = a.sums + (size_t)row * (a.d / a.G) * 2;
  auto emit = [&](int c, const V8& v) {
    float st = 0.f, sp = 0.f;
    if (c < nch) {
      half8v o;
      const uint32_t ce = (uint32_t)(a.cls_exp >> (12 * ((c >> 2) & 3)));   // this step's 4 exponents
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = (int)((ce >> (3 * (j >> 1))) & 7u);
        const half_t xt = (half_t)ldexpf((float)v[j], -E);
        const half_t xp = (half_t)ldexpf((float)xt, e);
        o[j] = xp;
        st += (float)xt;
        sp += (float)xp;
      }
      *reinterpret_cast<half8v*>(xo + 8 * c) = o;
    }
    st = group_sum<CPG>(st);
    sp = group_sum<CPG>(sp);
    if (c < nch && (c % CPG) == 0) {
      sums[2 * (c / CPG)] = st;
      sums[2 * (c / CPG) + 1] = sp;
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

template <typename T>
__device__ void prep_rows(const PrepArgs& a, int rows, int blk, float* s_red) {
  switch (a.G >> 3) {
    case 4: prep_row<T, 4>(a, rows, blk, s_red); break;
    case 8: prep_row<T, 8>(a, rows, blk, s_red); break;
    case 16: prep_row<T, 16>(a, rows, blk, s_red); break;
    default: prep_row<T, 32>(a, rows, blk, s_red); break;
  }
}

// Column stage for one (16-row tile, 1024-input slab, rank-fragment group
// fg: fragments fg and fg + 4 of r_pad / 16).  Wave w is k-group w (k-steps
// w + 4 i of the slab).  All loads of a wave are issued before its MFMAs;
// steps outside the slab, rows outside the tile and missing fragments read
// zeros through out-of-range offsets.
template <typename T>
__device__ void col_tile(const ColArgs& a, int blk, int* s_res, float* s_red /*[4][16][32]*/) {
  typedef typename Vec8<T>::type V8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fg = blk & 3;
  const int split = (blk >> 2) % a.nsplit;
  const int tile = (blk >> 2) / a.nsplit;
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
  // k-groups meet in LDS: s_red[kg][row][q][16]
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      s_red[(kg * 16 + 4 * (lane >> 4) + v) * 32 + 16 * q + (lane & 15)] = acc[q][v];
  }
  __syncthreads();
  float* P = a.P + (size_t)split * a.rows_cap * a.r_pad;
  for (int i = tid; i < 16 * 32; i += DS_THREADS) {
    const int r = i >> 5, qc = i & 31;
    const int f = fg + 4 * (qc >> 4), c = 16 * f + (qc & 15);
    const int row = row0 + r;
    if (row < row_end && f < nfrag) {
      const float v = s_red[r * 32 + qc] + s_red[(16 + r) * 32 + qc] +
                      s_red[(32 + r) * 32 + qc] + s_red[(48 + r) * 32 + qc];
      P[(size_t)row * a.r_pad + c] = v * a.sigma[c];
    }
  }
}

struct PrepColArgs {
  PrepArgs prep;
  int prep_rows, prep_blocks;
  ColArgs col[2];
  int ncol, col_blocks;          // column-stage blocks per projection (tiles x slabs)
  int route;                     // 1: workgroup 0 runs the routing (independent of the rest)
  RouteArgs ra;
};

constexpr int DS_ROUTE_SMAX = 1024;
constexpr int DS_LDS_FLOATS = 5680;      // >= routing scratch, 4 x 16 x 32 reduction, 4 maxima

template <typename T>
__global__ __launch_bounds__(DS_THREADS) void prep_col_kernel(PrepColArgs a) {
  __shared__ float s_red[DS_LDS_FLOATS];
  __shared__ int s_res;
  static_assert(route_lds_ints(DS_ROUTE_SMAX) <= DS_LDS_FLOATS && 4 * 16 * 32 <= DS_LDS_FLOATS, "LDS");
  int b = blockIdx.x;
  if (a.route) {
    if (b == 0) {
      route_block<DS_ROUTE_SMAX, DS_THREADS>(a.ra, reinterpret_cast<int*>(s_red));
      return;
    }
    --b;
  }
  if (b < a.prep_blocks) {
    prep_rows<T>(a.prep, a.prep_rows, b, s_red);
  } else {
    const int c = b - a.prep_blocks;
    const int z = c / a.col_blocks;
    col_tile<T>(a.col[z], c - z * a.col_blocks, &s_res, s_red);
  }
}

int decode_col_splits(int d_in) { return ((d_in >> 5) + DS_SLAB_STEPS - 1) / DS_SLAB_STEPS; }

bool prep_col_can_route(const RouteArgs& ra) {
  return ra.S <= DS_ROUTE_SMAX && ra.T <= DS_ROUTE_SMAX && ((ra.S + 63) / 64) * ra.K <= DS_ROUTE_SMAX;
}

void launch_prep_col(const PrepArgs* prep, int prep_rows, const ColArgs* col, int ncol,
                     int col_tiles, const RouteArgs* route, Act act, hipStream_t s) {
  PrepColArgs a{};
  if (route) {
    a.route = 1;
    a.ra = *route;
  }
  if (prep) {
    a.prep = *prep;
    a.prep.cls_exp = prep_class_exponents(prep->bits);
    a.prep_rows = prep_rows;
    a.prep_blocks = prep_rows;
  }
  a.ncol = ncol;
  for (int z = 0; z < ncol; ++z) a.col[z] = col[z];
  a.col_blocks = ncol ? col_tiles * col[0].nsplit * 4 : 0;   // x 4 rank-fragment groups
  const int blocks = a.route + a.prep_blocks + ncol * a.col_blocks;
  if (blocks == 0) return;
  if (act == ACT_F16)
    hipLaunchKernelGGL(prep_col_kernel<half_t>, dim3(blocks), dim3(DS_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(prep_col_kernel<__bf16>, dim3(blocks), dim3(DS_THREADS), 0, s, a);
}

}  // namespace tq
