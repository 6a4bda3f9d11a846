// Column stage of the fused low-rank forward.
//
// "TileQ" technical summary, section 2.2 (Mechanism): the batch is projected
// onto a shared factor once.  Here that is P[row][:] = V_n^T a_row for every
// row of a column's work list: for gate/up/single projections a row is a
// unique (column n, token t) pair, so V_n^T x_t is computed once for all the
// experts of column n that token t routes to; for the down projection a row
// is a slot (its input h differs per expert).  (Order of the two factor
// products: the input meets V first, as y = W x requires; see the design
// notes on the summary's wording.)
//
// MFMA 16x16x32 in the activation dtype, fp32 accumulation.  A operand =
// activation rows (16 rows x 32 inputs), B operand = V_n^T rows (r-columns).
// Split-K over `nsplit` slabs: slab s holds the partial sum over its k-range;
// consumers add the slabs (deterministic, no float atomics).
#include "tq_device.h"

namespace tq {

// WR = row fragments per workgroup (4 waves).  WR == 4: each wave owns 16
// rows; WR == 1: the 4 waves split the k-steps of the slab and reduce in LDS.
struct ColArgs2 {
  ColArgs c[2];
};

template <typename T, int WR>
__global__ __launch_bounds__(256) void colproj_kernel(ColArgs2 args) {
  typedef typename Vec8<T>::type V8;
  const ColArgs& a = args.c[blockIdx.z];
  __shared__ int s_res;
  __shared__ int s_last;
  __shared__ float s_red[(WR == 1) ? 4 * 16 * 128 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int seg = find_segment(a.tile_off, a.nseg, tile, &s_res);
  if (seg < 0) return;
  const int rt = 16 * WR;
  const int row0 = a.seg_off[seg] + (tile - a.tile_off[seg]) * rt;
  const int row_end = a.seg_off[seg + 1];
  const int vblk = a.seg_vblk ? a.seg_vblk[seg] : seg;
  const int nfrag = a.r_pad >> 4;

  const int split = blockIdx.y;
  const int st0 = split * a.steps_per_split;
  const int st1 = min(a.d_in >> 5, st0 + a.steps_per_split);

  // this wave's rows and k-steps
  const int rbase = (WR == 4) ? row0 + 16 * wave : row0;
  const int myrow = rbase + (lane & 15);
  const bool rvalid = myrow < row_end;
  int src = 0;
  if (rvalid) src = a.row_src ? a.row_src[myrow] : myrow;
  const T* arow = reinterpret_cast<const T*>(a.A) + (size_t)src * a.lda + 8 * (lane >> 4);
  const T* vt = reinterpret_cast<const T*>(a.Vt) + (size_t)vblk * a.r_pad * a.d_in;

  f32x4 acc[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kstart = (WR == 4) ? st0 : st0 + wave;
  const int kstride = (WR == 4) ? 1 : 4;
  for (int st = kstart; st < st1; st += kstride) {
    V8 av;
    if (rvalid) {
      av = *reinterpret_cast<const V8*>(arow + st * 32);
    } else {
      av = __builtin_bit_cast(V8, u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfrag) {
        const V8 bv = *reinterpret_cast<const V8*>(
            vt + (size_t)(16 * f + (lane & 15)) * a.d_in + st * 32 + 8 * (lane >> 4));
        acc[f] = mfma16(av, bv, acc[f]);
      }
    }
  }

  float* P = a.P + (size_t)split * a.rows_cap * a.r_pad;
  if (WR == 1) {
    // reduce the 4 waves' partials: s_red[wave][row 0..15][r]
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfrag) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          s_red[(wave * 16 + 4 * (lane >> 4) + v) * 128 + 16 * f + (lane & 15)] = acc[f][v];
      }
    }
    __syncthreads();
    for (int i = tid; i < 16 * a.r_pad; i += 256) {
      const int r = i / a.r_pad, c = i - r * a.r_pad;
      const int row = row0 + r;
      if (row < row_end) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) v += s_red[(w * 16 + r) * 128 + c];
        P[(size_t)row * a.r_pad + c] = v;
      }
    }
  } else {
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfrag) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = rbase + 4 * (lane >> 4) + v;
          if (row < row_end) P[(size_t)row * a.r_pad + 16 * f + (lane & 15)] = acc[f][v];
        }
      }
    }
  }
  // split-K: the last workgroup of a tile to arrive sums the slabs in slab
  // order into slab 0 (deterministic; no float atomics)
  if (a.nsplit > 1) {
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&a.counters[tile], 1) == a.nsplit - 1) ? 1 : 0;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int i = tid; i < rt * a.r_pad; i += 256) {
      const int r = i / a.r_pad, c = i - r * a.r_pad;
      const int row = row0 + r;
      if (row < row_end) {
        // slabs summed in slab order; loads issued 8 at a time
        const float* src = a.P + (size_t)row * a.r_pad + c;
        const size_t slab = (size_t)a.rows_cap * a.r_pad;
        float v = 0.f;
        int sp = 0;
        for (; sp + 8 <= a.nsplit; sp += 8) {
          float t[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) t[u] = __builtin_nontemporal_load(src + (sp + u) * slab);
#pragma unroll
          for (int u = 0; u < 8; ++u) v += t[u];
        }
        for (; sp < a.nsplit; ++sp) v += __builtin_nontemporal_load(src + sp * slab);
        a.P[(size_t)row * a.r_pad + c] = v;
      }
    }
  }
}

void launch_colproj(const ColArgs* a, int nproj, int rt, int max_tiles, Act act, hipStream_t s) {
  ColArgs2 args;
  args.c[0] = a[0];
  args.c[1] = a[nproj > 1 ? 1 : 0];
  const dim3 grid(max_tiles, a[0].nsplit, nproj);
  if (act == ACT_F16) {
    if (rt == 16) hipLaunchKernelGGL((colproj_kernel<half_t, 1>), grid, dim3(256), 0, s, args);
    else hipLaunchKernelGGL((colproj_kernel<half_t, 4>), grid, dim3(256), 0, s, args);
  } else {
    if (rt == 16) hipLaunchKernelGGL((colproj_kernel<__bf16, 1>), grid, dim3(256), 0, s, args);
    else hipLaunchKernelGGL((colproj_kernel<__bf16, 4>), grid, dim3(256), 0, s, args);
  }
}

}  // namespace tq
