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
// Prefill shape (the decode column stage is in decode_stages.hip).  MFMA
// 16x16x32 in the activation dtype, fp32 accumulation.  A operand =
// activation rows (16 rows x 32 inputs), B operand = V_n^T rows (r-columns).
// Split-K over `nsplit` slabs: slab s holds the partial sum over its k-range;
// consumers add the slabs (deterministic, no float atomics).  The stored rank
// vectors are already multiplied by Sigma (in fp32), which every consumer
// needs.
#include "tq_device.h"

namespace tq {

// 4 waves, each owning 16 rows of a 64-row tile, over the whole k-range.
struct ColArgs2 {
  ColArgs c[2];
};

template <typename T>
__global__ __launch_bounds__(256) void colproj_kernel(ColArgs2 args) {
  typedef typename Vec8<T>::type V8;
  const ColArgs& a = args.c[blockIdx.z];
  __shared__ int s_res;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  constexpr int rt = 64;
  int seg, row0, row_end;
  if (a.ap_T > 0) {
    // every (column, token) pair: column seg owns rows seg * T ... seg * T + T - 1
    const int tpc = (a.ap_T + rt - 1) / rt;
    seg = tile / tpc;
    if (seg >= a.nseg) return;
    row0 = seg * a.ap_T + (tile - seg * tpc) * rt;
    row_end = (seg + 1) * a.ap_T;
  } else {
    seg = find_segment(a.tile_off, a.nseg, tile, &s_res);
    if (seg < 0) return;
    row0 = a.seg_off[seg] + (tile - a.tile_off[seg]) * rt;
    row_end = a.seg_off[seg + 1];
  }
  const int vblk = a.seg_vblk ? a.seg_vblk[seg] : seg;
  const int nfrag = a.r_pad >> 4;
  const int split = blockIdx.y;
  const int st0 = split * a.steps_per_split;
  const int st1 = min(a.d_in >> 5, st0 + a.steps_per_split);

  const int rbase = row0 + 16 * wave;
  const int myrow = rbase + (lane & 15);
  const bool rvalid = myrow < row_end;
  int src = 0;
  if (rvalid) src = (a.ap_T > 0) ? myrow - seg * a.ap_T : (a.row_src ? a.row_src[myrow] : myrow);
  const T* arow = reinterpret_cast<const T*>(a.A) + (size_t)src * a.lda + 8 * (lane >> 4);
  const T* vt = reinterpret_cast<const T*>(a.Vt) + (size_t)vblk * a.r_pad * a.d_in;   // [steps][r_pad][32]

  f32x4 acc[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int st = st0; st < st1; ++st) {
    V8 avv;
    if (rvalid) avv = *reinterpret_cast<const V8*>(arow + st * 32);
    else avv = __builtin_bit_cast(V8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfrag) {
        const V8 bvv = *reinterpret_cast<const V8*>(
            vt + ((size_t)st * a.r_pad + 16 * f + (lane & 15)) * 32 + 8 * (lane >> 4));
        acc[f] = mfma16(avv, bvv, acc[f]);
      }
    }
  }
  float* P = a.P + (size_t)split * a.rows_cap * a.r_pad;
  T* PH = reinterpret_cast<T*>(P);
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    if (f < nfrag) {
      const float sg = a.sigma[16 * f + (lane & 15)];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = rbase + 4 * (lane >> 4) + v;
        if (row >= row_end) continue;
        const float val = acc[f][v] * sg;
        if (a.hilo) {
          // the operand of the row stage's MFMAs: value = high + low, both in
          // the activation dtype
          const T hi = from_f32<T>(val);
          T* dst = PH + (size_t)row * 2 * a.r_pad + 16 * f + (lane & 15);
          dst[0] = hi;
          dst[a.r_pad] = from_f32<T>(val - to_f32(hi));
        } else {
          P[(size_t)row * a.r_pad + 16 * f + (lane & 15)] = val;
        }
      }
    }
  }
}

// Split-K reduction of the column stage: slab 0 += slabs 1.. (in slab
// order, deterministic).  Rows past the segment total are skipped.
struct RedArgs {
  float* P[2];
  const int* total[2];           // device row count of each projection (or nullptr)
  int total_host[2];             // row count when total is nullptr
  int r_pad[2];
  int nsplit, rows_cap;
};

__global__ __launch_bounds__(256) void colproj_reduce_kernel(RedArgs a) {
  const int z = blockIdx.y;
  const int rp = a.r_pad[z];
  const int rows = a.total[z] ? *a.total[z] : a.total_host[z];
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * rp) return;
  const size_t slab = (size_t)a.rows_cap * rp;
  float* P = a.P[z];
  float v = 0.f;
  for (int sp = 0; sp < a.nsplit; sp += 16) {
    float t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) t[u] = (sp + u < a.nsplit) ? P[i + (sp + u) * slab] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) v += t[u];
  }
  P[i] = v;
}

void launch_colproj_reduce(const ColArgs* a, int nproj, hipStream_t s) {
  if (a[0].nsplit <= 1) return;
  RedArgs r{};
  int rp_max = 0;
  for (int z = 0; z < nproj; ++z) {
    r.P[z] = a[z].P;
    r.total[z] = (a[z].ap_T > 0) ? nullptr : a[z].seg_off + a[z].nseg;
    r.total_host[z] = a[z].nseg * a[z].ap_T;
    r.r_pad[z] = a[z].r_pad;
    rp_max = a[z].r_pad > rp_max ? a[z].r_pad : rp_max;
  }
  r.nsplit = a[0].nsplit;
  r.rows_cap = a[0].rows_cap;
  const dim3 rg((unsigned)(((size_t)a[0].rows_cap * rp_max + 255) / 256), nproj);
  hipLaunchKernelGGL(colproj_reduce_kernel, rg, dim3(256), 0, s, r);
}

void launch_colproj(const ColArgs* a, int nproj, int rt, int max_tiles, Act act, hipStream_t s) {
  (void)rt;                      // 64-row tiles
  ColArgs2 args;
  args.c[0] = a[0];
  args.c[1] = a[nproj > 1 ? 1 : 0];
  const dim3 grid(max_tiles, a[0].nsplit, nproj);
  if (act == ACT_F16) hipLaunchKernelGGL((colproj_kernel<half_t>), grid, dim3(256), 0, s, args);
  else hipLaunchKernelGGL((colproj_kernel<__bf16>), grid, dim3(256), 0, s, args);
  launch_colproj_reduce(a, nproj, s);
}

}  // namespace tq
