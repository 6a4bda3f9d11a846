// Column stage of the fused low-rank forward, and the dense shared expert.
//
// "TileQ" technical summary, section 2.2 (Mechanism): the batch is projected
// onto a shared factor once.  Here that is P[row][:] = V_n^T a_row for every
// row of a column's work list: for gate/up/single projections a row is a
// unique (column n, token t) pair, so V_n^T x_t is computed once for all the
// experts of column n that token t routes to; for the down projection a row
// is a slot (its input h differs per expert).  The input meets V first, as
// y = W x requires.
//
// Prefill shape (the decode column stage is in decode_stages.hip): one
// workgroup covers the whole k-range of its rows, except for the column
// stage that feeds the combine, which may split the k-range over
// blockIdx.z into fp32 slabs (summed by the combine) when its tiles alone
// would leave half the grid's workgroup slots empty.  MFMA 16x16x32 in the
// activation dtype, fp32 accumulation; A operand = V_n^T rows (rank rows),
// B operand = activation rows.  The stored rank vectors are already
// multiplied by Sigma (in fp32), which every consumer needs.
#include "tq_device.h"

namespace tq {

// ---- dense weights x gathered activation rows (prefill) ---------------------
// out(row n, m) = sum_k W[m][k] a[src(n)][k] for weight rows m of one M tile
// and a tile of 128 activation rows.  Both operands stream through LDS in a
// ring of RG_NSLOT slots of 64 inputs (two MFMA k-steps): per stage, 128
// weight rows and 128 activation rows arrive by 16-byte loads with the LDS
// destination, already in MFMA fragment order (one 1 KB fragment per load
// instruction), RG_DEPTH stages ahead of the MFMAs.  8 waves: wave (wm, wn)
// takes weight fragments wm and wm + 4 against activation fragments
// 4 wn .. 4 wn + 3.
//   RG_COL:   column stage, W = V_n^T of the row's segment (rank rows), out =
//             Sigma-scaled rank vectors (fp32, or high/low parts).
//   RG_DUAL:  dense SwiGLU input: the first half of the weight fragments
//             from W0 (gate), the second from W1 (up) for the same output
//             rows; out = RND_act(silu(g) u).
// Weights of every mode are stored in k-step blocks ([d_in / 32][rows][32]:
// V^T at upload, dense weights by launch_block_rows), so each fragment load
// reads 1 KB of contiguous memory.
//   RG_PLAIN: dense single projection, 128 output rows, fp32 out; split-K
//             over blockIdx.z into separate slabs.
enum RgMode { RG_COL = 0, RG_DUAL = 1, RG_PLAIN = 2 };
constexpr int RG_WAVES = 8;
constexpr int RG_A = 0;                          // [KS][4 FA frags][64 lanes] x 16 B, then
                                                 // the activations, [KS][8 frags][64 lanes]

struct RgArgs {
  ColArgs c[2];                  // RG_COL: per projection (blockIdx.z)
  DenseArgs d;                   // RG_DUAL / RG_PLAIN
  int nsplit;                    // RG_PLAIN: k-splits (blockIdx.z), slab stride T * d_out
  int ntiles;                    // row tiles of the grid (before the XCD remap)
  int nwt;                       // RG_DUAL / RG_PLAIN: weight tiles
};

// KS: MFMA k-steps (32 inputs) per stage: 2 (32 KB slots, one workgroup per
// CU) or 1 (16 KB slots, two workgroups per CU).  FA: weight fragments per
// wave, 2 (a tile of 128 weight rows) or 4 (256 rows, dense modes: half the
// LDS reads per MFMA; 48 KB slots, a ring of three).
template <typename T, int MODE, int KS, int FA = 2>
__global__ __launch_bounds__(64 * RG_WAVES) void rowgemm_kernel(RgArgs args) {
  typedef typename Vec8<T>::type V8;
  static_assert(FA == 2 || (FA == 4 && MODE != RG_COL), "weight fragments per wave");
  constexpr int RG_KS = KS;
  constexpr int NFA = 4 * FA;                        // weight fragments of the tile
  constexpr int RG_B = RG_KS * NFA * 1024;
  constexpr int RG_BYTES = RG_KS * (NFA + 8) * 1024;
  constexpr int RG_NI = RG_KS * (NFA + 8) / RG_WAVES;   // loads per wave per stage
  constexpr int SIN = 32 * KS;                       // inputs per stage
  constexpr int RG_NSLOT = (3 * RG_BYTES > 96 * 1024) ? 3 : 4, RG_DEPTH = RG_NSLOT - 1;
  static_assert(RG_NSLOT * RG_BYTES <= 150 * 1024, "LDS budget");
  static_assert(RG_NI * RG_WAVES == RG_KS * (NFA + 8), "loads split evenly over the waves");
  __shared__ __attribute__((aligned(16))) char s0[RG_BYTES];
  __shared__ __attribute__((aligned(16))) char s1[RG_BYTES];
  __shared__ __attribute__((aligned(16))) char s2[RG_BYTES];
  __shared__ __attribute__((aligned(16))) char s3[RG_NSLOT > 3 ? RG_BYTES : 16];
  __shared__ int s_src[128];
  __shared__ int s_res;
  char* const slot[4] = {s0, s1, s2, s3};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave & 3, wn = wave >> 2;

  // Workgroup W runs on XCD W mod 8.  Column stage: consecutive row tiles on
  // one XCD, so the workgroups of one segment share its weights in that
  // XCD's L2.  Dense modes (1D grid): the row tiles of one weight tile on
  // one XCD (its weights come from HBM once into that L2), the weight tiles
  // dealt to the 8 XCDs in turn, so every XCD gets an equal share even when
  // there are fewer row tiles than XCDs.
  int tile, wtile;
  if constexpr (MODE == RG_COL) {
    // the routed tile count (the last tile prefix; the grid covers the
    // bound args.ntiles): each XCD takes an equal run of the routed tiles
    const int* toff = blockIdx.z ? args.c[1].tile_off : args.c[0].tile_off;
    const int nseg = blockIdx.z ? args.c[1].nseg : args.c[0].nseg;
    const int ntot = min(args.ntiles, sload(toff, nseg));
    const int per = (ntot + 7) >> 3;
    if ((int)(blockIdx.x >> 3) >= per) return;
    tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    wtile = blockIdx.y;
    if (tile >= ntot) return;
  } else {
    const int j = blockIdx.x >> 3;
    tile = j % args.ntiles;
    wtile = (j / args.ntiles) * 8 + (blockIdx.x & 7);
    if (wtile >= args.nwt) return;
  }
  if (tile >= args.ntiles) return;

  int n0, n_end, d_in, M, lda;
  const void* X;
  const char* wbase[2];
  uint32_t wbytes, wrs, wks;           // weight buffer size, row and k-step strides (bytes)
  int st0 = 0, st1;
  int sp = 0;                          // RG_COL k-split (fp32 slab) of this workgroup
  // (a copy, not a pointer into the kernel arguments: the fields stay scalar)
  ColArgs ca{};
  if constexpr (MODE == RG_COL) {
    if (blockIdx.z) ca = args.c[1];
    else ca = args.c[0];
    const ColArgs& a = ca;
    const int seg = find_segment(a.tile_off, a.nseg, tile, &s_res);
    if (seg < 0) return;
    n0 = a.seg_off[seg] + (tile - a.tile_off[seg]) * 128;
    n_end = a.seg_off[seg + 1];
    const int vblk = a.seg_vblk ? a.seg_vblk[seg] : seg;
    d_in = a.d_in;
    M = a.r_pad;
    lda = a.lda;
    X = a.A;
    const size_t vsz = (size_t)(d_in >> 5) * a.r_pad * 64;
    wbase[0] = wbase[1] = reinterpret_cast<const char*>(a.Vt) + (size_t)vblk * vsz;
    wbytes = (uint32_t)vsz;
    wrs = 64u;
    wks = (uint32_t)a.r_pad * 64u;
    st1 = d_in / SIN;
    if (a.nsplit > 1) {
      // one projection split over blockIdx.z into k-ranges, each its own slab
      sp = blockIdx.z;
      const int sps = __builtin_amdgcn_readfirstlane((st1 + a.nsplit - 1) / a.nsplit);
      st0 = min(st1, sp * sps);
      st1 = min(st1, st0 + sps);
    }
    if (tid < 128) {
      const int n = n0 + tid;
      s_src[tid] = (n < n_end) ? (a.row_src ? a.row_src[n] : n) : -1;
    }
  } else {
    const DenseArgs& a = args.d;
    n0 = tile * 128;
    n_end = a.T;
    d_in = a.d_in;
    M = a.d_out;
    lda = a.d_in;
    X = a.X;
    wbase[0] = reinterpret_cast<const char*>(a.W0);
    wbase[1] = reinterpret_cast<const char*>(MODE == RG_DUAL ? a.W1 : a.W0);
    // k-step-blocked weights (launch_block_rows), like V^T above
    wbytes = (uint32_t)((size_t)M * d_in * 2);
    wrs = 64u;
    wks = (uint32_t)M * 64u;
    const int nst = d_in / SIN;
    // (uniform: the division may be done in vector registers)
    const int sps = __builtin_amdgcn_readfirstlane((nst + args.nsplit - 1) / args.nsplit);
    st0 = blockIdx.z * sps;
    st1 = min(nst, st0 + sps);
    if (tid < 128) {
      const int n = n0 + tid;
      s_src[tid] = (n < n_end) ? n : -1;
    }
  }
  // weight rows of this M tile: RG_DUAL 32 FA output rows (x2 matrices),
  // else 64 FA
  const int m0 = wtile * (MODE == RG_DUAL ? 32 * FA : 64 * FA);
  __syncthreads();
  const int nv = min(128, n_end - n0);
  // (uniform: the activation buffer resource lives in scalar registers)
  const int row_lo = __builtin_amdgcn_readfirstlane(s_src[0]);
  const int row_hi = __builtin_amdgcn_readfirstlane(s_src[max(nv - 1, 0)]);

  // per-lane offsets of this wave's loads: load q = wave * NI + i; q < NFA
  // KS: weight fragment (k-step q / NFA, fragment q % NFA), else activation
  // fragment (k-step, fragment q % 8 of the rest)
  uint32_t vo[RG_NI];
  bool isw[RG_NI];
  int wsel[RG_NI], ks_of[RG_NI], fr_of[RG_NI];
#pragma unroll
  for (int i = 0; i < RG_NI; ++i) {
    const int q = wave * RG_NI + i;
    const bool w = q < NFA * RG_KS;
    const int qq = w ? q : q - NFA * RG_KS;
    const int ks = w ? qq / NFA : qq >> 3, f = w ? qq % NFA : qq & 7;
    isw[i] = w;
    ks_of[i] = ks;
    fr_of[i] = f;
    if (w) {
      // weight row of fragment f (dual: the first half gate, the second up)
      int m;
      if (MODE == RG_DUAL) {
        wsel[i] = f / (NFA / 2);
        m = m0 + 16 * (f % (NFA / 2)) + l16;
      } else {
        wsel[i] = 0;
        m = m0 + 16 * f + l16;
      }
      // k-step-blocked weights: the k-step goes into the uniform offset
      vo[i] = (m < M) ? (uint32_t)m * wrs + lg * 16u : OOB;
    } else {
      wsel[i] = 0;
      const int src = s_src[16 * f + l16];
      vo[i] = (src >= 0) ? ((uint32_t)(src - row_lo) * lda + ks * 32 + 8 * lg) * 2u : OOB;
    }
  }
  __amdgpu_buffer_rsrc_t rw[2];
  rw[0] = make_rsrc(wbase[0], wbytes);
  rw[1] = make_rsrc(wbase[1], wbytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(
      reinterpret_cast<const T*>(X) + (size_t)max(row_lo, 0) * lda,
      (uint32_t)min<size_t>((size_t)(row_hi - row_lo + 1) * lda * 2u, (size_t)OOB));
  const int nstage = st1 - st0;

  auto issue = [&](int b, char* base) {
    const bool live = b < nstage;
    const int st = __builtin_amdgcn_readfirstlane(st0 + (live ? b : 0));   // a scalar offset
#pragma unroll
    for (int i = 0; i < RG_NI; ++i) {
      char* dst = isw[i] ? base + RG_A + (ks_of[i] * NFA + fr_of[i]) * 1024
                         : base + RG_B + (ks_of[i] * 8 + fr_of[i]) * 1024;
      if (isw[i]) {
        // k-step offset: whole k-step blocks of the blocked weights
        const uint32_t so = (uint32_t)(KS * st + ks_of[i]) * wks;
        dma16(wsel[i] ? rw[1] : rw[0], dst, live ? vo[i] : OOB, so);
      } else {
        dma16(rx, dst, live ? vo[i] : OOB, (uint32_t)st * (SIN * 2u));
      }
    }
  };

  // wave (wm, wn): weight fragments wm + 4 i (i < FA) against activation
  // fragments 4 wn + j (j < 4)
  f32x4 acc[FA][4];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const char* base) {
#pragma unroll
    for (int ks = 0; ks < RG_KS; ++ks) {
      V8 av[FA];
#pragma unroll
      for (int i = 0; i < FA; ++i)
        av[i] = *reinterpret_cast<const V8*>(base + RG_A + (ks * NFA + wm + 4 * i) * 1024 + lane * 16);
      V8 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const V8*>(base + RG_B + (ks * 8 + 4 * wn + j) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < FA; ++i) acc[i][j] = mfma16(av[i], b[j], acc[i][j]);
    }
  };

  // ring over stages (protocol of the grouped residual GEMMs): whole rounds,
  // stage-times past the end only wait and issue empty loads
#pragma unroll
  for (int b = 0; b < RG_DEPTH; ++b) issue(b, slot[b]);
  for (int t = 0; t < nstage; t += RG_NSLOT) {
#pragma unroll
    for (int u = 0; u < RG_NSLOT; ++u) {
      const int tau = t + u;
      wait_vm<RG_NI * (RG_DEPTH - 1)>();
      bar_nofence();
      if (tau < nstage) compute(slot[u]);
      issue(tau + RG_DEPTH, slot[(u + RG_DEPTH) % RG_NSLOT]);
    }
  }
  wait_vm<0>();

  // epilogue: lane holds out(row n0 + 16 (4 wn + j) + l16, weight rows
  // m(i) + 4 lg + v) in acc[i][j][v]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nl = 16 * (4 * wn + j) + l16;
    const int n = n0 + nl;
    if (nl >= nv) continue;
    if constexpr (MODE == RG_COL) {
      const ColArgs& a = ca;
      T* PH = reinterpret_cast<T*>(a.P);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = 16 * (wm + 4 * i) + 4 * lg;
        if (m >= a.r_pad) continue;
        const f32x4 sg = *reinterpret_cast<const f32x4*>(a.sigma + m);
        const f32x4 v = acc[i][j] * sg;
        if (a.hilo) {
          T hi[4], lo[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            hi[c] = from_f32<T>(v[c]);
            lo[c] = from_f32<T>(v[c] - to_f32(hi[c]));
          }
          T* dst = PH + (size_t)n * 2 * a.r_pad + m;
          *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, hi);
          *reinterpret_cast<u32x2*>(dst + a.r_pad) = __builtin_bit_cast(u32x2, lo);
        } else {
          *reinterpret_cast<f32x4*>(a.P + ((size_t)sp * a.rows_cap + n) * a.r_pad + m) = v;
        }
      }
    } else if constexpr (MODE == RG_DUAL) {
      // gate fragment wm + 4 i pairs with up fragment wm + 4 i + NFA / 2
      const DenseArgs& a = args.d;
#pragma unroll
      for (int i = 0; i < FA / 2; ++i) {
        const int o = m0 + 16 * (wm + 4 * i) + 4 * lg;
        if (o >= a.d_out) continue;
        half_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) hv[v] = (half_t)(silu_f(acc[i][j][v]) * acc[i + FA / 2][j][v]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<half_t*>(a.out_h) + (size_t)n * a.d_out + o) =
            __builtin_bit_cast(u32x2, hv);
      }
    } else {
      const DenseArgs& a = args.d;
      float* out = a.out_f + (size_t)blockIdx.z * a.T * a.d_out;
#pragma unroll
      for (int i = 0; i < FA; ++i) {
        const int o = m0 + 16 * (wm + 4 * i) + 4 * lg;
        if (o >= a.d_out) continue;
        *reinterpret_cast<f32x4*>(out + (size_t)n * a.d_out + o) = acc[i][j];
      }
    }
  }
}

void launch_colproj(const ColArgs* a, int nproj, int rt, int max_tiles, Act act, hipStream_t s) {
  (void)rt;                      // 128-row tiles
  RgArgs args{};
  args.c[0] = a[0];
  args.c[1] = a[nproj > 1 ? 1 : 0];
  args.ntiles = max_tiles;
  // z: the projection (gate, up), or the k-split of a single projection
  const int nz = nproj > 1 ? nproj : (a[0].nsplit > 1 ? a[0].nsplit : 1);
  const dim3 grid((unsigned)(((max_tiles + 7) / 8) * 8), 1, nz);
  // A grid that fits one workgroup per CU streams each workgroup's long
  // k-range in stages of 64 inputs (32 KB slots; half the ring round trips
  // per input; d_in a multiple of 64); a larger grid keeps stages of 32
  // inputs and 16 KB slots, so that two workgroups share a CU.
  const bool d64 = (a[0].d_in % 64) == 0 && (nproj < 2 || (a[1].d_in % 64) == 0);
  if (d64 && (long)grid.x * nz <= device_cus()) {
    if (act == ACT_F16) hipLaunchKernelGGL((rowgemm_kernel<half_t, RG_COL, 2>), grid, dim3(64 * RG_WAVES), 0, s, args);
    else hipLaunchKernelGGL((rowgemm_kernel<__bf16, RG_COL, 2>), grid, dim3(64 * RG_WAVES), 0, s, args);
  } else {
    if (act == ACT_F16) hipLaunchKernelGGL((rowgemm_kernel<half_t, RG_COL, 1>), grid, dim3(64 * RG_WAVES), 0, s, args);
    else hipLaunchKernelGGL((rowgemm_kernel<__bf16, RG_COL, 1>), grid, dim3(64 * RG_WAVES), 0, s, args);
  }
}

void launch_dense(const DenseArgs& a, int dual, int nsplit, hipStream_t s) {
  RgArgs args{};
  args.d = a;
  args.nsplit = dual ? 1 : nsplit;
  args.ntiles = (a.T + 127) / 128;
  // 256 weight rows per workgroup (128 output rows of the dual gate/up)
  if (dual) {
    args.nwt = (a.d_out + 127) / 128;
    const dim3 grid(8 * args.ntiles * ((args.nwt + 7) / 8), 1, 1);
    hipLaunchKernelGGL((rowgemm_kernel<half_t, RG_DUAL, 2, 4>), grid, dim3(64 * RG_WAVES), 0, s, args);
  } else {
    args.nwt = (a.d_out + 255) / 256;
    const dim3 grid(8 * args.ntiles * ((args.nwt + 7) / 8), 1, args.nsplit);
    hipLaunchKernelGGL((rowgemm_kernel<half_t, RG_PLAIN, 2, 4>), grid, dim3(64 * RG_WAVES), 0, s, args);
  }
}

}  // namespace tq
