// Decode-path residual kernel: streams each active expert's 2-bit codes once
// from HBM and applies them to that expert's few slots.
//
// "TileQ" technical summary, section 4 (Inference Latency, Decode): decode is
// memory bound; the layout is contiguous and read with wide vector accesses.
//
// Work: a workgroup (4 waves) owns 4/KW row fragments (16 rows each) of one
// expert -- in MODE_GATEUP the gate and the up rows together -- and KW waves
// split the k-stages of a fragment.  A stage is 8 MFMA k-steps (256 inputs).
// Per stage-time every wave issues, DEPTH stage-times ahead, buffer loads for
// its codes (16 B per lane per projection), a share of the stage's
// activations, its rows' scale/zero words and a share of the group sums; when
// they land it writes the shared parts to a double-buffered LDS slot, the
// workgroup synchronizes, and the MFMAs read their B operands and fold
// constants from LDS.  Only codes stay in registers, so the HBM stream is
// DEPTH stages deep per wave.
//
// The codes enter v_mfma_f32_16x16x32_f16 as the raw packed values 1 + q*c
// (one and-or per pair, no dequantization) against the class-scaled
// activations x' = x~/c from act_prep.hip; each quantization group's fp32
// partial is folded with acc += s * (C_g - X'_g - z * X~_g).
// Epilogue: undo the row scaling 2^E, add the low-rank row stage U_m Sigma p
// as MFMA K-steps (MODE_GATEUP; p from the column stage), then SwiGLU into h,
// or (MODE_RES) the slot's routing weight into the fp32 per-slot buffer.
#include "tq_device.h"

namespace tq {

constexpr int DEPTH = 3;          // stage-times of loads in flight per wave
constexpr int ALD = 256 + 8;      // LDS activation row stride (halves)

template <int NP, int KW>
struct DecRing {
  u32x4 code[NP];
  u32x4 act[2 * KW];              // this thread's share of the stage activations
  u32x2 sz[NP];                   // scale/zero words of this wave's rows
  u32x2 sum;                      // one (X~, X') pair of the group sums
};

template <int NP, int KW, int NG>
struct DecLds {
  static constexpr int ACT = KW * 16 * ALD * 2;           // bytes
  static constexpr int SUM = KW * 16 * NG * 8;
  static constexpr int SZ = 4 * NP * NG * 64;
  static constexpr int SLOT = ACT + SUM + SZ;
};

template <typename T, int MODE, int KW, int GS>
__global__ __launch_bounds__(256) void gemm_dec_kernel(DecArgs a) {
  typedef typename Vec8<T>::type V8;
  constexpr int NP = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int RPW = 4 / KW;            // row fragments per workgroup
  constexpr int NG = 8 / GS;             // groups per stage
  typedef DecLds<NP, KW, NG> LD;
  __shared__ __attribute__((aligned(16))) char lds[2 * LD::SLOT];
  __shared__ float s_red[(KW > 1) ? (KW - 1) * RPW * NP * 256 : 1];

  const int e = blockIdx.x;
  const int cnt = a.cnt[e];
  if (cnt == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l16 = lane & 15, lg = lane >> 4;
  const int rsub = wave / KW, kw = wave - rsub * KW;
  const int nrb = a.d_out >> 4;
  const int rb_raw = blockIdx.y * RPW + rsub;
  const bool rvalid = rb_raw < nrb;
  const int rb = rvalid ? rb_raw : nrb - 1;          // clamped: loads stay in bounds
  const int nsteps = a.d_in >> 5;
  const int nfull = nsteps >> 3;
  const bool tail = (nsteps & 7) != 0;
  const int ng = a.p[0].ng;
  const int ntau = (nfull + KW - 1) / KW;            // stage-times
  const size_t cpe = (size_t)a.d_out * (a.d_in >> 4);

  __amdgpu_buffer_rsrc_t rc[NP], rs[NP];
  const uint32_t* cbase[NP];
  const uint32_t* szb[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    cbase[p] = a.p[p].codes + (size_t)e * cpe + (size_t)rb * nsteps * 32;
    szb[p] = a.p[p].sz + ((size_t)e * nrb + rb) * ng * 16;
    rc[p] = make_rsrc(cbase[p], (uint32_t)nsteps * 128u);
    rs[p] = make_rsrc(szb[p], (uint32_t)ng * 64u);
  }
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.Xp, (uint32_t)a.rows * a.d_in * 2u);
  const __amdgpu_buffer_rsrc_t rsm = make_rsrc(a.sums, (uint32_t)a.rows * ng * 8u);

  for (int t0 = 0; t0 < cnt; t0 += 16) {
    const int ncol = min(16, cnt - t0);
    const bool cvalid = l16 < ncol;
    const int pos = a.off[e] + t0 + (cvalid ? l16 : 0);
    const int slot = a.perm[pos];
    const int arow = a.gather ? slot / a.topk : pos;

    // this thread's shares of the shared per-stage-time loads (invalid columns
    // read the tile's first column; MFMA columns are independent and those
    // are never stored)
    uint32_t act_voff[2 * KW];
    int act_lds[2 * KW];
#pragma unroll
    for (int i = 0; i < 2 * KW; ++i) {
      const int c = tid + 256 * i;                     // 16 B chunk of [KW][16][256]
      const int ks = c >> 9, col = (c >> 5) & 15, kc = c & 31;
      const int cc = (col < ncol) ? col : 0;
      const int r = a.gather ? a.perm[a.off[e] + t0 + cc] / a.topk : a.off[e] + t0 + cc;
      act_voff[i] = ((uint32_t)r * a.d_in + ks * 256 + kc * 8) * 2u;
      act_lds[i] = ((ks * 16 + col) * ALD + kc * 8) * 2;
    }
    const int nsum = KW * NG * 16;                     // (stage, group, column) triples
    const int sidx = tid % nsum;
    uint32_t sum_voff;
    int sum_lds;
    {
      const int col = sidx & 15, gis = sidx >> 4;      // gis = ks * NG + gi
      const int cc = (col < ncol) ? col : 0;
      const int r = a.gather ? a.perm[a.off[e] + t0 + cc] / a.topk : a.off[e] + t0 + cc;
      sum_voff = ((uint32_t)r * ng + gis) * 8u;
      sum_lds = LD::ACT + (gis * 16 + col) * 8;
    }
    const int szl = lane % (NG * 8);                   // u32x2 index within NG*16 words
    const int sz_lds = LD::ACT + LD::SUM + (wave * NP) * NG * 64 + szl * 8;

    auto issue = [&](int tau, DecRing<NP, KW>& R) {
      const int st = tau * KW + kw;
#pragma unroll
      for (int p = 0; p < NP; ++p) R.code[p] = bload128(rc[p], lane * 16u, st * 1024u);
#pragma unroll
      for (int i = 0; i < 2 * KW; ++i) R.act[i] = bload128(rx, act_voff[i], tau * KW * 512u);
#pragma unroll
      for (int p = 0; p < NP; ++p) R.sz[p] = bload64(rs[p], szl * 8u, st * NG * 64u);
      R.sum = bload64(rsm, sum_voff, tau * KW * NG * 8u);
    };
    auto deposit = [&](const DecRing<NP, KW>& R, int sl) {
      char* base = lds + sl * LD::SLOT;
#pragma unroll
      for (int i = 0; i < 2 * KW; ++i) *reinterpret_cast<u32x4*>(base + act_lds[i]) = R.act[i];
      *reinterpret_cast<u32x2*>(base + sum_lds) = R.sum;
#pragma unroll
      for (int p = 0; p < NP; ++p) *reinterpret_cast<u32x2*>(base + sz_lds + p * NG * 64) = R.sz[p];
    };

    f32x4 acc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto fold = [&](const f32x4 (&C)[NP], const char* base, int gi) {
      const float2 xs = *reinterpret_cast<const float2*>(
          base + LD::ACT + ((kw * NG + gi) * 16 + l16) * 8);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(
            base + LD::ACT + LD::SUM + ((wave * NP + p) * NG + gi) * 64 + lg * 16);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float sc = (float)__builtin_bit_cast(half_t, (uint16_t)(w[v] & 0xFFFFu));
          const float z = (float)__builtin_bit_cast(half_t, (uint16_t)(w[v] >> 16));
          acc[p][v] += sc * (C[p][v] - xs.y - z * xs.x);
        }
      }
    };

    auto compute = [&](const u32x4 (&code)[NP], int sl) {
      const char* base = lds + sl * LD::SLOT;
      const char* ab = base + ((kw * 16 + l16) * ALD + 8 * lg) * 2;
      f32x4 C[NP];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4 fr[NP][2];
#pragma unroll
        for (int p = 0; p < NP; ++p) unpack16_frags(code[p][d], fr[p][0], fr[p][1]);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int j = 2 * d + b;
          const half8v bv = *reinterpret_cast<const half8v*>(ab + j * 64);
          if (j % GS == 0) {
#pragma unroll
            for (int p = 0; p < NP; ++p) C[p] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int p = 0; p < NP; ++p) C[p] = mfma16(as_half8(fr[p][b]), bv, C[p]);
          if (j % GS == GS - 1) fold(C, base, j / GS);
        }
      }
    };

    // full stages: ring of DEPTH stage-times in registers, double-buffered LDS
    if (ntau > 0) {
      DecRing<NP, KW> R[DEPTH];
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) issue(u, R[u]);
      for (int t = 0; t < ntau; t += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
          const int tau = t + u;
          if (tau >= ntau) break;
          const int sl = tau & 1;
          deposit(R[u], sl);
          u32x4 code[NP];
#pragma unroll
          for (int p = 0; p < NP; ++p) code[p] = R[u].code[p];
          issue(tau + DEPTH, R[u]);        // refill the slot; past the end the buffers read zeros
          __syncthreads();
          if (tau * KW + kw < nfull) compute(code, sl);
        }
      }
      __syncthreads();
    }

    // 4-step tail stage (d_in % 256 == 128; then GS <= 4): direct loads
    if (tail && kw == nfull % KW) {
      const int st = nfull;
      const half_t* xrow = reinterpret_cast<const half_t*>(a.Xp) + (size_t)arow * a.d_in + 8 * lg;
      const float* srow = a.sums + (size_t)arow * ng * 2;
      u32x2 cd[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p)
        cd[p] = *reinterpret_cast<const u32x2*>(cbase[p] + st * 256 + lane * 2);
      half8v bt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bt[j] = *reinterpret_cast<const half8v*>(xrow + (8 * st + j) * 32);
      f32x4 C[NP];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        u32x4 fr[NP][2];
#pragma unroll
        for (int p = 0; p < NP; ++p) unpack16_frags(cd[p][d], fr[p][0], fr[p][1]);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int j = 2 * d + b;
          if (GS > 4 || j % GS == 0) {
#pragma unroll
            for (int p = 0; p < NP; ++p) C[p] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int p = 0; p < NP; ++p) C[p] = mfma16(as_half8(fr[p][b]), bt[j], C[p]);
          if (GS <= 4 && j % GS == GS - 1) {
            const int g = (8 * st + j) / GS;
            const float Xt = srow[2 * g], Xq = srow[2 * g + 1];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const u32x4 w = *reinterpret_cast<const u32x4*>(szb[p] + (size_t)g * 16 + 4 * lg);
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float sc = (float)__builtin_bit_cast(half_t, (uint16_t)(w[v] & 0xFFFFu));
                const float z = (float)__builtin_bit_cast(half_t, (uint16_t)(w[v] >> 16));
                acc[p][v] += sc * (C[p][v] - Xq - z * Xt);
              }
            }
          }
        }
      }
    }

    if constexpr (KW > 1) {
      if (kw > 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            s_red[(((rsub * (KW - 1) + kw - 1) * NP + p) * 64 + lane) * 4 + v] = acc[p][v];
      }
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int q = 0; q < KW - 1; ++q)
#pragma unroll
          for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[p][v] += s_red[(((rsub * (KW - 1) + q) * NP + p) * 64 + lane) * 4 + v];
      }
    }

    if (kw == 0 && rvalid) {
      const int E = a.ex[arow];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[p][v] = ldexpf(acc[p][v], E);
      const int o = rb * 16 + 4 * lg;
      if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const ProjDev& pd = a.p[p];
          if (pd.rank == 0) continue;
          const int rp = pd.r_pad;
          const T* up = reinterpret_cast<const T*>(pd.U) +
                        ((size_t)pd.m_of[e] * a.d_out + rb * 16 + l16) * rp + 8 * lg;
          const int col = a.slot2col[p][slot];
          const float* prow = a.P[p] + (size_t)col * rp + 8 * lg;
          const float* sg = pd.sigma + 8 * lg;
          for (int s2 = 0; s2 < rp; s2 += 32) {
            const V8 av = *reinterpret_cast<const V8*>(up + s2);
            V8 bh, bl;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float v = prow[s2 + i] * sg[s2 + i];
              const T hi = from_f32<T>(v);
              bh[i] = hi;
              bl[i] = from_f32<T>(v - to_f32(hi));
            }
            acc[p] = mfma16(av, bh, acc[p]);
            acc[p] = mfma16(av, bl, acc[p]);
          }
        }
        if (cvalid) {
          T hv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) hv[v] = from_f32<T>(silu_f(acc[0][v]) * acc[1][v]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(a.h) + (size_t)pos * a.d_out + o) =
              __builtin_bit_cast(u32x2, hv);
        }
      } else {
        if (cvalid) {
          const float g = a.gates[slot];
          *reinterpret_cast<f32x4*>(a.dres + (size_t)pos * a.d_out + o) = acc[0] * g;
        }
      }
    }
    if constexpr (KW > 1) __syncthreads();
  }
}

template <typename T, int MODE, int KW>
static void dec_gs(const DecArgs& a, hipStream_t s) {
  const int nrb = a.d_out >> 4;
  const dim3 grid(a.K, (nrb + (4 / KW) - 1) / (4 / KW));
  switch (a.p[0].group >> 5) {
    case 1: hipLaunchKernelGGL((gemm_dec_kernel<T, MODE, KW, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_dec_kernel<T, MODE, KW, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_dec_kernel<T, MODE, KW, 4>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_dec_kernel<T, MODE, KW, 8>), grid, dim3(256), 0, s, a); break;
  }
}

template <typename T, int MODE>
static void dec_kw(const DecArgs& a, int kw, hipStream_t s) {
  // the group-sum table of a stage-time (KW * NG * 16 entries) must fit the
  // 256 threads of a workgroup: KW = 4 needs groups of >= 64 inputs
  if (kw == 4 && (a.p[0].group >> 5) == 1) kw = 2;
  if (kw == 1) dec_gs<T, MODE, 1>(a, s);
  else if (kw == 2) dec_gs<T, MODE, 2>(a, s);
  else dec_gs<T, MODE, 4>(a, s);
}

void launch_gemm_decode(const DecArgs& a, GemmMode mode, int kw, Act act, hipStream_t s) {
  if (act == ACT_F16) {
    if (mode == MODE_GATEUP) dec_kw<half_t, MODE_GATEUP>(a, kw, s);
    else dec_kw<half_t, MODE_RES>(a, kw, s);
  } else {
    if (mode == MODE_GATEUP) dec_kw<__bf16, MODE_GATEUP>(a, kw, s);
    else dec_kw<__bf16, MODE_RES>(a, kw, s);
  }
}

}  // namespace tq
