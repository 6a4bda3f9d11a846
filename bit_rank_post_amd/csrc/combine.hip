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
// S is built in LDS per 16-token tile (split into a high and a low part in
// the activation dtype for the MFMA), never in HBM.
#include "tq_device.h"

namespace tq {

// Workgroup: 16 tokens x a range of output chunks (64 outputs, 16 per wave).
// The rank-space vectors S[t][m] of the grid rows m active in the tile are
// built once in LDS (high and low parts) when they fit CB_LDS bytes, then
// every chunk of the range runs its MFMAs against them; otherwise they are
// rebuilt per chunk and grid row.
constexpr int CB_KMAX = 32;                 // slots per token
constexpr int CB_MMAX = 1024;               // grid rows
constexpr int CB_LDS = 64 * 1024;           // resident S budget (dynamic LDS, at most)

// PERSLOT: the residual outputs of a token are gathered slot by slot with
// all k-chunk slabs of a slot requested together (few slots, several slabs:
// decode); else the first slab of every slot is requested together and
// further slabs follow one round trip each.
template <typename T, typename YT, bool PERSLOT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, int cpw, int lds_bytes) {
  typedef typename Vec8<T>::type V8;
  constexpr int KR = 8;                     // slots per token held in registers
  constexpr int UG = 8;                     // U fragments requested together
  extern __shared__ __attribute__((aligned(16))) char s_dyn[];
  __shared__ int s_i[16 * CB_KMAX];         // active-row index of each slot (-1: none)
  __shared__ int s_row[16 * CB_KMAX];       // row of P of each slot
  __shared__ float s_g[16 * CB_KMAX];       // routing weight of each slot
  __shared__ unsigned s_bits[CB_MMAX / 32];
  __shared__ int s_base[CB_MMAX / 32];
  __shared__ int s_ml[16 * CB_KMAX];        // active grid rows, ascending
  __shared__ int s_nact;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int k = a.topk;
  const int rp = a.r_pad;
  const int SLD = rp + 8;
  T* s_hi = reinterpret_cast<T*>(s_dyn);

  int nact = 0;
  bool resident = false;
  if (rp > 0) {
    for (int i = tid; i < CB_MMAX / 32; i += 256) s_bits[i] = 0u;
    __syncthreads();
    // per-slot data of the tile, once (s_i holds the grid row until the
    // active rows are numbered)
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
          atomicOr(&s_bits[m >> 5], 1u << (m & 31));
        }
      }
      s_i[tt * CB_KMAX + j] = m;
      s_row[tt * CB_KMAX + j] = row;
      s_g[tt * CB_KMAX + j] = g;
    }
    __syncthreads();
    // active grid rows in ascending order (wave 0, one bitmap word per lane)
    static_assert(CB_MMAX / 32 <= 64, "bitmap words fit one wave");
    if (wave == 0) {
      const unsigned wd = (lane < CB_MMAX / 32) ? s_bits[lane] : 0u;
      const int c = __popc(wd);
      const int inc = wave_incl_scan_i(c, lane);
      int pos = inc - c;
      if (lane < CB_MMAX / 32) s_base[lane] = pos;
      for (unsigned w = wd; w; w &= w - 1) s_ml[pos++] = lane * 32 + __ffs(w) - 1;
      if (lane == 63) s_nact = inc;
    }
    __syncthreads();
    nact = s_nact;
    resident = (size_t)nact * 16 * SLD * 2 * sizeof(T) <= (size_t)lds_bytes;
    for (int i = tid; i < 16 * k; i += 256) {
      const int tt = i / k, j = i - tt * k;
      const int m = s_i[tt * CB_KMAX + j];
      if (m >= 0) {
        const unsigned below = s_bits[m >> 5] & ((1u << (m & 31)) - 1u);
        s_i[tt * CB_KMAX + j] = s_base[m >> 5] + __popc(below);
      }
    }
    __syncthreads();
  }
  // S[t][m_i][:] = sum_{j : row(e_tj) = m_i} g_tj (Sigma p_tj) for active rows
  // i0 <= i < i1 (LDS block i - i0), split into high and low parts.  Item =
  // (token, 4 ranks): the token's slot vectors are requested together, then
  // summed per active row.
  auto build = [&](int i0, int i1) {
    T* s_lo = s_hi + (size_t)(i1 - i0) * 16 * SLD;
    const int nc4 = rp >> 2;
    for (int q = tid; q < 16 * nc4; q += 256) {
      const int tt = q / nc4, c = 4 * (q - tt * nc4);
      if (k <= KR) {
        f32x4 pv[KR];
        int ij[KR];
        float gj[KR];
#pragma unroll
        for (int j = 0; j < KR; ++j) {
          ij[j] = (j < k) ? s_i[tt * CB_KMAX + j] : -1;
          gj[j] = (j < k) ? s_g[tt * CB_KMAX + j] : 0.f;
          pv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (ij[j] >= i0 && ij[j] < i1) {
            const float* pp = a.P + (size_t)s_row[tt * CB_KMAX + j] * rp + c;
            pv[j] = *reinterpret_cast<const f32x4*>(pp);
            for (int sp = 1; sp < a.nsplit; ++sp)     // k-split slabs of the column stage
              pv[j] += *reinterpret_cast<const f32x4*>(pp + (size_t)sp * a.rows_cap * rp);
          }
        }
        for (int i = i0; i < i1; ++i) {
          f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < KR; ++j)
            if (ij[j] == i) v += gj[j] * pv[j];
          T hi[4], lo[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            hi[u] = from_f32<T>(v[u]);
            lo[u] = from_f32<T>(v[u] - to_f32(hi[u]));
          }
          const int o = ((i - i0) * 16 + tt) * SLD + c;
          *reinterpret_cast<u32x2*>(&s_hi[o]) = __builtin_bit_cast(u32x2, hi);
          *reinterpret_cast<u32x2*>(&s_lo[o]) = __builtin_bit_cast(u32x2, lo);
        }
      } else {
        for (int i = i0; i < i1; ++i) {
          f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int j = 0; j < k; ++j)
            if (s_i[tt * CB_KMAX + j] == i) {
              const float* pp = a.P + (size_t)s_row[tt * CB_KMAX + j] * rp + c;
              f32x4 pj = *reinterpret_cast<const f32x4*>(pp);
              for (int sp = 1; sp < a.nsplit; ++sp)
                pj += *reinterpret_cast<const f32x4*>(pp + (size_t)sp * a.rows_cap * rp);
              v += s_g[tt * CB_KMAX + j] * pj;
            }
          T hi[4], lo[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            hi[u] = from_f32<T>(v[u]);
            lo[u] = from_f32<T>(v[u] - to_f32(hi[u]));
          }
          const int o = ((i - i0) * 16 + tt) * SLD + c;
          *reinterpret_cast<u32x2*>(&s_hi[o]) = __builtin_bit_cast(u32x2, hi);
          *reinterpret_cast<u32x2*>(&s_lo[o]) = __builtin_bit_cast(u32x2, lo);
        }
      }
    }
  };
  // MFMAs of active rows i0 <= i < i1 for output rows o_w .. o_w + 15; the
  // U fragments (one per active row and 32 ranks) are requested UG at a time
  auto lowrank = [&](int i0, int i1, int o_w, f32x4& acc) {
    const T* s_lo = s_hi + (size_t)(i1 - i0) * 16 * SLD;
    const int nf = (i1 - i0) * (rp >> 5);
    int fi = i0, fs = 0;                    // (active row, rank offset) of fragment f0
    for (int f0 = 0; f0 < nf; f0 += UG) {
      V8 uf[UG];
      int bo[UG];
      int ci = fi, cs = fs;
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        if (f0 + u < nf) {
          uf[u] = *reinterpret_cast<const V8*>(reinterpret_cast<const T*>(a.U) +
                                               ((size_t)s_ml[ci] * a.d_out + o_w + l16) * rp +
                                               cs + 8 * lg);
          bo[u] = ((ci - i0) * 16 + l16) * SLD + cs + 8 * lg;
        }
        cs += 32;
        if (cs == rp) {
          cs = 0;
          ++ci;
        }
      }
      fi = ci;
      fs = cs;
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        if (f0 + u < nf) {
          const V8 bh = *reinterpret_cast<const V8*>(&s_hi[bo[u]]);
          const V8 bl = *reinterpret_cast<const V8*>(&s_lo[bo[u]]);
          acc = mfma16(uf[u], bh, acc);
          acc = mfma16(uf[u], bl, acc);
        }
      }
    }
  };
  if (resident && nact > 0) {
    build(0, nact);
    __syncthreads();
  }

  const int nch = (a.d_out + 63) >> 6;
  const int c0 = blockIdx.y * cpw, c1 = min(nch, c0 + cpw);
  const int t = t0 + l16;
  // positions of the token's slots (constant over the chunks)
  int pj[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) pj[j] = (t < a.T && j < k) ? a.inv[t * k + j] : -1;
  for (int ch = c0; ch < c1; ++ch) {
    const int o_w = ch * 64 + wave * 16;
    const bool ovalid = o_w < a.d_out;
    const int o = o_w + 4 * lg;
    // residual outputs of the token's slots and the shared expert, requested
    // before the MFMAs
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ovalid && t < a.T) {
      if (k <= KR && !PERSLOT) {
        // the first slab of every slot requested together, further slabs
        // (if any) one round trip each
        f32x4 dv[KR];
#pragma unroll
        for (int j = 0; j < KR; ++j) {
          dv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (pj[j] >= 0) dv[j] = *reinterpret_cast<const f32x4*>(a.dres + (size_t)pj[j] * a.d_out + o);
        }
        for (int c = 1; c < a.nks; ++c)
#pragma unroll
          for (int j = 0; j < KR; ++j)
            if (pj[j] >= 0)
              dv[j] += *reinterpret_cast<const f32x4*>(a.dres + ((size_t)c * a.S + pj[j]) * a.d_out + o);
#pragma unroll
        for (int j = 0; j < KR; ++j) v += dv[j];
      } else if (k <= KR) {
        // few slots, several k-chunk slabs (decode): per slot, up to NKB
        // slabs requested together (one round trip per slot instead of one
        // per slab), summed in slab order
        constexpr int NKB = 8;
#pragma unroll
        for (int j = 0; j < KR; ++j) {
          if (pj[j] < 0) continue;
          const float* dp = a.dres + (size_t)pj[j] * a.d_out + o;
          const size_t slab = (size_t)a.S * a.d_out;
          f32x4 sv[NKB];
#pragma unroll
          for (int c = 0; c < NKB; ++c)
            sv[c] = (c < a.nks) ? *reinterpret_cast<const f32x4*>(dp + c * slab) : f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 dv = sv[0];
#pragma unroll
          for (int c = 1; c < NKB; ++c)
            if (c < a.nks) dv += sv[c];
          for (int c = NKB; c < a.nks; ++c) dv += *reinterpret_cast<const f32x4*>(dp + c * slab);
          v += dv;
        }
      } else {
        for (int j = 0; j < k; ++j) {
          const int pos = a.inv[t * k + j];
          if (pos < 0) continue;
          for (int c = 0; c < a.nks; ++c)
            v += *reinterpret_cast<const f32x4*>(a.dres + ((size_t)c * a.S + pos) * a.d_out + o);
        }
      }
      if (a.ys)
        for (int c = 0; c < a.nys; ++c)
          v += *reinterpret_cast<const f32x4*>(a.ys + ((size_t)c * a.T + t) * a.d_out + o);
    }
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (resident) {
      if (ovalid) lowrank(0, nact, o_w, acc);
    } else {
      for (int i = 0; i < nact; ++i) {
        __syncthreads();
        build(i, i + 1);
        __syncthreads();
        if (ovalid) lowrank(i, i + 1, o_w, acc);
      }
    }
    if (!ovalid || t >= a.T) continue;
    v += acc;
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
}

template <bool PERSLOT>
static void combine_dt(const CombineArgs& a, Act act, dim3 grid, size_t lds, int lb, int cpw,
                       hipStream_t s) {
  if (act == ACT_F16) {
    if (a.y_dtype == 0) hipLaunchKernelGGL((combine_kernel<half_t, half_t, PERSLOT>), grid, dim3(256), lds, s, a, cpw, lb);
    else if (a.y_dtype == 1) hipLaunchKernelGGL((combine_kernel<half_t, __bf16, PERSLOT>), grid, dim3(256), lds, s, a, cpw, lb);
    else hipLaunchKernelGGL((combine_kernel<half_t, float, PERSLOT>), grid, dim3(256), lds, s, a, cpw, lb);
  } else {
    if (a.y_dtype == 0) hipLaunchKernelGGL((combine_kernel<__bf16, half_t, PERSLOT>), grid, dim3(256), lds, s, a, cpw, lb);
    else if (a.y_dtype == 1) hipLaunchKernelGGL((combine_kernel<__bf16, __bf16, PERSLOT>), grid, dim3(256), lds, s, a, cpw, lb);
    else hipLaunchKernelGGL((combine_kernel<__bf16, float, PERSLOT>), grid, dim3(256), lds, s, a, cpw, lb);
  }
}

void launch_combine(const CombineArgs& a, Act act, hipStream_t s) {
  // output chunks per workgroup: about 4 workgroups per CU over the grid
  const int tiles = (a.T + 15) / 16;
  const int nch = (a.d_out + 63) / 64;
  int os = (1024 + tiles - 1) / tiles;
  os = os < 1 ? 1 : (os > nch ? nch : os);
  const int cpw = (nch + os - 1) / os;
  const dim3 grid(tiles, (nch + cpw - 1) / cpw);
  // LDS: S of every grid row a tile can touch (min(M, 16 k)) if that fits
  // CB_LDS, else one grid row at a time
  size_t lds = 0;
  if (a.r_pad > 0) {
    const size_t per_row = (size_t)16 * (a.r_pad + 8) * 2 * 2;
    const int rows = a.M < 16 * a.topk ? a.M : 16 * a.topk;
    lds = (size_t)rows * per_row <= (size_t)CB_LDS ? (size_t)rows * per_row : per_row;
  }
  const int lb = (int)lds;
  if (a.nks > 1 && a.topk <= 2) combine_dt<true>(a, act, grid, lds, lb, cpw, s);
  else combine_dt<false>(a, act, grid, lds, lb, cpw, s);
}

}  // namespace tq
