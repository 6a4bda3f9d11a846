// Grouped 2-bit residual GEMM of the fused forward, with the low-rank row
// stage folded in as extra K-steps and the epilogues fused.
//
// "TileQ" technical summary, section 2.1 step 5: each expert's weight is the
// shared low-rank block plus its quantized residual; section 2.2: the
// low-rank part is done once per shared factor for all active experts, the
// residual product is per expert.  Work item = (expert, tile of that
// expert's slots, block of output rows).  For each 32-input k-step the 2-bit
// codes of a 16-row fragment arrive as one 16-bit field per lane (coalesced
// 8-byte loads of the repacked layout), are unpacked in registers into the
// exact dequantized fp16 weights RND_f16(s (q - z)) and fed to
// v_mfma_f32_16x16x32_f16 against activation fragments staged in LDS
// (bfloat16 activations are staged as fp16 after an exact per-row power-of-two
// scaling, undone on the fp32 result).
//
// MODE_GATEUP: the gate and the up projection of the same expert and rows are
//   computed together; the row stage of section 2.2 (U_m Sigma p, p = V_n^T x
//   from the column stage) is added as r extra K-steps per projection with
//   U_m as the A operand and Sigma p (split into a high and a low part in the
//   activation dtype) as the B operand; then h = RND_act(silu(gate) * up).
// MODE_RES: one projection (down, or a single projection); the result, times
//   the slot's routing weight, goes to an fp32 per-slot buffer that the
//   combine stage sums per token together with the rank-space low-rank term.
#include "tq_device.h"

namespace tq {

constexpr int KS = 4;                 // k-steps per LDS stage (128 inputs)
constexpr int ACT_LD = KS * 32 + 8;   // LDS row stride in halves (272 B)

template <typename T, int MODE, int BMF, int RF>
__global__ __launch_bounds__(256) void moe_gemm_kernel(GemmArgs a) {
  typedef typename Vec8<T>::type V8;
  constexpr int NP = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int BMS = 16 * BMF;
  constexpr int ACT_HALVES = BMS * ACT_LD;
  constexpr int EXT_LD = 64 + 8;       // rank chunk of 64 (+ pad)
  constexpr int EXT_HALVES = 2 * BMS * EXT_LD;
  constexpr int LDS_HALVES = (MODE == MODE_GATEUP && EXT_HALVES > ACT_HALVES) ? EXT_HALVES : ACT_HALVES;
  __shared__ __attribute__((aligned(16))) half_t s_act[LDS_HALVES];
  __shared__ int s_src[BMS];
  __shared__ int s_exp[BMS];
  __shared__ int s_res;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int e = find_segment(a.tile_off, a.K, blockIdx.x, &s_res);
  if (e < 0) return;
  const int lt = blockIdx.x - a.tile_off[e];
  const int pos0 = a.off[e] + lt * BMS;
  const int nv = min(BMS, a.cnt[e] - lt * BMS);
  const int o_wave = blockIdx.y * (64 * RF) + wave * (16 * RF);

  // slot rows of this tile: source activation row and exponent
  if (tid < BMS) {
    int src = -1, ex = 0;
    if (tid < nv) {
      const int pos = pos0 + tid;
      src = a.gather ? a.perm[pos] / a.topk : pos;
      if (a.ex) ex = a.ex[src];
      if (a.hamax) {
        const float m = __uint_as_float(a.hamax[pos]);
        int e2 = 0;
        if (m > 0.f) {
          frexpf(m, &e2);
          ex = e2 - 15;
        }
      }
    }
    s_src[tid] = src;
    s_exp[tid] = ex;
  }

  f32x4 acc[NP][RF][BMF];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int r = 0; r < RF; ++r)
#pragma unroll
      for (int f = 0; f < BMF; ++f) acc[p][r][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool rvalid[RF];
#pragma unroll
  for (int r = 0; r < RF; ++r) rvalid[r] = (o_wave + 16 * r) < a.d_out;

  const int nsteps = a.d_in >> 5;
  const int gsteps = a.p[0].group >> 5;           // k-steps per quantization group
  const int ng = a.p[0].ng;
  const size_t codes_per_expert = (size_t)a.d_out * (a.d_in >> 4);

  DeqConst cst[NP][RF];
  int cur_g = -1;

  for (int st = 0; st < nsteps; st += KS) {
    // (1) codes of this stage: 2 dwords per lane per (projection, fragment)
    u32x2 cw[NP][RF];
    const int sg = st >> 3, gs = min(8, nsteps - (sg << 3));
    const int within = lane * gs + (st & 7);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < RF; ++r) {
        if (rvalid[r]) {
          const int rb = (o_wave >> 4) + r;
          const uint32_t* src = a.p[p].codes + (size_t)e * codes_per_expert +
                                (((size_t)rb * nsteps + (sg << 3)) * 64 + within) / 2;
          cw[p][r] = *reinterpret_cast<const u32x2*>(src);
        } else {
          cw[p][r] = u32x2{0u, 0u};
        }
      }

    // (2) stage activations [BMS][128] as fp16
    __syncthreads();
    for (int i = tid; i < BMS * 16; i += 256) {
      const int row = i >> 4, c = i & 15;
      const int src = s_src[row];
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (src >= 0) {
        const T* ap = reinterpret_cast<const T*>(a.A) + (size_t)src * a.d_in + st * 32 + 8 * c;
        if constexpr (sizeof(T) == 2 && __is_same(T, half_t)) {
          v = *reinterpret_cast<const u32x4*>(ap);
        } else {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(ap);
          const int ex = s_exp[row];
          half8v hv;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float lo = __uint_as_float(raw[q] << 16);
            const float hi = __uint_as_float(raw[q] & 0xFFFF0000u);
            hv[2 * q] = (half_t)ldexpf(lo, -ex);
            hv[2 * q + 1] = (half_t)ldexpf(hi, -ex);
          }
          v = as_u32x4(hv);
        }
      }
      *reinterpret_cast<u32x4*>(&s_act[row * ACT_LD + 8 * c]) = v;
    }
    __syncthreads();

    // (3) two dwords = four k-steps.  With G >= 64 the two steps of a dword
    //     (an even-aligned pair) share a quantization group; G == 32 gives
    //     each step its own group.
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int s0 = st + 2 * d;
      half8v bfr[2][BMF];
#pragma unroll
      for (int f = 0; f < BMF; ++f) {
        const half_t* bp = &s_act[(16 * f + l16) * ACT_LD + (2 * d) * 32 + 8 * lg];
        bfr[0][f] = *reinterpret_cast<const half8v*>(bp);
        bfr[1][f] = *reinterpret_cast<const half8v*>(bp + 32);
      }
      if (gsteps >= 2) {
        const int g = s0 / gsteps;
        if (g != cur_g) {
#pragma unroll
          for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int r = 0; r < RF; ++r) {
              const int rb = (o_wave >> 4) + r;
              const uint32_t w = rvalid[r]
                  ? a.p[p].sz[(((size_t)e * a.p[p].nrb + rb) * ng + g) * 16 + l16] : 0u;
              cst[p][r] = deq_const(w);
            }
          cur_g = g;
        }
      }
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int r = 0; r < RF; ++r) {
          if (!rvalid[r]) continue;
          half8v a0, a1;
          if (gsteps >= 2) {
            deq_dword(cw[p][r][d], cst[p][r], cst[p][r], a0, a1);
          } else {
            const size_t base = (((size_t)e * a.p[p].nrb + (o_wave >> 4) + r) * ng) * 16 + l16;
            const DeqConst c0 = deq_const(a.p[p].sz[base + (size_t)s0 * 16]);
            const DeqConst c1 = deq_const(a.p[p].sz[base + (size_t)(s0 + 1) * 16]);
            deq_dword(cw[p][r][d], c0, c1, a0, a1);
          }
#pragma unroll
          for (int f = 0; f < BMF; ++f) {
            acc[p][r][f] = mfma16(a0, bfr[0][f], acc[p][r][f]);
            acc[p][r][f] = mfma16(a1, bfr[1][f], acc[p][r][f]);
          }
        }
    }
  }

  // undo the per-row power-of-two scaling of bfloat16 activations
  if constexpr (!__is_same(T, half_t)) {
#pragma unroll
    for (int f = 0; f < BMF; ++f) {
      const int ex = s_exp[16 * f + l16];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int r = 0; r < RF; ++r)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[p][r][f][v] = ldexpf(acc[p][r][f][v], ex);
    }
  }

  if constexpr (MODE == MODE_GATEUP) {
    // low-rank row stage as extra K-steps: A = U_m rows, B = Sigma p (hi, lo)
    T* s_ext = reinterpret_cast<T*>(s_act);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const ProjDev& pd = a.p[p];
      const int rp = pd.r_pad;
      if (pd.rank == 0) continue;
      const int m = pd.m_of[e];
      for (int rc = 0; rc < rp; rc += 64) {
        const int rw = min(64, rp - rc);
        __syncthreads();
        for (int i = tid; i < BMS * rw; i += 256) {
          const int row = i / rw, c = i - row * rw;
          T hi = from_f32<T>(0.f), lo = from_f32<T>(0.f);
          if (row < nv) {
            const int slot = a.perm[pos0 + row];
            const int col = a.slot2col[p][slot];
            float v = 0.f;
            for (int sp = 0; sp < a.nsplit[p]; ++sp)
              v += a.P[p][((size_t)sp * a.rows_cap[p] + col) * rp + rc + c];
            v *= pd.sigma[rc + c];
            hi = from_f32<T>(v);
            lo = from_f32<T>(v - to_f32(hi));
          }
          s_ext[row * EXT_LD + c] = hi;
          s_ext[BMS * EXT_LD + row * EXT_LD + c] = lo;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RF; ++r) {
          if (!rvalid[r]) continue;
          const T* up = reinterpret_cast<const T*>(pd.U) +
                        ((size_t)m * a.d_out + o_wave + 16 * r + l16) * rp + rc + 8 * lg;
          for (int s2 = 0; s2 < rw; s2 += 32) {
            const V8 av = *reinterpret_cast<const V8*>(up + s2);
#pragma unroll
            for (int f = 0; f < BMF; ++f) {
              const T* bp = &s_ext[(16 * f + l16) * EXT_LD + s2 + 8 * lg];
              const V8 bh = *reinterpret_cast<const V8*>(bp);
              const V8 bl = *reinterpret_cast<const V8*>(bp + BMS * EXT_LD);
              acc[p][r][f] = mfma16(av, bh, acc[p][r][f]);
              acc[p][r][f] = mfma16(av, bl, acc[p][r][f]);
            }
          }
        }
      }
    }
    // SwiGLU epilogue: h = RND_act(silu(gate) * up), stored per slot position
    T* h = reinterpret_cast<T*>(a.h);
#pragma unroll
    for (int f = 0; f < BMF; ++f) {
      const int row = 16 * f + l16;
      if (row >= nv) continue;
      const int pos = pos0 + row;
      float amax = 0.f;
#pragma unroll
      for (int r = 0; r < RF; ++r) {
        if (!rvalid[r]) continue;
        const int o = o_wave + 16 * r + 4 * lg;
        T hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          hv[v] = from_f32<T>(silu_f(acc[0][r][f][v]) * acc[1][r][f][v]);
          amax = fmaxf(amax, fabsf(to_f32(hv[v])));
        }
        *reinterpret_cast<u32x2*>(h + (size_t)pos * a.d_out + o) =
            __builtin_bit_cast(u32x2, hv);
      }
      if (a.hamax_out) atomicMax(a.hamax_out + pos, __float_as_uint(amax));
    }
  } else {
    // gated per-slot residual output (fp32)
#pragma unroll
    for (int f = 0; f < BMF; ++f) {
      const int row = 16 * f + l16;
      if (row >= nv) continue;
      const int pos = pos0 + row;
      const float g = a.gates[a.perm[pos]];
#pragma unroll
      for (int r = 0; r < RF; ++r) {
        if (!rvalid[r]) continue;
        const int o = o_wave + 16 * r + 4 * lg;
        f32x4 v = acc[0][r][f] * g;
        *reinterpret_cast<f32x4*>(a.dres + (size_t)pos * a.d_out + o) = v;
      }
    }
  }
}

template <typename T, int MODE>
static void launch_t(const GemmArgs& a, int path, int max_tiles, hipStream_t s) {
  if (path == 1) {          // decode: 16-slot tiles, 4 fragments (64 rows) per wave
    const dim3 grid(max_tiles, (a.d_out + 255) / 256);
    hipLaunchKernelGGL((moe_gemm_kernel<T, MODE, 1, 4>), grid, dim3(256), 0, s, a);
  } else {                  // prefill: 128-slot tiles, 2 fragments per wave
    const dim3 grid(max_tiles, (a.d_out + 127) / 128);
    hipLaunchKernelGGL((moe_gemm_kernel<T, MODE, 8, 2>), grid, dim3(256), 0, s, a);
  }
}

void launch_gemm(const GemmArgs& a, GemmMode mode, int path, Act act, int max_tiles,
                 hipStream_t s) {
  if (act == ACT_F16) {
    if (mode == MODE_GATEUP) launch_t<half_t, MODE_GATEUP>(a, path, max_tiles, s);
    else launch_t<half_t, MODE_RES>(a, path, max_tiles, s);
  } else {
    if (mode == MODE_GATEUP) launch_t<__bf16, MODE_GATEUP>(a, path, max_tiles, s);
    else launch_t<__bf16, MODE_RES>(a, path, max_tiles, s);
  }
}

}  // namespace tq
