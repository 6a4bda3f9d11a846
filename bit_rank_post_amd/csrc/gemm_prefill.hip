// Prefill-path grouped 2-bit residual GEMM, with the low-rank row stage folded
// in as extra MFMA k-steps and the epilogues fused.
//
// "TileQ" technical summary, section 2.1 step 5: each expert's weight is the
// shared low-rank block plus its quantized residual; section 2.2: the
// low-rank part is done once per shared factor for all active experts (here
// the column stage computed p = V_n^T x once per (column, token) beforehand),
// the residual product is per expert, over the whole batch.
//
// Work item (one workgroup of 8 waves) = (expert, tile of BN = 16 NF of that
// expert's slots, 16 RF WAVES output rows).  Each wave owns RF 16-row
// fragments (of both gate and up in MODE_GATEUP) against all NF token
// fragments.  K advances in stages of 128 inputs (4 MFMA k-steps); each
// stage's activation tile (BN x 128, fp16), the waves' codes and their
// scale/zero words arrive in LDS by buffer loads with the LDS destination, in
// a ring of DEPTH + 1 slots, so loads run DEPTH stages ahead of the MFMAs.
// The codes of a k-step pair are unpacked in registers into the exact fp16
// weights RND_f16(s (q - z)) (deq_dword; deq_dword_lut, a byte-table lookup,
// when a scale or zero point is outside the packed arithmetic's range) and
// fed to v_mfma_f32_16x16x32_f16.
//
// MODE_GATEUP: gate and up rows of the same expert together; the row stage
//   U_m (Sigma p) follows as extra k-steps (U_m rows as A, Sigma p split into
//   a high and a low part in the activation dtype as B); then
//   h = RND_act(silu(gate) * up).
// MODE_RES: one projection (down, or single); result times the slot's routing
//   weight into the fp32 per-slot buffer summed by the combine kernel.
// Activations are fp16 here; bfloat16 rows were converted exactly to fp16
// after a per-row power-of-two scaling 2^-E (rows_to_f16), undone on the
// fp32 result.
#include "tq_device.h"

namespace tq {

constexpr int PF_WAVES = 8;

// GS: k-steps per quantization group when G is a power of two >= 32
// (1, 2, 4, 8); GS = 0: any G (constants per k-step).  NGS: groups a stage
// needs constants for (k-step granularity when GS <= 1).
template <int GS> struct PfGroups { static constexpr int NGS = (GS <= 1) ? 4 : (GS == 2 ? 2 : 1); };

// LDS slot layout (bytes).  Scale/zero words of a wave and projection: word
// gi * SZG + r * 16 + row for group slot gi, fragment r, row; loaded by NSZ
// dword loads of 64 lanes.
template <int NP, int RF, int NF, int GS, int BITS>
struct PfSlot {
  static constexpr int NGS = PfGroups<GS>::NGS;
  static constexpr int SZG = (GS == 0) ? 64 : RF * 16;
  static constexpr int NSZ = (GS == 0) ? 4 : (NGS * RF * 16 + 63) / 64;
  static constexpr int NCW = BITS;                             // code dwords per lane per stage
  static constexpr int B = 0;                                  // [4][NF][64] x 16 B
  static constexpr int CODE = B + 4 * NF * 1024;                // [W][RF][NP][NCW][64] x 4 B
  static constexpr int SZ = CODE + PF_WAVES * RF * NP * NCW * 256;   // [W][NP][NSZ][64] x 4 B
  static constexpr int BYTES = SZ + PF_WAVES * NP * NSZ * 256;
  static constexpr int NB = 4 * NF / PF_WAVES;                 // activation loads per wave
  static constexpr int NI = NB + RF * NP * NCW + NP * NSZ;     // loads per wave per stage
};

// Super-block of row tiles x slot tiles that one XCD's 32 CUs (one
// workgroup each) work on together: up to 8 row tiles, 32 workgroups.
__host__ __device__ inline void pf_superblock(int nrt, int* sbr, int* sbc) {
  *sbr = nrt < 8 ? nrt : 8;
  *sbc = 32 / *sbr;
}

template <typename T, int MODE, int RF, int NF, int GS, bool LUT, int BITS>
__global__ __launch_bounds__(64 * PF_WAVES) void gemm_pre_kernel(GemmArgs a) {
  typedef typename Vec8<T>::type V8;
  constexpr int NP = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int BN = 16 * NF;
  constexpr int NGS = PfGroups<GS>::NGS;
  typedef PfSlot<NP, RF, NF, GS, BITS> SL;
  constexpr int DEPTH = 2;
  constexpr int NSLOT = DEPTH + 1;
  static_assert(NSLOT * SL::BYTES <= 160 * 1024 - 2048, "LDS budget");
  static_assert(SL::NI * (DEPTH - 1) < 64, "vmcnt range");
  static_assert(RF * 16 <= 64, "scale/zero load covers the wave's rows");
  __shared__ __attribute__((aligned(16))) char s0[SL::BYTES];
  __shared__ __attribute__((aligned(16))) char s1[SL::BYTES];
  __shared__ __attribute__((aligned(16))) char s2[SL::BYTES];
  __shared__ int s_src[BN];
  __shared__ int s_exp[BN];
  __shared__ int s_col[NP][BN];     // GATEUP: column-stage row of each slot (-1: none)
  __shared__ int s_res;
  char* const slot[3] = {s0, s1, s2};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int nrb = a.d_out >> 4;
  const int rows_per_wg = 16 * RF * PF_WAVES;
  const int nrt = (a.d_out + rows_per_wg - 1) / rows_per_wg;
  // Workgroup -> (row tile rt, slot-tile unit tq).  Items are grouped in
  // super-blocks of SBR row tiles x SBC slot tiles (row tile fastest inside
  // one; super-blocks step over the row tiles first); the 32 workgroups of a
  // super-block run together on one XCD, on the same stage order, so each
  // stage's codes (per row tile) and activations (per slot tile) come from
  // HBM once per XCD and are shared through its L2.  Workgroup W runs on XCD
  // W mod 8.  When the routed tiles (the grid covers the bound a.ntq) make
  // at least four super-blocks per XCD, they are dealt to the XCDs in turn
  // (all XCDs then work on neighbouring super-blocks at any time); with
  // fewer, each XCD takes an equal run of consecutive items in whole
  // slot-tile columns, so that no XCD idles while another works on one more
  // super-block (the 512-token Qwen-shaped batch makes 12).
  int sbr, sbc;
  pf_superblock(nrt, &sbr, &sbc);
  const int nrtb = (nrt + sbr - 1) / sbr;
  const int nreal = min(a.ntq, sload(a.tile_off, a.K) << (a.tile_half ? 1 : 0));
  const int nsb = nrtb * ((nreal + sbc - 1) / sbc);
  const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3;
  int sb, within;
  if (nsb >= 32) {
    const int sbl = li / (sbr * sbc);
    within = li - sbl * (sbr * sbc);
    sb = sbl * 8 + xcd;
    if (sb >= nsb) return;
  } else {
    const int nitems = nsb * (sbr * sbc);
    const int per = ((((nitems + 7) >> 3) + sbr - 1) / sbr) * sbr;
    if (li >= per) return;
    const int item = xcd * per + li;
    if (item >= nitems) return;
    sb = item / (sbr * sbc);
    within = item - sb * (sbr * sbc);
  }
  const int rt = (sb % nrtb) * sbr + within % sbr;
  const int tq = (sb / nrtb) * sbc + within / sbr;
  if (rt >= nrt || tq >= nreal) return;
  // the routing tiles hold 128 slots; with 64-slot tiles each is done in two
  // halves (tile_half)
  const int tile = a.tile_half ? tq >> 1 : tq;
  const int e = find_segment(a.tile_off, a.K, tile, &s_res);
  if (e < 0) return;
  const int lt = tile - a.tile_off[e];
  const int pos0 = a.off[e] + lt * 128 + (a.tile_half ? (tq & 1) * 64 : 0);
  const int nv = min(BN, a.cnt[e] - (pos0 - a.off[e]));
  if (nv <= 0) return;
  const int rb0 = rt * RF * PF_WAVES + wave * RF;     // first row block of this wave

  if (tid < BN) {
    int src = -1, ex = 0, col[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) col[p] = -1;
    if (tid < nv) {
      const int pos = pos0 + tid;
      const int slotid = a.perm[pos];
      src = a.gather ? slotid / a.topk : pos;
      if (a.ex) ex = a.ex[src];
      if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
          if (a.P[p]) col[p] = a.slot2col[p][slotid];
      }
    }
    s_src[tid] = src;
    s_exp[tid] = ex;
    if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
      for (int p = 0; p < NP; ++p) s_col[p][tid] = col[p];
    }
  }
  __syncthreads();

  const int nstage = a.d_in >> 7;
  const int nfull = a.d_in >> 8;                  // full 8-step code groups
  const bool has_tail = (a.d_in & 255) != 0;      // last stage is a 4-step tail group
  const int ng = a.p[0].ng;
  const int G = a.p[0].group;
  // code dwords per expert, and per row block and k-step (16 rows x 32 inputs)
  const size_t cpe = (size_t)a.d_out * BITS * (a.d_in >> 5);
  constexpr int WPS = 16 * BITS;

  const int row_lo = s_src[0];
  const int row_hi = s_src[max(nv - 1, 0)];
  // per-lane load offsets
  // activations: load i of this wave is (k-step j, token fragment f)
  uint32_t b_vo[SL::NB];
#pragma unroll
  for (int i = 0; i < SL::NB; ++i) {
    const int q = wave * SL::NB + i;
    const int j = q / NF, f = q - j * NF;
    const int src = s_src[16 * f + l16];
    b_vo[i] = (src >= 0) ? ((uint32_t)(src - row_lo) * a.d_in + 32 * j + 8 * lg) * 2u : OOB;
  }
  // codes and scale/zero words: one buffer per (fragment, projection)
  __amdgpu_buffer_rsrc_t rc[RF][NP], rs[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int r = 0; r < RF; ++r) {
      const int rb = min(rb0 + r, nrb - 1);
      rc[r][p] = make_rsrc(a.p[p].codes + (size_t)e * cpe + (size_t)rb * (a.d_in >> 5) * WPS,
                           (uint32_t)(a.d_in >> 5) * WPS * 4u);
    }
    const int rbc = min(rb0, nrb - 1);
    rs[p] = make_rsrc(a.p[p].sz + ((size_t)e * nrb + rbc) * ng * 16,
                      (uint32_t)(min(RF, nrb - rbc) * ng * 64));
  }
  // activation rows of the tile, addressed from its first row (rows ascend
  // inside a tile)
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(
      reinterpret_cast<const half_t*>(a.A) + (size_t)max(row_lo, 0) * a.d_in,
      (uint32_t)min<size_t>((size_t)(row_hi - row_lo + 1) * a.d_in * 2u, (size_t)OOB));
  // scale/zero loads: load n, lane l -> word w = 64 n + l = gi * SZG + r * 16 + row
  uint32_t sz_vo[SL::NSZ];
#pragma unroll
  for (int n = 0; n < SL::NSZ; ++n) {
    const int w = 64 * n + lane;
    const int gi = w / SL::SZG, r = (w % SL::SZG) >> 4, row = w & 15;
    const bool ok = gi < NGS && r < RF && rb0 + r < nrb;
    const int gofs = (GS == 0) ? 0 : gi;       // generic G: one load per group slot
    sz_vo[n] = ok ? (((uint32_t)(r * ng + gofs)) * 16u + row) * 4u : OOB;
  }
  // stage order rotated by super-block (the same inside one)
  const int r0 = sb % nstage;

  auto issue = [&](int b, char* base) {
    const bool live = b < nstage;
    int st = b + r0;
    st = (st >= nstage) ? st - nstage : st;
    st = live ? st : 0;
#pragma unroll
    for (int i = 0; i < SL::NB; ++i) {
      const int q = wave * SL::NB + i;
      dma16(rx, base + SL::B + q * 1024, live ? b_vo[i] : OOB, st * 256u);
    }
    const bool tl = has_tail && st == nstage - 1;
    // lane offsets of the stage's code dwords: 2-bit, dword 2 (st % 2) + i of
    // the lane's 16 B of its 8-step group (8 B in a 4-step tail); 3-bit, unit
    // st % 2 of the group (dwords 0..2 or 3..5, see upload.hip) or the tail's
    // three planes
    uint32_t c_vo[SL::NCW];
    uint32_t c_so;
    if constexpr (BITS == 3) {
      c_so = (st >> 1) * 1536u;
      const bool u1 = (st & 1) != 0;
#pragma unroll
      for (int i = 0; i < 3; ++i)
        c_vo[i] = tl ? i * 256u + lane * 4u
                     : (u1 ? (i == 0 ? lane * 16u + 12u : 1024u + (i - 1) * 256u + lane * 4u)
                           : lane * 16u + i * 4u);
    } else {
      c_so = tl ? nfull * 1024u : (st >> 1) * 1024u + (st & 1) * 8u;
#pragma unroll
      for (int i = 0; i < 2; ++i) c_vo[i] = (tl ? lane * 8u : lane * 16u) + i * 4u;
    }
#pragma unroll
    for (int r = 0; r < RF; ++r)
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < SL::NCW; ++i)
          dma4(rc[r][p], base + SL::CODE + (((wave * RF + r) * NP + p) * SL::NCW + i) * 256,
               live ? c_vo[i] : OOB, c_so);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int n = 0; n < SL::NSZ; ++n) {
        // first group of the stage (power-of-two G: the stage's groups are
        // consecutive), or the group of k-step n (any G)
        const int g = (GS == 0) ? (st * 128 + n * 32) / G : (st * 128) / (32 * (GS == 0 ? 1 : GS));
        dma4(rs[p], base + SL::SZ + ((wave * NP + p) * SL::NSZ + n) * 256,
             live ? sz_vo[n] : OOB, g * 64u);
      }
  };

  f32x4 acc[NP][RF][NF];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int r = 0; r < RF; ++r)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[p][r][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const char* base) {
    // the stage's code dwords and scale/zero words are read first, so the
    // first fragment's dequantization waits for them alone
    uint32_t cw[SL::NCW][RF][NP];
#pragma unroll
    for (int d = 0; d < SL::NCW; ++d)
#pragma unroll
      for (int r = 0; r < RF; ++r)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          cw[d][r][p] = *reinterpret_cast<const uint32_t*>(
              base + SL::CODE + (((wave * RF + r) * NP + p) * SL::NCW + d) * 256 + lane * 4);
    uint32_t zw[RF][NP][NGS];
#pragma unroll
    for (int r = 0; r < RF; ++r)
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int g = 0; g < NGS; ++g)
          zw[r][p][g] = *reinterpret_cast<const uint32_t*>(
              base + SL::SZ + (wave * NP + p) * SL::NSZ * 256 + (g * SL::SZG + r * 16 + l16) * 4);
    if constexpr (BITS == 3) {
      // one k-step at a time: its activation fragments, then per (fragment,
      // projection) the step's dequantized operand and the MFMAs
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8v bfr[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f)
          bfr[f] = *reinterpret_cast<const half8v*>(base + SL::B + ((j * NF + f) * 64 + lane) * 16);
        const int gi = (NGS == 4) ? j : (NGS == 2 ? j >> 1 : 0);
#pragma unroll
        for (int r = 0; r < RF; ++r)
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const uint32_t D0 = cw[0][r][p], D1 = cw[1][r][p], D2 = cw[2][r][p];
            half8v aj;
            if constexpr (LUT) {
              const DeqLut3 t = deq_lut3(zw[r][p][gi]);
              aj = (j == 0) ? lut3_step<0>(D0, D1, D2, t)
                 : (j == 1) ? lut3_step<1>(D0, D1, D2, t)
                 : (j == 2) ? lut3_step<2>(D0, D1, D2, t) : lut3_step<3>(D0, D1, D2, t);
            } else {
              const DeqConst3 c = deq_const3(zw[r][p][gi]);
              aj = (j == 0) ? deq3_step<0>(D0, D1, D2, c)
                 : (j == 1) ? deq3_step<1>(D0, D1, D2, c)
                 : (j == 2) ? deq3_step<2>(D0, D1, D2, c) : deq3_step<3>(D0, D1, D2, c);
            }
#pragma unroll
            for (int f = 0; f < NF; ++f) acc[p][r][f] = mfma16(aj, bfr[f], acc[p][r][f]);
          }
      }
      return;
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      half8v bfr[2][NF];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          bfr[b][f] = *reinterpret_cast<const half8v*>(
              base + SL::B + (((2 * d + b) * NF + f) * 64 + lane) * 16);
#pragma unroll
      for (int r = 0; r < RF; ++r)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          // scale/zero words of this lane's row for k-steps 2d and 2d+1
          const int gi0 = (NGS == 4) ? 2 * d : (NGS == 2 ? d : 0);
          const int gi1 = (NGS == 4) ? 2 * d + 1 : gi0;
          half8v a0, a1;
          if constexpr (LUT) {
            const DeqLut t0 = deq_lut(zw[r][p][gi0]);
            if (gi1 == gi0) {
              deq_dword_lut(cw[d][r][p], t0, t0, a0, a1);
            } else {
              const DeqLut t1 = deq_lut(zw[r][p][gi1]);
              deq_dword_lut(cw[d][r][p], t0, t1, a0, a1);
            }
          } else {
            const DeqConst c0 = deq_const(zw[r][p][gi0]);
            if (gi1 == gi0) {
              deq_dword(cw[d][r][p], c0, c0, a0, a1);
            } else {
              const DeqConst c1 = deq_const(zw[r][p][gi1]);
              deq_dword(cw[d][r][p], c0, c1, a0, a1);
            }
          }
#pragma unroll
          for (int f = 0; f < NF; ++f) acc[p][r][f] = mfma16(a0, bfr[0][f], acc[p][r][f]);
#pragma unroll
          for (int f = 0; f < NF; ++f) acc[p][r][f] = mfma16(a1, bfr[1][f], acc[p][r][f]);
        }
    }
  };

  // ring over stages (see gemm_decode.hip for the protocol): whole rounds
  // always run, stage-times past the end only wait and issue empty loads
#pragma unroll
  for (int b = 0; b < DEPTH; ++b) issue(b, slot[b]);
  for (int t = 0; t < nstage; t += NSLOT) {
#pragma unroll
    for (int u = 0; u < NSLOT; ++u) {
      const int tau = t + u;
      wait_vm<SL::NI * (DEPTH - 1)>();
      bar_nofence();
      if (tau < nstage) compute(slot[u]);
      issue(tau + DEPTH, slot[(u + DEPTH) % NSLOT]);
    }
  }
  wait_vm<0>();
  __syncthreads();

  // undo the per-row power-of-two scaling of converted bfloat16 rows
  if (a.ex) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
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
    // Low-rank row stage as extra k-steps: A = U_m rows (straight from global
    // memory in the A-fragment layout), B = Sigma p of each slot as a high
    // and a low part in the activation dtype (the column stage wrote them so,
    // row [high r_pad | low r_pad]).  One pass per block of up to KBB rank
    // steps of each projection: the wave's U fragments are requested, the
    // slots' rows are gathered into the idle ring by LDS-destination loads
    // as 1 KB B fragments (unit = one projection's rank step: [hi|lo][NF]
    // fragments), then the MFMAs run.
    constexpr int KBB = 4;                          // rank steps per projection and pass
    constexpr int NU = NP * KBB;                    // units per pass
    constexpr int UB = 2 * NF * 1024;               // bytes of a unit
    constexpr int UPS = SL::BYTES / UB;             // units per ring slot
    constexpr int CPW = NU * 2 * NF / PF_WAVES;     // fragment loads per wave and pass
    static_assert(NSLOT * UPS >= NU, "one pass of units fits the ring");
    static_assert(CPW * PF_WAVES == NU * 2 * NF, "fragment loads split evenly over the waves");
    int nk[NP], rp[NP];
    size_t mrow[NP];
    __amdgpu_buffer_rsrc_t rph[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      rp[p] = a.p[p].r_pad;
      nk[p] = (a.p[p].rank > 0 && a.P[p]) ? rp[p] >> 5 : 0;
      mrow[p] = nk[p] ? (size_t)a.p[p].m_of[e] * a.d_out : 0;
      rph[p] = make_rsrc(a.P[p], nk[p] ? (uint32_t)((size_t)a.p_rows * rp[p] * 4u) : 0u);
    }
    const int nkmax = (NP > 1) ? max(nk[0], nk[NP - 1]) : nk[0];
    auto slot_of = [&](int i) { return i == 0 ? s0 : (i == 1 ? s1 : s2); };
    for (int kb0 = 0; kb0 < nkmax; kb0 += KBB) {
      V8 uf[NP][RF][KBB];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int r = 0; r < RF; ++r)
#pragma unroll
          for (int i = 0; i < KBB; ++i) {
            uf[p][r][i] = __builtin_bit_cast(V8, u32x4{0u, 0u, 0u, 0u});
            if (kb0 + i < nk[p] && rb0 + r < nrb) {
              const T* up = reinterpret_cast<const T*>(a.p[p].U) +
                            (mrow[p] + (rb0 + r) * 16 + l16) * rp[p] + (kb0 + i) * 32 + 8 * lg;
              uf[p][r][i] = *reinterpret_cast<const V8*>(up);
            }
          }
      bar_nofence();               // nothing reads the ring any more (the U loads stay in flight)
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int c = wave * CPW + i;              // (unit, hi/lo, fragment)
        const int u = c / (2 * NF), hl = (c / NF) & 1, f = c % NF;
        const int p = (NP > 1) ? u / KBB : 0, kb = kb0 + u % KBB;
        const int np = (NP > 1 && p) ? nk[NP - 1] : nk[0];
        const int rpp = (NP > 1 && p) ? rp[NP - 1] : rp[0];
        const int col = s_col[p][16 * f + l16];
        const uint32_t vo = (kb < np && col >= 0)
                                ? ((uint32_t)col * rpp * 2u + hl * rpp + kb * 32 + 8 * lg) * 2u
                                : OOB;
        dma16((NP > 1 && p) ? rph[NP - 1] : rph[0],
              slot_of(u / UPS) + (u % UPS) * UB + (hl * NF + f) * 1024, vo, 0u);
      }
      wait_vm<0>();
      __syncthreads();
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < KBB; ++i) {
          if (kb0 + i >= nk[p]) continue;
          const int u = p * KBB + i;
          const char* ub = slot_of(u / UPS) + (u % UPS) * UB + lane * 16;
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const V8 bh = *reinterpret_cast<const V8*>(ub + f * 1024);
            const V8 bl = *reinterpret_cast<const V8*>(ub + (NF + f) * 1024);
#pragma unroll
            for (int r = 0; r < RF; ++r) {
              acc[p][r][f] = mfma16(uf[p][r][i], bh, acc[p][r][f]);
              acc[p][r][f] = mfma16(uf[p][r][i], bl, acc[p][r][f]);
            }
          }
        }
    }
    // SwiGLU epilogue: h = RND_act(silu(gate) * up), stored per slot position
    T* h = reinterpret_cast<T*>(a.h);
    // fp16 copy for bfloat16 layers: |silu(g) u| <= |g||u| <= B_g B_u max|x|^2
    // with B the row bounds of |W| (< 2^bg, 2^bu) and max|x| < 2^(ex + 15),
    // so h * 2^-(bg + bu + 2 ex + 15) stays below 2^15
    int bgu = 0;
    if (a.h16) {
      int bg, bu;
      frexpf(a.p[0].l1max[e], &bg);
      frexpf(a.p[1].l1max[e], &bu);
      bgu = bg + bu + 15;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int row = 16 * f + l16;
      if (row >= nv) continue;
      const int pos = pos0 + row;
      const int eh = bgu + 2 * s_exp[row];
      if (a.h16 && rt == 0 && wave == 0 && lg == 0) a.exh[pos] = eh;
#pragma unroll
      for (int r = 0; r < RF; ++r) {
        if (rb0 + r >= nrb) continue;
        const int o = (rb0 + r) * 16 + 4 * lg;
        T hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) hv[v] = from_f32<T>(silu_f(acc[0][r][f][v]) * acc[1][r][f][v]);
        *reinterpret_cast<u32x2*>(h + (size_t)pos * a.d_out + o) = __builtin_bit_cast(u32x2, hv);
        if (a.h16) {
          half_t hs[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) hs[v] = (half_t)ldexpf(to_f32(hv[v]), -eh);
          *reinterpret_cast<u32x2*>(reinterpret_cast<half_t*>(a.h16) + (size_t)pos * a.d_out + o) =
              __builtin_bit_cast(u32x2, hs);
        }
      }
    }
  } else {
    // gated per-slot residual output (fp32)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int row = 16 * f + l16;
      if (row >= nv) continue;
      const int pos = pos0 + row;
      const float g = a.gates[a.perm[pos]];
#pragma unroll
      for (int r = 0; r < RF; ++r) {
        if (rb0 + r >= nrb) continue;
        const int o = (rb0 + r) * 16 + 4 * lg;
        *reinterpret_cast<f32x4*>(a.dres + (size_t)pos * a.d_out + o) = acc[0][r][f] * g;
      }
    }
  }
}

template <int NP, int RF, int NF, int GS, int BITS>
constexpr bool pre_fits() {
  return 3 * PfSlot<NP, RF, NF, GS, BITS>::BYTES <= 160 * 1024 - 2048;
}

static int pf_grid(int nrt, int ntq) {
  int sbr, sbc;
  pf_superblock(nrt, &sbr, &sbc);
  const int nsb = ((nrt + sbr - 1) / sbr) * ((ntq + sbc - 1) / sbc);
  return ((nsb + 7) / 8) * 8 * sbr * sbc;
}

template <typename T, int MODE, int RF, int NF, int GS, bool LUT, int BITS>
static void pre_launch(const GemmArgs& a, int max_tiles, hipStream_t s) {
  constexpr int NP = (MODE == MODE_GATEUP) ? 2 : 1;
  const int rows_per_wg = 16 * RF * PF_WAVES;
  const int nrt = (a.d_out + rows_per_wg - 1) / rows_per_wg;
  GemmArgs b = a;
  if constexpr (pre_fits<NP, RF, NF, GS, BITS>()) {
    if (!a.narrow) {
      b.ntq = max_tiles;
      const dim3 grid(pf_grid(nrt, b.ntq)), block(64 * PF_WAVES);
      hipLaunchKernelGGL((gemm_pre_kernel<T, MODE, RF, NF, GS, LUT, BITS>), grid, block, 0, s, b);
      return;
    }
  }
  // a 128-slot tile as two 64-slot units (when the wide ring does not fit,
  // or when experts hold few slots: half the MFMA work on padding)
  static_assert(NF == 8, "smaller tiles always fit");
  static_assert(pre_fits<NP, RF, 4, GS, BITS>(), "64-slot tiles fit");
  b.tile_half = 1;
  b.ntq = 2 * max_tiles;
  const dim3 grid(pf_grid(nrt, b.ntq)), block(64 * PF_WAVES);
  hipLaunchKernelGGL((gemm_pre_kernel<T, MODE, RF, 4, GS, LUT, BITS>), grid, block, 0, s, b);
}

template <typename T, int MODE, int RF, int NF, bool LUT, int BITS>
static void pre_gs(const GemmArgs& a, int max_tiles, hipStream_t s) {
  const int G = a.p[0].group;
  const bool pow2 = (G & (G - 1)) == 0;
  if (!pow2 || G > 256) {
    // any group size: 2-bit codes only (upload requires a power of two from
    // 32 to 256 with 3-bit codes)
    if constexpr (BITS == 2) pre_launch<T, MODE, RF, NF, 0, LUT, BITS>(a, max_tiles, s);
  } else if (G == 32) pre_launch<T, MODE, RF, NF, 1, LUT, BITS>(a, max_tiles, s);
  else if (G == 64) pre_launch<T, MODE, RF, NF, 2, LUT, BITS>(a, max_tiles, s);
  else if (G == 128) pre_launch<T, MODE, RF, NF, 4, LUT, BITS>(a, max_tiles, s);
  else pre_launch<T, MODE, RF, NF, 8, LUT, BITS>(a, max_tiles, s);
}

// The table dequantization when any projection of the launch has scales or
// zero points outside the packed-arithmetic range (both give the same
// canonical weights where both apply).
template <typename T, int MODE, int RF, int NF, int BITS>
static void pre_lut(const GemmArgs& a, int max_tiles, hipStream_t s) {
  constexpr int NP = (MODE == MODE_GATEUP) ? 2 : 1;
  bool lut = false;
  for (int p = 0; p < NP; ++p) lut = lut || a.p[p].deq_lut;
  if (lut) pre_gs<T, MODE, RF, NF, true, BITS>(a, max_tiles, s);
  else pre_gs<T, MODE, RF, NF, false, BITS>(a, max_tiles, s);
}

// This translation unit holds the kernels of one code width (the build
// compiles it once per width, TQ_PREFILL_BITS = 2 and 3).
#ifndef TQ_PREFILL_BITS
#define TQ_PREFILL_BITS 2
#endif

#if TQ_PREFILL_BITS == 3
void launch_gemm_prefill_b3(const GemmArgs& a, GemmMode mode, Act act, int max_tiles,
                            hipStream_t s) {
#else
void launch_gemm_prefill_b2(const GemmArgs& a, GemmMode mode, Act act, int max_tiles,
                            hipStream_t s) {
#endif
  constexpr int B = TQ_PREFILL_BITS;
  if (act == ACT_F16) {
    if (mode == MODE_GATEUP) pre_lut<half_t, MODE_GATEUP, 2, 8, B>(a, max_tiles, s);
    else pre_lut<half_t, MODE_RES, 4, 8, B>(a, max_tiles, s);
  } else {
    if (mode == MODE_GATEUP) pre_lut<__bf16, MODE_GATEUP, 2, 8, B>(a, max_tiles, s);
    else pre_lut<__bf16, MODE_RES, 4, 8, B>(a, max_tiles, s);
  }
}

}  // namespace tq
