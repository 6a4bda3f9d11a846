// Decode-path residual kernel: streams each active expert's 2-bit codes once
// from HBM and applies them to that expert's few slots.
//
// "TileQ" technical summary, section 4 (Inference Latency, Decode): decode is
// memory bound; the layout is contiguous and read with wide vector accesses.
//
// Work: a workgroup of WAVES waves, rows_per of which own a row fragment (16
// rows each) of one expert -- in MODE_GATEUP the gate and the up rows
// together -- walks a range of k-stages (8 MFMA k-steps = 256 inputs each)
// for a column tile of 16 of the expert's slots.  With NCT = 2 (many slots
// per expert) the waves form two groups that take two column tiles at once,
// reading each stage's codes from LDS once loaded: the codes are streamed
// once for 32 slots.  For a single projection (down) a wave may instead own
// two adjacent fragments in the places of gate and up (MODE_RES2), so each
// stage streams twice the code bytes.  Everything a stage
// needs (each wave's codes, the stage's activations shared by all waves, the
// scale/zero words and the activation group sums) is brought straight into
// LDS by buffer loads with the LDS destination (no registers in between), in
// a ring of DEPTH + 1 slots: DEPTH stages are in flight while one is
// computed.  Two 8-wave workgroups share a CU when their ring fits half the
// LDS.  Each wave waits for its own loads with an explicit vmcnt (loads
// complete in issue order) before the stage's barrier; the barrier carries
// no memory fence, which would wait for every load in flight.
//
// The codes enter v_mfma_f32_16x16x32_f16 as the raw packed values 1 + q*c
// (one and-or per pair, no dequantization) against the class-scaled
// activations x' = x~/c (decode_stages.hip), so a group's fp32 partial is
// C_g = X'_g + sum q x~ and the residual output of a row is
//     sum_g s_g (C_g - X'_g - z_g X~_g)
//   = sum_g s_g C_g  -  sum_g (s_g X'_g + s_g z_g X~_g).
// The first sum costs one fma per group; the second is a small product
// (rows x 2 NG) . (2 NG x columns) per stage, done by v_mfma_f32_16x16x4_f32
// into a separate accumulator.
// Epilogue: undo the row scaling 2^E, add the low-rank row stage U_m Sigma p
// as MFMA K-steps (MODE_GATEUP; in MODE_RES by the first k-chunk when P is
// given; p from the column stage), then SwiGLU into h, or (MODE_RES) the
// slot's routing weight into the fp32 per-slot buffer of the workgroup's
// k-range (split-K slabs, summed by the combine kernel).
#include "tq_device.h"

namespace tq {

// Kernel-internal mode: one projection (as MODE_RES) with two row fragments
// per wave, 2 u and 2 u + 1 of row unit u, in the places the gate and up
// fragments take in MODE_GATEUP: each wave streams twice the code bytes per
// stage for the same fixed costs per stage.
constexpr int MODE_RES2 = 2;
template <int MODE> constexpr int dec_np() { return MODE == MODE_RES ? 1 : 2; }

// LDS slot layout (bytes) for NP projections, WAVES waves, NG groups/stage,
// BITS-bit codes and NCT column tiles of 16 slots: the waves form NCT groups
// of WR = WAVES / NCT (group c computes column tile c); wave slot w of every
// group owns row fragment w, whose codes all groups read, each wave loading
// those of NPL projections
template <int NP, int WAVES, int NG, int BITS, int NCT = 1>
struct DecSlot {
  static constexpr int WR = WAVES / NCT;
  static constexpr int NPL = (NP + NCT - 1) / NCT;
  // codes of a wave and projection per stage: 2-bit 64 lanes x 16 B; 3-bit
  // 64 lanes x 16 B (dwords 0..3) then dwords 4 and 5 of the 64 lanes
  static constexpr int CB = (BITS == 3) ? 1536 : 1024;
  static constexpr int NCL = (BITS == 3) ? 3 : 1;    // code loads per projection
  // scale/zero words of a stage: per projection a [WAVES][NG][16 rows] table,
  // brought in by 64-word loads that the waves share out
  static constexpr int NSZP = (WR * NG + 3) / 4;     // 64-word loads per projection
  static constexpr int NSZW = (NP * NSZP + WAVES - 1) / WAVES;   // ... per wave
  static constexpr int NSUM = NG >= 2 ? NG / 2 : 1;  // dword loads of the group sums per tile
  static constexpr int NACT = (8 * NCT + WAVES - 1) / WAVES;   // activation loads per wave
  static constexpr int CODE = 0;                     // [WR][NP] x CB
  static constexpr int ACT = CODE + WR * NP * CB;    // [NCT][8 k-steps][64 lanes] x 16 B
  static constexpr int SZ = ACT + NCT * 8 * 1024;    // [NP][NSZP * 64] x 4 B
  static constexpr int SUM = SZ + NP * NSZP * 256;   // [NCT][NG][16 cols] float2
  static constexpr int BYTES = SUM + NCT * NSUM * 256;
  // loads per wave per stage (the same for every wave)
  static constexpr int NI = NPL * NCL + NACT + NSZW + 1;
  // two tiles: wave w loads k-steps w NACT .. w NACT + NACT - 1 of the
  // activations, all of its own tile
  static_assert(NCT == 1 || NACT * WR == 8, "activation loads of a tile group");
};

// Two workgroups share a CU when an 8-wave workgroup's ring of three slots
// fits half the LDS: then one workgroup's routing reads, ring fill and
// epilogue overlap the other's streaming.
template <int BYTES, int WAVES>
constexpr bool dec_dual() {
  return WAVES <= 8 && 3 * BYTES + 1024 <= 80 * 1024;
}

// ring length: as many slots as fit the LDS budget (half the LDS for two
// workgroups per CU, else about 150 KB), at most DMAX + 1
template <int BYTES, int DMAX, bool DUAL>
constexpr int ring_depth() {
  constexpr int budget = DUAL ? 79 * 1024 : 150 * 1024;
  return (budget / BYTES - 1 < DMAX) ? budget / BYTES - 1 : DMAX;
}

template <int MODE, int GS, int WAVES, int BITS, int NCT = 1>
constexpr bool dec_dual_cfg() {
  return dec_dual<DecSlot<dec_np<MODE>(), WAVES, 8 / GS, BITS, NCT>::BYTES, WAVES>();
}

// Raw A operand (1 + q c per fp16 half) of k-step J of a stage from the
// lane's code dwords: 2-bit, dword J / 2 (unpack16); 3-bit, unit J / 4 of
// dwords (0, 1, 2) or (3, 4, 5) (raw3_step).  J folds to a constant.
template <int BITS>
__device__ __forceinline__ u32x4 dec_raw(int J, const u32x4& c, uint32_t c4, uint32_t c5) {
  if constexpr (BITS == 3) {
    const uint32_t D0 = J < 4 ? c[0] : c[3], D1 = J < 4 ? c[1] : c4, D2 = J < 4 ? c[2] : c5;
    switch (J & 3) {
      case 0: return raw3_step<0>(D0, D1, D2);
      case 1: return raw3_step<1>(D0, D1, D2);
      case 2: return raw3_step<2>(D0, D1, D2);
      default: return raw3_step<3>(D0, D1, D2);
    }
  } else {
    return unpack16_step(c[J >> 1], J & 1);
  }
}

template <typename T, int MODE, int GS, int WAVES, int DMAX, int BITS, int NCT>
__global__ __launch_bounds__(64 * WAVES, (dec_dual_cfg<MODE, GS, WAVES, BITS, NCT>() ? 4 : 1))
void gemm_dec_kernel(DecArgs a) {
  typedef typename Vec8<T>::type V8;
  // The kernel arguments read before the first stage, requested together:
  // the empty asm needs them all in scalar registers, so their loads go out
  // at once with one wait, instead of one round trip per use site.
  asm volatile("" ::"s"(a.K), "s"(a.d_in), "s"(a.d_out), "s"(a.rows_per), "s"(a.nks),
               "s"(a.spec), "s"(a.arec), "s"(a.etab), "s"(a.S), "s"(a.off), "s"(a.cnt));
  asm volatile("" ::"s"(a.p[0].ng), "s"(a.p[0].codes), "s"(a.p[0].sz), "s"(a.p[0].rank),
               "s"(a.p[0].m_of), "s"(a.p[0].n_of), "s"(a.P[0]), "s"(a.Xp), "s"(a.rows),
               "s"(a.sums), "s"(a.gather), "s"(a.topk), "s"(a.ex));
  if constexpr (dec_np<MODE>() > 1)
    asm volatile("" ::"s"(a.p[1].codes), "s"(a.p[1].sz), "s"(a.p[1].rank), "s"(a.p[1].m_of),
                 "s"(a.p[1].n_of), "s"(a.P[1]));
  constexpr int NP = dec_np<MODE>();
  constexpr bool PAIR = MODE == MODE_RES2;   // the NP "projections" are two row fragments
  constexpr int NPG = PAIR ? 1 : NP;         // projections whose Sigma p the row stage gathers
  constexpr int NG = 8 / GS;             // groups per stage
  typedef DecSlot<NP, WAVES, NG, BITS, NCT> SL;
  constexpr int WR = SL::WR;
  constexpr bool DUAL = dec_dual<SL::BYTES, WAVES>();
  constexpr int DEPTH = ring_depth<SL::BYTES, DMAX, DUAL>();
  constexpr int NSLOT = DEPTH + 1;
  static_assert(DEPTH >= 2, "ring depth");
  static_assert(SL::NI * (DEPTH - 1) < 64, "vmcnt range");
  static_assert(NSLOT <= 8, "ring length");
  static_assert(SL::BYTES >= NP * 2 * 16 * (128 + 8) * 2, "row-stage staging");
  constexpr int NCORR = (2 * NG + 3) / 4;   // fp32 MFMAs of the group correction
  __shared__ __attribute__((aligned(16))) char s0[SL::BYTES];
  __shared__ __attribute__((aligned(16))) char s1[SL::BYTES];
  __shared__ __attribute__((aligned(16))) char s2[NSLOT > 2 ? SL::BYTES : 16];
  __shared__ __attribute__((aligned(16))) char s3[NSLOT > 3 ? SL::BYTES : 16];
  __shared__ __attribute__((aligned(16))) char s4[NSLOT > 4 ? SL::BYTES : 16];
  __shared__ __attribute__((aligned(16))) char s5[NSLOT > 5 ? SL::BYTES : 16];
  __shared__ __attribute__((aligned(16))) char s6[NSLOT > 6 ? SL::BYTES : 16];
  __shared__ __attribute__((aligned(16))) char s7[NSLOT > 7 ? SL::BYTES : 16];
  // target of unused loads (activation loads past the 8th k-step are 16 B
  // per lane, the others 4 B)
  __shared__ __attribute__((aligned(16))) char s_dummy[(WAVES * SL::NACT > 8 * NCT || NCT > 1) ? 1024 : 256];
  char* const slot[8] = {s0, s1, s2, s3, s4, s5, s6, s7};

  // Workgroup -> (expert, row-fragment group, k-chunk).  Consecutive
  // workgroups go to the 8 XCDs in turn.  With every expert expected to be
  // routed to (a.spec), consecutive workgroups of one XCD take different
  // experts and every XCD gets an equal share of every expert's rows.  Else
  // (compact mapping, a.arec) the workgroups of active expert i come i-th:
  // the routing's record says which expert that is, and the workgroups past
  // the active ones end at once instead of being interleaved with the work.
  const int nrb = a.d_out >> 4;
  // row units of a wave: a 16-row fragment, or (PAIR) two
  const int nun = PAIR ? (nrb + 1) >> 1 : nrb;
  // a.rows_per (<= WAVES) waves of a workgroup own row units; the others
  // only help with the shared loads
  const int rpw = a.rows_per;
  const int nby = (nun + rpw - 1) / rpw;
  const int nby8 = (nby + 7) >> 3;
  const int wg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  int e, ks, by, q, cnt = 0, offe = 0;
  const int* rec = nullptr;
  if (a.arec) {
    const int ue = nby8 * 8 * a.nks;               // workgroups per expert
    const int ei = wg / ue, rem = wg - ei * ue;
    rec = a.arec + ei * ROUTE_AREC;
    const int na = sload(a.arec, a.K * ROUTE_AREC);
    e = sload(rec, 0);
    cnt = sload(rec, 1);
    offe = sload(rec, 2);
    ks = rem / (nby8 * 8);
    by = rem - ks * nby8 * 8;
    q = rem >> 3;
    if (ei >= na || by >= nby) return;
  } else {
    q = wg >> 3;
    e = q % a.K;
    const int jq = q / a.K;
    ks = jq / nby8;
    by = (jq - ks * nby8) * 8 + (wg & 7);
    if (by >= nby) return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  // row-fragment slot and column tile of this wave
  const int wr = (NCT == 1) ? wave : wave % WR, wc = (NCT == 1) ? 0 : wave / WR;
  const int rb_raw = by * rpw + wr;
  const bool rvalid = wr < rpw && rb_raw < nun;
  const int rb = rvalid ? rb_raw : nun - 1;          // clamped: loads stay in bounds
  // row fragment of "projection" p (PAIR: 2 rb + p, clamped; the second of
  // an odd count is computed but not stored)
  int rbp[NP];
  bool fvalid[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    rbp[p] = PAIR ? min(2 * rb + p, nrb - 1) : rb;
    fvalid[p] = rvalid && (!PAIR || 2 * rb_raw + p < nrb);
  }
  const int nsteps = a.d_in >> 5;
  const int nfull = nsteps >> 3;
  // k-chunk of this workgroup: stages [k0, k0 + ntau); the 4-step tail stage
  // (d_in % 256 == 128) goes with the last chunk
  const int k0 = (int)(((long)nfull * ks) / a.nks);
  const int ntau = (int)(((long)nfull * (ks + 1)) / a.nks) - k0;
  const bool tail = ((nsteps & 7) != 0) && ks == a.nks - 1;
  const int ng = a.p[0].ng;
  // Stage order is rotated per workgroup (stage-time tau works on stage
  // k0 + (tau + r0) mod ntau): workgroups running together on an XCD read
  // different activation chunks and code pages instead of all hitting the
  // same L2 channels.
  const int r0 = ntau > 0 ? q % ntau : 0;
  // code dwords per expert, and per row block and k-step (16 rows x 32 inputs)
  const size_t cpe = (size_t)a.d_out * BITS * (a.d_in >> 5);
  constexpr int WPS = 16 * BITS;

  __amdgpu_buffer_rsrc_t rc[NP], rs[NP];
  const uint32_t* cbase[NP];
  const uint32_t* szb[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const ProjDev& pd = a.p[PAIR ? 0 : p];
    cbase[p] = pd.codes + (size_t)e * cpe + (size_t)rbp[p] * nsteps * WPS;
    szb[p] = pd.sz + ((size_t)e * nrb + rbp[p]) * ng * 16;
    rc[p] = make_rsrc(cbase[p], (uint32_t)nsteps * WPS * 4u);
    rs[p] = make_rsrc(pd.sz + (size_t)e * nrb * ng * 16, (uint32_t)nrb * ng * 64u);
  }
  // scale/zero loads of this wave: load i = wave + WAVES * k of the stage
  // covers words 64 (i mod NSZP) + lane of projection i / NSZP's table, i.e.
  // (wave' = w / (16 NG), group w / 16 mod NG, row w mod 16)
  uint32_t sz_vo[SL::NSZW];
  int sz_p[SL::NSZW], sz_lds[SL::NSZW];
#pragma unroll
  for (int k = 0; k < SL::NSZW; ++k) {
    const int i = wave + WAVES * k;
    const bool ok = i < NP * SL::NSZP;
    sz_p[k] = ok ? i / SL::NSZP : 0;
    sz_lds[k] = ok ? SL::SZ + i * 256 : -1;
    const int w = (ok ? i - sz_p[k] * SL::NSZP : 0) * 64 + lane;
    const int wv = w / (16 * NG), g = (w / 16) % NG, row = w & 15;
    const int rbw = min(PAIR ? 2 * (by * rpw + wv) + sz_p[k] : by * rpw + wv, nrb - 1);
    sz_vo[k] = (ok && wv < rpw) ? (((uint32_t)rbw * ng + g) * 16u + row) * 4u : OOB;
  }
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.Xp, (uint32_t)a.rows * a.d_in * 2u);
  const __amdgpu_buffer_rsrc_t rsm = make_rsrc(a.sums, (uint32_t)a.rows * ng * 8u);

  // Loads of batch b (stage-time b of the ring) into the slot at base: the
  // expert's codes and scale/zero words (known before the routing) ...
  auto issue_w = [&](int b, char* base) {
    const bool live = b < ntau;
    int tr = b + r0;
    tr = (tr >= ntau) ? tr - ntau : tr;
    const int st = live ? k0 + tr : 0;
#pragma unroll
    for (int i = 0; i < SL::NPL; ++i) {
      // projection p of this wave's row fragment (none: a load of nothing)
      const int p = wc * SL::NPL + i;
      const bool has = p < NP;
      const int pc = has ? p : 0;
      char* cb = has ? base + SL::CODE + (wr * NP + pc) * SL::CB : s_dummy;
      const bool ld = live && rvalid && has;
      dma16(rc[pc], cb, ld ? lane * 16u : OOB, st * (uint32_t)SL::CB);
      if constexpr (BITS == 3) {
        dma4(rc[pc], has ? cb + 1024 : s_dummy, ld ? 1024u + lane * 4u : OOB, st * (uint32_t)SL::CB);
        dma4(rc[pc], has ? cb + 1280 : s_dummy, ld ? 1280u + lane * 4u : OOB, st * (uint32_t)SL::CB);
      }
    }
#pragma unroll
    for (int k = 0; k < SL::NSZW; ++k)
      dma4(sz_p[k] == 0 ? rs[0] : rs[NP - 1], sz_lds[k] >= 0 ? base + sz_lds[k] : s_dummy,
           live ? sz_vo[k] : OOB, st * NG * 64u);
  };
  // ... and the activations and group sums of the column tile's slots
  uint32_t act_vo = OOB, sum_vo = OOB;
  auto issue_x = [&](int b, char* base) {
    const bool live = b < ntau;
    int tr = b + r0;
    tr = (tr >= ntau) ? tr - ntau : tr;
    const int st = live ? k0 + tr : 0;
#pragma unroll
    for (int i = 0; i < SL::NACT; ++i) {
      // k-step j of tile j / 8 (the wave's own tile); loads past the last
      // step load nothing
      const int j = wave * SL::NACT + i;
      dma16(rx, j < 8 * NCT ? base + SL::ACT + j * 1024 : s_dummy,
            (live && j < 8 * NCT && act_vo != OOB) ? act_vo + (j & 7) * 64u : OOB, st * 512u);
    }
    // group sums of the wave's tile: the first NSUM waves of each group
    dma4(rsm, wr < SL::NSUM ? base + SL::SUM + (wc * SL::NSUM + wr) * 256 : s_dummy,
         live ? sum_vo : OOB, st * NG * 8u);
  };

  // With the expert expected to be routed to (a.spec), the codes of the
  // first DEPTH stages are requested before the routing reads return.
  const bool spec = a.spec && ntau > 0;
  if (spec) {
#pragma unroll
    for (int b = 0; b < DEPTH; ++b) issue_w(b, slot[b]);
  }

  // routing reads, none waiting for another and all scalar (they do not
  // queue behind the code loads above): the expert's slot count and offset,
  // the slot ids of its first 16 positions (entries past the count are stale
  // and never used; the table has 16 entries of padding) and its tile row /
  // column (row stage)
  const int* etab = a.etab + (size_t)e * a.S;
  if (!rec) {
    cnt = sload(a.cnt, e);
    offe = sload(a.off, e);
  }
  const int sl_first = rec ? sload16(rec + 4, 0, l16) : sload16(etab, 0, l16);
  // (the tile row / column loads are unconditional -- every uploaded
  // projection has its maps -- so that all of these go out together
  // instead of behind a branch each)
  int m_e[NP], n_e[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const ProjDev& pm = a.p[PAIR ? 0 : p];
    const bool lr = a.P[p] != nullptr && a.p[p].rank > 0;
    const int mv = sload(pm.m_of, e), nv = sload(pm.n_of, e);
    m_e[p] = lr ? mv : 0;
    n_e[p] = lr ? nv : 0;
  }
  if (cnt == 0) {
    wait_vm<0>();                          // no load may land after the workgroup ends
    return;
  }

  // One column tile (16 slot positions from t0).  The first tile is a
  // straight-line copy ahead of the loop over further tiles: reached from a
  // loop header, the compiler's waits would count loads of an earlier tile
  // and stall on the code loads in flight.
  auto tile = [&](const int t0) __attribute__((always_inline)) {
    // this wave's column tile starts at position tt0; an empty one (second
    // tile past the count) reads the group's first tile instead and computes
    // nothing
    const int tt0 = t0 + 16 * wc;
    const int ncol = max(0, min(16, cnt - tt0));
    const bool tlive = ncol > 0;
    const int ts = tlive ? tt0 : t0;
    const bool cvalid = l16 < ncol;
    const int pos = offe + ts + (cvalid ? l16 : 0);
    // (no cross-lane reads here: an LDS-pipe instruction would make the
    // compiler wait for the code loads above to land)
    const int* slp = (rec && ts == 0) ? rec + 4 : etab + ts;   // slot ids from position ts
    int slotid = (ts == 0) ? sl_first : sload16(slp, 0, l16);
    slotid = cvalid ? slotid : sload(slp, 0);            // column 0 always holds a slot
    const int arow = a.gather ? slotid / a.topk : pos;
    const int E = a.ex[arow];              // row exponent, used by the epilogue

    // per-lane load offsets (columns past the tile's slots are not loaded:
    // their MFMA columns are never stored, and columns do not mix)
    // activations: lane = (lg, col) of k-step j; the k-step adds 64 bytes
    act_vo = cvalid ? ((uint32_t)arow * a.d_in + 8 * lg) * 2u : OOB;
    // group sums: word w = 64 * wr + lane of the stage's [NG][16][2] table
    // of the wave's tile
    sum_vo = OOB;
    {
      const int w = 64 * wr + lane;
      const int gi = w >> 5, col = (w >> 1) & 15, comp = w & 1;
      const int r = a.gather ? sload16(slp, 0, col) / a.topk : offe + ts + col;
      if (wr < SL::NSUM && gi < NG && col < ncol) sum_vo = (((uint32_t)r * ng + gi) * 2u + comp) * 4u;
    }
    auto issue = [&](int b, char* base) {
      issue_w(b, base);
      issue_x(b, base);
    };

    f32x4 acc[NP], corr[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
      corr[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One stage: every LDS read first (the codes, the 8 activation k-steps,
    // the scale/zero words and the group sums), then the arithmetic, so the
    // reads overlap instead of each waiting for the one before.
    //   acc  += s_g * C_g                 for the wave's rows 4 lg + v
    //   corr += A . B   with A[row][t] = s_t (t < NG) or s z of group t - NG
    //                   and B[t][col] = X'_t resp. X~_(t - NG); MFMA m of the
    //                   fp32 product covers terms t = 4 m + lg
    auto compute = [&](const char* base) {
      u32x4 code[NP];
      uint32_t code4[NP], code5[NP];
      half8v bv[8];
      u32x4 szw[NP][NG];
      float cbx[NCORR];
      uint32_t cw[NP][NCORR];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const char* cb = base + SL::CODE + (wr * NP + p) * SL::CB;
        code[p] = *reinterpret_cast<const u32x4*>(cb + lane * 16);
        code4[p] = code5[p] = 0u;
        if constexpr (BITS == 3) {
          code4[p] = *reinterpret_cast<const uint32_t*>(cb + 1024 + lane * 4);
          code5[p] = *reinterpret_cast<const uint32_t*>(cb + 1280 + lane * 4);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bv[j] = *reinterpret_cast<const half8v*>(base + SL::ACT + lane * 16 + (wc * 8 + j) * 1024);
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          szw[p][gi] = *reinterpret_cast<const u32x4*>(
              base + SL::SZ + (p * SL::NSZP * 64 + (wr * NG + gi) * 16 + 4 * lg) * 4);
#pragma unroll
      for (int m = 0; m < NCORR; ++m) {
        const int t = 4 * m + lg;
        const int g = (t < NG) ? t : t - NG;
        cbx[m] = 0.f;
        if (t < 2 * NG)
          cbx[m] = *reinterpret_cast<const float*>(base + SL::SUM + wc * SL::NSUM * 256 +
                                                   ((g * 16 + l16) * 2 + (t < NG)) * 4);
#pragma unroll
        for (int p = 0; p < NP; ++p)
          cw[p][m] = (t < 2 * NG) ? *reinterpret_cast<const uint32_t*>(
                                        base + SL::SZ + (p * SL::NSZP * 64 + (wr * NG + g) * 16 + l16) * 4)
                                  : 0u;
      }

      f32x4 C[NP];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j % GS == 0) {
#pragma unroll
          for (int p = 0; p < NP; ++p) C[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int p = 0; p < NP; ++p)
          C[p] = mfma16(as_half8(dec_raw<BITS>(j, code[p], code4[p], code5[p])), bv[j], C[p]);
        if (j % GS == GS - 1) {
          const int gi = j / GS;
#pragma unroll
          for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[p][v] += (float)__builtin_bit_cast(half_t, (uint16_t)(szw[p][gi][v] & 0xFFFFu)) * C[p][v];
        }
      }
#pragma unroll
      for (int m = 0; m < NCORR; ++m) {
        const int t = 4 * m + lg;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const float sc = (float)__builtin_bit_cast(half_t, (uint16_t)(cw[p][m] & 0xFFFFu));
          const float z = (float)__builtin_bit_cast(half_t, (uint16_t)(cw[p][m] >> 16));
          const float av = (t < 2 * NG) ? ((t < NG) ? sc : sc * z) : 0.f;
          corr[p] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, cbx[m], corr[p], 0, 0, 0);
        }
      }
    };

    // full stages.  Ring: batch b lands in slot b % NSLOT; at stage-time tau
    // the wave waits for batch tau (DEPTH - 1 newer batches may stay in
    // flight) and for its own LDS reads, the barrier makes every wave's part
    // visible and every wave's reads of stage tau - 1 complete, batch
    // tau + DEPTH is issued into the slot of tau - 1, and the stage is
    // computed while DEPTH batches are in flight.  Slots are distinct LDS
    // arrays indexed by constants: the ring is unrolled by its length and
    // whole rounds always run (stage-times past the end only wait and issue
    // empty loads), so the loop has a single back edge and the compiler's
    // own wait counts stay exact.
    if (ntau > 0) {
      // prologue: batches 0 .. DEPTH-1 (their codes may already be in flight)
      if (spec && t0 == 0) {
#pragma unroll
        for (int b = 0; b < DEPTH; ++b) issue_x(b, slot[b]);
      } else {
#pragma unroll
        for (int b = 0; b < DEPTH; ++b) issue(b, slot[b]);
      }
      for (int t = 0; t < ntau; t += NSLOT) {
#pragma unroll
        for (int u = 0; u < NSLOT; ++u) {
          const int tau = t + u;
          // first round: the prologue issued batches 0 .. DEPTH-1 whole, or
          // (first tile, weights requested early) every batch's code and
          // scale/zero loads first and then its NACT + 1 activation and
          // group-sum loads; later rounds: the DEPTH - 1 newer batches
          if (t == 0 && u < DEPTH - 1) wait_vm_first<SL::NI, SL::NACT + 1, DEPTH>(u);
          else wait_vm<SL::NI * (DEPTH - 1)>();
          wait_lgkm0();          // this wave's reads of the slot refilled below are done
          bar_nofence();
          // the next batch's loads go out at raised wave priority, ahead of
          // the other workgroup's arithmetic on the same SIMDs
          __builtin_amdgcn_s_setprio(3);
          issue(tau + DEPTH, slot[(u + DEPTH) % NSLOT]);
          __builtin_amdgcn_s_setprio(0);
          if (tau < ntau && rvalid && tlive) compute(slot[u]);
        }
      }
      // every load has landed and every wave is done with the ring before
      // the next tile (or the row stage) reuses it
      wait_vm<0>();
      wait_lgkm0();
      bar_nofence();
    }

    // 4-step tail stage (d_in % 256 == 128; then GS <= 4): direct loads
    // (two column tiles are only launched without it)
    if (NCT == 1 && tail && rvalid) {
      // addresses from opaque copies: computed here, not held across the ring
      const int st = nfull;
      const int lane_t = opaque(lane), lg_t = lane_t >> 4, arow_t = opaque(arow);
      const half_t* xrow = reinterpret_cast<const half_t*>(a.Xp) + (size_t)arow_t * a.d_in + 8 * lg_t;
      const float* srow = a.sums + (size_t)arow_t * ng * 2;
      // the tail group: 2-bit, 8 B per lane; 3-bit, three planes of 64 dwords
      u32x4 cd[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if constexpr (BITS == 3) {
          const uint32_t* tb = cbase[p] + st * 384;
          cd[p] = u32x4{tb[lane_t], tb[64 + lane_t], tb[128 + lane_t], 0u};
        } else {
          const u32x2 c2 = *reinterpret_cast<const u32x2*>(cbase[p] + st * 256 + lane_t * 2);
          cd[p] = u32x4{c2[0], c2[1], 0u, 0u};
        }
      }
      half8v bt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bt[j] = *reinterpret_cast<const half8v*>(xrow + (8 * st + j) * 32);
      f32x4 C[NP];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        u32x4 fr[NP][2];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          fr[p][0] = dec_raw<BITS>(2 * d, cd[p], cd[p][2], 0u);
          fr[p][1] = dec_raw<BITS>(2 * d + 1, cd[p], cd[p][2], 0u);
        }
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
              const u32x4 w = *reinterpret_cast<const u32x4*>(szb[p] + (size_t)g * 16 + 4 * lg_t);
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

    // Row stage U_m (Sigma p) as extra MFMA K-steps, p split into hi + lo
    // halves of the activation type: the gate/up projections of MODE_GATEUP,
    // and in MODE_RES the projection when P is given, done by the workgroups
    // of the first k-chunk.  P row of a column: its (tile column, token) pair
    // when ap_T > 0, else the slot's position.  The columns are the same for
    // every wave of a tile group, so Sigma p is gathered once per group:
    // every thread loads whole float4 runs of all split-K slabs at once
    // (slabs past the count read zeros), adds them in slab order and writes
    // hi/lo into slot c of the (drained) ring for tile c.  The U fragments of each wave
    // go out right after, in the same round trip.  Every address here
    // derives from an opaque copy of the thread id, so none of it is computed
    // ahead and held in registers across the ring.
    constexpr int RC = 4;                  // rank chunks of 32 (r_pad <= 128)
    constexpr int NTH = 64 * WR;           // threads of a tile group
    constexpr int IMAX = (16 * 32 + NTH - 1) / NTH;   // float4 runs per thread
    constexpr int SPMAX = (NP == 2) ? (IMAX > 1 ? 2 : 4) : (IMAX > 1 ? 4 : 16);   // slabs loaded together
    V8 uf[NP][RC];
    const bool rowstage = (MODE == MODE_GATEUP) || (ks == 0 && a.P[0] != nullptr && a.p[0].rank > 0);
    if (rowstage) {
      const int tid_e = opaque(tid) % NTH;  // thread of the tile group
      const int l16e = tid_e & 15, lge = (tid_e >> 4) & 3;
      T* sh = reinterpret_cast<T*>(wc == 0 ? s0 : s1);   // [NP][hi, lo][16 columns][r_pad + 8]
      const int tok = slotid / a.topk;
      const int ns = a.p_nsplit;
      f32x4 ld[NP][IMAX][SPMAX];
      int cix[NP][IMAX], kix[NP][IMAX];
      bool ok[NP][IMAX];
#pragma unroll
      for (int p = 0; p < NPG; ++p) {
        const ProjDev& pd = a.p[p];
        const int rp = pd.r_pad, q4 = rp >> 2;
        const int prow = (a.ap_T > 0) ? n_e[p] * a.ap_T + tok : pos;
        const int mycol = (cvalid && pd.rank > 0) ? prow : -1;
        const __amdgpu_buffer_rsrc_t rp4 = make_rsrc(a.P[p], OOB);
        const uint32_t slab = (uint32_t)a.p_rows_cap * rp * 4u;
#pragma unroll
        for (int j = 0; j < IMAX; ++j) {
          const int i = tid_e + j * NTH;
          ok[p][j] = pd.rank > 0 && i < 16 * q4;
          const int c = ok[p][j] ? i / q4 : 0;
          cix[p][j] = c;
          kix[p][j] = i - c * q4;
          const int col = __shfl(mycol, c, 64);   // lane c holds column c
          const bool live = ok[p][j] && col >= 0;
          const uint32_t vo = ((uint32_t)col * rp + 4 * kix[p][j]) * 4u;
#pragma unroll
          for (int sp = 0; sp < SPMAX; ++sp)
            ld[p][j][sp] = __builtin_bit_cast(f32x4, bload128(rp4, (live && sp < ns) ? vo + sp * slab : OOB, 0u));
          for (int sp = SPMAX; sp < ns; ++sp)       // more slabs than one batch: serial
            ld[p][j][SPMAX - 1] += __builtin_bit_cast(f32x4, bload128(rp4, live ? vo + sp * slab : OOB, 0u));
        }
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pp = PAIR ? 0 : p;
        const ProjDev& pd = a.p[pp];
        if (pd.rank == 0) continue;
        const int rp = pd.r_pad;
        const T* up = reinterpret_cast<const T*>(pd.U) +
                      ((size_t)m_e[pp] * a.d_out + rbp[p] * 16 + l16e) * rp + 8 * lge;
#pragma unroll
        for (int c = 0; c < RC; ++c)
          if (32 * c < rp) uf[p][c] = *reinterpret_cast<const V8*>(up + 32 * c);
      }
#pragma unroll
      for (int p = 0; p < NPG; ++p) {
        const int rps = a.p[p].r_pad + 8;
#pragma unroll
        for (int j = 0; j < IMAX; ++j) {
          if (!ok[p][j]) continue;
          f32x4 f = ld[p][j][0];
#pragma unroll
          for (int sp = 1; sp < SPMAX; ++sp) f += ld[p][j][sp];
          T hi[4], lo[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            hi[v] = from_f32<T>(f[v]);
            lo[v] = from_f32<T>(f[v] - to_f32(hi[v]));
          }
          T* d0 = sh + ((2 * p) * 16 + cix[p][j]) * rps + 4 * kix[p][j];
          *reinterpret_cast<u32x2*>(d0) = __builtin_bit_cast(u32x2, hi);
          *reinterpret_cast<u32x2*>(d0 + 16 * rps) = __builtin_bit_cast(u32x2, lo);
        }
      }
      __syncthreads();
    }

    if (rvalid) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[p][v] = ldexpf(acc[p][v] - corr[p][v], E);
      const int o = rb * 16 + 4 * lg;
      if (rowstage) {
        const T* sh = reinterpret_cast<const T*>(wc == 0 ? s0 : s1);
        const int tid_e = opaque(tid) % NTH;
        const int l16e = tid_e & 15, lge = (tid_e >> 4) & 3;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int pp = PAIR ? 0 : p;
          const ProjDev& pd = a.p[pp];
          if (pd.rank == 0) continue;
          const int rp = pd.r_pad, rps = rp + 8;
          const T* bh = sh + ((2 * pp) * 16 + l16e) * rps + 8 * lge;
#pragma unroll
          for (int c = 0; c < RC; ++c) {
            if (32 * c < rp) {
              acc[p] = mfma16(uf[p][c], *reinterpret_cast<const V8*>(bh + 32 * c), acc[p]);
              acc[p] = mfma16(uf[p][c], *reinterpret_cast<const V8*>(bh + 16 * rps + 32 * c), acc[p]);
            }
          }
        }
      }
      // output addresses from opaque copies: computed here, not held across the ring
      const int pos_e = opaque(pos), o_e = opaque(o);
      if constexpr (MODE == MODE_GATEUP) {
        if (cvalid) {
          T hv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) hv[v] = from_f32<T>(silu_f(acc[0][v]) * acc[1][v]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(a.h) + (size_t)pos_e * a.d_out + o_e) =
              __builtin_bit_cast(u32x2, hv);
        }
      } else if constexpr (PAIR) {
        if (cvalid) {
          const float g = a.gates[opaque(slotid)];
#pragma unroll
          for (int p = 0; p < NP; ++p)
            if (fvalid[p])
              *reinterpret_cast<f32x4*>(a.dres + ((size_t)ks * a.S + pos_e) * a.d_out + opaque(rbp[p] * 16 + 4 * lg)) =
                  acc[p] * g;
        }
      } else {
        if (cvalid) {
          const float g = a.gates[opaque(slotid)];
          *reinterpret_cast<f32x4*>(a.dres + ((size_t)ks * a.S + pos_e) * a.d_out + o_e) = acc[0] * g;
        }
      }
    }
    // slots 0 .. NCT-1 hold the gathered Sigma p until every wave has used it
    if (rowstage && t0 + 16 * NCT < cnt) __syncthreads();
  };
  tile(0);
  for (int t0 = 16 * NCT; t0 < cnt; t0 += 16 * NCT) tile(t0);
}

template <typename T, int MODE, int GS, int WAVES, int DMAX, int BITS, int NCT = 1>
static void dec_launch(const DecArgs& a, hipStream_t s) {
  constexpr int NP = dec_np<MODE>();
  constexpr int BYTES = DecSlot<NP, WAVES, 8 / GS, BITS, NCT>::BYTES;
  if constexpr (WAVES > 8 && ring_depth<BYTES, DMAX, false>() < 2) {
    // slots too large for a ring of three: fall back to 8 waves, one tile
    DecArgs b = a;
    b.nct = 1;
    dec_launch<T, MODE, GS, 8, DMAX, BITS>(b, s);
  } else {
    constexpr int WR = WAVES / NCT;
    DecArgs b = a;
    b.rows_per = (a.rows_per >= 1 && a.rows_per <= WR) ? a.rows_per : WR;
    const int nrb = b.d_out >> 4;
    const int nun = (MODE == MODE_RES2) ? (nrb + 1) >> 1 : nrb;   // row units
    const int nby = (nun + b.rows_per - 1) / b.rows_per;
    const dim3 grid(b.K * ((nby + 7) / 8) * 8 * b.nks);
    hipLaunchKernelGGL((gemm_dec_kernel<T, MODE, GS, WAVES, DMAX, BITS, NCT>), grid, dim3(64 * WAVES),
                       0, s, b);
  }
}

template <typename T, int MODE, int WAVES, int DMAX, int BITS, int NCT = 1>
static void dec_gs(const DecArgs& a, hipStream_t s) {
  switch (a.p[0].group >> 5) {
    case 1: dec_launch<T, MODE, 1, WAVES, DMAX, BITS, NCT>(a, s); break;
    case 2: dec_launch<T, MODE, 2, WAVES, DMAX, BITS, NCT>(a, s); break;
    case 4: dec_launch<T, MODE, 4, WAVES, DMAX, BITS, NCT>(a, s); break;
    default: dec_launch<T, MODE, 8, WAVES, DMAX, BITS, NCT>(a, s); break;
  }
}

template <typename T, int MODE, int BITS>
static void dec_waves(const DecArgs& a, hipStream_t s) {
  if constexpr (MODE == MODE_GATEUP && BITS == 2) {
    if (a.nct == 2 && decode_two_tiles_ok(2, a.p[0].group, a.p[0].bits, a.d_in)) {
      // two column tiles of 16 slots: two groups of waves share each
      // stage's codes (two 8-wave workgroups per CU, groups of 4 waves)
      if ((a.p[0].group >> 5) == 4) dec_launch<T, MODE, 4, 8, 6, BITS, 2>(a, s);
      else dec_launch<T, MODE, 8, 8, 6, BITS, 2>(a, s);
      return;
    }
  }
  if constexpr (MODE == MODE_GATEUP) {
    switch (a.waves) {
      case 16: dec_gs<T, MODE, 16, 6, BITS>(a, s); break;
      case 14: dec_gs<T, MODE, 14, 6, BITS>(a, s); break;
      case 12: dec_gs<T, MODE, 12, 6, BITS>(a, s); break;
      default: dec_gs<T, MODE, 8, 6, BITS>(a, s); break;
    }
  } else {
    if (a.waves == 16) dec_gs<T, MODE, 16, 6, BITS>(a, s);
    else dec_gs<T, MODE, 8, 6, BITS>(a, s);
  }
}

// Ring depth: as many slots as fit the LDS budget (at most 7).  With 16 waves
// a 2-bit gate/up slot holds 32 KB of codes (3 slots), a down / single slot
// 16 KB (5 slots); with 8 waves 16 resp. 8 KB (5 resp. 7 slots).  One
// workgroup per CU either way.  3-bit slots hold 1.5 times the codes.
template <int MODE, int BITS>
static bool dual_gs(int group) {
  switch (group >> 5) {
    case 1: return dec_dual_cfg<MODE, 1, 8, BITS>();
    case 2: return dec_dual_cfg<MODE, 2, 8, BITS>();
    case 4: return dec_dual_cfg<MODE, 4, 8, BITS>();
    default: return dec_dual_cfg<MODE, 8, 8, BITS>();
  }
}

// Two column tiles per workgroup (two groups of 4 or 8 waves) for gate/up
// with 2-bit codes, groups of 128 or 256 inputs (the instances that keep to
// the register budget) and no 4-step tail stage.  (The down projection's
// split-K launch measured slower with two tiles.)
bool decode_two_tiles_ok(int np, int group, int bits, int d_in) {
  return np == 2 && bits == 2 && (group == 128 || group == 256) && d_in % 256 == 0;
}

bool decode_dual(int np, int group, int bits) {
  if (bits == 3) return np == 2 ? dual_gs<MODE_GATEUP, 3>(group) : dual_gs<MODE_RES, 3>(group);
  return np == 2 ? dual_gs<MODE_GATEUP, 2>(group) : dual_gs<MODE_RES, 2>(group);
}

template <typename T>
static void dec_bits(const DecArgs& a, GemmMode mode, hipStream_t s) {
  if (a.p[0].bits == 3) {
    if (mode == MODE_GATEUP) dec_waves<T, MODE_GATEUP, 3>(a, s);
    else if (a.pair) dec_waves<T, MODE_RES2, 3>(a, s);
    else dec_waves<T, MODE_RES, 3>(a, s);
  } else {
    if (mode == MODE_GATEUP) dec_waves<T, MODE_GATEUP, 2>(a, s);
    else if (a.pair) dec_waves<T, MODE_RES2, 2>(a, s);
    else dec_waves<T, MODE_RES, 2>(a, s);
  }
}

void launch_gemm_decode(const DecArgs& a, GemmMode mode, Act act, hipStream_t s) {
  if (act == ACT_F16) dec_bits<half_t>(a, mode, s);
  else dec_bits<__bf16>(a, mode, s);
}

}  // namespace tq
