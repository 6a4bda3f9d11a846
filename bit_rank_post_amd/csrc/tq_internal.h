// Internal declarations shared by the host runtime (tileq_host.cpp) and the
// gfx950 kernels (*.hip).  Plain structs of device pointers and sizes; no
// torch, no HIP types beyond hipStream_t.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq {

enum Act { ACT_F16 = 0, ACT_BF16 = 1 };

// Device image of one uploaded projection.
//   codes : repacked 2-bit codes, per expert nrb row blocks of 16 rows; within a
//           row block, step groups of 8 MFMA k-steps (32 inputs each, the last
//           group may hold 4); a group stores, for each of the 64 lanes, the
//           lane's codes of those steps contiguously (16 B, or 8 B in a 4-step
//           tail).  Lane l owns row 16*rb + l%16 and inputs 32*step + 8*(l/16)
//           + 0..7 of every step (the A-operand layout of
//           v_mfma_f32_16x16x32_f16).  Bit positions inside a dword: see
//           unpack16() in tq_device.h.
//   sz    : [K][nrb][ng][16] u32, scale bits | zero bits << 16 (fp16 each)
//   U     : [M*d_out][r_pad] act, r zero-padded to a multiple of 32
//   Vt    : [N][d_in/32][r_pad][32] act (V_n transposed per 32-input k-step,
//           zero-padded ranks)
//   sigma : [r_pad] f32, zero padded
struct ProjDev {
  int K, M, N, d_in, d_out, rank, r_pad, group, ng, nrb, nsteps;
  int bits;       // residual code width: 2, or 3 (codes in the 3-bit layout of
                  // repack_codes3_kernel, upload.hip)
  int deq_lut;    // 1: some scale or zero point is outside the packed dequantization's
                  // range (zero point not an integer in 0..3, or |s| >= 1024); the
                  // prefill kernels then dequantize through byte tables (deq_lut)
  uint32_t* codes;
  uint32_t* sz;
  void* U;
  void* Vt;
  float* sigma;
  int* m_of;
  int* n_of;
  float* l1max;   // [K] bound on max_o sum_i |W_e[o][i]| (effective weight)
};

struct SharedDev {
  int d_ff;       // 0: no shared expert
  void* wg;       // [d_ff][d_model] f16
  void* wu;
  void* wd;       // [d_model][d_ff] f16
};

// ---- routing --------------------------------------------------------------
struct RouteArgs {
  const int* ids;                // [T][k]; written by the router first when logits is set
  const float* logits;           // optional [T][K] router logits: top-k router fused in
                                 // front (one-workgroup routing only)
  float* gates_out;              // with logits: the routing weights [T][k]
  int T, k, S, K;
  int ncol;                      // column lists to build (1 single, 2 gate+up)
  const int* n_of[2];
  int N[2];
  int bm_gemm;                   // GEMM slot-tile height
  int rt_col;                    // column-stage row-tile height
  int* flags;                    // [0] = dropped slot count
  int* cnt;                      // [K]
  int* off;                      // [K+1]
  int* perm;                     // [S]
  int* inv;                      // [S]
  int* etab;                     // optional [K][S]: slot ids of expert e at e * S + c
  int* arec;                     // optional [K][ROUTE_AREC] + 1: active-expert records, see below
  int* tile_gemm;                // [K+1] prefix of ceil(cnt/bm_gemm)
  int* tile_colx;                // [K+1] prefix of ceil(cnt/rt_col) (down column stage)
  int* col_off[2];               // [N+1]
  int* col_tok[2];               // [S]
  int* slot2col[2];              // [S]
  int* tile_col[2];              // [N+1] prefix of ceil(col count/rt_col)
  int* cntw;                     // scratch chunk counts: [ceil(S/64)][K] (one-workgroup routing), [K][ceil(S/64)] (multi-workgroup)
  int* rank;                     // scratch [S]
  int* colmask;                  // scratch [2][T]
  int* wgcnt;                    // scratch [2][ceil(S/1024)][32] (multi-workgroup path)
  int* dropw;                    // scratch [ceil(S/1024)]
  unsigned* zero_init;           // optional region zeroed by the kernel
  int zero_n;
};
void launch_route(const RouteArgs& a, hipStream_t s);
// Active-expert record i (i < number of active experts, stored after the K
// records): expert id, slot count, offset, 0, slot ids of its first 16
// positions (entries past the count are stale).
constexpr int ROUTE_AREC = 20;

// ---- column stage: P[split][row][r] = sigma_r sum_{k in split} a_row[k] V_n[k][r]
struct ColArgs {
  const void* A;                 // activations, row stride lda
  int lda;
  const int* seg_off;            // [nseg+1] row offsets
  const int* tile_off;           // [nseg+1] tile prefix (rt rows per tile)
  const int* row_src;            // row -> activation row (nullptr: identity)
  const int* seg_vblk;           // segment -> V block (nullptr: segment id)
  int nseg;
  const void* Vt;
  int r_pad, d_in;
  int nsplit, steps_per_split;
  const float* sigma;            // [r_pad]: P holds Sigma (V_n^T a)
  float* P;
  int rows_cap;                  // rows per split slab
  int hilo;                      // 1 (nsplit 1 only): each row of P holds Sigma (V_n^T a)
                                 // as [high part | low part] in the activation dtype
  int ap_T;                      // > 0: every (column, token) pair, row = n * ap_T + t
                                 // (no work lists; seg_off/tile_off/row_src unused)
};
// prefill column stage (ap_T == 0; nsplit > 1 only for an fp32 P consumed
// by the combine: k-ranges over blockIdx.z, slab stride rows_cap rows):
// tiles of 128 rows (route rt_col 128)
void launch_colproj(const ColArgs* a, int nproj, int rt, int max_tiles, Act act,
                    hipStream_t s);
// compute units of the current device (cached per device id)
int device_cus();

// ---- residual grouped GEMM (+ low-rank K-extension, SwiGLU) ---------------
enum GemmMode { MODE_GATEUP = 0, MODE_RES = 1 };
struct GemmArgs {
  int K, d_in, d_out, topk, S;
  const void* A;                 // x [T][d_in] (gather by token) or h [S][d_in]
  int gather;                    // 1: row of slot = token of perm[pos]; 0: pos
  const int* perm;
  const int* off;
  const int* cnt;
  const int* tile_off;           // [K+1]
  const int* ex;                 // per-row exponent of converted bf16 rows, or nullptr
  // projections (1 for RES, 2 for GATEUP)
  ProjDev p[2];
  // low-rank extension (GATEUP): Sigma p rows of each projection as written
  // by the column stage with hilo set ([row][high r_pad | low r_pad] in the
  // activation dtype, p_rows rows) and the column-stage row of every slot
  const float* P[2];
  int p_rows;
  const int* slot2col[2];
  // outputs
  void* h;                       // GATEUP: [S][d_out] act
  // GATEUP, bfloat16 layers: also h * 2^-exh[pos] as fp16 (the operand of
  // down), exh from the weights' row bounds and the token's exponent ex
  void* h16;
  int* exh;
  float* dres;                   // RES: [S][d_out] f32 (gate weight applied)
  const float* gates;            // RES: topk weights [T*topk]
  int rows;                      // rows of A
  int narrow;                    // host: few slots per expert, use 64-slot halves
  int tile_half;                 // set by the launcher: 64-slot halves of 128-slot tiles
  int ntq;                       // set by the launcher: slot-tile units of the grid
};
// prefill grouped GEMM; A is fp16 (bfloat16 rows converted by rows_to_f16,
// exponents in ex); tiles of 128 slots (route bm_gemm = 128)
// (the kernels of each code width live in their own translation unit)
void launch_gemm_prefill_b2(const GemmArgs& a, GemmMode mode, Act act, int max_tiles,
                            hipStream_t s);
void launch_gemm_prefill_b3(const GemmArgs& a, GemmMode mode, Act act, int max_tiles,
                            hipStream_t s);
inline void launch_gemm_prefill(const GemmArgs& a, GemmMode mode, Act act, int max_tiles,
                                hipStream_t s) {
  if (a.p[0].bits == 3) launch_gemm_prefill_b3(a, mode, act, max_tiles, s);
  else launch_gemm_prefill_b2(a, mode, act, max_tiles, s);
}
// bfloat16 rows -> fp16 rows scaled by 2^-E, max|row| * 2^-E in [2^14, 2^15)
void launch_rows_to_f16(const void* X, int rows, int d, const int* row_src, int* ex,
                        void* Y, hipStream_t s);

// ---- decode streaming residual kernel --------------------------------------
struct DecArgs {
  int K, d_in, d_out, topk;
  const int* etab;               // [K][S] slot ids of each expert, in position order
  const int* off;
  const int* cnt;
  int gather;                    // 1: activation row of a slot = its token; 0: pos
  const void* Xp;                // class-scaled fp16 activations [rows][d_in]
  int rows;                      // rows of Xp / sums / ex
  const float* sums;             // [rows][d_in/G][2]: (X~_g, X'_g)
  const int* ex;                 // [rows] row exponent E
  ProjDev p[2];
  const float* P[2];             // column-stage results Sigma p, [rows][r_pad] (GATEUP)
  const int* slot2col[2];
  void* h;                       // GATEUP out [S][d_out] act
  float* dres;                   // RES out [nks][S][d_out] f32 (one slab per k-chunk)
  const float* gates;
  int nks;                       // k-chunks (RES; 1 for GATEUP)
  int S;                         // slots (slab stride of dres)
  int waves;                     // waves per workgroup: 8, 12, 14 or 16 (GATEUP), 8 or 16
  int rows_per;                  // waves that own a row unit: a 16-row fragment, or two with pair (<= waves / nct)
  int nct;                       // column tiles of 16 slots per pass: 1, or 2 (16 waves in two
                                 // groups of 8 sharing each stage's codes; no 4-step tail)
  int ap_T;                      // GATEUP: P rows are (column, token) pairs n * ap_T + t
  int p_nsplit, p_rows_cap;      // GATEUP: P slabs to add, rows per slab
  int pair;                      // RES: 1 = each wave takes two 16-row fragments (row units of 32 rows)
  int spec;                      // 1: request the first stages' codes before the routing reads return
  const int* arec;               // active-expert records (compact mapping) or nullptr
};
void launch_gemm_decode(const DecArgs& a, GemmMode mode, Act act, hipStream_t s);
// true when 8-wave decode workgroups of np projections, this group size and
// code width run two per CU
bool decode_dual(int np, int group, int bits);
// true when the decode kernel can take two 16-slot column tiles per
// workgroup for np projections of this group size, code width and d_in
bool decode_two_tiles_ok(int np, int group, int bits, int d_in);

// ---- activation preparation for the decode kernel ---------------------------
struct PrepArgs {
  const void* X;                 // [*][d] act
  int d, G;
  int bits;                      // code width of the projection reading the rows (class pattern)
  uint64_t cls_exp;              // set by the launcher: class exponents of that pattern
  const int* row_src;            // output row -> input row (nullptr: identity)
  void* Xp;                      // [rows][d] f16: x~ / c
  float* sums;                   // [rows][d/G][2]
  int* ex;                       // [rows]
};
// decode: activation preparation of `prep_rows` rows and the column stage of
// `ncol` projections (col_tiles 16-row tiles x slabs of 1024 inputs) in one
// launch; prep may be nullptr
void launch_prep_col(const PrepArgs* prep, int prep_rows, const ColArgs* col, int ncol,
                     int col_tiles, const RouteArgs* route, Act act, hipStream_t s);
// true when the decode companion launch can also run the routing (small batch)
bool prep_col_can_route(const RouteArgs& ra);
int decode_col_splits(int d_in);

// ---- combine: y_t = sum_j dres[inv(t,j)] + U_cat S_t (+ shared) ------------
struct CombineArgs {
  int T, topk, K, d_out, M, r_pad;
  const int* ids;
  const float* gates;
  const int* inv;
  const int* prow;               // slot -> row of P (inv for down, slot2col for single)
  int ap_T;                      // single projection, all-pairs P: row = n_of[e] * ap_T + t
  const int* n_of;
  const int* m_of;
  const float* P;
  int nsplit, rows_cap;
  const void* U;
  const float* dres;             // [nks][S][d_out]
  int nks, S;
  const float* ys;               // shared expert output [nys][T][d_out] f32 slabs or nullptr
  int nys;
  void* y;
  int y_dtype;                   // 0 f16, 1 bf16, 2 f32
};
void launch_combine(const CombineArgs& a, Act act, hipStream_t s);

// ---- dense fp16 shared expert --------------------------------------------
struct DenseArgs {
  int T, d_in, d_out;
  const void* X;                 // [T][d_in] f16
  const void* W0;                // [d_in / 32][d_out][32] f16 (k-step blocks, launch_block_rows)
  const void* W1;                // second weight (dual SwiGLU) or nullptr
  void* out_h;                   // dual: [T][d_out] f16
  float* out_f;                  // single: [T][d_out] f32
};
// dual: SwiGLU input (W0 gate, W1 up) -> out_h; else fp32 out_f in nsplit
// k-split slabs [nsplit][T][d_out]
void launch_dense(const DenseArgs& a, int dual, int nsplit, hipStream_t s);

// ---- upload-time kernels --------------------------------------------------
void launch_repack_codes(const uint32_t* src, uint32_t* dst, int K, int d_out, int d_in, int bits,
                         hipStream_t s);
void launch_pack_sz(const uint16_t* scales, const uint16_t* zeros, uint32_t* dst,
                    int K, int d_out, int ng, int bits, int* bad, hipStream_t s);
// per-expert bound on the effective weight's row sums of |W| (upload time)
struct RowBoundArgs {
  const uint32_t* codes;         // user layout [K][d_out][d_in/16]
  const uint16_t* scales;        // [K][d_out][d_in/G] f16
  const uint16_t* zeros;
  const void* U;                 // [M*d_out][r] activation dtype (r > 0)
  const float* sigma;            // [r]
  const void* V;                 // [N*d_in][r]
  const int* m_of;               // [K] device
  const int* n_of;
  int K, N, d_out, d_in, G, r, bf, bits;
  float* vn;                     // scratch [N][r]
  float* l1max;                  // [K], zero on entry
};
void launch_row_bound(const RowBoundArgs& b, hipStream_t s);
// top-k router: logits [T][K] (K <= 256) -> ids, weights [T][k] (k <= 32)
void launch_router_topk(const float* logits, int T, int K, int k, int* ids, float* w,
                        hipStream_t s);
void launch_pad_u(const void* U, void* dst, int rows, int r, int r_pad, hipStream_t s);
// sigma [r] as f16 (f16 = 1) or f32 -> [r_pad] f32, zero padded
void launch_sigma_to_f32(const void* src, int f16, float* dst, int r, int r_pad, hipStream_t s);
void launch_transpose_v(const void* V, void* dst, int N, int d_in, int r, int r_pad,
                        hipStream_t s);
// benchmark calibration: one plain streaming read of bytes (a multiple of 16)
void launch_stream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s);
// row-major f16 [rows][d_in] (d_in % 32 == 0) -> k-step blocks [d_in / 32][rows][32]
void launch_block_rows(const void* W, void* dst, int rows, int d_in, hipStream_t s);
void launch_debug_dequant(const ProjDev& p, int expert, void* w_out, hipStream_t s);

// ---- offline packer (pack.hip) -----------------------------------------------
struct PackArgs {
  int K, M, N, d_in, d_out, rank, group, bits;
  int l;                         // sketch width (rank + oversampling), <= 136
  int power_iters;
  int act_bf16;                  // U, V stored as bf16 (else fp16)
  const void* W;                 // [K][d_out][d_in] expert weights
  int wdt;                       // 0 f16, 1 bf16, 2 f32, 3 f64
  const int* tile_host;          // HOST [K] tile of each expert
  const int* emap_host;          // HOST [M*N] expert at each tile, -1 empty
  const double* omega;           // [N*d_in][l]
  void* U;                       // outputs in tq_proj_desc's layout
  float* sigma;
  void* V;
  uint32_t* codes;
  uint16_t* scales;
  uint16_t* zeros;
};
// enqueue the packer on s (the caller synchronizes before emap_host goes away)
void run_pack(const PackArgs& a, void* ws, hipStream_t s);
size_t pack_workspace_bytes(int M, int N, int d_in, int d_out, int r, int l);
constexpr int PACK_SKETCH_MAX = 136;

}  // namespace tq
