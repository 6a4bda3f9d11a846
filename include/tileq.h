/*
 * tileq.h -- C ABI of the MI355X (gfx950) TileQ MoE expert forward.
 *
 * Method: "TileQ: Efficient Low-Rank Quantization of Mixture-of-Experts with
 * 2D Tiling" (gist.science technical summary).
 *   - Section 2.1, step 4: the K experts of a projection are tiles of one
 *     block matrix W_big on an M x N grid.
 *   - Section 2.1, step 5, and "Key Technical Insight": W_big is factored
 *     once, U Sigma V^T; the experts of grid row m share the left (output
 *     space) block U_m, the experts of grid column n share the right (input
 *     space) block V_n, and each expert keeps a quantized residual.  So the
 *     weight of expert e at tile (m, n) is  W_e = U_m Sigma V_n^T + R_e.
 *   - Section 2.2 ("Efficient Fused Sparse Low-Rank Inference"): the forward
 *     takes the whole token batch and the routing weights, projects onto a
 *     shared factor once, applies routing weights in rank space through an
 *     in-place accumulation buffer, and multiplies by the other shared factor
 *     in one batched product.
 *
 * Two calls carry the method: tq_upload_proj() (the tile map, the shared
 * factors and the packed 2- or 3-bit residual of one projection) and tq_forward()
 * (token activations plus top-k routing).  Everything else is set-up,
 * workspace sizing and test hooks.
 *
 * Conventions for every call:
 *   - Every call returns a tq_status and never aborts across the ABI; the text
 *     of the last non-OK status of the calling thread is tq_last_error().
 *   - "DEVICE" pointers are device memory of the current HIP device; "HOST"
 *     pointers are read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Storage formats: f16 = IEEE binary16, bf16 = bfloat16 (both 2 bytes);
 *     integers little endian.
 */
#ifndef TILEQ_H
#define TILEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tq_layer tq_layer; /* opaque; owns the uploaded device weights */

/* The enumerations are 32-bit integers on both sides of the boundary; any
 * int32 value may be passed and out-of-range ones are rejected (C++ sees them
 * with a fixed int32_t underlying type, so such a value is well defined). */
#ifdef __cplusplus
#define TQ_ENUM(tag) enum tag : int32_t
#else
#define TQ_ENUM(tag) enum tag
#endif

typedef TQ_ENUM(tq_status_e) {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* invalid argument value (map, pointer, dtype, ...) */
  TQ_ESHAPE = 2,        /* shapes inconsistent or unsupported sizes          */
  TQ_ENOMEM = 3,        /* device allocation failed                          */
  TQ_EHIP = 4,          /* a HIP runtime call failed (text in last_error)    */
  TQ_EUNSUPPORTED = 5,  /* valid request this library does not implement     */
  TQ_ESTATE = 6         /* call order (e.g. forward before every upload)     */
} tq_status;

typedef TQ_ENUM(tq_dtype_e) { TQ_F16 = 0, TQ_BF16 = 1, TQ_F32 = 2, TQ_F64 = 3 } tq_dtype;

/* TQ_SINGLE: one projection  y_t = sum_j g_tj W_e x_t.
 * TQ_SWIGLU: gate, up and down projections,
 *            h = RND_act(silu(W_gate,e x) * (W_up,e x)),
 *            y_t = sum_j g_tj W_down,e h_tj  (+ optional dense shared expert). */
typedef TQ_ENUM(tq_kind_e) { TQ_SINGLE = 0, TQ_SWIGLU = 1 } tq_kind;

/* projection selectors */
#define TQ_P_SINGLE 0
#define TQ_P_GATE 0
#define TQ_P_UP 1
#define TQ_P_DOWN 2

/* One projection as stored after the offline quantization of section 2.1.
 * Sizes: K experts on an M x N grid (K <= M*N <= 1024, K <= 256, N <= 32),
 * d_in and d_out the projection's input and output widths, rank r >= 0,
 * residual group size G along d_in, code width `bits`.  Requirements:
 * d_in % 128 == 0, d_out % 16 == 0, G % 32 == 0, d_in % G == 0, r <= 128,
 * bits 2 or 3 (3: G a power of two, 32 .. 256).
 *   tile_of_expert HOST   int32 [K]: tile index m*N + n of each expert;
 *                         must be injective and in [0, M*N) (empty tiles allowed).
 *   U      DEVICE act   [M*d_out][r] row-major; block m = rows m*d_out ...
 *   sigma  DEVICE sigma_dtype [r] (the diagonal of Sigma, any order);
 *          sigma_dtype TQ_F16 or TQ_F32 (kept as f32 either way, exactly)
 *   V      DEVICE act   [N*d_in][r]  row-major; block n = rows n*d_in ...
 *   codes  DEVICE u32   bits 2: [K][d_out][d_in/16], the code of input i at
 *                       bits 2*(i%16) .. 2*(i%16)+1 of word i/16;
 *                       bits 3 (the pages' 3-bit setting, section 4):
 *                       [K][d_out][3*d_in/32], each row one little-endian
 *                       bit string with the code of input i at bits 3i ..
 *                       3i+2 (bit n = bit n%32 of word n/32)
 *   scales DEVICE f16   [K][d_out][d_in/G]   any finite value
 *   zeros  DEVICE f16   [K][d_out][d_in/G]   any finite value (fractional too)
 * The residual weight is R_e[o][i] = s[e][o][i/G] * (q[e][o][i] - z[e][o][i/G]).
 * The prefill kernels multiply fp16 weights RND_f16(fl32(fl32(q - z) * s)), so
 * that value must be finite for every code q of every group (checked).
 * U, V and sigma may be NULL when r == 0. */
typedef struct {
  int32_t K, M, N, d_in, d_out, rank, group, bits;
  const int32_t *tile_of_expert;
  const void *U;
  const void *sigma;
  int32_t sigma_dtype;
  const void *V;
  const uint32_t *codes;
  const uint16_t *scales;
  const uint16_t *zeros;
} tq_proj_desc;

/* Create an empty layer.  act: TQ_F16 or TQ_BF16, the dtype of activations, of
 * U and V and of the SwiGLU intermediate.  SINGLE: d_model = d_in,
 * d_ff = d_out of the one projection.  SWIGLU: gate/up are d_model -> d_ff,
 * down is d_ff -> d_model.  No device memory is touched.
 * Errors: TQ_EINVAL (bad kind/dtype, out == NULL), TQ_ESHAPE (sizes <= 0). */
tq_status tq_layer_create(tq_kind kind, tq_dtype act, int32_t d_model, int32_t d_ff,
                          int32_t K, tq_layer **out);

/* Call (1): upload one projection (TileQ technical summary, section 2.1 step 5
 * "Quantization": the global factors U, Sigma, V are kept once for the whole
 * grid and every expert keeps its own quantized residual).  The map is
 * validated on the host before any device work; the device arrays are copied
 * (and re-laid-out) into library-owned memory on `stream`; scales/zeros are
 * validated on the device, after which the call synchronizes `stream` and
 * returns.  The caller may free its arrays when the call returns.
 * Re-uploading a projection replaces it.
 * Errors: TQ_EINVAL (non-injective or out-of-range map, NULL pointers, bad
 * sigma_dtype, a scale or zero point that is not finite or whose dequantized
 * weight overflows fp16), TQ_ESHAPE (sizes inconsistent with the layer or the
 * requirements above), TQ_EUNSUPPORTED (bits other than 2 or 3; 3-bit codes with
 * a group size that is not a power of two from 32 to 256), TQ_ENOMEM, TQ_EHIP. */
tq_status tq_upload_proj(tq_layer *L, int32_t which, const tq_proj_desc *d, void *stream);

/* Optional dense shared expert, added to every token with weight 1 (SWIGLU
 * layers with act = TQ_F16 only): wg, wu DEVICE f16 [d_ff_shared][d_model],
 * wd DEVICE f16 [d_model][d_ff_shared]; d_ff_shared % 128 == 0.  Copied like
 * tq_upload_proj (re-laid-out in blocks of 32 inputs per row; the call
 * synchronizes `stream`, after which the caller may free its arrays).  Errors: TQ_EINVAL, TQ_ESHAPE, TQ_EUNSUPPORTED, TQ_ENOMEM, TQ_EHIP. */
tq_status tq_upload_shared_expert(tq_layer *L, int32_t d_ff_shared, const void *wg,
                                  const void *wu, const void *wd, void *stream);

/* Bytes of device workspace tq_forward needs for T tokens with top-k routing
 * (valid for both execution paths).  Errors: TQ_ESHAPE (T < 0, topk < 1 or
 * T*topk > 2^20), TQ_ESTATE (a projection not uploaded yet). */
tq_status tq_workspace_size(const tq_layer *L, int32_t T, int32_t topk, size_t *bytes);

/* Call (2): the forward (section 2.2) for T tokens.
 *   x        DEVICE act [T][d_in of the first projection]
 *   topk_ids DEVICE int32 [T][topk] expert ids; an id outside [0, K) makes
 *            that slot contribute nothing and is counted (see below)
 *   topk_w   DEVICE f32 [T][topk] routing weights, applied as given
 *   y        DEVICE y_dtype [T][d_out of the last projection]; written once,
 *            rounded to nearest-even from fp32 accumulation
 *   ws       DEVICE workspace of at least tq_workspace_size() bytes, 256-byte
 *            aligned.  After the call, ((int32_t*)ws)[0] holds the number of
 *            slots whose id was outside [0, K).
 * Only enqueues work on `stream`: no allocation, no synchronization, no read
 * back, so it can be captured in a HIP graph.  T == 0 is a no-op.  Buffers may
 * not overlap.  Calls on one layer must not run concurrently (issue them on
 * one stream, or order them): the layer owns the side stream of its shared
 * expert, the events that fork it from and join it into the caller's stream,
 * and the profiling events.  Calls on different layers may run concurrently
 * when they use distinct workspaces.
 * Errors (all checked before any launch): TQ_EINVAL (NULL pointers, y_dtype),
 * TQ_ESHAPE (T, topk, ws_bytes too small), TQ_ESTATE, TQ_EUNSUPPORTED
 * (T * d_model * 2 >= 2^31 bytes of activations; gate and up uploaded with
 * different code widths), TQ_EHIP (launch failure). */
tq_status tq_forward(const tq_layer *L, const void *x, int32_t T, const int32_t *topk_ids,
                     const float *topk_w, int32_t topk, void *y, tq_dtype y_dtype,
                     void *ws, size_t ws_bytes, void *stream);

/* Call (2) fed by router logits: the top-k router of tq_router_topk (below)
 * followed by tq_forward, in one call.  logits DEVICE f32 [T][K]; the routing
 * it produces is written to topk_ids (DEVICE int32 [T][topk]) and topk_w
 * (DEVICE f32 [T][topk]) -- bit-identical to tq_router_topk's -- and used by
 * the forward.  At decode batch sizes the router runs inside the first launch
 * of the forward (the workgroup that groups the slots by expert runs it just
 * before), so it costs no launch of its own; otherwise it is one launch ahead
 * of the routing.  Other arguments, results and errors as tq_forward, plus
 * TQ_ESHAPE for topk > min(K, 32). */
tq_status tq_forward_from_logits(const tq_layer *L, const void *x, int32_t T,
                                 const float *logits, int32_t topk, int32_t *topk_ids,
                                 float *topk_w, void *y, tq_dtype y_dtype, void *ws,
                                 size_t ws_bytes, void *stream);

/* Size of the static scratch array behind tq_forward_noalloc (64 MiB per GPU
 * the library runs on, held until the process ends). */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* tq_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels with the same arguments and results, minus the workspace,
 * which here is a file-scope device array of TQ_NOALLOC_SCRATCH_BYTES bytes
 * inside the library.  The call allocates nothing (no hipMalloc, no library
 * allocation).  Every call on one GPU shares that GPU's array and the array
 * keeps the last call's contents (the forward never needs it zeroed), so
 * calls that overlap in time on one GPU -- on any layers, from any thread or
 * stream -- race: the caller must order them.  The dropped-slot count of
 * tq_forward is not reported.  Errors: as tq_forward, plus TQ_ESHAPE when
 * tq_workspace_size(L, T, topk) exceeds TQ_NOALLOC_SCRATCH_BYTES (decode
 * batches and prefills of a few hundred tokens of the Mixtral- and
 * Qwen-MoE-shaped layers fit; larger prefills need tq_forward). */
tq_status tq_forward_noalloc(const tq_layer *L, const void *x, int32_t T,
                             const int32_t *topk_ids, const float *topk_w, int32_t topk,
                             void *y, tq_dtype y_dtype, void *stream);

/* Free the layer and its device memory (synchronizes the device first).
 * NULL is accepted. */
tq_status tq_layer_destroy(tq_layer *L);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char *tq_last_error(void);

/* ABI version (increments on incompatible changes). */
int32_t tq_abi_version(void);

/* ---- test hooks (exported and documented as such) ---------------------- */

/* Execution path: 0 = automatic (chosen on the host from T, topk and K),
 * 1 = decode kernels (16-slot tiles), 2 = prefill kernels (large tiles). */
tq_status tq_layer_set_path(tq_layer *L, int32_t path);

/* The execution path tq_forward takes for T tokens with top-k routing, as
 * written to *path: 1 = decode kernels (16-slot tiles, streaming residual
 * GEMV on MFMA), 2 = prefill kernels (grouped dequantizing GEMM).  The choice
 * depends on T * topk against K, the override above, the group sizes and the
 * size of the activations.  Errors: TQ_EINVAL, TQ_ESTATE, TQ_ESHAPE. */
tq_status tq_forward_path(const tq_layer *L, int32_t T, int32_t topk, int32_t *path);

/* Run only the routing/grouping step of tq_forward (the expert grouping of
 * section 2.2 that replaces per-token sparse dispatch) and copy its lists to
 * caller buffers (all DEVICE int32):
 *   cnt[K], off[K+1], perm[T*topk] (slots t*topk+j ordered by (expert, slot);
 *   entries past off[K] are unspecified), inv[T*topk] (position of each slot,
 *   -1 if dropped), col_off[N+1], col_tok[T*topk], slot2col[T*topk]: the
 *   unique (column n of the expert, token t) pairs of projection `which`
 *   sorted by (n, t), and each slot's index into them (-1 if dropped).
 * `which` must be TQ_P_GATE/TQ_P_UP (SWIGLU) or TQ_P_SINGLE.  ws as tq_forward. */
tq_status tq_debug_route(const tq_layer *L, int32_t which, const int32_t *topk_ids, int32_t T,
                         int32_t topk, void *ws, size_t ws_bytes, int32_t *cnt, int32_t *off,
                         int32_t *perm, int32_t *inv, int32_t *col_off, int32_t *col_tok,
                         int32_t *slot2col, void *stream);

/* Write the dequantized residual weights of one expert exactly as the forward
 * multiplies them: w_out DEVICE f16 [d_out][d_in],
 * w[o][i] = RND_f16(s * (q - z)) (one rounding of the exact product). */
tq_status tq_debug_dequant(const tq_layer *L, int32_t which, int32_t expert, void *w_out,
                           void *stream);

/* Top-k router feeding tq_forward (section 2.2 takes the routing weights of
 * the active experts as given; the pages name no router, this is the plain
 * top-k one).  For each of T rows of logits (DEVICE f32 [T][K]): the k
 * largest logits in descending order, ties to the lower expert id, NaN read
 * as -inf, written to ids (DEVICE int32 [T][k]); weights (DEVICE f32 [T][k])
 * = softmax over the k selected logits (uniform 1/k when the largest
 * selected logit is -inf).  Asynchronous on `stream`; no layer needed.
 * Errors: TQ_EINVAL (NULL pointer with T > 0), TQ_ESHAPE (T < 0, K outside
 * [1, 256], k outside [1, min(K, 32)]), TQ_EHIP. */
tq_status tq_router_topk(const float *logits, int32_t T, int32_t K, int32_t k, int32_t *ids,
                         float *weights, void *stream);

/* ---- offline packer ----------------------------------------------------- */

/* Dense expert weights in, one projection's stored form out (the input of
 * tq_upload_proj): TileQ technical summary, section 2.1 step 4 (the experts
 * are tiles of W_big; a tile without an expert is a zero block) and step 5
 * (a global low-rank decomposition of W_big approximated by Gaussian
 * sketching instead of a full SVD; the factors are stored; each expert's
 * residual is quantized).  All arithmetic in fp64 on the device:
 *   Y = W_big Omega, an orthonormal basis Q of range(Y) (power_iters times
 *   refined by Y = W_big (W_big^T Q)), the small SVD of B = Q^T W_big, the
 *   rank leading triplets stored as U, V (act) and sigma (f32); each expert's
 *   residual against those stored factors quantized by asymmetric
 *   round-to-nearest per group: s = RND_f16((mx - mn) / (2^bits - 1)) with
 *   mn = min(min w, 0), mx = max(max w, 0) (1 when 0), z = clamp(rint(-mn/s)),
 *   q = clamp(rint(w/s) + z).  (The pages quantize the residual with
 *   calibration-based GPTQ/GPTVQ; this is the calibration-free reading.)
 * Fields: sizes and requirements as tq_proj_desc (K <= M*N, injective map);
 *   sketch   columns of Omega (rank + oversampling), rank <= sketch <= 136
 *   power_iters >= 0; act TQ_F16 or TQ_BF16 (storage of U and V)
 *   tile_of_expert HOST int32 [K]
 *   W        DEVICE w_dtype [K][d_out][d_in], w_dtype F16, BF16, F32 or F64
 *   omega    DEVICE f64 [N*d_in][sketch] (the sketch's random numbers, given)
 *   outputs  DEVICE, caller-owned, in tq_proj_desc's layouts: U [M*d_out][rank]
 *            act, sigma [rank] f32 (descending), V [N*d_in][rank] act, codes,
 *            scales, zeros.
 * The call enqueues on `stream` and synchronizes it before returning.
 * Errors: TQ_EINVAL (NULL pointers, dtypes, map), TQ_ESHAPE (sizes, sketch,
 * ws_bytes), TQ_EUNSUPPORTED (bits), TQ_EHIP. */
typedef struct {
  int32_t K, M, N, d_in, d_out, rank, group, bits;
  int32_t sketch, power_iters;
  tq_dtype act;
  const int32_t *tile_of_expert;
  const void *W;
  tq_dtype w_dtype;
  const double *omega;
  void *U;
  float *sigma;
  void *V;
  uint32_t *codes;
  uint16_t *scales;
  uint16_t *zeros;
} tq_pack_desc;

/* Bytes of device workspace tq_pack_proj needs (fp64 sketch, basis and
 * Gram matrices, the fp64 stored factors, one expert's low-rank block).
 * Errors: as tq_pack_proj's size checks. */
tq_status tq_pack_workspace_size(const tq_pack_desc *d, size_t *bytes);
tq_status tq_pack_proj(const tq_pack_desc *d, void *ws, size_t ws_bytes, void *stream);

/* Copy the per-expert row bound of one projection to l1_out (HOST f32 [K]):
 * an upper bound on max_o sum_i |W_e[o][i]| of the effective weight
 * W_e = U_m Sigma V_n^T + R_e (section 2.1), the sum over the residual's
 * |s (q - z)| plus sum_r |U_m[o][r]| |sigma_r| sum_i |V_n[i][r]|, computed
 * in fp32 at upload (3e38 where that overflows or is NaN).  The
 * forward of bfloat16 SWIGLU layers at prefill scales its fp16 copy of the
 * intermediate h by a power of two derived from the gate and up bounds.
 * Synchronous.  Errors: TQ_EINVAL, TQ_ESTATE (not uploaded), TQ_EHIP. */
tq_status tq_debug_row_bound(const tq_layer *L, int32_t which, float *l1_out);

/* Stage timing for benchmarks: with profiling on, tq_forward records a HIP
 * event on `stream` before its first stage and after each of its stages
 * (pre-created events: the forward still allocates nothing).  Stage order:
 * 0 routing, 1 bf16 row exponents, 2 column stage of the input projection(s),
 * 3 residual GEMM of gate+up (SWIGLU) or of the single projection,
 * 4 column stage of down, 5 shared expert, 6 residual GEMM of down, 7 combine
 * (stages a layer does not run take ~0 ms).  tq_profile_read waits for the
 * last recorded forward and writes its 8 stage durations in ms.
 * Errors: TQ_EINVAL, TQ_ESTATE (read without a profiled forward), TQ_EHIP. */
tq_status tq_profile_enable(tq_layer *L, int32_t on);
tq_status tq_profile_read(const tq_layer *L, float *stage_ms);

/* Benchmark calibration, not part of the method: enqueue on `stream` one
 * plain streaming read of `bytes` bytes of DEVICE memory at `buf` (16-byte
 * loads over the whole grid; nothing is written in practice: `scratch` is a
 * DEVICE uint32 that the kernel may write only for one fixed data pattern).
 * Timing such launches gives the read bandwidth the device attains, the
 * practical ceiling beside the nominal HBM peak.
 * Errors: TQ_EINVAL (NULL pointer, buf or bytes not a multiple of 16), TQ_EHIP. */
tq_status tq_calibrate_read(const void *buf, size_t bytes, uint32_t *scratch, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TILEQ_H */
