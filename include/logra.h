/*
 * logra.h -- C ABI of the LoGRA low-rank gradient-sketch library for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources cited below:
 *   [paper]   "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
 *             Sketches", paper text on paperpeel.com.
 *   [zh]      Chinese review of the paper (shibing624.github.io ai-paper-analysis).
 *   [ko]      Korean summary of the paper (onedev.kr).
 *   [rgc]     "Randomized Gradient Compression" blog (iluvatarlabs), "How it works"
 *             (a different method; used for the orientation of the contraction
 *             and the meaning of stochastic rounding only).
 *   [summary] paperlayer.ai section summary of the paper ("B. RowAdam", "D.1").
 *
 * For one selected linear weight W in R^{d x k} (out x in, row-major), with
 * layer input X [T x k] and backward derivative D [T x d] of a microbatch of
 * T tokens, the library computes
 *
 *   A      = sigma / sqrt(r), sigma in {+1,-1}^{r x k} from a counter-based
 *            generator keyed by (seed, matrix_id, step)       [paper] §2.1-2.2
 *   XAt    = X A^T                        [T x r]  fp32       [paper] §2.1
 *   S     += D^T XAt                      [d x r]  fp32       [paper] §2.1 (Eq. 2)
 *   U      = RowAdam(S) or S (SGD)        [d x r]  fp32       [summary] B
 *   q      = 1/(2|P| tau^2) sum_s Var_{p_s}[zdot_s]           [paper] §2.3 (Eq. 6)
 *   alpha  = min(alpha_max, sqrt(delta/q))                    [paper] §2.3, App. A.2
 *   W     <- round(W - scale * U A)       in place, bf16/fp32 [paper] §2.1-2.2
 *
 * Conventions (every entry point):
 *   - Matrices are row-major.  Device pointers are caller-owned device memory;
 *     the library never allocates or frees device memory except where an entry
 *     point says so.  Workspace arguments are caller-allocated device memory
 *     of at least the size the matching *_ws_bytes() query returns.
 *   - Every device call is asynchronous on the caller's stream (NULL = the
 *     default stream); outputs are valid once that stream has synchronised.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation failure nothing is launched and a status other than
 *     LOGRA_OK is returned.  logra_last_error() gives a message for the
 *     calling thread's most recent failure.  No C++ exception crosses the ABI.
 *   - Alignment: X, D and W base pointers must be 16-byte aligned and their
 *     leading dimensions (in elements) must make every row start 16-byte
 *     aligned; XAt, S, U, v, z and zdot must be 16-byte aligned.
 *   - Results are deterministic: the same input bits and shapes give the same
 *     output bits, run after run; no floating-point atomics are used.
 *
 * Generator (this library's choice -- the pages fix only that A is
 * regenerated from a seed and metadata, [paper] §2.2 "Memory and
 * synchronization"): the Philox family (Salmon et al., SC'11).
 *   key of a projection      = (seed, (step << 32) | matrix_id)
 *   sign of A[j, l]          = bit (l & 31) of word ((l & 127) >> 5) of
 *                              Philox4x32-10 with 32-bit counter words
 *                              (l >> 7, j | 2^31, matrix_id, step) under the
 *                              32-bit key words (seed & 0xFFFFFFFF, seed >> 32);
 *                              1 -> -1
 *   stochastic-rounding draw = for element e = (row0 + i) * k + l of W, the
 *                              16 bits [16*(e & 1), +16) of word ((e & 7) >> 1)
 *                              of Philox4x32-10 with 32-bit counter words
 *                              (g & 0xFFFFFFFF, g >> 32, matrix_id, step),
 *                              g = e >> 3, under the 32-bit key words
 *                              (sr_seed & 0xFFFFFFFF, sr_seed >> 32)
 */
#ifndef LOGRA_H_
#define LOGRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOGRA_API __attribute__((visibility("default")))

/* Opaque stream handle: a hipStream_t (NULL = default stream). */
typedef void* logra_stream;

typedef enum logra_status {
  LOGRA_OK = 0,
  LOGRA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  LOGRA_ERR_SHAPE = 2,     /* a size is out of range or inconsistent             */
  LOGRA_ERR_DTYPE = 3,     /* unsupported element type or type combination       */
  LOGRA_ERR_ALIGN = 4,     /* pointer or leading dimension breaks 16-B alignment */
  LOGRA_ERR_ALIAS = 5,     /* output overlaps an input it must not overlap      */
  LOGRA_ERR_DOMAIN = 6,    /* scalar out of its domain (q<0, NaN, delta<=0, ...) */
  LOGRA_ERR_HIP = 7,       /* the HIP runtime reported an error                  */
  LOGRA_ERR_WORKSPACE = 8, /* workspace or packed buffer missing or too small    */
  LOGRA_ERR_HOST = 9        /* host-side failure inside the call (out of host
                               memory); nothing was launched                     */
} logra_status;

typedef enum logra_dtype {
  LOGRA_F32 = 0,   /* IEEE binary32                           */
  LOGRA_BF16 = 1,  /* bfloat16 (top half of a binary32)       */
  LOGRA_I8 = 2     /* int8, used only for the signs of A      */
} logra_dtype;

typedef enum logra_round {
  LOGRA_ROUND_NEAREST = 0,    /* round to nearest, ties to even               */
  LOGRA_ROUND_STOCHASTIC = 1  /* deterministic stochastic rounding (bf16 W)   */
} logra_round;

/* Identifies one projection A: [paper] §2.2 -- each matrix has its own A,
 * refreshed every update; a fixed basis keeps `step` constant. */
typedef struct logra_key {
  uint64_t seed;
  uint32_t matrix_id;
  uint32_t step;
} logra_key;

/* Largest supported rank r (register-resident accumulators). */
#define LOGRA_MAX_RANK 256

/* ---------------------------------------------------------------- helpers */

/* Library version string (static storage). */
LOGRA_API const char* logra_version(void);

/* Message for the calling thread's last failed call ("" if none). */
LOGRA_API const char* logra_last_error(void);

/* Bytes of one fp32 sketch, 4*d*r: [paper] §2.2 "Memory and synchronization"
 * (d = k = 4096, r = 64 gives 1 MiB against 64 MiB dense).  Returns -1 for
 * negative sizes. */
LOGRA_API int64_t logra_sketch_bytes(int64_t d, int64_t r);

/* ------------------------------------------------------------- projection */

/* Materialise A [r x k] (row-major, contiguous) for `key`.
 * out = LOGRA_I8: A[j,l] = sigma (+1/-1, int8).
 * out = LOGRA_F32: A[j,l] = sigma * fl32(1/sqrt(r)).
 * Bit-identical to the A used inside logra_project_input and logra_merge.
 * Sources: [paper] §2.1 (A in R^{r x k}), §2.2 (regenerated from its seed);
 * [zh], [ko] (entries +-1/sqrt(r)).
 * Errors: NULL key/A; r < 1, r > LOGRA_MAX_RANK, k < 1; out not I8/F32. */
LOGRA_API int logra_regen_A(const logra_key* key, int64_t r, int64_t k,
                            logra_dtype out, void* A, logra_stream stream);

/* XAt [T x r] = X [T x k] A^T, overwritten (fp32, contiguous, ld = r).
 * X is bf16 or fp32 with leading dimension ldx >= k.  [paper] §2.1: the
 * inputs of the weight-gradient product are projected before they meet the
 * backward derivatives; [rgc] the layer keeps X A^T instead of X.
 * Errors: NULL pointers; T < 1, k < 1, r < 1, r > LOGRA_MAX_RANK, ldx < k;
 * alignment; XAt overlapping X. */
LOGRA_API int logra_project_input(const logra_key* key, int64_t T, int64_t k, int64_t r,
                                  const void* X, logra_dtype x_dtype, int64_t ldx,
                                  float* XAt, logra_stream stream);

/* ------------------------------------------------------------ diagnostic */

/* Workspace bytes of logra_reconstruction_cosine (0 for invalid sizes). */
LOGRA_API size_t logra_reconstruction_cosine_ws_bytes(int64_t d, int64_t k, int64_t r);

/* How much of a dense gradient the sketch keeps: the Frobenius cosine
 * between G [d x k] and its reconstruction (G A^T) A, A from `key` ([paper]
 * App. D.3 "Reconstruction heatmaps"; Fig. 5 reports 0.046 at r = 4 up to
 * 0.348 at r = 256 for Qwen2.5-1.5B gradients).  Written to out_dev (4
 * doubles on the device): {cos, ||G||_F^2, ||G A^T||_F^2, ||(G A^T) A||_F^2}.
 * Computed as ||S||^2 / (||G|| sqrt(sum_i S_i (A A^T) S_i^T)) with
 * S = G A^T from the projection (bf16 G on matrix cores, fp32 G in fp64)
 * and A A^T exact from the sign bits; sums in fp64, fixed order.  G is bf16
 * or fp32 with leading dimension ldg >= k.  The dense G exists only for this
 * diagnostic; the method never forms it.
 * Errors: NULL pointers; d < 1, k < 1, r < 1, r > LOGRA_MAX_RANK, ldg < k;
 * alignment; workspace too small; G, output and workspace overlapping. */
LOGRA_API int logra_reconstruction_cosine(const logra_key* key, int64_t d, int64_t k, int64_t r,
                                          const void* G, logra_dtype g_dtype, int64_t ldg,
                                          double* out_dev, void* ws, size_t ws_bytes,
                                          logra_stream stream);

/* ------------------------------------------ Gaussian projection variant */

/* The Gaussian projection the pages ablate against Rademacher signs
 * ([paper] §3.4.1, App. D.3; Fig. 5: the mean reconstruction cosine drops by
 * less than 2e-4): A[j][l] = fl32(z / sqrt(r)), z standard normal by
 * Box-Muller (1958) on the same Philox stream -- for row j and 4-column group
 * c = l >> 2 the block with counter (j, c, 2, 0) gives words w0..w3, uniforms
 * u_i = ((w_i >> 11) + 1/2) 2^-53, and z = sqrt(-2 ln u0) cos(2 pi u1),
 * sqrt(-2 ln u0) sin(2 pi u1), sqrt(-2 ln u2) cos(2 pi u3), sqrt(-2 ln u2)
 * sin(2 pi u3) for columns 4c .. 4c + 3 (fp64, rounded once).  A [r x k] fp32
 * row-major.  Unlike the signs, these entries are not exact in bf16, so
 * projections with an explicit A carry it as bf16 hi + lo.
 * Errors: NULL pointers; k < 1, r < 1, r > LOGRA_MAX_RANK; alignment. */
LOGRA_API int logra_regen_A_gaussian(const logra_key* key, int64_t r, int64_t k, float* A,
                                     logra_stream stream);

/* Bytes of an explicit projection packed as the projection kernel's B
 * operands: for each 256-column block, 32-column step and 16-rank block
 * (rank blocks padded to 1, 2, 4, 6, 8, 12 or 16), a 1 KiB hi operand then a
 * 1 KiB lo operand in which lane l holds rank 16nb + (l & 15), columns
 * 256b + 32s + 8(l >> 4) .. +7.  0 for invalid sizes. */
LOGRA_API size_t logra_projection_packed_bytes(int64_t r, int64_t k);

/* Pack an explicit A [r x k] (fp32 row-major) into that form (hi = RNE(a),
 * lo = RNE(a - hi); padding zero).
 * Errors: NULL pointers; k < 1, r < 1, r > LOGRA_MAX_RANK; packed_bytes too
 * small; alignment; A overlapping the packed output. */
LOGRA_API int logra_pack_projection(int64_t r, int64_t k, const float* A, void* A_packed,
                                    size_t packed_bytes, logra_stream stream);

/* XAt = X A^T with an explicit projection (packed as above) instead of the
 * key's signs, written as fp32 [T x r] (XAt) and/or in the accumulate's
 * packed input form (planes, logra_packed_input_bytes(T, r) bytes); either
 * may be NULL but not both.  X bf16.  [paper] §2.1.
 * Errors: NULL pointers; T < 1, k < 1, r < 1, r > LOGRA_MAX_RANK, ldx < k;
 * X not bf16; sizes; alignment; outputs overlapping an input or each other. */
LOGRA_API int logra_project_input_explicit(int64_t T, int64_t k, int64_t r, const void* X,
                                           logra_dtype x_dtype, int64_t ldx, const void* A_packed,
                                           size_t packed_bytes, float* XAt, void* planes,
                                           size_t planes_bytes, logra_stream stream);

/* logra_reconstruction_cosine with an explicit projection: A (fp32) for the
 * exact A A^T and A_packed (its packed form) for G A^T.  G bf16.  Same
 * output and workspace as logra_reconstruction_cosine.
 * Errors: as logra_reconstruction_cosine; G not bf16; packed_bytes too small. */
LOGRA_API int logra_reconstruction_cosine_explicit(int64_t d, int64_t k, int64_t r, const void* G,
                                                   logra_dtype g_dtype, int64_t ldg, const float* A,
                                                   const void* A_packed, size_t packed_bytes,
                                                   double* out_dev, void* ws, size_t ws_bytes,
                                                   logra_stream stream);

/* ---------------------------------------------------------------- sketch */

/* Workspace bytes one logra_sketch_accumulate call (or one descriptor of a
 * grouped call) needs for bf16 D: XAt repacked as two bf16 terms (hi, lo) in
 * matrix-core operand order, ranks padded to 32, 64, 128 or 256 and tokens
 * to 16.  d is accepted for future layouts and does not change the
 * size today.  A multiple of 256 bytes; 0 for invalid sizes. */
LOGRA_API size_t logra_sketch_accumulate_ws_bytes(int64_t T, int64_t d, int64_t r);

/* S [d x r] += D^T XAt for one microbatch (fp32 accumulate; G = D^T X is
 * never formed).  D [T x d] is bf16 or fp32 with leading dimension ldd >= d;
 * XAt [T x r] fp32 contiguous; S [d x r] fp32 contiguous, read and written.
 * The caller zeroes S at the start of each update.  [paper] §2.1 (S = G A^T,
 * accumulated per microbatch in fp32), [rgc] "How it works" (C += D^T (X P)).
 * bf16 D runs on bf16 MFMA with XAt split into two bf16 terms (hi + lo), which
 * needs the workspace above (ignored for fp32 D, may be NULL then).  The
 * summation order is a function of T and r alone: the 16-token steps s are
 * dealt to classes by s mod c (c = 4 for r <= 64, 2 for r <= 128, else 1);
 * each class sums its steps in ascending order (hi term, then lo term, per
 * step) and S receives S + ((Q0 + Q1) + (Q2 + Q3)), S + (Q0 + Q1) or
 * S + Q0 -- so a grouped call gives the same bits as single calls.
 * Errors: NULL pointers; T < 1, d < 1, r < 1, r > LOGRA_MAX_RANK, ldd < d;
 * alignment; S or the workspace overlapping an operand; workspace too small. */
LOGRA_API int logra_sketch_accumulate(int64_t T, int64_t d, int64_t r,
                                      const void* D, logra_dtype d_dtype, int64_t ldd,
                                      const float* XAt, float* S, void* ws, size_t ws_bytes,
                                      logra_stream stream);

/* One matrix of a grouped accumulate. */
/* One projection of logra_project_input_table. */
typedef struct logra_project_desc {
  logra_key key;     /* key of this projection's A                          */
  const void* X;     /* [T x k] bf16, row-major, leading dimension ldx      */
  int64_t k;
  int64_t ldx;
  float* XAt;        /* [T x r] fp32 contiguous, or NULL                    */
  void* planes;      /* packed projected input, or NULL                     */
  size_t planes_bytes; /* bytes available at planes: at least
                          logra_packed_input_bytes(T, r) when planes is set */
} logra_project_desc;

#define LOGRA_MAX_PROJECT_TABLE 1024

/* Workspace bytes of logra_project_input_table for n projections (the table
 * the kernel reads and an item counter); 0 for n out of range. */
LOGRA_API size_t logra_project_input_table_ws_bytes(int n);

/* logra_project_input_packed for up to LOGRA_MAX_PROJECT_TABLE projections
 * sharing T and r (e.g. every projection of every layer for one microbatch)
 * in one persistent launch ([paper] Sec. 2.1; [rgc] "How it works").  Each
 * descriptor gets XAt (fp32) and/or its packed planes.  The work items are
 * (projection group, two 16-token steps), the groups ordered widest X first
 * (so the launch ends on its shortest items); each wave of the grid computes
 * one item whole (all k columns, all ranks) and takes the next unclaimed one
 * from a counter in the workspace, so projections of any width mix without
 * idle compute units.  The outputs do not depend on the order.  Summation order: for each token and rank,
 * the 256-column blocks in ascending order, each block's 32-column MFMA
 * steps in order; deterministic, and equal to logra_project_input_packed's
 * result up to the last bits (that call adds its column blocks in eight
 * interleaved partial sums).  Several descriptors may share one X;
 * consecutive descriptors with the same X, k and ldx (up to three, at
 * r <= 64) are projected together, reading X once, with each projection's
 * sums formed as they would be alone (the same bits either way).  The
 * descriptor array is read on the host during the call and copied, with the
 * zeroed counter, into the workspace on the stream; calls that share a
 * workspace must not overlap in time.
 * Errors: NULL pointers or a descriptor without outputs; T < 1, k < 1, r out
 * of range, ldx < k, n out of range; alignment (X rows, outputs 16 bytes);
 * workspace too small; two outputs overlapping, or an output or the
 * workspace overlapping any X. */
LOGRA_API int logra_project_input_table(int64_t T, int64_t r, const logra_project_desc* descs,
                                        int n, void* ws, size_t ws_bytes, logra_stream stream);

typedef struct logra_acc_desc {
  const void* D;       /* [T x d], row-major, leading dimension ldd */
  const float* XAt;    /* [T x r] fp32 contiguous                    */
  float* S;            /* [d x r] fp32 contiguous                    */
  int64_t d;
  int64_t ldd;
} logra_acc_desc;

#define LOGRA_MAX_GROUP 16

/* Grouped form: n <= LOGRA_MAX_GROUP accumulates that share T, r and the
 * dtype of D, in one launch (e.g. the seven projections of one layer for one
 * microbatch).  Same result bits as n separate logra_sketch_accumulate calls.
 * The descriptor array is read on the host during the call.  For bf16 D the
 * workspace holds n consecutive per-descriptor workspaces, descriptor i's of
 * logra_sketch_accumulate_ws_bytes(T, descs[i].d, r) bytes, in order.
 * Errors: as logra_sketch_accumulate for each descriptor; n < 1 or
 * n > LOGRA_MAX_GROUP; two descriptors writing overlapping S. */
LOGRA_API int logra_sketch_accumulate_grouped(int64_t T, int64_t r, logra_dtype d_dtype,
                                              const logra_acc_desc* descs, int n,
                                              void* ws, size_t ws_bytes,
                                              logra_stream stream);

/* ------------------------------------------------- packed projected input */

/* Bytes of the packed projected input for T tokens and rank r: XAt as two
 * bf16 terms (hi = RNE(x), lo = RNE(x - hi)) in the matrix-core operand
 * order the accumulate reads -- for each 16-token step and 32-rank block, a
 * 1 KiB hi operand and a 1 KiB lo operand in which 16-byte lane l holds
 * tokens 8(l>>5) .. +7 of the step for rank 32b + (l & 31); ranks padded as
 * for logra_sketch_accumulate_ws_bytes, padding zero.  0 for invalid sizes. */
LOGRA_API size_t logra_packed_input_bytes(int64_t T, int64_t r);

/* logra_project_input writing its result straight in the packed form above
 * (and, when XAt is not NULL, also as fp32 [T x r]), so the accumulate
 * needs no repacking pass.  Same projection as logra_project_input ([paper]
 * §2.1, §2.2); X must be bf16.  planes needs logra_packed_input_bytes(T, r)
 * bytes, 16-byte aligned.
 * Errors: as logra_project_input; X not bf16; planes NULL, too small,
 * misaligned or overlapping X or XAt. */
LOGRA_API int logra_project_input_packed(const logra_key* key, int64_t T, int64_t k, int64_t r,
                                         const void* X, logra_dtype x_dtype, int64_t ldx,
                                         float* XAt, void* planes, size_t planes_bytes,
                                         logra_stream stream);

typedef struct logra_acc_packed_desc {
  const void* D;            /* [T x d] bf16, row-major, leading dimension ldd */
  const uint16_t* planes;   /* packed projected input of this matrix          */
  float* S;                 /* [d x r] fp32 contiguous                         */
  int64_t d;
  int64_t ldd;
  size_t planes_bytes;      /* bytes available at planes: at least
                               logra_packed_input_bytes(T, r)                 */
} logra_acc_packed_desc;

/* logra_sketch_accumulate_grouped for bf16 D with the projected inputs
 * already packed (by logra_project_input_packed): the same result bits, one
 * kernel, no workspace.  Several descriptors may share one packed input.
 * Errors: NULL pointers; T < 1, d < 1, r out of range, ldd < d; alignment;
 * planes_bytes below logra_packed_input_bytes(T, r) (LOGRA_ERR_WORKSPACE);
 * S overlapping D, a packed input or another S; n out of range. */
LOGRA_API int logra_sketch_accumulate_grouped_packed(int64_t T, int64_t r,
                                                     const logra_acc_packed_desc* descs, int n,
                                                     logra_stream stream);

/* Workspace bytes of logra_sketch_accumulate_table for n matrices (the
 * matrix table the kernel reads and eight tile counters). */
LOGRA_API size_t logra_sketch_accumulate_table_ws_bytes(int n);

/* logra_sketch_accumulate_grouped_packed over any number of matrices in one
 * persistent launch (e.g. all projections of all layers for one
 * microbatch).  The matrices' 256-column tiles, in descriptor order, are cut
 * into eight contiguous ranges, one per XCD; the blocks resident on an XCD
 * take its range's tiles in turn from a counter in the workspace, so the
 * tiles of one matrix run close together on one XCD and share its L2 copy of
 * the packed input, and the compute units one layer's tiles leave idle and
 * the ramp of separate launches are shared by the whole table.  Each tile is
 * computed whole by one block in the documented summation order, so S has
 * the same bits as with grouped or single calls.  The descriptor array is
 * read on the host during the call and copied, with the zeroed counters,
 * into the workspace on the stream; calls that share a workspace must not
 * overlap in time.
 * Errors: as logra_sketch_accumulate_grouped_packed for each descriptor;
 * n < 1; workspace too small or misaligned; two sketches overlapping, or a
 * sketch or the workspace overlapping another descriptor's operands. */
LOGRA_API int logra_sketch_accumulate_table(int64_t T, int64_t r, const logra_acc_packed_desc* descs,
                                            int n, void* ws, size_t ws_bytes, logra_stream stream);

/* ------------------------------------------------------------- optimiser */

/* Workspace bytes logra_rowadam needs for d rows. */
LOGRA_API size_t logra_rowadam_ws_bytes(int64_t d);

/* RowAdam ([summary] B; [paper] App. D.1 Table 4: beta2, no first moment,
 * relative eps).  With t the 1-based index of this update:
 *   m_i = sum_j S_ij^2;  v_i <- beta v_i + (1-beta) m_i;  vh_i = v_i/(1-beta^t)
 *   rho = sqrt(mean_i vh_i);  Ut_ij = S_ij / (sqrt(vh_i) + eps*rho)
 *   U = Ut * ||S||_F / ||Ut||_F   (U = 0 when Ut = 0)
 * S [d x r], U [d x r] fp32 contiguous (U may equal S: in place); v [d]
 * fp32, read and written.  beta and eps are taken in fp64 (0.999 in fp32
 * would move 1 - beta by 1.3e-5).  Reductions run in fp64 in a fixed order.
 * Errors: NULL pointers; d < 1, r < 1; t < 1; beta not in [0,1); eps < 0 or
 * non-finite; workspace too small; U partially overlapping S. */
LOGRA_API int logra_rowadam(int64_t d, int64_t r, const float* S, float* v, int64_t t,
                            double beta, double eps, float* U, void* ws, size_t ws_bytes,
                            logra_stream stream);

/* -------------------------------------------------------- step control */

/* Workspace bytes logra_predicted_kl_q needs for P contexts of V logits. */
LOGRA_API size_t logra_predicted_kl_q_ws_bytes(int64_t P, int64_t V);

/* q = 1/(2 P tau^2) * sum_s Var_{v ~ softmax(z_s/tau)}[zdot_s,v], written to
 * q_dev (one float on the device).  z, zdot [P x V] row-major contiguous,
 * bf16 or fp32 (same dtype).  A logit of -inf marks a masked entry
 * (probability 0); each context needs at least one finite logit.  zdot must
 * be finite.  [paper] §2.3 (Eq. 6), App. A.1.
 * Errors: NULL pointers; P < 1, V < 1; tau not finite and > 0; workspace too
 * small. */
LOGRA_API int logra_predicted_kl_q(int64_t P, int64_t V, const void* z, const void* zdot,
                                   logra_dtype dtype, float tau, float* q_dev,
                                   void* ws, size_t ws_bytes, logra_stream stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): logra_predicted_kl_q
 * with no workspace argument, the same result bits.  The partial moments go to
 * a scratch array the library holds on each GPU (LOGRA_NOALLOC_MAX_CONTEXTS
 * contexts, 512 bytes each: 2 MiB per GPU, held until the process ends); its
 * device address is looked up once per device, on the first call there.  The
 * call allocates nothing.  Calls on one GPU share that array, so calls that
 * overlap in time on one GPU (on two streams, or from two threads) race;
 * calls in one stream, or on different GPUs, do not.
 * Errors: as logra_predicted_kl_q; P > LOGRA_NOALLOC_MAX_CONTEXTS
 * (LOGRA_ERR_SHAPE); the scratch address unavailable (LOGRA_ERR_HIP). */
#define LOGRA_NOALLOC_MAX_CONTEXTS 4096
LOGRA_API int logra_predicted_kl_q_noalloc(int64_t P, int64_t V, const void* z, const void* zdot,
                                           logra_dtype dtype, float tau, float* q_dev,
                                           logra_stream stream);

/* Workspace bytes of logra_exact_kl for P contexts. */
LOGRA_API size_t logra_exact_kl_ws_bytes(int64_t P);

/* The finite-difference check of the predicted KL: the mean over the P
 * contexts of KL(softmax(z_s/tau) || softmax((z_s + alpha zdot_s)/tau)),
 * logits linear in the step ([paper] §2.3, Eq. 5 approximates it by
 * alpha^2 q; App. A.1).  Written to out_dev (one double on the device).
 * Evaluated per context as log E_p[exp(c (zdot - E_p[zdot]))], c = alpha/tau,
 * through log1p/expm1 in fp64, so small steps keep their digits.  z, zdot as
 * for logra_predicted_kl_q.
 * Errors: NULL pointers; P < 1, V < 1; tau not finite and > 0; alpha not
 * finite; workspace too small. */
LOGRA_API int logra_exact_kl(int64_t P, int64_t V, const void* z, const void* zdot,
                             logra_dtype dtype, double alpha, double tau, double* out_dev,
                             void* ws, size_t ws_bytes, logra_stream stream);

/* alpha = min(alpha_max, sqrt(delta / q)) on the host (fp64); q = 0 gives
 * alpha_max.  [paper] §2.3 and App. A.2 (root restored from alpha^2 q <= delta;
 * [zh], [ko]).  Errors: NULL alpha; q < 0 or NaN, delta <= 0, alpha_max <= 0
 * (LOGRA_ERR_DOMAIN). */
LOGRA_API int logra_step_alpha(double q, double delta, double alpha_max, double* alpha);

/* KL budget of update u (1-based) on a cosine schedule over H updates
 * ([paper] App. D.1 "KL budget", Table 4: 2e-4 down to 2e-5 over H = 300):
 *   delta_u = delta_min + (delta_max - delta_min)/2 * (1 + cos(pi (u-1)/(H-1)))
 * for u <= H, held at delta_min afterwards ([paper] App. D.2: annealed over
 * the horizon, then held constant).  Host, fp64.
 * Errors: NULL delta_u; u < 1, H < 2; delta_min < 0, delta_max < delta_min
 * or non-finite (LOGRA_ERR_DOMAIN). */
LOGRA_API int logra_kl_budget(int64_t u, int64_t H, double delta_max, double delta_min,
                              double* delta_u);

/* Smoothed rollout-versus-trainer log-probability mismatch kappa ([summary]
 * D.1: averaged over completed non-truncated responses, smoothed with weight
 * 0.3, clamped below at zero).  valid = 0 until a first measurement. */
typedef struct logra_mismatch_state {
  double kappa;
  int32_t valid;
  int32_t reserved;
} logra_mismatch_state;

/* Fold one measurement into the state: kappa <- max(0, w m + (1 - w) kappa),
 * or max(0, m) for the first one.  A NaN measurement (no valid measurement
 * this update) leaves the state unchanged.  weight is 0.3 in the pages.
 * Errors: NULL state; weight outside (0, 1]; infinite measurement. */
LOGRA_API int logra_mismatch_update(logra_mismatch_state* state, double measurement, double weight);

/* delta_eff = max(delta_u - kappa, 0.5 delta_u) ([paper] App. D.1, Table 4
 * "budget floor 50%"); delta_u itself while the state holds no measurement.
 * Errors: NULL pointers; delta_u < 0 or non-finite. */
LOGRA_API int logra_effective_budget(double delta_u, const logra_mismatch_state* state,
                                     double* delta_eff);

/* Device form: *alpha_dev = min(alpha_max, sqrt(delta / *q_dev)) in fp32;
 * q = 0 gives alpha_max; q < 0 or NaN gives NaN (checked on the host by the
 * caller if needed).  Errors: NULL pointers; delta <= 0 or alpha_max <= 0. */
LOGRA_API int logra_step_alpha_dev(const float* q_dev, float delta, float alpha_max,
                                   float* alpha_dev, logra_stream stream);

/* -------------------------------------------------------------- merge */

/* W [d x k] <- round(W - s * U A) in place, A regenerated from `key`.
 * s = scale * (*scale_dev if scale_dev != NULL else 1): on the trainer
 * scale = alpha*eta (or eta with alpha on the device); on the rollout side U
 * is the received alpha*eta*U and scale = 1 ([paper] §2.2 "Memory and
 * synchronization").  W is bf16 (mode NEAREST or STOCHASTIC) or fp32 (NEAREST
 * only), leading dimension ldw >= k.  U [d x r] fp32 contiguous.  The update
 * is formed in fp32 and rounded once to W's type; for bf16 W a NaN becomes
 * the quiet NaN of its sign and an infinity stays itself.  row0 is the global index
 * of W's first row (for row-sharded merges: stochastic-rounding draws are
 * indexed by (row0 + i) * k + l, so a merge of a row block equals the same
 * rows of a whole-matrix merge).  Two merges of equal W with equal
 * (U, key, s, mode, sr_seed, row0) give identical bits -- the rollout-sync
 * invariant.  [paper] §2.1-2.2, [rgc] "How it works" (stochastic rounding).
 * Errors: NULL pointers; d < 1, k < 1, r < 1, r > LOGRA_MAX_RANK, ldw < k,
 * row0 < 0; fp32 W with STOCHASTIC; non-finite scale; W overlapping U. */
LOGRA_API int logra_merge(const logra_key* key, int64_t d, int64_t k, int64_t r,
                          void* W, logra_dtype w_dtype, int64_t ldw, const float* U,
                          double scale, const float* scale_dev, logra_round mode,
                          uint64_t sr_seed, int64_t row0, logra_stream stream);

typedef struct logra_merge_desc {
  logra_key key;       /* key of this matrix's A                        */
  void* W;             /* [d x k] bf16, row-major, leading dimension ldw */
  int64_t d;
  int64_t k;
  int64_t ldw;
  const float* U;      /* [d x r] fp32 contiguous                        */
  int64_t row0;        /* global index of W's first row                  */
} logra_merge_desc;

/* Grouped form of logra_merge for bf16 W: n <= LOGRA_MAX_GROUP merges that
 * share r, the scale (scale, scale_dev), the rounding mode and sr_seed, in
 * one launch (e.g. the seven projections of one layer).  Each descriptor's
 * result has the same bits as the single call with its key, W, d, k, ldw,
 * U and row0.  The descriptor array is read on the host during the call.
 * Errors: as logra_merge for each descriptor; n < 1 or n > LOGRA_MAX_GROUP;
 * a W overlapping another descriptor's W or any U. */
LOGRA_API int logra_merge_grouped(int64_t r, const logra_merge_desc* descs, int n, double scale,
                                  const float* scale_dev, logra_round mode, uint64_t sr_seed,
                                  logra_stream stream);

/* --------------------------------------------------------- packed update */

/* Bytes of the packed update of d rows at rank r: U split into two bf16
 * terms (hi = RNE(u), lo = RNE(u - hi)) in the merge's matrix-core operand
 * order -- for each 32-row band g and 16-rank step s (steps padded to 1, 2,
 * 4, 8 or 16), a 1 KiB hi operand then a 1 KiB lo operand in which 16-byte
 * lane l holds rows 32g + (l & 31), ranks 16s + 8(l >> 5) .. +7; rows >= d
 * and ranks >= r are zero.  The same bytes as fp32 U with rows padded to 32
 * and ranks to 16, 32, 64, 128 or 256.  0 for invalid sizes. */
LOGRA_API size_t logra_packed_update_bytes(int64_t d, int64_t r);

/* Pack fp32 U [d x r] (contiguous) into the form above, so that a merge
 * reads its operands as they are ([paper] §2.2: the update U is what the
 * merge applies; the split is the hi + lo carrying of U in bf16 arithmetic).
 * Errors: NULL pointers; d < 1, r < 1, r > LOGRA_MAX_RANK; packed_bytes too
 * small; alignment; U overlapping the packed update. */
LOGRA_API int logra_pack_update(int64_t d, int64_t r, const float* U, void* U_packed,
                                size_t packed_bytes, logra_stream stream);

/* logra_rowadam writing the packed update instead of fp32 U: the same fp32
 * values as logra_rowadam's U, packed as by logra_pack_update, in one pass.
 * Errors: as logra_rowadam; r > LOGRA_MAX_RANK; packed_bytes too small; the
 * packed update overlapping S, v or the workspace. */
LOGRA_API int logra_rowadam_packed(int64_t d, int64_t r, const float* S, float* v, int64_t t,
                                   double beta, double eps, void* U_packed, size_t packed_bytes,
                                   void* ws, size_t ws_bytes, logra_stream stream);

/* One sketch of a grouped RowAdam. */
typedef struct logra_rowadam_desc {
  const float* S;         /* [d x r] fp32 sketch, contiguous                   */
  float* v;               /* [d] fp32 row second moments, updated in place     */
  void* U_packed;         /* packed update output (logra_packed_update_bytes)  */
  size_t packed_bytes;    /* bytes available at U_packed                       */
  int64_t d;              /* rows                                              */
} logra_rowadam_desc;

/* Workspace bytes logra_rowadam_packed_grouped needs for n sketches of
 * total_rows rows in all (0 if n < 1 or total_rows < n). */
LOGRA_API size_t logra_rowadam_grouped_ws_bytes(int n, int64_t total_rows);

/* logra_rowadam_packed for n sketches sharing r, t, beta and eps in three
 * launches instead of 3n (one RowAdam per selected matrix of a model, [summary]
 * "B. RowAdam": the statistics are per matrix).  Every sketch's results (v and
 * the packed update) are bit-identical to its own logra_rowadam_packed call.
 * The workspace holds a copy of the descriptor table and each sketch's
 * statistics.  Errors: as logra_rowadam_packed for each descriptor; n < 1 or
 * n > LOGRA_MAX_ROWADAM_GROUP; an output (v, packed update, workspace)
 * overlapping another output or any sketch. */
#define LOGRA_MAX_ROWADAM_GROUP 65536
LOGRA_API int logra_rowadam_packed_grouped(int64_t r, const logra_rowadam_desc* descs, int n,
                                           int64_t t, double beta, double eps, void* ws,
                                           size_t ws_bytes, logra_stream stream);

typedef struct logra_merge_packed_desc {
  logra_key key;          /* key of this matrix's A                          */
  void* W;                /* [d x k] bf16, row-major, leading dimension ldw  */
  int64_t d;
  int64_t k;
  int64_t ldw;
  const void* U_packed;   /* packed update of this matrix                     */
  int64_t row0;           /* global index of W's first row                    */
  size_t packed_bytes;    /* bytes available at U_packed: at least
                             logra_packed_update_bytes(d, r)                  */
} logra_merge_packed_desc;

/* logra_merge_grouped with each U given as its packed update.  Same result
 * bits as logra_merge_grouped with the fp32 U the update was packed from.
 * Errors: as logra_merge_grouped; packed_bytes below
 * logra_packed_update_bytes(d, r) (LOGRA_ERR_WORKSPACE). */
LOGRA_API int logra_merge_grouped_packed(int64_t r, const logra_merge_packed_desc* descs, int n,
                                         double scale, const float* scale_dev, logra_round mode,
                                         uint64_t sr_seed, logra_stream stream);

/* Bytes of an explicit projection packed as the merge's A operands (the
 * merge's column order: column block cb of BC = 512 columns when the rank
 * takes at most four 16-rank steps, else 256; for each wave w, instance e and
 * rank step s, a 1 KiB hi then a 1 KiB lo operand in which lane l holds
 * column BC cb + 32(E w + e) + 16((m >> 2) & 1) + 4(m >> 3) + (m & 3), m =
 * l & 31, and ranks 16s + 8(l >> 5) .. +7).  0 for invalid sizes. */
LOGRA_API size_t logra_merge_projection_packed_bytes(int64_t r, int64_t k);

/* Pack an explicit A [r x k] (fp32 row-major, e.g. from logra_regen_A_gaussian)
 * into that form (hi = RNE(a), lo = RNE(a - hi); padding zero).
 * Errors: as logra_pack_projection. */
LOGRA_API int logra_pack_merge_projection(int64_t r, int64_t k, const float* A, void* A_packed,
                                          size_t packed_bytes, logra_stream stream);

typedef struct logra_merge_explicit_desc {
  logra_key key;          /* key of the matrix (stochastic-rounding draws only) */
  void* W;                /* [d x k] bf16, leading dimension ldw                */
  int64_t d;
  int64_t k;
  int64_t ldw;
  const void* U_packed;   /* packed update of this matrix                      */
  const void* A_packed;   /* the projection in the merge's operand order       */
  int64_t row0;
  size_t packed_bytes;    /* bytes at U_packed: >= logra_packed_update_bytes(d, r) */
  size_t A_packed_bytes;  /* bytes at A_packed: >= logra_merge_projection_packed_bytes(r, k) */
} logra_merge_explicit_desc;

/* logra_merge_grouped_packed with an explicit projection (the Gaussian
 * variant) instead of the key's signs: W <- round(W - s U A), s = scale *
 * (*scale_dev if given) with A taken as given (no 1/sqrt(r) applied).  A and
 * U both enter as bf16 hi + lo; the product keeps A hi x U hi, A hi x U lo
 * and A lo x U hi (the dropped lo x lo term is below 2^-16 relative).
 * Errors: as logra_merge_grouped_packed; NULL projection; misaligned or
 * overlapping projection. */
LOGRA_API int logra_merge_grouped_explicit(int64_t r, const logra_merge_explicit_desc* descs, int n,
                                           double scale, const float* scale_dev, logra_round mode,
                                           uint64_t sr_seed, logra_stream stream);

/* ------------------------------------------------------ policy sync */

/* What the trainer sends the rollout side for one matrix ([paper] §2.2
 * "Memory and synchronization": the engine regenerates A from its seed and
 * applies the received alpha*eta*U, O(d r) instead of the d k weights).  The
 * payload is the packed update of fl32(s U), s the merge step size; both
 * sides then merge from the same payload with scale 1, so their weights stay
 * bit-identical.  Transport is the caller's: the header is plain data (host
 * memory) and the payload payload_bytes of device memory. */
#define LOGRA_SYNC_MAGIC 0x4C475253u  /* "LGRS" */
#define LOGRA_SYNC_VERSION 1u
typedef struct logra_sync_header {
  uint32_t magic;          /* LOGRA_SYNC_MAGIC                               */
  uint32_t version;        /* LOGRA_SYNC_VERSION                             */
  logra_key key;           /* key of the matrix's A                          */
  int64_t d, k, r;         /* W [d x k], rank r                              */
  int32_t mode;            /* logra_round                                    */
  int32_t reserved;
  uint64_t sr_seed;        /* stochastic-rounding seed                       */
  int64_t row0;            /* global index of the first row                  */
  uint64_t payload_bytes;  /* logra_packed_update_bytes(d, r)                */
} logra_sync_header;

/* Build one matrix's payload: header filled on the host, payload (device,
 * payload_bytes >= logra_packed_update_bytes(d, r)) = packed fl32(s U) with
 * s = scale * (*scale_dev if scale_dev != NULL else 1).
 * Errors: NULL pointers; d < 1, k < 1, r < 1, r > LOGRA_MAX_RANK, row0 < 0;
 * unknown mode; non-finite scale; payload too small or misaligned; U
 * overlapping the payload. */
LOGRA_API int logra_sync_pack(const logra_key* key, int64_t d, int64_t k, int64_t r,
                              const float* U, double scale, const float* scale_dev,
                              logra_round mode, uint64_t sr_seed, int64_t row0,
                              logra_sync_header* header, void* payload, size_t payload_bytes,
                              logra_stream stream);

/* One matrix to apply: its header and payload, and the local bf16 W. */
typedef struct logra_sync_desc {
  const logra_sync_header* header;
  const void* payload;
  void* W;        /* [d x k] bf16, leading dimension ldw */
  int64_t ldw;
} logra_sync_desc;

/* Apply n <= LOGRA_MAX_GROUP payloads sharing r, mode and sr_seed in one
 * launch: W <- round(W - (P as U) A) with scale 1 -- the merge both sides run.
 * Errors: NULL pointers; a bad magic or version, or a header whose
 * payload_bytes does not match its d and r (LOGRA_ERR_DOMAIN); mixed r, mode
 * or sr_seed; otherwise as logra_merge_grouped_packed. */
LOGRA_API int logra_sync_apply(const logra_sync_desc* descs, int n, logra_stream stream);

/* ------------------------------------------------- measurement helper */

typedef enum logra_probe {
  LOGRA_PROBE_READ = 0,  /* read src                    */
  LOGRA_PROBE_COPY = 1   /* copy src to dst             */
} logra_probe;

/* Not a step of the method: a streaming read of `bytes` of src, or a copy of
 * them to dst, with 16-byte accesses spread over every compute unit
 * (blocks_per_cu blocks of 256 threads per unit, grid-strided, non-temporal
 * loads).
 * Timed by the caller, it gives the read and copy ceilings the kernels are
 * measured against, and a transfer of known size to calibrate HBM byte
 * counters with.  READ writes 4 KiB of fold values to dst (their values are
 * meaningless).  bytes must be a positive multiple of 16; blocks_per_cu in
 * [1, 32].
 * Errors: NULL pointers; bytes not a positive multiple of 16 or above 2^50;
 * blocks_per_cu out of range; unknown mode; src or dst not 16-byte aligned;
 * src and dst overlapping. */
LOGRA_API int logra_bandwidth_probe(logra_probe mode, const void* src, void* dst, size_t bytes,
                                    int blocks_per_cu, logra_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* LOGRA_H_ */
