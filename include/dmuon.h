/*
 * dmuon.h -- C ABI of the MI355X (gfx950) owner-side Muon step.
 *
 * What is computed.  DMuon gives every Muon-target matrix parameter one owner
 * rank; the owner holds the full parameter, receives the reduced gradient,
 * and alone runs Newton-Schulz on it once per step (DMuon landing page,
 * intro and "LLM Pretraining"; "Z2 vs Z3 Modes", "Byte cost per step").  This
 * library is that owner's step over its list of matrices, on one GPU:
 *
 *   M <- mu*M + G                                  momentum accumulation
 *   X <- U / (||U||_F + eps), U = M (or G + mu*M with Nesterov)
 *        transposed to m x n, m = min(rows, cols) (wide orientation)
 *   ns_steps times:  A = X X^T ;  X <- a X + (b A + c A^2) X
 *   O = X back in rows x cols orientation
 *   P <- P - lr * scale * O
 *
 * The pages name the iteration but print no coefficients, momentum rule,
 * epsilon or scale; all are passed in (see dmuon_step_config).  The pack /
 * unpack calls build the owner's single contiguous buffer of its matrices
 * ("Z2 vs Z3 Modes", "The two packed-buffer lifecycles").  dmuon_partition_lpt
 * is the balanced owner assignment (landing page, "MoE": balanced partition).
 *
 * Conventions for every call.
 *   - Matrices are row-major and contiguous: element (i, j) of an r x c
 *     matrix is at base[i*c + j].  Rows/cols are the PyTorch [out, in] shape.
 *   - Device pointers must be 16-byte aligned; the workspace 256-byte aligned.
 *   - The caller owns every buffer.  The library keeps no pointer after a
 *     call returns; it does not allocate device memory.  It holds small
 *     pinned host staging buffers for the per-call descriptor tables.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Device calls only
 *     enqueue work and return; results are valid once the stream is
 *     synchronised, and no buffer may be reused or freed before that.
 *   - Return value: DMUON_OK (0) or a negative dmuon_status.  Every argument
 *     is validated before the first launch: on an error nothing is enqueued
 *     and no buffer is touched.  dmuon_last_error() gives a message (per
 *     thread).  No C++ exception crosses this interface.
 *   - Results are deterministic: the same inputs give bitwise equal outputs
 *     (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef DMUON_H
#define DMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DMUON_ABI_VERSION 1

typedef enum {
  DMUON_OK = 0,
  DMUON_ERR_INVALID_ARG = -1,       /* null pointer, bad size, bad value     */
  DMUON_ERR_UNSUPPORTED_DTYPE = -2, /* dtype code unknown or not allowed     */
  DMUON_ERR_ALIAS = -3,             /* an output overlaps another buffer     */
  DMUON_ERR_WORKSPACE_TOO_SMALL = -4,
  DMUON_ERR_MISALIGNED = -5,        /* pointer alignment rule broken         */
  DMUON_ERR_HIP = -6                /* a HIP call or launch failed           */
} dmuon_status;

typedef enum { DMUON_BF16 = 0, DMUON_F32 = 1 } dmuon_dtype;

/* Field selector of dmuon_pack / dmuon_unpack. */
enum { DMUON_FIELD_PARAM = 0, DMUON_FIELD_GRAD = 1 };

/* dmuon_step_config.flags */
enum {
  /* Keep X, A, B in fp32 through the Newton-Schulz chain (fp32 MFMA) instead
   * of bf16.  A checking mode: slower, closer to exact arithmetic.
   * Without it (the bf16 chain): from ns_steps = 6 on, B = bA + cA^2 (from
   * the third iteration on), and every P and T = P^2 of the Gram-space
   * chain, are stored as a pair of bf16 values, hi = RNE(v) and
   * lo = RNE(v - hi), and each product that reads one runs one more pass
   * over lo, because the default quintic amplifies rounding errors on part
   * of its band and B's rounding is the largest contributor; and a matrix
   * with min(rows, cols) < 128 runs its whole chain in fp32 (its own
   * launches), because its singular values stay in that band for most
   * iterations, where bf16 storage alone cannot keep it within 2e-2. */
  DMUON_FLAG_NS_FP32 = 1u << 0,
  /* Orthogonalise the look-ahead G + mu*M (after the momentum update)
   * instead of M. */
  DMUON_FLAG_NESTEROV = 1u << 1,
  /* Gram-space Newton-Schulz (the pages credit a "Gram Newton-Schulz"
   * kernel: landing page, "VLA and VLM" and the credits) for every matrix
   * with max(r,c) >= 2 min(r,c) and min(r,c) >= 128 when ns_steps >= 5; the
   * others, and every matrix at fewer iterations, keep the direct chain.  All iterates are
   * polynomials in A = X X^T, so the chain runs on m x m matrices: per
   * iteration P = aI + bA + cA^2, A <- A P^2, Q <- Q P, and X <- Q X once
   * per phase.  Same result in exact arithmetic; about 1.35x fewer flops at
   * n = 3.5m and ns_steps = 5.  Phases are two iterations (5 -> 2 + 2 + 1),
   * each restarting from an explicit X, which bounds the bf16 rounding of the
   * accumulated Q: on a rank-one-plus-noise input (GPU test) the error stays
   * within 1.2x of the direct chain's, and on Gaussian gradients within the
   * 2e-2 bar.  Its limit: when the singular values spread over one or two
   * decades, the bf16 storage of its m x m products makes it 2-3x less
   * accurate than the direct chain and above 2e-2 (GPU test on 256 x 1024:
   * 3.0e-2 against 1.1e-2).  Hence opt-in. */
  DMUON_FLAG_GRAM_NS = 1u << 2,
  /* Record, per matrix, whether the Newton-Schulz input U (M after the
   * momentum update, or the Nesterov look-ahead) holds a NaN or an Inf:
   * one int32 per matrix (1 or 0) in the workspace, at the offset
   * dmuon_nonfinite_flags_offset() gives.  It only reports: non-finite
   * values still propagate through that matrix's step, as without it. */
  DMUON_FLAG_CHECK_FINITE = 1u << 3,
  /* Run every bf16 Newton-Schulz product of the step as one dependency-
   * driven launch (this library's own design; the pages describe no kernel
   * structure): each matrix's tiles
   * of all its stages go to one XCD, whose work-groups take them in stage
   * order and wait, per matrix, for the previous stage's tiles; no launch
   * boundary separates stages.  Same tile code as the grouped launches
   * (256 x 256 tiles, no split K, no 128-tiles), so results match the
   * grouped launches bit for bit where those use whole 256-tiles.
   * Matrices that run their chain in fp32 keep their grouped launches.  A
   * wait that exceeds about a second gives up (the result is then wrong, the
   * step always ends, and the status word of dmuon_chain_status_offset
   * reads 1).  Off by default: pinning each matrix to one XCD
   * makes the XCDs stream different matrices at once, and on the
   * Llama-3.1-8B owner share the step is about a third slower than with
   * the grouped launches (a quarter even with every wait removed). */
  DMUON_FLAG_CHAIN_LAUNCH = 1u << 4
};

/* Launch kinds reported by dmuon_step_launches. */
enum {
  DMUON_LAUNCH_MOMENTUM_SUMSQ = 0,  /* ns_steps = 0: M update + sum of squares   */
  DMUON_LAUNCH_MOMENTUM_ORIENT = 1, /* M update + sum of squares + wide X^T      */
  DMUON_LAUNCH_NORM = 2,            /* 1 / (||U||_F + eps) per matrix           */
  DMUON_LAUNCH_UPDATE_DIRECT = 3,   /* ns_steps = 0: P -= lr*s*U/(||U||+eps)   */
  DMUON_LAUNCH_GRAM = 4,            /* A = X X^T                                */
  DMUON_LAUNCH_SQUARE = 5,          /* symmetric m x m product (+ bA + diag)    */
  DMUON_LAUNCH_APPLY = 6,           /* X <- aX + BX (Gram-space: X <- Q X)      */
  DMUON_LAUNCH_FINAL = 7,           /* last apply + parameter update            */
  DMUON_LAUNCH_GRAM_SQUARE = 8,     /* Gram tiles of some matrices and Square
                                       tiles of others, in one launch          */
  DMUON_LAUNCH_CHAIN = 9            /* DMUON_FLAG_CHAIN_LAUNCH: every bf16
                                       product of the step, one launch         */
};

/* One launch of a step, as dmuon_step_launches describes it. */
typedef struct {
  int32_t kind;         /* DMUON_LAUNCH_*                                    */
  int32_t tile;         /* GEMM launches: the output tile edge, 256, or 128
                           for a bf16 Square launch of whole tiles whose
                           256-tiles would leave CUs idle; 0 for the
                           element-wise launches                             */
  double flops;         /* flops the GEMM launches execute (symmetric
                           products as their upper triangle: m(m+1)n for
                           A = X X^T, m^2(m+1) for an m x m product, 2m^2 n
                           for an apply, times the passes over bf16 hi + lo
                           pairs, summed over the launch's matrices); 0 for
                           the element-wise launches                         */
} dmuon_launch_info;

/* One matrix of the owner's share. */
typedef struct {
  void *param;          /* rows x cols, param_dtype, updated in place        */
  int32_t param_dtype;  /* DMUON_BF16 or DMUON_F32                           */
  int32_t grad_dtype;   /* DMUON_BF16 or DMUON_F32                           */
  const void *grad;     /* rows x cols, read only; may point into a packed
                           gradient buffer                                   */
  float *momentum;      /* rows x cols fp32 momentum buffer, updated in place */
  void *orth_out;       /* NULL, or rows x cols in param_dtype: receives the
                           Newton-Schulz output O                            */
  int64_t rows, cols;   /* >= 1 each                                         */
  float scale;          /* per-matrix update scale (finite)                  */
  int32_t reserved;     /* must be 0                                         */
  int64_t packed_offset;/* element offset of this matrix in the packed
                           buffer (read by dmuon_pack, dmuon_unpack and
                           dmuon_muon_step_packed only)                      */
} dmuon_matrix;

/* Step hyper-parameters.  The landing page's optimizer call uses lr = 0.02
 * and ns_steps = 5 ("LLM Pretraining"); a, b, c, momentum and eps are not on
 * the pages.  The public Muon quintic is (3.4445, -4.7750, 2.0315). */
typedef struct {
  float a, b, c;        /* iteration coefficients                            */
  int32_t ns_steps;     /* 0 .. 64; 0 = normalised momentum update           */
  float lr;             /* finite                                            */
  float momentum;       /* mu, finite                                        */
  float eps;            /* finite, >= 0                                      */
  uint32_t flags;       /* DMUON_FLAG_*                                      */
} dmuon_step_config;

/* ABI version (DMUON_ABI_VERSION of the built library). */
int dmuon_abi_version(void);

/* Static text for a status code. */
const char *dmuon_error_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char *dmuon_last_error(void);

/* ---------------------------------------------------------------------------
 * Host-only planning calls (no GPU needed).
 */

/* Balanced owner assignment, largest matrix first (landing page, "MoE").
 * Matrices are visited by element count, largest first, equal counts in input
 * order; each goes to the owner with the smallest load so far, equal loads to
 * the lowest owner id.
 *   numel[n]          element count of each matrix (>= 0)
 *   owner_out[n]      receives the owner id of each matrix
 *   load_out[n_owners] nullable; receives each owner's total element count
 * Errors: INVALID_ARG for n < 0, n_owners < 1, negative numel, or a null
 * array that n or n_owners requires. */
int dmuon_partition_lpt(const int64_t *numel, int32_t n, int32_t n_owners,
                        int32_t *owner_out, int64_t *load_out);

/* Offsets of consecutive matrices in one packed buffer ("Z2 vs Z3 Modes",
 * "The two packed-buffer lifecycles": one contiguous buffer per owner group).
 * Matrix i starts at the end of matrix i-1 rounded up to a multiple of
 * `align` elements; *total_out is the end of the last one rounded up too.
 * Errors: INVALID_ARG for n < 0, align < 1, negative numel, null outputs. */
int dmuon_pack_offsets(const int64_t *numel, int32_t n, int64_t align,
                       int64_t *offset_out, int64_t *total_out);

/* The launch sequence dmuon_muon_step runs for these matrices and flags, in
 * order (the events of dmuon_muon_step_traced follow it).  Writes the first
 * min(cap, count) entries of out[] and the total to *count.  Host-only;
 * validates like dmuon_workspace_bytes, and checks the plan beyond what a
 * step checks: every GEMM launch computes each output tile of each of its
 * matrices exactly once (split launches: its pieces cover the tile's K
 * steps without gap or overlap).
 * Errors: INVALID_ARG (count NULL, cap < 0, out NULL with cap > 0, or a plan
 * that fails those checks, which is an internal error) and those of
 * dmuon_workspace_bytes. */
int dmuon_step_launches(const dmuon_matrix *mats, int32_t n,
                        const dmuon_step_config *cfg, dmuon_launch_info *out,
                        int32_t cap, int32_t *count);

/* Byte offset in the workspace of the int32[n] non-finite flags that a step
 * with DMUON_FLAG_CHECK_FINITE writes (flag i for mats[i]; valid once the
 * step has completed on its stream, until the workspace is used again).
 * Host-only.
 * Errors: INVALID_ARG (offset_out NULL, the flag not set in cfg) and those
 * of dmuon_workspace_bytes. */
int dmuon_nonfinite_flags_offset(const dmuon_matrix *mats, int32_t n,
                                 const dmuon_step_config *cfg, size_t *offset_out);

/* Byte offset in the workspace of the int32 status word of a step with
 * DMUON_FLAG_CHAIN_LAUNCH: the step clears it, and a wait that gives up
 * sets it to 1 (that step's result is then wrong).  Valid once the step
 * has completed on its stream, until the workspace is used again.  The
 * step that allocates nothing keeps this word in its own scratch instead.
 * Host-only.
 * Errors: INVALID_ARG (offset_out NULL, the flag not set in cfg, or a step
 * with no chained launch: ns_steps = 0, or every matrix in fp32) and those
 * of dmuon_workspace_bytes. */
int dmuon_chain_status_offset(const dmuon_matrix *mats, int32_t n,
                              const dmuon_step_config *cfg, size_t *offset_out);

/* Bytes of device workspace dmuon_muon_step needs for these matrices and
 * flags.  Host-only; validates like dmuon_muon_step except for pointers. */
int dmuon_workspace_bytes(const dmuon_matrix *mats, int32_t n,
                          const dmuon_step_config *cfg, size_t *out_bytes);

/* ---------------------------------------------------------------------------
 * Device calls.
 */

/* Copy the selected field (param or grad) of every matrix into `packed`:
 *   packed[mats[i].packed_offset + r*cols + c] = field_i[r, c]
 * Bit copy: packed_dtype must equal each matrix's field dtype.  Elements of
 * `packed` outside the matrices are not written.
 *   packed_numel  size of `packed` in elements; every matrix must fit.
 * Errors: INVALID_ARG, UNSUPPORTED_DTYPE, MISALIGNED (packed + offset not
 * 16-byte aligned), ALIAS (matrices overlap each other in `packed`, or
 * `packed` overlaps a source), HIP. */
int dmuon_pack(const dmuon_matrix *mats, int32_t n, int32_t field, void *packed,
               int32_t packed_dtype, int64_t packed_numel, void *stream);

/* Inverse of dmuon_pack: field_i[r, c] = packed[packed_offset + r*cols + c].
 * For the grad field this writes through the (const) grad pointer: the
 * caller must own that memory as writable. */
int dmuon_unpack(const dmuon_matrix *mats, int32_t n, int32_t field,
                 const void *packed, int32_t packed_dtype, int64_t packed_numel,
                 void *stream);

/* One owner-side Muon step over n matrices (n = 0 is a no-op).
 *   workspace  device scratch of at least dmuon_workspace_bytes(); its
 *              contents on entry do not matter and are undefined on exit.
 * Writes: every param, momentum and (non-null) orth_out.  Reads: grads.
 * Errors: INVALID_ARG (null pointer, rows/cols < 1 or > 2^22, ns_steps out of range,
 * non-finite lr/momentum/scale, eps < 0, unknown flag, reserved != 0),
 * UNSUPPORTED_DTYPE, MISALIGNED, ALIAS (a written buffer overlaps any other
 * buffer of the call, the workspace included), WORKSPACE_TOO_SMALL, HIP. */
int dmuon_muon_step(const dmuon_matrix *mats, int32_t n,
                    const dmuon_step_config *cfg, void *workspace,
                    size_t workspace_bytes, void *stream);

/* One tensor of the AdamW step: any shape, numel contiguous elements. */
typedef struct {
  void *param;          /* numel elements, param_dtype, updated in place      */
  int32_t param_dtype;  /* DMUON_BF16 or DMUON_F32                           */
  int32_t grad_dtype;   /* DMUON_BF16 or DMUON_F32                           */
  const void *grad;     /* numel elements, read only                         */
  float *exp_avg;       /* numel fp32 first moment, updated in place         */
  float *exp_avg_sq;    /* numel fp32 second moment, updated in place        */
  int64_t numel;        /* >= 1                                              */
} dmuon_tensor;

/* AdamW hyper-parameters.  The landing page's optimizer call takes an
 * adamw_lr (1e-3 in its example, "LLM Pretraining"); betas, eps and weight
 * decay are not on the pages. */
typedef struct {
  float lr;             /* finite                                            */
  float beta1, beta2;   /* in [0, 1)                                         */
  float eps;            /* finite, > 0                                       */
  float weight_decay;   /* finite (decoupled: P <- P - lr*wd*P)              */
  int32_t step;         /* 1-based step count t, for the bias corrections    */
} dmuon_adamw_config;

/* AdamW on the parameters the Muon step does not own (landing page, "VLA and
 * VLM": parameters the predicate does not select stay under the ordinary
 * sharded setup; "LLM Pretraining": adamw_lr).  Per element, in fp32:
 *   P <- P - lr*wd*P;  M <- b1*M + (1-b1)*G;  V <- b2*V + (1-b2)*G^2
 *   P <- P - lr * (M / (1 - b1^t)) / (sqrt(V / (1 - b2^t)) + eps)
 * n = 0 is a no-op.  Pointers 16-byte aligned.
 * Errors: INVALID_ARG (NULL pointer, numel < 1, step < 1, beta outside
 * [0, 1), eps <= 0, non-finite value), UNSUPPORTED_DTYPE, MISALIGNED, ALIAS
 * (a written buffer overlaps another buffer of the call), HIP. */
int dmuon_adamw_step(const dmuon_tensor *tensors, int32_t n,
                     const dmuon_adamw_config *cfg, void *stream);

/* dmuon_muon_step that also writes every updated param into a packed buffer,
 * the buffer an owner broadcasts its updated params from ("Z2 vs Z3 Modes",
 * "The two packed-buffer lifecycles").  The result equals dmuon_muon_step
 * followed on the same stream by
 *   dmuon_pack(mats, n, DMUON_FIELD_PARAM, packed, packed_dtype, packed_numel)
 * bit for bit, but the last launch (the last Apply, or the direct update when
 * ns_steps = 0) stores each updated element to both places, so the params are
 * not read back.
 *   packed        packed_numel elements of packed_dtype; matrix i occupies
 *                 [packed_offset_i, packed_offset_i + rows*cols); elements
 *                 outside the matrices are not written
 *   events, n_events  as for dmuon_muon_step_traced (n_events = 0: none)
 * Errors: those of dmuon_muon_step_traced; INVALID_ARG (NULL packed, a slot
 * outside the buffer), UNSUPPORTED_DTYPE (param dtype != packed_dtype),
 * MISALIGNED (slot not 16-byte aligned), ALIAS (a slot overlaps another slot
 * or any buffer of the step, the workspace included). */
int dmuon_muon_step_packed(const dmuon_matrix *mats, int32_t n,
                           const dmuon_step_config *cfg, void *workspace,
                           size_t workspace_bytes, void *packed,
                           int32_t packed_dtype, int64_t packed_numel,
                           void *stream, void *const *events, int32_t n_events);

/* dmuon_muon_step that also records caller-created HIP events (hipEvent_t,
 * passed as void*) on `stream`, for per-kernel timing: events[0] before the
 * first launch and events[j] right after the j-th launch.  Launch order:
 * with ns_steps = 0: momentum + sum of squares, norm, direct update; with
 * ns_steps >= 1: momentum + sum of squares + wide orientation, norm, then
 * the Newton-Schulz launches.  The direct chain runs Gram, Square, Apply
 * per iteration (the last Apply carries the parameter update); with
 * DMUON_FLAG_GRAM_NS the Gram-space chain's launches are merged into that
 * sequence, each chain keeping its order: a launch of each chain becomes one
 * grouped launch where both have the same kind, or where one is a Gram and
 * the other a Square launch (kind DMUON_LAUNCH_GRAM_SQUARE), the pairs
 * chosen to maximise 2 per same-kind pair plus 1 per mixed pair over the
 * two kind sequences; dmuon_step_launches lists the result.
 * Only the first
 * n_events are recorded; n_events = 0 makes this dmuon_muon_step.
 * Errors: those of dmuon_muon_step; INVALID_ARG for n_events < 0 or a NULL
 * list with n_events > 0; HIP if an event cannot be recorded. */
int dmuon_muon_step_traced(const dmuon_matrix *mats, int32_t n,
                           const dmuon_step_config *cfg, void *workspace,
                           size_t workspace_bytes, void *stream,
                           void *const *events, int32_t n_events);

/* Bytes of the static device scratch dmuon_muon_step_noalloc works in. */
#define DMUON_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* dmuon_muon_step for callers that cannot allocate device memory (tight
 * serving loops, harnesses that forbid hipMalloc): no workspace argument,
 * and no device or pinned allocation in the call.  Its workspace is a
 * file-scope device array of DMUON_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds from the library's module load until the process
 * ends; its address is looked up once per device on the first call there.
 * The launch tables go through a static host buffer of 4 MiB, reused after
 * the previous call's copy from it has completed (the call may wait for
 * that).  Results are bitwise those of dmuon_muon_step with a workspace.
 * Limits: the matrices' dmuon_workspace_bytes() must not exceed
 * DMUON_NOALLOC_SCRATCH_BYTES, else WORKSPACE_TOO_SMALL and nothing is
 * enqueued.  Every call on one GPU shares that GPU's scratch, which keeps the
 * last call's contents (nothing in it needs clearing: each step writes every
 * workspace byte it reads, the zero padding included).  Calls in stream order
 * are safe; calls that overlap on one GPU (other streams, other host
 * threads whose work is in flight together) race on the scratch.  Not meant
 * for stream capture: the table upload is a copy from pageable host memory.
 * Errors: those of dmuon_muon_step, WORKSPACE_TOO_SMALL as above, HIP if
 * the scratch cannot be looked up. */
int dmuon_muon_step_noalloc(const dmuon_matrix *mats, int32_t n,
                            const dmuon_step_config *cfg, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DMUON_H */
