/*
 * muonh.h - C ABI of the MI355X (gfx950) MuonH optimizer step.
 *
 * MuonH updates a set of weight matrices with Muon's orthogonalized momentum
 * update and then puts every matrix back on the sphere of the Frobenius norm
 * it had at initialization. Sources, cited by page title and section:
 *   - digest page "Puro-2B trains for $6.9K, attention sinks hit 99%,
 *     LoopArena tops at 24.69%", section "The load-bearing tricks aren't in
 *     the abstract" and footnotes 3-4: MuonH extends Muon, fixes each matrix's
 *     Frobenius norm at its initialization value by projecting updates onto a
 *     fixed hypersphere; Muon's overhead is its Newton-Schulz iterations;
 *   - model card "Puro", section "Training": MuonH with hyperball projection
 *     and zero weight decay on the matrix group; master weights and optimizer
 *     state in FP32 or BF16 (W fp32 here; G and M fp32 or bf16 by plan flag).
 *
 * One step, per matrix (rows x cols, row-major fp32):
 *   M  <- beta*M + G                                  (heavy-ball momentum)
 *   X0  = M / (||M||_F + 1e-7), transposed when rows > cols
 *   ns_iters times:  A = X X^T;  B = b*A + c*A*A;  X <- a*X + B*X
 *                    (a, b, c) = (3.4445, -4.7750, 2.0315)
 *   O   = X (transposed back)
 *   W'  = W - lr*O
 *   W  <- (R / ||W'||_F) * W'        (W <- W' when ||W'||_F == 0)
 * with R = ||W0||_F captured once by muonh_init. The pages give neither the
 * momentum rule, nor the polynomial, nor the normalisation: the readings above
 * are the plainest ones consistent with the pages (no update scale, no weight
 * decay, no Nesterov).
 *
 * Conventions for every call below
 *   - Matrices are grouped by shape: a plan lists groups {rows, cols, count};
 *     matrix index i runs over group 0's matrices, then group 1's, etc.
 *   - W, G, M are DEVICE arrays of n_matrices DEVICE pointers (the layout of
 *     batched-BLAS pointer arrays); each points to a contiguous row-major
 *     rows x cols matrix: W in fp32; G and M in fp32, or in bf16 (bits of
 *     IEEE binary32's upper half) under the plan flags MUONH_GRAD_BF16 and
 *     MUONH_MOM_BF16 (so G and M are typed void). R is a DEVICE array of
 *     n_matrices floats. Pointers aligned to 4 elements (16 bytes fp32,
 *     8 bytes bf16) take the vector path; others work through a scalar path.
 *     W, G and M must not overlap.
 *   - The workspace is a DEVICE buffer of at least muonh_workspace_bytes(plan)
 *     bytes, 256-byte aligned, owned by the caller. It holds the
 *     Newton-Schulz operands (bf16, split bf16 or fp32 by plan flag) and the
 *     norm partials. After a step it holds that step's update O until the
 *     next call that uses it.
 *   - All device work is enqueued asynchronously on `stream` (a hipStream_t;
 *     NULL is the default stream). No call synchronises the device, except
 *     muonh_step_status, which waits for `stream`.
 *   - Calls that share a workspace must be ordered by the caller (same stream,
 *     or events). A plan itself is read-only after creation and may be shared.
 *   - All argument checks run before any work is enqueued; a call that returns
 *     an error has enqueued nothing. Negative return values are errors;
 *     muonh_last_error() gives a message for the calling thread.
 *   - Non-finite inputs are not errors: they propagate into the results. A
 *     step records in the workspace whether a norm it took was not finite
 *     (muonh_step_status reads that record).
 */
#ifndef MUONH_H
#define MUONH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUONH_ABI_VERSION 3

typedef struct muonh_plan muonh_plan;

typedef struct {
  int32_t rows;   /* rows of every matrix in the group, >= 1 */
  int32_t cols;   /* columns of every matrix in the group, >= 1 */
  int32_t count;  /* number of matrices in the group, >= 1 */
} muonh_group_desc;

enum {
  MUONH_OK = 0,
  MUONH_EINVAL = -1,     /* bad argument (null pointer, value out of range) */
  MUONH_ESHAPE = -2,     /* bad group description or matrix index */
  MUONH_EWORKSPACE = -3, /* workspace missing, too small or misaligned */
  MUONH_EHIP = -4,       /* a HIP runtime call failed (see muonh_last_error) */
  MUONH_ENOMEM = -5,     /* host allocation failed */
  MUONH_EALIAS = -6      /* two of the W, G, M matrices overlap in memory */
};

/* Newton-Schulz plan flags (at most one). Default: operands in bf16, bf16
 * MFMA with fp32 accumulation; about 1e-2 relative error of O at 5
 * iterations, about 1.8e-2 at 8. With bf16 or split operands and
 * ns_iters >= 1, X0's factor 1/(||M||_F + 1e-7) is applied inside the first
 * iteration's products rather than before rounding M to the operand format
 * (the same value up to that rounding; matrices of at most 65536 entries,
 * and momentum norms outside [2^-40, 2^40], are normalised first). For
 * matrices of more than 65536 entries the polynomial stores
 * B' = a*I + b*A + c*A*A and the update is X <- B' X: the same algebra as
 * a*X + B*X, with a better-conditioned rounding of B'. */
enum {
  /* fp32 operands and fp32 MFMA. Debug/reference mode: about 1e-6 relative
   * error, an order of magnitude slower. */
  MUONH_NS_FP32 = 1u,
  /* Split-bf16 operands: every stored value v is kept as hi = bf16(v) plus
   * lo = bf16(v - hi), and each product takes hi*hi + hi*lo + lo*hi on bf16
   * MFMA (fp32 accumulation). About 1e-4 relative error of O at 8
   * iterations, for about 3x the Newton-Schulz time and twice its
   * workspace. */
  MUONH_NS_SPLIT_BF16 = 2u
};

/* Storage plan flags (any combination with the above; model card "Puro",
 * section "Training": master weights and optimizer state in FP32 or BF16).
 * W always stays fp32. */
enum {
  /* G is bf16: its values are taken as given. */
  MUONH_GRAD_BF16 = 4u,
  /* M is stored in bf16: the new momentum is the exact beta*M + G (beta
   * as the fp32 value passed) rounded once to the nearest bf16, ties to
   * even; that stored value is the momentum whose norm and Newton-Schulz
   * update the step uses. Cuts the momentum pass from 12 to 8 bytes per parameter
   * (6 with MUONH_GRAD_BF16). */
  MUONH_MOM_BF16 = 8u
};

/* Limits. */
#define MUONH_MAX_GROUPS 4096
#define MUONH_MAX_MATRICES (1 << 20)
#define MUONH_MAX_DIM 65536      /* rows and cols */
#define MUONH_MAX_NS_ITERS 32
#define MUONH_MAX_TENSOR_ELEMS (1LL << 40) /* elements per AdamW tensor */

/* Library ABI version (MUONH_ABI_VERSION of the built library). */
int32_t muonh_abi_version(void);

/*
 * Create a plan for `n_groups` shape groups. Host-only: no HIP call.
 * flags: at most one of MUONH_NS_FP32 and MUONH_NS_SPLIT_BF16, or'd with any
 * of MUONH_GRAD_BF16 and MUONH_MOM_BF16. On success *out owns a plan
 * that must be released with muonh_plan_destroy. Errors: MUONH_EINVAL (null
 * out/groups, n_groups out of [1, MUONH_MAX_GROUPS], unknown or conflicting
 * flags), MUONH_ESHAPE (a dim out
 * of [1, MUONH_MAX_DIM], count < 1, too many matrices, or more than 2^31
 * 64x64 tiles of the 256-padded matrices in total), MUONH_ENOMEM.
 */
int muonh_plan_create(muonh_plan** out, const muonh_group_desc* groups, int32_t n_groups,
                      uint32_t flags);

/* Release a plan (NULL is ignored). The caller must not have work in flight
 * that still needs it: plans hold no device memory, so this never syncs. */
void muonh_plan_destroy(muonh_plan* plan);

/* Number of matrices, and of matrix entries (parameters), in the plan. */
int64_t muonh_plan_num_matrices(const muonh_plan* plan);
int64_t muonh_plan_num_params(const muonh_plan* plan);

/* Bytes of device workspace that muonh_init/muonh_step need. */
size_t muonh_workspace_bytes(const muonh_plan* plan);

/*
 * R[i] <- ||W[i]||_F for every matrix (fp32 result of a fixed-order
 * reduction: squares summed 4 at a time in fp32, fp64 beyond that). Capture the
 * radius once, from the initial weights. Deterministic.
 * Errors: MUONH_EINVAL (null plan/W/R), MUONH_EWORKSPACE, MUONH_EHIP.
 */
int muonh_init(const muonh_plan* plan, float* const* W, float* R, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * One MuonH step over every matrix of the plan (formula at the top of this
 * file). W and M are updated in place; G and R are read only.
 * lr: finite, >= 0 (the caller's effective rate; the model card applies a
 *     10x multiplier to the matrix group, section "Training").
 * beta: in [0, 1).  ns_iters: in [0, MUONH_MAX_NS_ITERS].
 * Results are bitwise deterministic for a given plan and input. A matrix's
 * result does not depend on the other matrices of the plan, except that bf16
 * Newton-Schulz phases whose GEMMs have few 256x256 tiles (at most 128)
 * run 128x128 tiles, which can change the last bits of the polynomial's
 * diagonal blocks and so of O (well within the tolerances).
 * Errors: MUONH_EINVAL, MUONH_EWORKSPACE, MUONH_EHIP.
 */
int muonh_step(const muonh_plan* plan, float* const* W, const void* const* G, void* const* M,
               const float* R, float lr, float beta, int32_t ns_iters, void* workspace,
               size_t workspace_bytes, void* stream);

/* Bytes of the fixed device workspace of muonh_step_noalloc (per GPU). */
#define MUONH_NOALLOC_WORKSPACE_BYTES (128u << 20)

/*
 * muonh_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step with the same arguments, but no caller workspace. The library
 * keeps one fixed array of MUONH_NOALLOC_WORKSPACE_BYTES (128 MiB) of
 * device memory per GPU for the life of the process, and this call runs in
 * the current device's array; it calls no allocating routine. Plans whose
 * muonh_workspace_bytes exceed that size are rejected (MUONH_EWORKSPACE),
 * before anything is enqueued. `stream` must belong to the current device.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (the step clears what must start at zero): calls that may overlap
 * on one GPU (other streams, other threads) race and must be ordered by the
 * caller. The update O is not kept for muonh_read_update, and the
 * non-finite record is not reachable through muonh_step_status. R comes
 * from muonh_init (with a workspace, at set-up) or from a checkpoint;
 * muonh_init also looks up this device's array, so that the first
 * muonh_step_noalloc on a device need not.
 * Errors: as muonh_step.
 */
int muonh_step_noalloc(const muonh_plan* plan, float* const* W, const void* const* G,
                       void* const* M, const float* R, float lr, float beta, int32_t ns_iters,
                       void* stream);

/*
 * muonh_step plus phase timing: the same work, with hipEventRecord of the
 * caller's events on `stream` at the phase boundaries, for profiling.
 * events: host array of n_events hipEvent_t (created by the caller, with
 * timing enabled); n_events must be 3*ns_iters + 3. Recorded, in order:
 *   [0] before the momentum update,
 *   [1] after momentum, its norm and the normalised cast (Newton-Schulz input),
 *   [2+3i], [3+3i], [4+3i] after iteration i's Gram, polynomial and apply,
 *   [3*ns_iters+2] after the trial update, its norm and the projection.
 * Errors: as muonh_step, plus MUONH_EINVAL for a NULL events array, a NULL
 * event or a wrong n_events.
 */
int muonh_step_timed(const muonh_plan* plan, float* const* W, const void* const* G,
                     void* const* M, const float* R, float lr, float beta, int32_t ns_iters,
                     void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                     int32_t n_events);

/*
 * The baseline MuonH is measured against: Muon with decoupled weight decay
 * (the digest page quotes MuonH's speedup against standard weight decay,
 * section "The load-bearing tricks aren't in the abstract"; the report page,
 * part 6/7, section 4.3 "Cost Estimation", its compute multiplier relative to
 * Muon; neither prints the update). The same momentum and Newton-Schulz as
 * muonh_step, then
 *   W <- (1 - lr*weight_decay) * W - lr*O
 * with no projection and no radius. Same plan, workspace and conventions as
 * muonh_step (the two may share a plan; W and M are updated in place).
 * weight_decay: finite, >= 0. Errors: as muonh_step.
 */
int muonh_step_muon_wd(const muonh_plan* plan, float* const* W, const void* const* G,
                       void* const* M, float lr, float beta, float weight_decay,
                       int32_t ns_iters, void* workspace, size_t workspace_bytes, void* stream);

/* muonh_step_muon_wd with the phase events of muonh_step_timed (the last one
 * after the decayed update). */
int muonh_step_muon_wd_timed(const muonh_plan* plan, float* const* W, const void* const* G,
                             void* const* M, float lr, float beta, float weight_decay,
                             int32_t ns_iters, void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events, int32_t n_events);

/*
 * AdamW for the parameters outside the MuonH group (model card page "Puro",
 * section "Training": AdamW with weight decay 0.1; the page gives no other
 * hyperparameter). One step at step number `step` (1-based), per element of
 * every tensor, in fp32 (decoupled decay, bias-corrected moments):
 *   p <- p*(1 - lr*weight_decay)
 *   m <- beta1*m + (1 - beta1)*g ;  v <- beta2*v + (1 - beta2)*g^2
 *   p <- p - lr*(m/(1 - beta1^step)) / (sqrt(v/(1 - beta2^step)) + eps)
 * sizes: HOST array of n_tensors element counts (0 allowed, at most
 *   MUONH_MAX_TENSOR_ELEMS). P, G, M, V: DEVICE arrays of n_tensors DEVICE
 *   pointers to flat fp32 tensors (parameters, gradients, first and second
 *   moments); P, M, V are updated in place, G is read. No plan and no
 *   workspace: tensors go in grouped launches of up to 128 tensors.
 * lr, weight_decay: finite, >= 0; beta1, beta2 in [0, 1); eps finite, >= 0.
 * n_tensors == 0 is a no-op. Deterministic; asynchronous on `stream`.
 * Errors: MUONH_EINVAL (bad scalar, NULL array, step < 1, n_tensors < 0),
 * MUONH_ESHAPE (a size out of range), MUONH_EHIP.
 */
int muonh_adamw_step(int32_t n_tensors, const int64_t* sizes, float* const* P,
                     const float* const* G, float* const* M, float* const* V, float lr,
                     float beta1, float beta2, float eps, float weight_decay, int32_t step,
                     void* stream);

/*
 * Copy the update O of matrix `index` computed by the last muonh_step (or
 * muonh_step_muon_wd) that used this workspace into dst, a DEVICE buffer of
 * rows x cols fp32 (row-major, the matrix's own orientation). For inspection
 * and tests.
 * Errors: MUONH_EINVAL, MUONH_ESHAPE (index out of range), MUONH_EWORKSPACE,
 * MUONH_EHIP.
 */
int muonh_read_update(const muonh_plan* plan, int64_t index, float* dst, const void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Non-finite report of the last muonh_step or muonh_step_muon_wd that used
 * this workspace (0 after muonh_init on it and before any step): each step
 * clears the record when it starts and then sets
 *   MUONH_NONFINITE_MOMENTUM  when ||M|| (after the momentum update) of any
 *                             matrix is NaN or infinite: its X0, O and W are
 *                             then not finite either;
 *   MUONH_NONFINITE_UPDATE    (muonh_step only) when ||W - lr*O|| of any
 *                             matrix is NaN or infinite, so the projected W
 *                             is not finite.
 * (the two norms the step divides by, formula at the top of this file). The
 * kernels that finalize the norms write the record; it never changes the
 * results. *flags (HOST) receives the bits.
 * This call copies 4 bytes to the host and waits for `stream` (the only
 * synchronising call of the library); order it after the step like any
 * other call on the workspace.
 * Errors: MUONH_EINVAL (NULL plan or flags), MUONH_EWORKSPACE, MUONH_EHIP.
 */
enum {
  MUONH_NONFINITE_MOMENTUM = 1,
  MUONH_NONFINITE_UPDATE = 2,
};
int muonh_step_status(const muonh_plan* plan, const void* workspace, size_t workspace_bytes,
                      void* stream, uint32_t* flags);

/*
 * Check that no two of the plan's W, G and M matrices overlap in memory
 * (model card "Puro", section "Training": the step updates W and M in place,
 * so W, G and M must be distinct storage). W, G and M are HOST arrays of
 * n_matrices DEVICE pointers: the values the caller puts into the device
 * pointer arrays it passes to muonh_step. Each matrix spans rows*cols
 * elements of its storage type (W fp32; G and M fp32 or bf16 by plan flag).
 * Host-only: no HIP call, nothing enqueued, and no pointer is dereferenced.
 * muonh_step itself cannot check this (its pointer arrays live in device
 * memory); a caller whose pointers change calls this before the step.
 * O(n log n) in the number of matrices.
 * Errors: MUONH_EINVAL (NULL plan or array), MUONH_EALIAS (the message names
 * the first overlapping pair, e.g. "G[3] overlaps W[3]"), MUONH_ENOMEM.
 */
int muonh_check_disjoint(const muonh_plan* plan, const void* const* W, const void* const* G,
                         const void* const* M);

/* Static description of a status code. */
const char* muonh_status_string(int status);

/* Message of the last error raised on the calling thread ("" if none). */
const char* muonh_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUONH_H */
