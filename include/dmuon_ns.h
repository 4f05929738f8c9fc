/*
 * dmuon_ns.h — C ABI of libdmuon_ns, the owner-rank Muon optimizer step on one
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources: the DMuon documentation pages and the
 * MindSpore parameter-grouping design page; see each entry point):
 *
 *   for every owned gradient tensor G (2-D, or 3-D = a batch of matrices over
 *   the last two dims), with momentum buffer B and fp32 master weight W:
 *     B ← μ·B + s·G                       (s: gradient-ingest scale, 1 or 1/N)
 *     for each 2-D slice: X₀ = B_slice / (‖B_slice‖_F + eps), oriented so that
 *       the Gram matrix is on the short side (a slice with rows > cols is
 *       treated as its transpose); then k times
 *       X ← a·X + b·(X Xᵀ) X + c·(X Xᵀ)² X;  O = X (original orientation)
 *     W ← (1 − lr·wd)·W − lr·O;  optionally P = bf16(W) (the published copy)
 *
 *   and, for the owner's small and 1-D parameters (the "adamw" route), one
 *   AdamW step per element (dmuon_adamw_step).
 *
 *   DMuon "架构设计" (Architecture design) page, §1 (the Newton–Schulz
 *   equation with coefficients α, β, γ = a, b, c) and §2 (the owner alone runs
 *   Newton–Schulz + momentum + weight decay + parameter update, on its local
 *   full-precision copy, with no communication); HSDP guide, section "底层发生了
 *   什么" (what happens underneath), step 3; routing page, dtype paragraph
 *   (master and optimizer arithmetic in fp32); parameter-grouping page §2.1 /
 *   §4.1 (fewer than 2 dims is an error) and §2.2 / §6 (more than 2 dims: the
 *   matrix is the last two dims).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named "device" must be device memory of the current HIP device;
 *   tensors are dense and row-major (C order), last dim contiguous.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   GPU entry point only ENQUEUES work on `stream` and returns; the caller keeps
 *   every buffer alive until that work completes.
 * - The caller owns and frees all memory, including the workspace, and every
 *   stream.  The library allocates no device or host memory that outlives a
 *   call and keeps no streams or events between calls; the one exception is
 *   the opt-in phase timing (dmuon_phase_timing), which holds its events until
 *   they are read.
 * - A call's tables (tensor descriptors, launch prefixes) are built on the host
 *   and copied into the workspace by small kernels whose arguments carry them,
 *   enqueued on `stream`; so every entry point may be captured into a HIP graph
 *   (replays copy the same bytes and launch the same kernels).
 * - Every argument is validated on the host, before anything is enqueued, so a
 *   rejected call leaves all buffers untouched.  Validation makes no HIP call.
 * - DMUON_TEST_FAIL_AT (environment, for failure-handling tests) makes a valid
 *   call return DMUON_E_HIP at a named point as a failed HIP call would:
 *   "plan" (before anything is enqueued), "table" (the table copy) or a phase
 *   name ("ingest", "norm", "gram", "square", "apply", "update", "adamw": that
 *   phase's first launch, the earlier launches being enqueued).
 * - DMUON_DEBUG_SYNC (environment, for debugging; set and not "0") waits for
 *   each launch to finish before the next is enqueued, so a call returns only
 *   when its work is done, and returns DMUON_E_HIP naming the launch ("table"
 *   or a phase name) whose wait reported an error.  The wait is skipped on a
 *   stream under graph capture.  Results are unchanged.
 * - Return value: DMUON_OK or a negative DMUON_E_* code; dmuon_last_error()
 *   then gives a message (thread-local, valid until the next call on the thread).
 * - After DMUON_E_HIP (a HIP launch/copy failed after validation) the contents
 *   of the momentum, master and output buffers are unspecified.
 * - Non-finite inputs are not checked; they propagate.
 * - Results are deterministic: identical inputs give bit-identical outputs
 *   (fixed-order reductions, no floating-point atomics).
 */
#ifndef DMUON_NS_H
#define DMUON_NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DMUON_OK = 0,
  DMUON_E_NULL = -1,      /* a required pointer is NULL */
  DMUON_E_NDIM = -2,      /* tensor with fewer than 2 (or more than 3) dims */
  DMUON_E_SHAPE = -3,     /* negative or too large dimension, bad count */
  DMUON_E_DTYPE = -4,     /* unknown dtype or precision code */
  DMUON_E_CFG = -5,       /* bad hyper-parameter (k out of range, eps < 0, non-finite) */
  DMUON_E_WORKSPACE = -6, /* workspace NULL, too small or misaligned */
  DMUON_E_ALIAS = -7,     /* forbidden overlap between buffers */
  DMUON_E_HIP = -8        /* HIP runtime error after validation */
};

typedef enum { DMUON_F32 = 0, DMUON_BF16 = 1 } dmuon_dtype;

/* Arithmetic of the Newton–Schulz contractions.
 * BF16_MFMA: bf16 matrix-core operands, fp32 accumulation; the iterate is
 *            computed in fp32 and kept between iterations as its bf16 operand
 *            copy plus the remainder quantised to a signed byte, with one
 *            power-of-two scale per 16 values (about 16 significant bits of
 *            each group's largest value).
 * F32:       fp32 matrix-core operands and accumulation, fp32 iterate (parity path).
 * Momentum, normalisation, the iterate's axpy and the update are fp32 in both. */
typedef enum { DMUON_PREC_BF16_MFMA = 0, DMUON_PREC_F32 = 1 } dmuon_prec;

/* One owned parameter.  shape = (rows, cols) for ndim 2 or (batch, rows, cols)
 * for ndim 3 (only shape[0..ndim-1] are read).  Every dim must be ≥ 0 and
 * rows, cols ≤ 65536; a tensor with a zero dim is skipped (no-op).
 *   grad       device, read-only, grad_dtype (bf16 or fp32): the reduced gradient,
 *              read in place (it may sit inside the owner's packed reduce buffer)
 *   momentum   device fp32, updated in place (B ← μB + s·G)
 *   master     device fp32, updated in place (W ← (1 − lr·wd)W − lr·O)
 *   ns_out     device fp32 or NULL: if set, receives O (same shape) as well
 *   param_out  device bf16 (raw 16-bit words) or NULL: if set, receives the
 *              updated master rounded to nearest-even bf16, same shape (the
 *              parameter the owner publishes: routing page, dtype paragraph,
 *              param_dtype; architecture page §2, owner broadcast); it may sit
 *              inside the owner's packed broadcast buffer
 * grad must not overlap momentum, master, ns_out or param_out; the written
 * buffers must not overlap each other or another tensor's buffers
 * (DMUON_E_ALIAS). */
typedef struct {
  int32_t ndim;
  int32_t grad_dtype;       /* dmuon_dtype */
  int64_t shape[3];
  const void* grad;
  float* momentum;
  float* master;
  float* ns_out;
  uint16_t* param_out;
} dmuon_tensor;

/* Step hyper-parameters.  lr, momentum (μ), weight_decay (wd): the HSDP guide's
 * example builds the optimizer with lr 0.02 and momentum 0.95.  eps ≥ 0 is added
 * to the Frobenius norm.  (a, b, c) are the page's (α, β, γ).  0 ≤ ns_steps ≤ 64.
 * prec is a dmuon_prec.  grad_scale (s, finite) multiplies the gradient as it is
 * read: 1 for an averaged reduce, 1/N for a summed one (HSDP guide, two-stage
 * gradient reduce: the net divisor is the number of contributing ranks).
 * 0 ≤ stream_groups ≤ 4. */
typedef struct {
  float lr;
  float momentum;
  float weight_decay;
  float eps;
  float a, b, c;
  int32_t ns_steps;
  int32_t prec;
  float grad_scale;
  int32_t stream_groups;    /* 0: the library's choice; 1..4: split the tensors
                               into this many work-balanced groups (see
                               dmuon_muon_step_run); the workspace layout
                               depends on it */
} dmuon_step_cfg;

/* Bytes of workspace dmuon_muon_step needs for these tensors and cfg (host only,
 * no HIP call).  The workspace must be device memory, 256-byte aligned. */
int dmuon_muon_step_workspace_size(const dmuon_tensor* tensors, int32_t n_tensors,
                                   const dmuon_step_cfg* cfg, size_t* bytes);

/* Number of work groups the step splits these tensors into (host only, no HIP
 * call): cfg->stream_groups if set, else 4 when the apply phase is short (under
 * 1024 rounds of 32-wide K stages of 256×256 output tiles on the 256 compute
 * units: the groups' tail rounds, epilogues and launch gaps then overlap each
 * other's contractions), else 1; never more than the number of non-empty
 * tensors. */
int dmuon_muon_step_groups(const dmuon_tensor* tensors, int32_t n_tensors, const dmuon_step_cfg* cfg,
                           int32_t* groups);

/* The owner-rank Muon step over n_tensors tensors (all slices of all tensors in
 * one grouped launch per phase and group): momentum, per-slice normalisation,
 * ns_steps Newton–Schulz iterations, decoupled decay + lr-scaled update.
 * DMuon architecture page §2 and §3.3 (owner-gated step); HSDP guide, "what
 * happens underneath", step 3.  n_tensors ≥ 0 (0 is a no-op); tensors may be
 * NULL only when n_tensors is 0.  The workspace (≥ the size reported above) is
 * scratch apart from its table region: its contents on entry are ignored and
 * on exit are unspecified.
 *
 * dmuon_muon_step = dmuon_muon_step_prepare followed by dmuon_muon_step_run.
 * A caller that steps the same tensors repeatedly prepares once and runs each
 * step: prepare writes the tables for exactly these tensor pointers, shapes,
 * dtypes, cfg->prec and cfg->stream_groups into the workspace; run only
 * launches the kernels, which read them.  The kernels of a run check a hash of
 * the host-built table in every table entry they read: if the workspace does not
 * hold the tables of a prepare with the same arguments (lr, momentum, weight
 * decay, eps, a, b, c, ns_steps and grad_scale may differ), every workgroup
 * exits at once and the run changes nothing.  The table region is written
 * only by prepare, so runs may follow each other without a new prepare.
 *
 * Group 0 runs on `stream`; group g ≥ 1 runs on side_streams[(g − 1) mod
 * n_side_streams], forked from `stream` and joined back to it with events
 * created and destroyed inside the call (with n_side_streams = 0 every group
 * runs on `stream`, in order).  The caller owns the side streams (non-NULL; use
 * default-priority streams).  Results do not depend on the grouping or on the
 * streams. */
int dmuon_muon_step(const dmuon_tensor* tensors, int32_t n_tensors, const dmuon_step_cfg* cfg,
                    void* workspace, size_t workspace_bytes, void* stream, void* const* side_streams,
                    int32_t n_side_streams);
int dmuon_muon_step_prepare(const dmuon_tensor* tensors, int32_t n_tensors, const dmuon_step_cfg* cfg,
                            void* workspace, size_t workspace_bytes, void* stream);
int dmuon_muon_step_run(const dmuon_tensor* tensors, int32_t n_tensors, const dmuon_step_cfg* cfg,
                        void* workspace, size_t workspace_bytes, void* stream, void* const* side_streams,
                        int32_t n_side_streams);

/* The same step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument, no device allocation and no allocating HIP call.  The
 * step's scratch (tables, iterate, operand copies, partial sums) lives in a
 * static device array of the library, 64 MiB per GPU, which each GPU the
 * library runs on holds until the process ends; a step whose
 * dmuon_muon_step_workspace_size with stream_groups = 1 exceeds 64 MiB returns
 * DMUON_E_WORKSPACE before anything is enqueued.  The step runs as one group
 * on `stream` (cfg->stream_groups must be 0 or 1) and gives the same bits as
 * dmuon_muon_step.  Every call on a GPU uses that GPU's one array and nothing
 * in it needs clearing between calls; calls that overlap on one GPU (on
 * different streams, or from different threads) race on it and must be
 * ordered by the caller.  Host-side planning uses the C++ heap. */
int dmuon_muon_step_noalloc(const dmuon_tensor* tensors, int32_t n_tensors, const dmuon_step_cfg* cfg,
                            void* stream);

/* Bytes of workspace dmuon_ns_batched needs (host only, no HIP call). */
int dmuon_ns_batched_workspace_size(int64_t batch, int64_t rows, int64_t cols, int32_t prec,
                                    int32_t steps, size_t* bytes);

/* Newton–Schulz alone on `batch` matrices rows×cols (contiguous, row-major):
 * out[i] = NS_k(x[i]) with the architecture page §1 equation.  With normalize=1
 * the start is x/(‖x‖_F + eps) per matrix; with normalize=0 it is x itself (for
 * fixed-point checks).  x: device, x_dtype (bf16 or fp32), read-only.  out:
 * device fp32, must not overlap x.  batch, rows, cols ≥ 0 (zero: no-op). */
int dmuon_ns_batched(const void* x, int32_t x_dtype, float* out, int64_t batch, int64_t rows,
                     int64_t cols, float a, float b, float c, int32_t steps, float eps,
                     int32_t normalize, int32_t prec, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Global greedy LPT partition of n Muon units over n_slots owner slots (host only,
 * synchronous, no HIP call).  DMuon architecture page §3.1 (partition, global LPT):
 * one pass over all units, largest first; units of one transformer layer go to
 * distinct slots; same-layer units below merge_below_elems elements (0 = off; the
 * page's default threshold is 5M) are merged into one unit with one owner.
 *   rows, cols, batch, layer_id   host arrays of n items (batch ≥ 1; layer_id < 0:
 *                                 no layer constraint)
 *   cost_kind                     0: cost = batch·rows·cols; 1: NS flops
 *                                 batch·(4m²n + 2m³), m = min, n = max
 * Order: stable sort by cost, largest first (ties keep input order; a merged unit
 * sits at its first member).  Each unit goes to the least-loaded slot holding no
 * unit of its layer (ties: lowest slot id), or to the least-loaded slot if all
 * hold its layer.
 * Outputs (host arrays, caller-allocated):
 *   slot_of[n]            slot of every item
 *   slot_load[n_slots]    summed cost per slot
 *   owner_order[n]        the items of owner_slot, grouped by exact shape
 *                         (batch, rows, cols), groups in order of first
 *                         assignment, items in assignment order; *n_owned of them
 *   group_offsets[n + 1]  start of each group in owner_order, then *n_owned;
 *                         *n_groups groups
 * owner_order, n_owned, group_offsets and n_groups may all be NULL together. */
int dmuon_lpt_assign(int64_t n, const int64_t* rows, const int64_t* cols, const int64_t* batch,
                     const int32_t* layer_id, int32_t n_slots, int64_t merge_below_elems,
                     int32_t cost_kind, int32_t* slot_of, int64_t* slot_load, int32_t owner_slot,
                     int64_t* owner_order, int64_t* n_owned, int64_t* group_offsets,
                     int32_t* n_groups);

/* ---- the "adamw" route ----------------------------------------------------
 * Routing page, route table: "adamw" runs AdamW on the owner for LayerNorm
 * weights, biases and other small parameters, which the owner then broadcasts;
 * the MindSpore parameter-grouping page §1 / §2.1 sends 1-D parameters to an
 * element-wise optimizer.  The pages do not restate AdamW; the step is the
 * published AdamW (decoupled weight decay, bias-corrected moments):
 *   g ← s·G;  p ← (1 − lr·wd)·p;  m ← β₁m + (1 − β₁)g;  v ← β₂v + (1 − β₂)g²
 *   p ← p − lr·m̂ / (√v̂ + eps),  m̂ = m / (1 − β₁ᵗ),  v̂ = v / (1 − β₂ᵗ)
 * in fp32, element by element; optionally P = bf16(p) (round to nearest even). */

/* One parameter of any shape, dense, numel ≥ 0 elements (0: skipped).
 *   grad        device, read-only, grad_dtype (bf16 or fp32)
 *   param       device fp32, updated in place
 *   exp_avg     device fp32 (m), updated in place
 *   exp_avg_sq  device fp32 (v), updated in place
 *   param_out   device bf16 (raw 16-bit words) or NULL: the published copy
 * Same overlap rules as dmuon_tensor (DMUON_E_ALIAS). */
typedef struct {
  int64_t numel;
  int32_t grad_dtype;       /* dmuon_dtype */
  int32_t reserved;         /* must be 0 */
  const void* grad;
  float* param;
  float* exp_avg;
  float* exp_avg_sq;
  uint16_t* param_out;
} dmuon_adamw_tensor;

/* lr ≥ 0, 0 ≤ beta1, beta2 < 1, eps > 0, weight_decay, grad_scale finite;
 * step ≥ 1 is the step number the bias correction uses (the first step is 1). */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  float grad_scale;
  int32_t step;
} dmuon_adamw_cfg;

/* Bytes of workspace dmuon_adamw_step needs (host only, no HIP call). */
int dmuon_adamw_step_workspace_size(const dmuon_adamw_tensor* tensors, int32_t n_tensors, size_t* bytes);

/* One AdamW step over n_tensors tensors in one grouped launch (asynchronous on
 * stream).  n_tensors ≥ 0; tensors may be NULL only when n_tensors is 0.  The
 * workspace (device, 256-byte aligned, ≥ the size above) is scratch. */
int dmuon_adamw_step(const dmuon_adamw_tensor* tensors, int32_t n_tensors, const dmuon_adamw_cfg* cfg,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Plain NT product C = A·Bᵀ on the matrix-core kernel the step uses (a test hook
 * for the contraction core).  A: M×K (lda elements per row), B: N×K (ldb), both
 * dtype (bf16 or fp32), device; C: M×N fp32 (ldc), device.  lda and ldb must be
 * multiples of 64 and the K..ld columns must be zero (they are summed). */
int dmuon_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int64_t ldc, int32_t dtype, void* stream);

/* Where one slice's intermediates sit in a step workspace (a test hook for the
 * per-phase checks of the contraction kernels).  Host only, no HIP call: the
 * call validates the arguments as dmuon_muon_step does, lays the plan out on
 * `workspace` (the layout dmuon_muon_step_prepare and dmuon_muon_step use for
 * the same tensors and cfg) and reports device addresses inside it, which it
 * never dereferences.  `tensor` indexes `tensors`, `slice` its leading dim
 * (0 for a 2-D tensor).  After a step with cfg.ns_steps = k ≥ 1 the buffers
 * hold:
 *   x_copy   the operand copy the first Gram read: bf16 path, bf16(B) of the
 *            new momentum in the tensor's own layout (x_rows = rows, x_ld ≥
 *            cols, x_oriented = 0); fp32 path, the oriented X₀ before its scale,
 *            m × n (x_rows = m, x_ld ≥ n, x_oriented = 1);
 *   a_prime  A′ = s²·X Xᵀ − d·I of the last Gram, m × m, row stride ld_m (both
 *            triangles), element type of the path (elem_bytes 2: bf16, 4: fp32),
 *            with s = inv at t = 0 and 1 later;
 *   b_prime  B′ = (b + 2cd)·A′ + c·A′² of the last square, same layout;
 *   scalars  fp32 [inv, d_0, d_1, …, d_{k−1}] with inv = 1/(‖B‖_F + eps) and
 *            d_t the shift of iteration t.
 * m = min(rows, cols), n = max; wide = 1 when rows ≤ cols.  DMUON_E_SHAPE if
 * tensor or slice is out of range. */
typedef struct {
  const void* x_copy;
  int64_t x_rows, x_ld;
  int32_t x_oriented;
  int32_t elem_bytes;
  const void* a_prime;
  const void* b_prime;
  int64_t ld_m;
  const float* scalars;
  int32_t m, n, wide;
  int32_t reserved;
} dmuon_debug_slice;

int dmuon_debug_slice_buffers(const dmuon_tensor* tensors, int32_t n_tensors, const dmuon_step_cfg* cfg,
                              void* workspace, size_t workspace_bytes, int32_t tensor, int64_t slice,
                              dmuon_debug_slice* out);

/* Phase timing for profiling (off by default).  enable = 1: every later kernel
 * launch of the library is bracketed by two hipEvents on its stream; enable = 0
 * stops it.  dmuon_phase_timing_read waits for the recorded events, writes for
 * each phase p < n the summed milliseconds ms[p] and the launch count count[p],
 * then clears the record.  Phases: 0 ingest (momentum, partial norms, operand
 * copies), 1 norm finalize, 2 Gram, 3 square+poly, 4 apply, 5 update (k = 0
 * only), 6 gemm_nt, 7 adamw. */
int dmuon_phase_timing(int32_t enable);
int dmuon_phase_timing_read(double* ms, int64_t* count, int32_t n);

/* Message for the last non-OK return on this thread ("" if none). */
const char* dmuon_last_error(void);

/* ABI version (bumped on any change of a signature, a struct or a documented
 * numbering such as the phases above): 5. */
int32_t dmuon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DMUON_NS_H */
