// Internal declarations shared by the host planner (plan.cpp, abi.cpp) and the
// HIP kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

namespace dmuon {

// ---- tiling constants -------------------------------------------------------
constexpr int kThreads = 256;          // threads per workgroup (4 wave64)
constexpr int kTile = 256;             // output tile edge of the contraction kernels
constexpr int kElemChunk = 16384;      // elements per workgroup of the momentum kernel
constexpr int kPrepTile = 64;          // tile edge of the ingest kernel
constexpr int kLdAlign = 64;           // operand leading dims are multiples of this
constexpr int kMaxSteps = 64;          // ns_steps upper bound
constexpr int kScalStride = 80;        // floats of per-slice scalars (inv, d[0..k])
constexpr size_t kScratchBytes = (size_t)64 << 20;   // static scratch of the allocation-free step

enum Phase : int {
  PH_INGEST = 0,     // momentum, partial sums of squares, unscaled operand copies
  PH_NORM = 1,       // per-slice norm finalize: inv = 1/(‖B‖_F + eps), d₀
  PH_GRAM = 2,       // A' = X Xᵀ − d I (upper tiles, mirrored)
  PH_SQUARE = 3,     // B' = (b + 2cd) A' + c A'²
  PH_APPLY = 4,      // X ← (a + bd + cd²) X + B' X (last: decay + update)
  PH_UPDATE = 5,     // W ← (1 − lr wd) W − lr X0 (only when k = 0)
  PH_GEMM = 6,       // test hook: plain NT product
  PH_ADAMW = 7,      // the adamw route (its own launch table)
  PH_COUNT = 8
};

// One tensor (2-D = batch 1, or 3-D batch of slices) as the kernels see it.
// All per-slice arrays are laid out slice after slice with the given strides
// (in elements of the array's type).
struct DevProblem {
  uint32_t tag;                // plan tag (see LaunchTable::tag)
  int32_t batch, rows, cols;   // storage shape of one slice (row-major)
  int32_t m, n;                // m = min(rows, cols), n = max
  int32_t wide;                // 1: rows <= cols (Gram X Xᵀ on rows), 0: tall
  int32_t ld_m;                // round_up(m, 64): ld of XA, A', B' (n×ld_m, m×ld_m)
  int32_t ld_n;                // round_up(n, 64): ld of XG (m×ld_n)
  int32_t grad_bf16;           // 1: grad is bf16, 0: fp32
  int32_t chunks;              // update-kernel workgroups per slice (k = 0)
  int32_t prep_tiles_r, prep_tiles_c;   // ingest-kernel 64×64 tiles per slice
  int32_t tiles_m;             // ceil(m / 256)
  int32_t apply_tr, apply_tc;  // apply tiles per slice over rows / cols of storage
  int32_t slice_base;          // global index of this problem's first slice
  int32_t ld_x;                // round_up(cols, 32): ld of xraw
  // per-phase workgroup prefix (first global workgroup of this problem)
  int32_t wg0[PH_COUNT];
  int32_t ld_x0;               // ld of x0
  int32_t pad_;                // explicit, so that the struct has no padding bytes (it is hashed)
  // caller buffers (slice stride = rows*cols)
  const void* grad;            // ingest input (grad, or x for ns_batched)
  float* mom;                  // momentum (NULL for ns_batched)
  float* master;               // master weight (NULL for ns_batched)
  float* out;                  // NS output (NULL if not wanted)
  uint16_t* pub;               // bf16 published parameter (NULL if not wanted)
  const float* x0;             // X₀ before its 1/(‖B‖_F + eps) scale: the momentum
                               // (ld cols), or for ns_batched xraw (ld ld_x)
  // workspace (operand element type = bf16 or fp32 per precision)
  float* xf;                   // iterate in the apply's register order, per 256×256 tile
                               // (row-major tile order): fp32 path kTile² fp32 values as
                               // [wave 8][block 8][16-byte piece 4][lane 64]; bf16 path the
                               // remainder below its bf16 copy, kTile² signed bytes as
                               // [wave 8][block 8][lane 64][16] then kTile²/16 exponent
                               // bytes as [wave 8][block 8][lane 64]
  float* xraw;                 // ns_batched only: x in fp32, storage layout rows×ld_x
  void* xs[2];                 // bf16 path: X in storage layout, rows×ld_s with
                               // ld_s = round_up(cols, 64) (ping-pong: the apply reads
                               // xs[t & 1] and writes xs[(t + 1) & 1]); every bf16
                               // contraction reads X from it, row-major or K-major
  // fp32 path (no K-major reads there): both orientations of X
  void* xg;                    // oriented X, m×ld_n, stride m*ld_n
  void* xa0;                   // oriented Xᵀ, n×ld_m, stride n*ld_m (ping)
  void* xa1;                   // (pong)
  void* ap;                    // A', m×ld_m, stride m*ld_m
  void* bp;                    // B', m×ld_m
  float* part_norm;            // [batch][prep_tiles_r*prep_tiles_c]
  float* part_apply;           // [batch][apply_tr*apply_tc]
};
static_assert(sizeof(DevProblem) == 112 + 17 * 8, "DevProblem must have no implicit padding");

// Scalars of one launch (passed by value).
struct LaunchScalars {
  float mu, lr, decay, eps;    // decay = 1 − lr·wd
  float a, b, c;
  int32_t t;                   // NS iteration index
  int32_t last;                // 1 on the last apply
  int32_t has_momentum;        // 0 for ns_batched
  int32_t normalize;
  int32_t write_master;
  float gscale;                // gradient-ingest scale s (B ← μB + s·G)
};

struct LaunchTable {
  const DevProblem* probs;     // device
  const int32_t* wg_prefix;    // device, [PH_COUNT][n_probs + 1]
  float* scal;                 // device, [total_slices][kScalStride]
  int32_t n_probs;
  int32_t total_wg;            // workgroups of this launch
  uint32_t tag;                // hash of the host-built table: a workgroup whose
                               // problem entry carries another tag (the workspace
                               // does not hold this plan's table) exits at once
};

// ---- the adamw route ----------------------------------------------------
struct AdamwProblem {
  int64_t numel;
  int32_t grad_bf16;
  int32_t chunks;              // workgroups (kElemChunk elements each)
  int32_t wg0;                 // first workgroup of this tensor
  uint32_t tag;                // plan tag (see AdamwTable::tag)
  const void* grad;
  float* param;
  float* m;
  float* v;
  uint16_t* pub;
};
static_assert(sizeof(AdamwProblem) == 24 + 5 * 8, "AdamwProblem must have no implicit padding");

struct AdamwScalars {
  float decay;                 // 1 − lr·wd
  float step_size;             // lr / (1 − β₁ᵗ)
  float inv_sqrt_bc2;          // 1 / √(1 − β₂ᵗ)
  float eps;
  float beta1, one_m_beta1, beta2, one_m_beta2;
  float gscale;
};

struct AdamwTable {
  const AdamwProblem* probs;   // device
  const int32_t* wg_prefix;    // device, [n_probs + 1]
  int32_t n_probs;
  int32_t total_wg;
  uint32_t tag;                // as LaunchTable::tag
};

// One piece of a host-built table, carried to the device in the kernel
// arguments of a one-workgroup copy kernel: no host buffer has to outlive the
// call, and a captured graph replays the same bytes.
constexpr int kChunkWords = 508;        // 2 KiB of kernel arguments per piece
struct TableChunk {
  uint32_t* dst;                        // device, 4-byte aligned
  int32_t n_words;
  int32_t pad;
  uint32_t words[kChunkWords];
};

// Kernel launchers (kernels.hip).  Return 0 or a hipError_t value.
int launch_phase(int phase, int prec_f32, const LaunchTable& tab, const LaunchScalars& s,
                 void* stream);
int launch_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc, int f32, void* stream);
int launch_adamw(const AdamwTable& tab, const AdamwScalars& s, void* stream);
// Copy `bytes` (a multiple of 4) of host data to device memory at `dst`, in
// kernel arguments of copy kernels enqueued on `stream`.
int launch_write_table(void* dst, const void* src, size_t bytes, void* stream);
const char* hip_error_string(int err);
// Device address of this GPU's static scratch (kScratchBytes, 256-byte aligned):
// looked up once per device with hipGetSymbolAddress, then cached.
int scratch_region(void** ptr);

// Phase timing (abi.cpp).
void timing_before(int phase, void* stream);
void timing_after(int phase, void* stream);

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t x, int64_t a) { return (x + a - 1) / a; }

}  // namespace dmuon
