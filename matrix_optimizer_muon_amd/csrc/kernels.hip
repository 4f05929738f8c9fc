// HIP kernels of the owner-rank Muon step for gfx950 (MI355X).
//
// The step (DMuon "架构设计" / Architecture design page, §1 NS equation and §2
// owner-local step) is run as one grouped launch per phase over every 2-D slice
// of every tensor:
//
//   momentum   B ← μB + G, per-workgroup partial Σ B² (HBM stream)
//   start      X₀ = B / (‖B‖_F + eps) → fp32 iterate + two operand copies
//              (oriented X row-major and its transpose), zero padding
//   k × { gram    A' = X Xᵀ − d·I          (upper 256×256 tiles, mirrored)
//         square  B' = (b + 2cd)·A' + c·A'²  (upper tiles, mirrored)
//         apply   X ← (a + bd + cd²)·X + B'·X; the last one fuses
//                 W ← (1 − lr·wd)·W − lr·X  }
//
// The diagonal shift A = d·I + A' is exact algebra for any scalar d:
//   aX + bAX + cA²X = (a + bd + cd²)X + [(b + 2cd)A' + cA'²]X.
// With d = ‖X‖²_F / m the matrix-core operands A', B' are centred, which keeps
// bf16 rounding of A's large diagonal out of the result; the iterate itself
// stays fp32.
//
// Every contraction is an "NT" product C[i][j] = Σ_k P[i][k]·Q[j][k] with both
// operands K-contiguous (rows of a row-major matrix): the Gram uses the oriented
// X (m×n) twice, the square uses the symmetric A' twice, and the apply uses B'
// and the oriented transpose Xᵀ (n×m), ordered so that the output tile is in the
// tensor's own storage layout.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace dmuon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN
  const __bf16 b = (__bf16)f;
  uint16_t u;
  __builtin_memcpy(&u, &b, 2);
  return u;
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T> struct Op;
template <> struct Op<uint16_t> {            // bf16 operand storage
  static __device__ __forceinline__ uint16_t from(float f) { return f32_to_bf16(f); }
  static __device__ __forceinline__ float to(uint16_t v) { return bf16_to_f32(v); }
};
template <> struct Op<float> {
  static __device__ __forceinline__ float from(float f) { return f; }
  static __device__ __forceinline__ float to(float v) { return v; }
};

// Sum over the workgroup in a fixed order (xor butterfly inside each wave64,
// then the four wave sums in a fixed tree): bit-identical on every run.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int find_prob(const int32_t* prefix, int n, int bid) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= bid) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Σ of a slice's partials in a fixed order.
__device__ __forceinline__ float sum_partials(const float* part, int count, float* red) {
  float v = 0.f;
  for (int i = threadIdx.x; i < count; i += kThreads) v += part[i];
  return block_sum(v, red);
}

// ---------------------------------------------------------------------------
// momentum: B ← μB + G (or, for NS alone, just read x) and partial Σ B²
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_momentum(LaunchTable tab, LaunchScalars s) {
  __shared__ float red[4];
  const int bid = blockIdx.x;
  const int p = find_prob(tab.wg_prefix + PH_MOMENTUM * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  const int local = bid - P.wg0[PH_MOMENTUM];
  const int slice = local / P.chunks, chunk = local % P.chunks;
  const int64_t per = (int64_t)P.rows * P.cols;
  const int64_t base = (int64_t)slice * per;
  const int64_t e0 = (int64_t)chunk * kElemChunk;
  const int64_t e1 = (e0 + kElemChunk < per) ? e0 + kElemChunk : per;
  const float mu = s.mu;
  float* mom = s.has_momentum ? P.mom + base : nullptr;
  const uint16_t* gb = (const uint16_t*)P.grad + base;
  const float* gf = (const float*)P.grad + base;
  float acc = 0.f;

  const bool aligned =
      ((P.grad_bf16 ? ((uintptr_t)(gb + e0) & 15) : ((uintptr_t)(gf + e0) & 15)) == 0) &&
      (!mom || (((uintptr_t)(mom + e0) & 15) == 0));
  int64_t done = e0;
  if (aligned) {
    const int64_t nvec = (e1 - e0) >> 3;
    for (int64_t g = threadIdx.x; g < nvec; g += kThreads) {
      const int64_t e = e0 + g * 8;
      float x[8];
      if (P.grad_bf16) {
        const uint4 raw = *(const uint4*)(gb + e);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[2 * q] = __uint_as_float(w[q] << 16);
          x[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
      } else {
        const float4 u = *(const float4*)(gf + e), v = *(const float4*)(gf + e + 4);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
      }
      if (mom) {
        float4 u = *(const float4*)(mom + e), v = *(const float4*)(mom + e + 4);
        u.x = fmaf(mu, u.x, x[0]); u.y = fmaf(mu, u.y, x[1]);
        u.z = fmaf(mu, u.z, x[2]); u.w = fmaf(mu, u.w, x[3]);
        v.x = fmaf(mu, v.x, x[4]); v.y = fmaf(mu, v.y, x[5]);
        v.z = fmaf(mu, v.z, x[6]); v.w = fmaf(mu, v.w, x[7]);
        *(float4*)(mom + e) = u;
        *(float4*)(mom + e + 4) = v;
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
      }
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) q = fmaf(x[i], x[i], q);
      acc += q;
    }
    done = e0 + nvec * 8;
  }
  for (int64_t e = done + threadIdx.x; e < e1; e += kThreads) {
    float x = P.grad_bf16 ? bf16_to_f32(gb[e]) : gf[e];
    if (mom) {
      x = fmaf(mu, mom[e], x);
      mom[e] = x;
    }
    acc = fmaf(x, x, acc);
  }
  const float tot = block_sum(acc, red);
  if (threadIdx.x == 0) P.part_norm[(int64_t)slice * P.chunks + chunk] = tot;
}

// ---------------------------------------------------------------------------
// start: X₀ = inv·B (inv = 1/(‖B‖_F + eps), or 1 without normalisation);
// fp32 iterate in storage layout, operand copy in storage layout, operand copy
// transposed (through LDS), zero padding up to the 64-element leading dims.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_start(LaunchTable tab, LaunchScalars s) {
  __shared__ float tile[kPrepTile][kPrepTile + 1];
  __shared__ float red[4];
  const int bid = blockIdx.x;
  const int p = find_prob(tab.wg_prefix + PH_START * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  const int local = bid - P.wg0[PH_START];
  const int per_slice = P.prep_tiles_r * P.prep_tiles_c;
  const int slice = local / per_slice, tt = local % per_slice;
  const int r0 = (tt / P.prep_tiles_c) * kPrepTile, c0 = (tt % P.prep_tiles_c) * kPrepTile;
  const int rows = P.rows, cols = P.cols;

  const float total = sum_partials(P.part_norm + (int64_t)slice * P.chunks, P.chunks, red);
  const float inv = s.normalize ? 1.0f / (sqrtf(total) + s.eps) : 1.0f;
  float* scal = tab.scal + (int64_t)(P.slice_base + slice) * kScalStride;
  if (tt == 0 && threadIdx.x == 0) {
    scal[0] = inv;
    scal[1] = total * inv * inv / (float)P.m;   // d₀ = ‖X₀‖²_F / m
  }

  const int64_t per = (int64_t)rows * cols;
  const float* srcf = s.has_momentum ? P.mom + (int64_t)slice * per
                                     : (P.grad_bf16 ? nullptr : (const float*)P.grad + (int64_t)slice * per);
  const uint16_t* srcb = (!s.has_momentum && P.grad_bf16) ? (const uint16_t*)P.grad + (int64_t)slice * per
                                                          : nullptr;
  float* xf = P.xf + (int64_t)slice * per;
  const int ld_s = P.wide ? P.ld_n : P.ld_m;    // straight copy: cols padded
  const int ld_t = P.wide ? P.ld_m : P.ld_n;    // transposed copy: rows padded
  T* cs = (T*)(P.wide ? P.xg : P.xa0) + (int64_t)slice * rows * ld_s;
  T* ct = (T*)(P.wide ? P.xa0 : P.xg) + (int64_t)slice * cols * ld_t;

  const int tr = threadIdx.x >> 4;          // 0..15
  const int tc = (threadIdx.x & 15) * 4;    // 0..60
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lr = q * 16 + tr;
    const int r = r0 + lr;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + tc + e;
      float x = 0.f;
      if (r < rows && c < cols) {
        const int64_t o = (int64_t)r * cols + c;
        x = (srcb ? bf16_to_f32(srcb[o]) : srcf[o]) * inv;
        xf[o] = x;
      }
      v[e] = x;
      tile[lr][tc + e] = x;
    }
    if (r < rows) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + tc + e;
        if (c < ld_s) cs[(int64_t)r * ld_s + c] = Op<T>::from(v[e]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lc = q * 16 + tr;            // storage column = transposed row
    const int c = c0 + lc;
    if (c >= cols) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + tc + e;           // storage row = transposed column
      if (r < ld_t) ct[(int64_t)c * ld_t + r] = Op<T>::from(tile[tc + e][lc]);
    }
  }
}

// ---------------------------------------------------------------------------
// update when k = 0: W ← (1 − lr·wd)·W − lr·X₀, out = X₀
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_update(LaunchTable tab, LaunchScalars s) {
  const int bid = blockIdx.x;
  const int p = find_prob(tab.wg_prefix + PH_UPDATE * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  const int local = bid - P.wg0[PH_UPDATE];
  const int slice = local / P.chunks, chunk = local % P.chunks;
  const int64_t per = (int64_t)P.rows * P.cols;
  const int64_t base = (int64_t)slice * per;
  const int64_t e0 = (int64_t)chunk * kElemChunk;
  const int64_t e1 = (e0 + kElemChunk < per) ? e0 + kElemChunk : per;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += kThreads) {
    const float x = P.xf[base + e];
    if (P.out) P.out[base + e] = x;
    if (s.write_master) P.master[base + e] = fmaf(-s.lr, x, s.decay * P.master[base + e]);
  }
}

// ---------------------------------------------------------------------------
// NT contraction core on the matrix cores: 256×256 output tile, 4 waves in a
// 2×2 grid of 128×128 wave tiles (4×4 blocks of 32×32), K staged through LDS in
// 128-byte rows (64 bf16 or 32 fp32), double buffered; 16-byte chunks of each
// LDS row are XOR-swizzled by (row & 7) so that ds_read_b128 of 32 rows and the
// row-contiguous ds_write_b128 are both bank-conflict free.
// ---------------------------------------------------------------------------
constexpr int kLdsRow = 128;                          // bytes per staged row
constexpr int kStageBytes = 2 * kTile * kLdsRow;      // A + B rows of one stage
constexpr int kGemmLds = 2 * kStageBytes;             // double buffered: 128 KiB

struct Operands {
  const char* a;     // first row of the tile's A rows (bytes)
  const char* b;
  int64_t lda_b;     // leading dims in bytes
  int64_t ldb_b;
  int rows_a;        // valid A rows from the tile start (≤ 0: none)
  int rows_b;
  int ktiles;        // K / (elements per 128-byte row)
};

template <typename T>
__device__ __forceinline__ void mfma_chunk(f32x16_t& acc, const uint4& a, const uint4& b);

template <>
__device__ __forceinline__ void mfma_chunk<uint16_t>(f32x16_t& acc, const uint4& a, const uint4& b) {
  bf16x8_t va, vb;
  __builtin_memcpy(&va, &a, 16);
  __builtin_memcpy(&vb, &b, 16);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
}

// fp32: the 16-byte chunk holds 4 consecutive k; element e of the lanes of both
// halves forms one K=2 step.  A and B use the same k permutation, so the sum
// over k is the same set of products.
template <>
__device__ __forceinline__ void mfma_chunk<float>(f32x16_t& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ void gemm_mainloop(const Operands& op, char* smem, f32x16_t (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lrow = tid >> 3;                 // 0..31, + 32·q
  const int chunk = tid & 7;
  const int sw = (chunk ^ (lrow & 7)) * 16;  // swizzled byte offset inside a row
  uint4 ra[8], rb[8];

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto gload = [&](int kt) {
    const int64_t koff = (int64_t)kt * kLdsRow + chunk * 16;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = lrow + 32 * q;
      ra[q] = row < op.rows_a ? *(const uint4*)(op.a + row * op.lda_b + koff) : make_uint4(0, 0, 0, 0);
      rb[q] = row < op.rows_b ? *(const uint4*)(op.b + row * op.ldb_b + koff) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    char* sa = smem + stage * kStageBytes;
    char* sb = sa + kTile * kLdsRow;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = lrow + 32 * q;
      *(uint4*)(sa + row * kLdsRow + sw) = ra[q];
      *(uint4*)(sb + row * kLdsRow + sw) = rb[q];
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < op.ktiles; ++kt) {
    const bool more = kt + 1 < op.ktiles;
    if (more) gload(kt + 1);
    const char* sa = smem + (kt & 1) * kStageBytes;
    const char* sb = sa + kTile * kLdsRow;
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      const int off = ((2 * ss + h) ^ (r32 & 7)) * 16;
      uint4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = *(const uint4*)(sa + (wr * 128 + i * 32 + r32) * kLdsRow + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = *(const uint4*)(sb + (wc * 128 + j * 32 + r32) * kLdsRow + off);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma_chunk<T>(acc[i][j], fa[i], fb[j]);
    }
    if (more) lstore((kt + 1) & 1);
    __syncthreads();
  }
}

// Position of accumulator register r of block (i, j) inside the 256×256 tile.
__device__ __forceinline__ int acc_row(int i, int r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 1) * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
__device__ __forceinline__ int acc_col(int j) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 1) * 128 + j * 32 + (lane & 31);
}

// upper-triangle tile u (row-major over ti ≤ tj) of a T×T tile grid
__device__ __forceinline__ void tri_tile(int u, int T, int& ti, int& tj) {
  int i = 0, start = 0;
  while (start + (T - i) <= u) { start += T - i; ++i; }
  ti = i;
  tj = i + (u - start);
}

template <typename T, int PH>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(LaunchTable tab, LaunchScalars s) {
  extern __shared__ __align__(16) char smem[];
  __shared__ float red[4];
  constexpr int kElemsPerRow = kLdsRow / (int)sizeof(T);
  const int bid = blockIdx.x;
  const int p = find_prob(tab.wg_prefix + PH * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  const int local = bid - P.wg0[PH];
  const int m = P.m;
  float* scal_base = tab.scal;

  Operands op;
  int slice, row0, col0, ti = 0, tj = 0, u;
  if (PH == PH_GRAM || PH == PH_SQUARE) {
    const int T_ = P.tiles_m;
    const int per = T_ * (T_ + 1) / 2;
    slice = local / per;
    u = local % per;
    tri_tile(u, T_, ti, tj);
    row0 = ti * kTile;
    col0 = tj * kTile;
    const int ld = PH == PH_GRAM ? P.ld_n : P.ld_m;
    const T* base = PH == PH_GRAM ? (const T*)P.xg + (int64_t)slice * m * P.ld_n
                                  : (const T*)P.ap + (int64_t)slice * m * P.ld_m;
    op.a = (const char*)(base + (int64_t)row0 * ld);
    op.b = (const char*)(base + (int64_t)col0 * ld);
    op.lda_b = op.ldb_b = (int64_t)ld * sizeof(T);
    op.rows_a = m - row0;
    op.rows_b = m - col0;
    op.ktiles = ld / kElemsPerRow;
  } else {  // PH_APPLY
    const int per = P.apply_tr * P.apply_tc;
    slice = local / per;
    u = local % per;
    row0 = (u / P.apply_tc) * kTile;
    col0 = (u % P.apply_tc) * kTile;
    const T* bp = (const T*)P.bp + (int64_t)slice * m * P.ld_m;
    const T* xa = (const T*)((s.t & 1) ? P.xa1 : P.xa0) + (int64_t)slice * P.n * P.ld_m;
    const T* pa = P.wide ? bp : xa;     // rows of the output = storage rows
    const T* pb = P.wide ? xa : bp;     // cols of the output = storage cols
    op.a = (const char*)(pa + (int64_t)row0 * P.ld_m);
    op.b = (const char*)(pb + (int64_t)col0 * P.ld_m);
    op.lda_b = op.ldb_b = (int64_t)P.ld_m * sizeof(T);
    op.rows_a = P.rows - row0;
    op.rows_b = P.cols - col0;
    op.ktiles = P.ld_m / kElemsPerRow;
  }
  float* scal = scal_base + (int64_t)(P.slice_base + slice) * kScalStride;

  // d_t: at t = 0 from the start kernel; later the sum of the previous apply's
  // per-tile Σ X² partials (fixed order, identical in every workgroup).
  float d;
  if (PH == PH_GRAM && s.t > 0) {
    const int cnt = P.apply_tr * P.apply_tc;
    d = sum_partials(P.part_apply + (int64_t)slice * cnt, cnt, red) / (float)m;
    if (u == 0 && threadIdx.x == 0) scal[1 + s.t] = d;
  } else {
    d = scal[1 + s.t];
  }

  f32x16_t acc[4][4];
  gemm_mainloop<T>(op, smem, acc);

  if (PH == PH_GRAM || PH == PH_SQUARE) {
    T* dst = (T*)(PH == PH_GRAM ? P.ap : P.bp) + (int64_t)slice * m * P.ld_m;
    const T* aprime = (const T*)P.ap + (int64_t)slice * m * P.ld_m;
    const float lin = s.b + 2.f * s.c * d;
    const int ldm = P.ld_m;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gc = col0 + acc_col(j);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gr = row0 + acc_row(i, r);
          float v = acc[i][j][r];
          if (PH == PH_GRAM) {
            if (gr == gc && gr < m) v -= d;
          } else {
            const float ap = (gr < m && gc < ldm) ? Op<T>::to(aprime[(int64_t)gr * ldm + gc]) : 0.f;
            v = fmaf(lin, ap, s.c * v);
          }
          const T tv = Op<T>::from(v);
          if (gr < m && gc < ldm) dst[(int64_t)gr * ldm + gc] = tv;
          if (ti != tj && gc < m && gr < ldm) dst[(int64_t)gc * ldm + gr] = tv;
        }
      }
  } else {  // PH_APPLY
    const float alpha = s.a + s.b * d + s.c * d * d;
    const int rows = P.rows, cols = P.cols;
    const int64_t per = (int64_t)rows * cols;
    float* xf = P.xf + (int64_t)slice * per;
    float acc_sq = 0.f;
    if (s.last) {
      float* out = P.out ? P.out + (int64_t)slice * per : nullptr;
      float* w = s.write_master ? P.master + (int64_t)slice * per : nullptr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int gc = col0 + acc_col(j);
          if (gc >= cols) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int gr = row0 + acc_row(i, r);
            if (gr >= rows) continue;
            const int64_t o = (int64_t)gr * cols + gc;
            const float xn = fmaf(alpha, xf[o], acc[i][j][r]);
            if (out) out[o] = xn;
            if (w) w[o] = fmaf(-s.lr, xn, s.decay * w[o]);
          }
        }
    } else {
      const int ld_s = P.wide ? P.ld_n : P.ld_m;
      const int ld_t = P.wide ? P.ld_m : P.ld_n;
      void* xa_next = (s.t & 1) ? P.xa0 : P.xa1;
      T* cs = (T*)(P.wide ? P.xg : xa_next) + (int64_t)slice * rows * ld_s;
      T* ct = (T*)(P.wide ? xa_next : P.xg) + (int64_t)slice * cols * ld_t;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int gc = col0 + acc_col(j);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int gr = row0 + acc_row(i, r);
            float xn = 0.f;
            if (gr < rows && gc < cols) {
              const int64_t o = (int64_t)gr * cols + gc;
              xn = fmaf(alpha, xf[o], acc[i][j][r]);
              xf[o] = xn;
              acc_sq = fmaf(xn, xn, acc_sq);
            }
            const T tv = Op<T>::from(xn);
            if (gr < rows && gc < ld_s) cs[(int64_t)gr * ld_s + gc] = tv;
            if (gc < cols && gr < ld_t) ct[(int64_t)gc * ld_t + gr] = tv;
          }
        }
      const float tot = block_sum(acc_sq, red);
      if (threadIdx.x == 0) P.part_apply[(int64_t)slice * P.apply_tr * P.apply_tc + u] = tot;
    }
  }
}

// plain C = A·Bᵀ (fp32 out) on the same core: the contraction test hook
struct GemmArgs {
  const void* A;
  const void* B;
  float* C;
  int64_t M, N, lda, ldb, ldc;
  int ktiles;
  int tiles_n;
};

template <typename T>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_plain(GemmArgs g) {
  extern __shared__ __align__(16) char smem[];
  const int row0 = (blockIdx.x / g.tiles_n) * kTile;
  const int col0 = (blockIdx.x % g.tiles_n) * kTile;
  Operands op;
  op.a = (const char*)((const T*)g.A + row0 * g.lda);
  op.b = (const char*)((const T*)g.B + col0 * g.ldb);
  op.lda_b = g.lda * (int64_t)sizeof(T);
  op.ldb_b = g.ldb * (int64_t)sizeof(T);
  op.rows_a = (int)(g.M - row0);
  op.rows_b = (int)(g.N - col0);
  op.ktiles = g.ktiles;
  f32x16_t acc[4][4];
  gemm_mainloop<T>(op, smem, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gc = col0 + acc_col(j);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gr = row0 + acc_row(i, r);
        if (gr < g.M && gc < g.N) g.C[gr * g.ldc + gc] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <typename K>
static int set_lds(K kernel) {
  return (int)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
}

static int lds_ready_bf16 = 0, lds_ready_f32 = 0;

static int ensure_lds(int f32) {
  int& flag = f32 ? lds_ready_f32 : lds_ready_bf16;
  if (flag) return 0;
  int e = 0;
  if (f32) {
    e |= set_lds(k_gemm<float, PH_GRAM>);
    e |= set_lds(k_gemm<float, PH_SQUARE>);
    e |= set_lds(k_gemm<float, PH_APPLY>);
    e |= set_lds(k_gemm_plain<float>);
  } else {
    e |= set_lds(k_gemm<uint16_t, PH_GRAM>);
    e |= set_lds(k_gemm<uint16_t, PH_SQUARE>);
    e |= set_lds(k_gemm<uint16_t, PH_APPLY>);
    e |= set_lds(k_gemm_plain<uint16_t>);
  }
  if (e == 0) flag = 1;
  return e;
}

int launch_phase(int phase, int prec_f32, const LaunchTable& tab, const LaunchScalars& s, void* stream) {
  if (tab.total_wg <= 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(tab.total_wg), block(kThreads);
  int e = ensure_lds(prec_f32);
  if (e) return e;
  timing_before(phase, stream);
  switch (phase) {
    case PH_MOMENTUM: hipLaunchKernelGGL(k_momentum, grid, block, 0, st, tab, s); break;
    case PH_START:
      if (prec_f32) hipLaunchKernelGGL(k_start<float>, grid, block, 0, st, tab, s);
      else hipLaunchKernelGGL(k_start<uint16_t>, grid, block, 0, st, tab, s);
      break;
    case PH_GRAM:
      if (prec_f32) hipLaunchKernelGGL((k_gemm<float, PH_GRAM>), grid, block, kGemmLds, st, tab, s);
      else hipLaunchKernelGGL((k_gemm<uint16_t, PH_GRAM>), grid, block, kGemmLds, st, tab, s);
      break;
    case PH_SQUARE:
      if (prec_f32) hipLaunchKernelGGL((k_gemm<float, PH_SQUARE>), grid, block, kGemmLds, st, tab, s);
      else hipLaunchKernelGGL((k_gemm<uint16_t, PH_SQUARE>), grid, block, kGemmLds, st, tab, s);
      break;
    case PH_APPLY:
      if (prec_f32) hipLaunchKernelGGL((k_gemm<float, PH_APPLY>), grid, block, kGemmLds, st, tab, s);
      else hipLaunchKernelGGL((k_gemm<uint16_t, PH_APPLY>), grid, block, kGemmLds, st, tab, s);
      break;
    case PH_UPDATE: hipLaunchKernelGGL(k_update, grid, block, 0, st, tab, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  e = (int)hipGetLastError();
  timing_after(phase, stream);
  return e;
}

int launch_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                   int64_t ldb, int64_t ldc, int f32, void* stream) {
  if (M == 0 || N == 0) return 0;
  int e = ensure_lds(f32);
  if (e) return e;
  GemmArgs g;
  g.A = A; g.B = B; g.C = C; g.M = M; g.N = N; g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  const int64_t kpad = round_up(K, kLdAlign);
  g.ktiles = (int)(kpad / (f32 ? 32 : 64));
  g.tiles_n = (int)cdiv(N, kTile);
  const dim3 grid((unsigned)(cdiv(M, kTile) * g.tiles_n)), block(kThreads);
  hipStream_t st = (hipStream_t)stream;
  timing_before(PH_GEMM, stream);
  if (f32) hipLaunchKernelGGL(k_gemm_plain<float>, grid, block, kGemmLds, st, g);
  else hipLaunchKernelGGL(k_gemm_plain<uint16_t>, grid, block, kGemmLds, st, g);
  e = (int)hipGetLastError();
  timing_after(PH_GEMM, stream);
  return e;
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

int upload_async(void* dst, const void* src, size_t bytes, void* stream) {
  return (int)hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
}

}  // namespace dmuon
