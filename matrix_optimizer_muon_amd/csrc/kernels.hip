// HIP kernels of the owner-rank Muon step for gfx950 (MI355X).
//
// The step (DMuon "架构设计" / Architecture design page, §1 NS equation and §2
// owner-local step) is run as one grouped launch per phase over every 2-D slice
// of every tensor:
//
//   ingest     B ← μB + s·G, per-tile partial Σ B², and the operand copy of B
//              in storage layout, zero padded (fp32 path: also its transpose)
//   norm       inv = 1/(‖B‖_F + eps), X₀ = inv·B (the scale is folded into the
//              first Gram and the first apply)
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
// Every contraction is C[i][j] = Σ_k P(i, k)·Q(j, k) on one core whose operands
// are read row-major (K-contiguous) or K-major (see the core below): on the bf16
// path the Gram reads X from its storage-layout copy (row-major for a wide slice,
// K-major for a tall one), the square reads the symmetric A' twice row-major, and
// the apply pairs B' with X so that the output tile is in the tensor's own
// storage layout; the fp32 path keeps X in both orientations and reads every
// operand row-major.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "internal.hpp"

namespace dmuon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Global-memory (address space 1) view of a pointer.  Pointers read out of the
// device-side problem table are generic to the compiler, which would otherwise
// emit flat accesses (counted on both vmcnt and lgkmcnt, hence coarse waits).
template <typename T> using gptr = __attribute__((address_space(1))) T*;
template <typename T> __device__ __forceinline__ gptr<T> glob(T* p) { return (gptr<T>)p; }

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
template <int W>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = (red[0] + red[1]) + (red[2] + red[3]);
  if (W == 8) r += (red[4] + red[5]) + (red[6] + red[7]);
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

// Σ of a slice's partials in a fixed order.  Each thread keeps eight running
// sums so that eight loads are in flight at once (long lists: one partial per
// 64×64 tile of a large matrix).
template <int W>
__device__ __forceinline__ float sum_partials(const float* part, int count, float* red) {
  constexpr int S = 64 * W;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int i = threadIdx.x;
  for (; i + 7 * S < count; i += 8 * S) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] += part[i + k * S];
  }
  for (; i < count; i += S) v[0] += part[i];
  const float t = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  return block_sum<W>(t, red);
}

// Store 4 consecutive elements of one destination row as one vector (8 bytes of
// bf16 or 16 bytes of fp32).
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  *(uint2*)p = make_uint2(lo, hi);
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}

// Byte offset of element (r, c) of a staged 128×256 fp32 half-tile: 1 KiB rows,
// 16-byte chunks XOR-swizzled by (r >> 3) & 15 so that row-contiguous 16-byte
// reads and reads of one column over 16 row groups both spread over all banks.
__device__ __forceinline__ int stage_off(int r, int c) {
  return r * 1024 + ((((c >> 2) ^ ((r >> 3) & 15)) << 4) | ((c & 3) << 2));
}

// The same half-tile for the square's epilogue, which reads 8 columns per lane:
// chunks XOR-swizzled by (r >> 3) & 15 as above, and chunk k's bit 0 flipped when bit 4 of k is
// set, so that the even (or the odd) chunks of a row, which one instruction of
// the row pass reads (8 columns per lane), fall in 16 different bank groups.
__device__ __forceinline__ int stage_off8(int r, int c) {
  const int k = c >> 2;
  return r * 1024 + (((k ^ ((k >> 4) & 1) ^ ((r >> 3) & 15)) << 4) | ((c & 3) << 2));
}

// 4 consecutive elements of one source row, read once per step (gradient,
// momentum): nontemporal loads, which measured faster here than plain ones
typedef unsigned u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
  const u32x2_nt u = __builtin_nontemporal_load((const u32x2_nt*)p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const f32x4_t u = __builtin_nontemporal_load((const f32x4_t*)p);
  v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}

// 16 bytes of one destination row: 8 bf16 or 4 fp32 values
__device__ __forceinline__ void store_row16(uint16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
  u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
  *(uint4*)p = u;
}
__device__ __forceinline__ void store_row16(float* p, const float (&v)[4]) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
// ---------------------------------------------------------------------------
// norm finalize: one workgroup per slice sums the ingest kernel's per-tile
// partials in a fixed order: inv = 1/(‖B‖_F + eps) (1 without normalisation),
// d₀ = ‖X₀‖²_F/m = inv²·‖B‖²_F/m
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_norm(LaunchTable tab, LaunchScalars s) {
  __shared__ float red[4];
  const int bid = blockIdx.x;
  const int p = find_prob(tab.wg_prefix + PH_NORM * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  if (P.tag != tab.tag) return;
  const int slice = bid - P.wg0[PH_NORM];
  const int cnt = P.prep_tiles_r * P.prep_tiles_c;
  const float total = sum_partials<4>(P.part_norm + (int64_t)slice * cnt, cnt, red);
  if (threadIdx.x == 0) {
    const float inv = s.normalize ? 1.0f / (sqrtf(total) + s.eps) : 1.0f;
    float* scal = tab.scal + (int64_t)(P.slice_base + slice) * kScalStride;
    scal[0] = inv;
    scal[1] = total * inv * inv / (float)P.m;
  }
}

// ---------------------------------------------------------------------------
// ingest: one 64×64 storage tile of one slice per workgroup
//   B ← μB + s·G into the momentum (for NS alone X = x, kept in fp32 in the
//   iterate buffer), the tile's partial Σ B², and the unscaled operand copy of B
//   in storage layout, with zero padding up to the 64-element leading dim (the
//   fp32 path also writes the transposed copy, through an LDS tile).
// The scale of X₀ = inv·B, inv = 1/(‖B‖_F + eps), is applied by the first Gram
// (A'₀ = inv²·B Bᵀ − d₀·I) and the first apply (X₁ = inv·(α·B + B'₀·B)), which
// is the same algebra, so B is read once and no scaled copy of it is written.
// Global accesses are 16-byte row vectors (8-byte for bf16 data) when the row
// length allows; every load of the tile is issued before the first store.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_ingest(LaunchTable tab, LaunchScalars s) {
  __shared__ float tile[kPrepTile][kPrepTile + 1];
  __shared__ float red[4];
  const int bid = blockIdx.x;
  const int p = find_prob(tab.wg_prefix + PH_INGEST * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  if (P.tag != tab.tag) return;
  const int local = bid - P.wg0[PH_INGEST];
  const int per_slice = P.prep_tiles_r * P.prep_tiles_c;
  const int slice = local / per_slice, tt = local % per_slice;
  const int r0 = (tt / P.prep_tiles_c) * kPrepTile, c0 = (tt % P.prep_tiles_c) * kPrepTile;
  const int rows = P.rows, cols = P.cols;
  const int64_t per = (int64_t)rows * cols;
  const uint16_t* gb = (const uint16_t*)P.grad + (int64_t)slice * per;
  const float* gf = (const float*)P.grad + (int64_t)slice * per;
  float* mom = s.has_momentum ? P.mom + (int64_t)slice * per : nullptr;
  float* xf = s.has_momentum ? nullptr : P.xraw + (int64_t)slice * rows * P.ld_x;
  const int ld_s = P.wide ? P.ld_n : P.ld_m;    // straight copy: cols padded
  const int ld_t = P.wide ? P.ld_m : P.ld_n;    // transposed copy: rows padded
  // bf16: the storage-layout copy only (every bf16 contraction reads X from it);
  // fp32: the storage-layout copy and the transposed one
  constexpr bool kBoth = sizeof(T) == 4;
  T* cs = (T*)(kBoth ? (P.wide ? P.xg : P.xa0) : P.xs[0]) + (int64_t)slice * rows * ld_s;
  T* ct = kBoth ? (T*)(P.wide ? P.xa0 : P.xg) + (int64_t)slice * cols * ld_t : nullptr;
  // rows of 4-element vectors are aligned when cols is a multiple of 4 and the
  // slice bases are (16 bytes for fp32 data, 8 for bf16)
  const bool vec = (cols & 3) == 0 &&
                   ((P.grad_bf16 ? ((uintptr_t)gb & 7) : ((uintptr_t)gf & 15)) == 0) &&
                   (!mom || ((uintptr_t)mom & 15) == 0);

  const int tr = threadIdx.x >> 4;          // 0..15
  const int tc = (threadIdx.x & 15) * 4;    // 0..60
  const int c = c0 + tc;
  // (1) loads: rows r0 + 16q + tr, columns c .. c+3; zero outside the slice
  float g[4][4], b[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + q * 16 + tr;
#pragma unroll
    for (int e = 0; e < 4; ++e) g[q][e] = b[q][e] = 0.f;
    if (r >= rows) continue;
    const int64_t o = (int64_t)r * cols + c;
    if (vec) {
      if (c < cols) {
        if (P.grad_bf16) load4(gb + o, g[q]); else load4(gf + o, g[q]);
        if (mom) load4(mom + o, b[q]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e < cols) {
          g[q][e] = P.grad_bf16 ? bf16_to_f32(gb[o + e]) : gf[o + e];
          if (mom) b[q][e] = mom[o + e];
        }
    }
  }
  // (2) the new B, stored to the momentum (or the fp32 x) and the straight copy
  float sq = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lr = q * 16 + tr;
    const int r = r0 + lr;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = mom ? fmaf(s.mu, b[q][e], s.gscale * g[q][e]) : g[q][e];
      sq = fmaf(v[e], v[e], sq);
    }
    if (r < rows) {
      const int64_t o = (int64_t)r * cols + c;
      if (mom) {
        if (vec) {
          if (c < cols) *(float4*)(mom + o) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < cols) mom[o + e] = v[e];
        }
      }
      if (xf && c < cols) *(float4*)(xf + (int64_t)r * P.ld_x + c) = make_float4(v[0], v[1], v[2], v[3]);
      if (c < ld_s) store4(cs + (int64_t)r * ld_s + c, v[0], v[1], v[2], v[3]);
    }
    if (kBoth) {
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[lr][tc + e] = v[e];
    }
  }
  // (3) the tile's Σ B² (its barriers also publish the LDS tile)
  const float tot = block_sum<4>(sq, red);
  if (threadIdx.x == 0) P.part_norm[(int64_t)slice * per_slice + tt] = tot;
  if (!kBoth) return;
  // (4) fp32: transposed copy: 64 storage columns × 64 storage rows = 16 chunks
  // of 4 rows per column
  constexpr int RPC = 16 / (int)sizeof(T);
  constexpr int CPC = kPrepTile / RPC;
#pragma unroll
  for (int k = 0; k < (kPrepTile * CPC) / kThreads; ++k) {
    const int id = threadIdx.x + kThreads * k;
    const int lc = id / CPC, rg = id % CPC;
    const int cc = c0 + lc;                 // storage column = transposed row
    const int r = r0 + rg * RPC;            // first storage row = transposed column
    if (cc >= cols || r >= ld_t) continue;
    float v[RPC];
#pragma unroll
    for (int e = 0; e < RPC; ++e) v[e] = tile[rg * RPC + e][lc];
    store_row16(ct + (int64_t)cc * ld_t + r, v);
  }
}

// ---------------------------------------------------------------------------
// update when k = 0: W ← (1 − lr·wd)·W − lr·X₀, out = X₀ = inv·B
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_update(LaunchTable tab, LaunchScalars s) {
  const int bid = blockIdx.x;
  const int p = find_prob(tab.wg_prefix + PH_UPDATE * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  if (P.tag != tab.tag) return;
  const int local = bid - P.wg0[PH_UPDATE];
  const int slice = local / P.chunks, chunk = local % P.chunks;
  const int64_t per = (int64_t)P.rows * P.cols;
  const int64_t base = (int64_t)slice * per;
  const float inv = tab.scal[(int64_t)(P.slice_base + slice) * kScalStride];
  const float* x0 = P.x0 + (int64_t)slice * P.rows * P.ld_x0;
  const int64_t e0 = (int64_t)chunk * kElemChunk;
  const int64_t e1 = (e0 + kElemChunk < per) ? e0 + kElemChunk : per;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += kThreads) {
    const int64_t r = e / P.cols, c = e - r * P.cols;
    const float x = inv * x0[r * P.ld_x0 + c];
    if (P.out) P.out[base + e] = x;
    if (s.write_master) {
      const float w = fmaf(-s.lr, x, s.decay * P.master[base + e]);
      P.master[base + e] = w;
      if (P.pub) P.pub[base + e] = f32_to_bf16(w);
    }
  }
}

// bf16 pair (lo, hi) packed into one dword, round to nearest even
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  const bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}
// ---------------------------------------------------------------------------
// the adamw route: one AdamW step per element over a grouped list of tensors
// (routing page, route table: the owner runs AdamW on small and 1-D parameters;
// the steps are the published AdamW: decoupled decay, bias-corrected moments)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void adamw_elem(float& p, float& m, float& v, float g, const AdamwScalars& s) {
  g *= s.gscale;
  p *= s.decay;
  m = fmaf(s.beta1, m, s.one_m_beta1 * g);
  v = fmaf(s.beta2, v, s.one_m_beta2 * g * g);
  const float denom = sqrtf(v) * s.inv_sqrt_bc2 + s.eps;   // √v̂ + eps
  p = p - s.step_size * (m / denom);                        // lr·m̂ / (√v̂ + eps)
}

__global__ __launch_bounds__(kThreads) void k_adamw(AdamwTable tab, AdamwScalars s) {
  const int bid = blockIdx.x;
  const AdamwProblem& P = tab.probs[find_prob(tab.wg_prefix, tab.n_probs, bid)];
  if (P.tag != tab.tag) return;
  const int64_t e0 = (int64_t)(bid - P.wg0) * kElemChunk;
  const int64_t e1 = (e0 + kElemChunk < P.numel) ? e0 + kElemChunk : P.numel;
  const gptr<float> pp = glob(P.param);
  const gptr<float> mm = glob(P.m);
  const gptr<float> vv = glob(P.v);
  const gptr<uint16_t> pub = P.pub ? glob(P.pub) : nullptr;
  const gptr<const uint16_t> gb = glob((const uint16_t*)P.grad);
  const gptr<const float> gf = glob((const float*)P.grad);
  const bool aligned = (((uintptr_t)(P.param + e0) | (uintptr_t)(P.m + e0) | (uintptr_t)(P.v + e0)) & 15) == 0 &&
                       (P.grad_bf16 ? ((uintptr_t)((const uint16_t*)P.grad + e0) & 15) == 0
                                    : ((uintptr_t)((const float*)P.grad + e0) & 15) == 0) &&
                       (!P.pub || ((uintptr_t)(P.pub + e0) & 15) == 0);
  int64_t done = e0;
  if (aligned) {
    // 8 elements per vector; each pass handles kVec vectors per thread and
    // issues all their loads before any store (the buffers may alias as far as
    // the compiler knows, so it would not move loads above earlier stores)
    constexpr int kVec = 4;
    const int64_t nvec = (e1 - e0) >> 3;
    auto load_vec = [&](int64_t e, float (&g)[8], float (&pv)[8], float (&mv)[8], float (&vw)[8]) {
      if (P.grad_bf16) {
        const u32x4_t raw = *(const gptr<const u32x4_t>)(gb + e);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          g[2 * k] = __uint_as_float(w[k] << 16);
          g[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4_t a = *(const gptr<const f32x4_t>)(gf + e + 4 * h);
          g[4 * h] = a.x; g[4 * h + 1] = a.y; g[4 * h + 2] = a.z; g[4 * h + 3] = a.w;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4_t a = *(const gptr<const f32x4_t>)(pp + e + 4 * h);
        const f32x4_t b = *(const gptr<const f32x4_t>)(mm + e + 4 * h);
        const f32x4_t c = *(const gptr<const f32x4_t>)(vv + e + 4 * h);
        pv[4 * h] = a.x; pv[4 * h + 1] = a.y; pv[4 * h + 2] = a.z; pv[4 * h + 3] = a.w;
        mv[4 * h] = b.x; mv[4 * h + 1] = b.y; mv[4 * h + 2] = b.z; mv[4 * h + 3] = b.w;
        vw[4 * h] = c.x; vw[4 * h + 1] = c.y; vw[4 * h + 2] = c.z; vw[4 * h + 3] = c.w;
      }
    };
    auto store_vec = [&](int64_t e, const float (&pv)[8], const float (&mv)[8], const float (&vw)[8]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        *(gptr<f32x4_t>)(pp + e + 4 * h) = f32x4_t{pv[4 * h], pv[4 * h + 1], pv[4 * h + 2], pv[4 * h + 3]};
        *(gptr<f32x4_t>)(mm + e + 4 * h) = f32x4_t{mv[4 * h], mv[4 * h + 1], mv[4 * h + 2], mv[4 * h + 3]};
        *(gptr<f32x4_t>)(vv + e + 4 * h) = f32x4_t{vw[4 * h], vw[4 * h + 1], vw[4 * h + 2], vw[4 * h + 3]};
      }
      if (pub)
        *(gptr<u32x4_t>)(pub + e) = u32x4_t{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                            pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
    };
    int64_t q = threadIdx.x;
    for (; q + (kVec - 1) * kThreads < nvec; q += kVec * kThreads) {
      float g[kVec][8], pv[kVec][8], mv[kVec][8], vw[kVec][8];
#pragma unroll
      for (int u = 0; u < kVec; ++u) load_vec(e0 + (q + u * kThreads) * 8, g[u], pv[u], mv[u], vw[u]);
#pragma unroll
      for (int u = 0; u < kVec; ++u) {
#pragma unroll
        for (int k = 0; k < 8; ++k) adamw_elem(pv[u][k], mv[u][k], vw[u][k], g[u][k], s);
        store_vec(e0 + (q + u * kThreads) * 8, pv[u], mv[u], vw[u]);
      }
    }
    for (; q < nvec; q += kThreads) {
      float g[8], pv[8], mv[8], vw[8];
      load_vec(e0 + q * 8, g, pv, mv, vw);
#pragma unroll
      for (int k = 0; k < 8; ++k) adamw_elem(pv[k], mv[k], vw[k], g[k], s);
      store_vec(e0 + q * 8, pv, mv, vw);
    }
    done = e0 + nvec * 8;
  }
  for (int64_t e = done + threadIdx.x; e < e1; e += kThreads) {
    float p = pp[e], m = mm[e], v = vv[e];
    adamw_elem(p, m, v, P.grad_bf16 ? bf16_to_f32(gb[e]) : gf[e], s);
    pp[e] = p;
    mm[e] = m;
    vv[e] = v;
    if (pub) pub[e] = f32_to_bf16(p);
  }
}

// Buffer resource over [p, p + bytes) (a null p gives an empty range).  Buffer
// accesses are range checked: a load beyond the range reads zero and a store
// beyond it is dropped, which replaces per-element predicates (and the branches
// they would need) in the apply epilogue.
constexpr unsigned kOob = 0x7ffffff0u;       // an offset beyond every range used here
// Word 3 of a buffer descriptor: data format 32 (bits 15–18 = 4), which raw
// (untyped) buffer accesses need to be non-zero; no swizzle, no index stride.
constexpr int kRsrcFlags = 0x00020000;
// The fields are workgroup-uniform; readfirstlane tells the compiler so (a
// descriptor it cannot prove uniform is rebuilt per lane in a loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* p, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(p ? (int)bytes : 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, n, kRsrcFlags);
}
__device__ __forceinline__ float buf_ld(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_st(__amdgpu_buffer_rsrc_t r, unsigned off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st(__amdgpu_buffer_rsrc_t r, unsigned off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}

// ---------------------------------------------------------------------------
// Contraction core on the matrix cores: C[i][j] = Σ_k A(i, k)·B(j, k).
//
// One workgroup = 8 wave64s (two per SIMD) computing a 256×256 output tile; each
// wave owns a 128×64 sub-tile (4×2 blocks of 32×32 fp32 accumulators; on the bf16
// path each block is computed as four 16×16×32 quarters, see mfma_quarter).  K is staged
// through LDS in 64-byte rows (32 bf16 or 16 fp32 per row and stage), four stages
// deep, filled by buffer_load … lds (global → LDS without VGPRs; rows beyond the
// operand read as zero through the buffer's range check).  The four 16-byte
// chunks of a row are XOR-swizzled with (row >> 2) & 3 so that 16 consecutive
// rows read at one logical chunk cover all 64 LDS banks.
//
// An operand is read either row-major ("NT": row i holds A(i, 0..K), staged as
// 256 rows of 64 bytes) or K-major (row k holds A(0..255, k) of the tile,
// staged as 32 rows of 512 bytes, bf16 only).  A K-major stage is filled with
// whole 512-byte row segments, so each DMA instruction moves 8 full cache lines
// (the NT stage moves 16 half lines); its MFMA fragments are read with the
// transposing ds_read_b64_tr_b16 (two 8-byte reads per 16-byte fragment).  Its
// 32-byte segments are XOR-swizzled by kmaj_swz(row), which spreads the rows and
// segments one half-wave of a fragment read touches over all 64 banks.  A K-major B operand
// made plain 2048- to 8192-sized products 5–16% faster than NT; with both
// operands K-major (twice the fragment reads) it is about even.  On the bf16
// path X is kept only in storage layout, so the apply reads X (wide) or the
// symmetric B′ (tall) K-major and the tall Gram reads both operands K-major; the
// square stays NT (measured faster there).
//
// Ping-pong schedule: the two waves sharing a SIMD belong to different groups
// (group = wave >> 2, the 128-row half of the tile they own), and the groups run
// one phase apart.  A phase is either an MFMA phase (the MFMAs on the fragments
// of one stage: 32 of 16×16×32 on bf16, 64 of 32×32×2 on fp32) or a memory
// phase (wait for the stage's DMA, read all of its fragments, issue the DMA of
// the stage three ahead); a workgroup barrier ends every phase.  While one group's waves keep the matrix cores busy, the other
// group's waves move data, so no barrier drains the MFMA pipeline.
// ---------------------------------------------------------------------------
constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kRowBytes = 64;                          // staged bytes per operand row
constexpr int kStageBytes = 2 * kTile * kRowBytes;     // A rows + B rows: 32 KiB
constexpr int kStages = 4;
constexpr int kGemmLds = kStages * kStageBytes;        // 128 KiB
constexpr int kDmaPerStage = 4;                        // buffer_load … lds per thread per stage
static_assert(kTile == 256 && kGemmWaves == 8, "fragment layout assumes 8 waves on a 256 tile");

struct Operands {
  const char* a;     // NT: first A row of the tile; K-major: start of k-row 0
  const char* b;     // NT: first B row of the tile; K-major: start of k-row 0
  int lda_b;         // leading dims in bytes (multiples of 128)
  int ldb_b;
  int rows_a;        // NT: valid rows from the tile start; K-major: valid k rows
  int rows_b;
  int cola_b;        // K-major: byte offset of the tile's first column in a k-row
  int colb_b;
  int ktiles;        // stages: K elements / 32 (bf16) or / 16 (fp32)
};

// K-major stage layout: 32-byte segment s of k-row r sits at segment s ^ kmaj_swz(r).
// A transposing fragment read has 16-lane groups read four consecutive k-rows of
// one 16-column segment, the two groups of a half-wave k-rows 8 apart: bits 0-1
// of r spread a group's rows over four segment pairs and bit 3 moves the other
// group's rows to the odd segments, so a half-wave touches 8 distinct segments.
__device__ __forceinline__ int kmaj_swz(int r) { return (2 * (r & 3)) ^ ((r >> 3) & 1); }

// f(std::integral_constant<int, 0>{}) … f(std::integral_constant<int, N − 1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// bf16 contraction step on one 16×16 quarter of a 32×32 accumulator block.
// During the K loop quarter (R, C) (rows 16R.., columns 16C.. of the block) lives
// in registers 4(2R + C) .. 4(2R + C) + 3 in the 16×16×32 output layout: lane l,
// register i holds row 4(l >> 4) + i, column l & 15.  The operands: lane l holds
// row (A) or column (B) l & 15 and k = 8(l >> 4) .. 8(l >> 4) + 7 of the 32-deep
// stage.  quarters_to_32x32 turns the block into the 32×32×16 output layout the
// epilogues read (acc_row / acc_col).
template <int Q>
__device__ __forceinline__ void mfma_quarter(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
  bf16x8_t va, vb;
  __builtin_memcpy(&va, &a, 16);
  __builtin_memcpy(&vb, &b, 16);
  f32x4_t q = {acc[4 * Q], acc[4 * Q + 1], acc[4 * Q + 2], acc[4 * Q + 3]};
  q = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, q, 0, 0, 0);
  acc[4 * Q] = q[0];
  acc[4 * Q + 1] = q[1];
  acc[4 * Q + 2] = q[2];
  acc[4 * Q + 3] = q[3];
}

// Quarter layout → 32×32×16 layout, in place.  In the 32×32 layout lane l,
// register 4g + i holds row 8g + 4(l >> 5) + i, column l & 31; that value sits in
// quarter (g >> 1, (l >> 4) & 1) at lane 32(g & 1) + 16(l >> 5) + (l & 15),
// register i.  Per register pair (quarters (R, 0) and (R, 1)) this is a swap of
// lane bit 4 with the pair index followed by a swap of lane bit 5 with it:
// v_permlane16_swap then v_permlane32_swap.
__device__ __forceinline__ void quarters_to_32x32(f32x16_t& acc) {
#pragma unroll
  for (int R = 0; R < 2; ++R)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[8 * R + i]),
                                                        __float_as_uint(acc[8 * R + 4 + i]), false, false);
      const auto s32 = __builtin_amdgcn_permlane32_swap(s16[0], s16[1], false, false);
      acc[8 * R + i] = __uint_as_float(s32[0]);
      acc[8 * R + 4 + i] = __uint_as_float(s32[1]);
    }
}

// fp32 contraction step on one 32×32 block: a 16-byte chunk holds 4 consecutive
// k; element e of the two lane halves forms one K = 2 step.  A and B use the same
// k permutation, so the sum covers the same products.
__device__ __forceinline__ void mfma_chunk_f32(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// s_waitcnt with only vmcnt constrained (expcnt 7, lgkmcnt 15 = no wait)
#define DMUON_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8) | ((n) & 15) | ((((n) >> 4) & 3) << 14))

// s_waitcnt with only lgkmcnt constrained to 0 (vmcnt 63, expcnt 7 = no wait)
#define DMUON_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4))

// The apply's α·X term on the matrix cores (bf16 path).  X enters the apply's
// contraction as its bf16 operand copy hi; α·hi is α·I times that operand, so
// in the K stages that cover the tile's own rows (wide: the diagonal block of
// the B′ operand) or columns (tall: of the B′ operand on the B side) each wave
// issues extra MFMAs against a diagonal fragment built in registers.  α is split
// into two bf16 values α1 = bf16(α), α2 = bf16(α − α1), so α1·hi + α2·hi is
// α·hi to about 2⁻¹⁷ relative; the products are exact and accumulate in fp32.
struct DiagTerm {
  int kd0;           // first K stage of the tile's diagonal block
  uint32_t a1, a2;   // bf16 bit patterns of α1, α2
};

template <typename T, bool TA = false, bool TB = false, int DIAG = 0>
__device__ __forceinline__ void gemm_mainloop(const Operands& op, char* smem, f32x16_t (&acc)[4][2],
                                              const DiagTerm& dg = DiagTerm{0, 0u, 0u}) {
  static_assert(!(TA || TB) || sizeof(T) == 2, "K-major operands are bf16");
  static_assert(DIAG == 0 || sizeof(T) == 2, "the diagonal term is for bf16 operands");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // wave-uniform
  const int wr = wave >> 2, wc = wave & 3, h = lane >> 5, r32 = lane & 31;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)op.a, 0, (op.rows_a < kTile ? op.rows_a : kTile) * op.lda_b, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)op.b, 0, (op.rows_b < kTile ? op.rows_b : kTile) * op.ldb_b, kRsrcFlags);
  // DMA: wave w fills rows [32w, 32w + 32) of A and of B, 16 rows per instruction;
  // lane l lands at byte 16·l of the instruction's 1 KiB = row l/4, physical chunk l%4.
  // K-major: the instruction's 1 KiB is k-rows 2(2w + q) and 2(2w + q) + 1; lane l
  // lands in k-row l/32 at physical 16-byte unit l%32.
  int offa[2], offb[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = (wave * 2 + q) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int kr = 2 * (wave * 2 + q) + (lane >> 5), un = lane & 31;
    const int lun = (((un >> 1) ^ kmaj_swz(kr)) << 1) | (un & 1);    // logical unit
    offa[q] = TA ? kr * op.lda_b + op.cola_b + lun * 16 : row * op.lda_b + c * 16;
    offb[q] = TB ? kr * op.ldb_b + op.colb_b + lun * 16 : row * op.ldb_b + c * 16;
  }
  // Fragments of one stage.  bf16 (16×16×32 quarters): fa[ss][i] is rows
  // 16(4ss + i) .. +15 of the wave's 128 and fb[ss][j] columns 16(2ss + j) .. +15
  // of its 64, all 32 k, lane l reading logical chunk l >> 4 of row l & 15.
  // fp32 (32×32×2): fa[ss][i] / fb[ss][j] are 32-row / 32-column blocks i / j and
  // 16-k chunk ss, lane l reading logical chunk 2·ss + (l >> 5) of row l & 31.
  constexpr bool kQ = sizeof(T) == 2;
  int fa_off[2][4], fb_off[2][2];
#pragma unroll
  for (int ss = 0; ss < 2; ++ss) {
    const int c = kQ ? lane >> 4 : 2 * ss + h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = kQ ? wr * 128 + 16 * (4 * ss + i) + (lane & 15) : wr * 128 + i * 32 + r32;
      fa_off[ss][i] = row * kRowBytes + ((c ^ ((row >> 2) & 3)) * 16);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = kQ ? wc * 64 + 16 * (2 * ss + j) + (lane & 15) : wc * 64 + j * 32 + r32;
      fb_off[ss][j] = kTile * kRowBytes + row * kRowBytes + ((c ^ ((row >> 2) & 3)) * 16);
    }
  }
  // K-major fragments (bf16, quarter layout): two transposing 8-byte reads (k
  // 0..3 and 4..7 of the lane's 8-k block 8(l >> 4)); in each 16-lane group,
  // source lane i reads k-row 8(l >> 4) + 4t + (i >> 2), columns 4(i & 3) .. +3 of
  // the quarter's 16 columns, and lane i receives column i of the quarter, four
  // consecutive k
  int ta_off[TA ? 2 : 1][4][2], tb_off[TB ? 2 : 1][2][2];
#pragma unroll
  for (int ss = 0; ss < 2; ++ss)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kr = 8 * (lane >> 4) + 4 * t + ((lane & 15) >> 2);
      const int sub = 4 * (lane & 3);
      if (TA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = wr * 128 + 16 * (4 * ss + i) + sub;
          ta_off[TA ? ss : 0][i][t] = kr * 512 + (((n >> 4) ^ kmaj_swz(kr)) << 5) + ((2 * n) & 31);
        }
      }
      if (TB) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = wc * 64 + 16 * (2 * ss + j) + sub;
          tb_off[TB ? ss : 0][j][t] = kTile * kRowBytes + kr * 512 + (((n >> 4) ^ kmaj_swz(kr)) << 5) + ((2 * n) & 31);
        }
      }
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4_t fa[2][4], fb[2][2];     // all fragments of one stage
  // K-major operands take a range per stage: exactly its 32 k-rows (fewer at the
  // K tail, whose missing rows read as zero), so byte offsets stay small for any
  // K and no read leaves the operand.  Reads past a row's end (tile columns past
  // the leading dim) see the next row or zero; they feed only output columns
  // past the matrix, which the epilogues drop.
  auto kmaj_rsrc = [&](const char* p, int ld_b, int rows, int kt) {
    const int left = rows - 32 * kt;
    return range_rsrc(p + (int64_t)kt * 32 * ld_b, (int64_t)(left < 0 ? 0 : (left < 32 ? left : 32)) * ld_b);
  };
  auto issue = [&](int kt) {
    char* base = smem + (kt % kStages) * kStageBytes;
    const __amdgpu_buffer_rsrc_t sa = TA ? kmaj_rsrc(op.a, op.lda_b, op.rows_a, kt) : ra;
    const __amdgpu_buffer_rsrc_t sb = TB ? kmaj_rsrc(op.b, op.ldb_b, op.rows_b, kt) : rb;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      char* da = base + (wave * 2 + q) * 16 * kRowBytes;
      char* db = da + kTile * kRowBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sa, (__attribute__((address_space(3))) void*)da, 16,
                                               offa[q] + (TA ? 0 : kt * kRowBytes), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sb, (__attribute__((address_space(3))) void*)db, 16,
                                               offb[q] + (TB ? 0 : kt * kRowBytes), 0, 0, 0);
    }
  };
  const int KT = op.ktiles;        // ≥ 2 (leading dims are multiples of 64 elements)
  const bool lead = wr == 1;       // group 1 runs one phase ahead of group 0

  // Memory phase of stage kt.  Every wave waited for its own share of stage kt
  // in its previous memory phase (or before the first barrier), so each share
  // a wave reads here landed before at least one barrier, like the other
  // group's share.  Here it waits for its share of stage kt + 1; stages up to
  // min(kt + 2, KT − 1) have been issued.
  auto mem_phase = [&](int kt) {
    if (kt + 2 < KT) DMUON_WAIT_VM(kDmaPerStage);
    else DMUON_WAIT_VM(0);
    const char* base = smem + (kt % kStages) * kStageBytes;
    auto tr16 = [&](int off0, int off1) {    // two transposing reads → one 16-byte fragment
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(base + off0));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(base + off1));
      u32x4_t r;
      r.x = (uint32_t)(uint16_t)lo.x | ((uint32_t)(uint16_t)lo.y << 16);
      r.y = (uint32_t)(uint16_t)lo.z | ((uint32_t)(uint16_t)lo.w << 16);
      r.z = (uint32_t)(uint16_t)hi.x | ((uint32_t)(uint16_t)hi.y << 16);
      r.w = (uint32_t)(uint16_t)hi.z | ((uint32_t)(uint16_t)hi.w << 16);
      return r;
    };
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[ss][i] = TA ? tr16(ta_off[TA ? ss : 0][i][0], ta_off[TA ? ss : 0][i][1])
                       : *(const u32x4_t*)(base + fa_off[ss][i]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[ss][j] = TB ? tr16(tb_off[TB ? ss : 0][j][0], tb_off[TB ? ss : 0][j][1])
                       : *(const u32x4_t*)(base + fb_off[ss][j]);
    }
    // the slot of stage kt − 1, read by both groups in earlier phases
    if (kt + kStages - 1 < KT) issue(kt + kStages - 1);
    // fragment reads complete before the barrier that releases this slot
    DMUON_WAIT_LGKM0();
  };
  // diagonal fragment of quarter R (A side: rows 16R .. of the 32-row block the
  // stage's k cover; B side: columns): this lane holds k = 8(l >> 4) + e (e < 8)
  // for row / column 16R + (l & 15); its only nonzero element is e = e0 + 16R
  // with e0 = (l & 15) − 8(l >> 4).
  // e0 passes through an empty asm so that the fragments are built inside the
  // (rarely taken) diagonal branch instead of being hoisted out of the K loop,
  // where they would hold registers for the whole contraction.
  auto diag_frag = [&](int e, uint32_t bits) {
    const uint32_t v = (e & 1) ? bits << 16 : bits;
    u32x4_t f;
    f.x = (unsigned)e < 2u ? v : 0u;
    f.y = (unsigned)(e - 2) < 2u ? v : 0u;
    f.z = (unsigned)(e - 4) < 2u ? v : 0u;
    f.w = (unsigned)(e - 6) < 2u ? v : 0u;
    return f;
  };
  auto mfma_phase = [&]() {
    __builtin_amdgcn_s_setprio(1);
    if constexpr (kQ) {
      // quarter (s, t): rows 16s of the wave's 128, columns 16t of its 64
      static_for<8>([&](auto S) {
        constexpr int qs = decltype(S)::value;
        static_for<4>([&](auto Tq) {
          constexpr int qt = decltype(Tq)::value;
          mfma_quarter<2 * (qs & 1) + (qt & 1)>(acc[qs >> 1][qt >> 1], fa[qs >> 2][qs & 3], fb[qt >> 1][qt & 1]);
        });
      });
    } else {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) mfma_chunk_f32(acc[i][j], fa[ss][i], fb[ss][j]);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // the extra MFMAs of a diagonal stage: block I of the wave's rows (A side) or
  // columns (B side)
  auto diag_phase = [&](auto I) {
    constexpr int b = decltype(I)::value;
    int e0 = (lane & 15) - 8 * (lane >> 4);
    asm volatile("" : "+v"(e0));
    __builtin_amdgcn_s_setprio(1);
    static_for<2>([&](auto Rq) {
      constexpr int R = decltype(Rq)::value;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32x4_t df = diag_frag(e0 + 16 * R, p ? dg.a2 : dg.a1);
        if constexpr (DIAG == 1) {
          // rows of quarter row R of block b against every column quarter
          static_for<4>([&](auto Tq) {
            constexpr int qt = decltype(Tq)::value;
            mfma_quarter<2 * R + (qt & 1)>(acc[b][qt >> 1], df, fb[qt >> 1][qt & 1]);
          });
        } else {
          // columns of quarter column R of block b against every row quarter
          static_for<8>([&](auto S) {
            constexpr int qs = decltype(S)::value;
            mfma_quarter<2 * (qs & 1) + R>(acc[qs >> 1][b], fa[qs >> 2][qs & 3], df);
          });
        }
      }
    });
    __builtin_amdgcn_s_setprio(0);
  };

  const int pro = KT < kStages - 1 ? KT : kStages - 1;
  for (int st = 0; st < pro; ++st) issue(st);
  if (pro == 3) DMUON_WAIT_VM(2 * kDmaPerStage);      // own share of stage 0
  else if (pro == 2) DMUON_WAIT_VM(kDmaPerStage);
  else DMUON_WAIT_VM(0);
  __builtin_amdgcn_s_barrier();
  if (!lead) __builtin_amdgcn_s_barrier();             // trailing group: one phase late
  __builtin_amdgcn_sched_barrier(0);
  auto step = [&](int kt) {
    mem_phase(kt);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfma_phase();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (DIAG == 0) {
#pragma unroll 1
    for (int kt = 0; kt < KT; ++kt) step(kt);
  } else {
    // every wave runs KT steps with the same barriers; its diagonal stages
    // [kb, kb + nb) (wide: its 4 row blocks, tall: its 2 column blocks) are
    // unrolled so that each names its accumulator block at compile time
    constexpr int nb = DIAG == 1 ? 4 : 2;
    const int kb = dg.kd0 + (DIAG == 1 ? 4 * wr : 2 * wc);
    const int k1 = kb < KT ? kb : KT;
#pragma unroll 1
    for (int kt = 0; kt < k1; ++kt) step(kt);
    auto dstep = [&](auto I) {
      const int kt = kb + decltype(I)::value;
      if (kt >= KT) return;
      mem_phase(kt);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      mfma_phase();
      diag_phase(I);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    dstep(std::integral_constant<int, 0>{});
    dstep(std::integral_constant<int, 1>{});
    if constexpr (nb == 4) {
      dstep(std::integral_constant<int, 2>{});
      dstep(std::integral_constant<int, 3>{});
    }
#pragma unroll 1
    for (int kt = kb + nb < KT ? kb + nb : KT; kt < KT; ++kt) step(kt);
  }
  if (lead) __builtin_amdgcn_s_barrier();              // every wave passes 2·KT + 2 barriers
  if constexpr (kQ) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) quarters_to_32x32(acc[i][j]);
  }
  // all LDS reads done before the caller reuses LDS
  __syncthreads();
}

// Position of accumulator register r of block (i, j) inside the 256×256 tile.
__device__ __forceinline__ int acc_row(int i, int rq) {   // rq = r >> 2; rows rq·8 + h·4 + 0..3
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 2) * 128 + i * 32 + rq * 8 + (lane >> 5) * 4;
}
__device__ __forceinline__ int acc_col(int j) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 3) * 64 + j * 32 + (lane & 31);
}

// Tile orders.  Consecutive logical tiles run on one XCD in runs of 16 or 64 (see
// xcd_logical_block), so the order decides how many operand panels one XCD's L2
// has to hold at once.  Both orders walk bands of tiles along one side of the
// output and advance the other side every band height, so the 32 apply tiles
// one XCD runs at once cover about 8 × 4 tiles and touch ~12 panels (a
// row-by-row order touched ~33: for an 8192 × 28672 matrix, all 32 panels of B'
// per XCD and round).  The Gram and the square, in runs of 16, walk bands of 4:
// a run covers about 4 × 4 tiles (8 panels, against 10 for 8 × 2).
constexpr int kBand = 8;
constexpr int kTriBand = 4;

// apply: R tiles along the short side, C along the long one; returns the
// short-side and long-side tile indices of logical tile u
__device__ __forceinline__ void band_tile(int u, int R, int C, int& ts, int& tl) {
  const int b = u / (kBand * C);
  const int r0 = b * kBand;
  const int gb = R - r0 < kBand ? R - r0 : kBand;
  const int v = u - b * kBand * C;
  ts = r0 + v % gb;
  tl = v / gb;
}

// Gram / square: upper-triangle tile u (ti ≤ tj) of a T×T grid.  Band b holds
// rows [BAND·b, BAND·b + h): first its triangle (tj from BAND·b to BAND·b + h − 1,
// each with the rows up to tj), then h rows for every later tj.
template <int BAND>
__device__ __forceinline__ void tri_tile(int u, int T, int& ti, int& tj) {
  int r0 = 0, start = 0;
  for (;;) {
    const int h = T - r0 < BAND ? T - r0 : BAND;
    const int n = h * (h + 1) / 2 + h * (T - r0 - h);
    if (u < start + n) {
      int v = u - start;
      const int tri = h * (h + 1) / 2;
      if (v < tri) {
        int k = 0;
        while ((k + 1) * (k + 2) / 2 <= v) ++k;
        ti = r0 + (v - k * (k + 1) / 2);
        tj = r0 + k;
      } else {
        v -= tri;
        ti = r0 + v % h;
        tj = r0 + h + v / h;
      }
      return;
    }
    start += n;
    r0 += BAND;
  }
}

// Logical workgroup index.  Workgroups are handed to the 8 XCDs round-robin in
// launch order, so workgroup b runs on XCD b % 8 as its (b / 8)-th workgroup.
// The logical tile list is consumed in windows of 8·RUN tiles: inside a window
// each XCD takes RUN consecutive tiles (neighbours share operand panels in that
// XCD's L2), and all XCDs advance through the list together, so tiles of
// unequal cost (long-K problems first) are spread over every XCD.  A last
// partial window of R tiles is split the same way into 8 contiguous runs (the
// first R % 8 XCDs take one tile more).  The map is a bijection on [0, G).
// Runs of 64 suit the apply (two rounds of 8 × 4 tiles per XCD); the Gram and
// the square (triangle tiles in bands of 4) measured faster with runs of 16.
template <int RUN>
__device__ __forceinline__ int xcd_logical_block() {
  const int G = gridDim.x, b = blockIdx.x;
  constexpr int win = 8 * RUN;
  const int w = b / win;
  const int xcd = b & 7, slot = (b >> 3) - w * RUN;
  if ((w + 1) * win <= G) return w * win + xcd * RUN + slot;
  const int R = G - w * win, per = R >> 3, rem = R & 7;
  return w * win + (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
}

// ---- Gram / square epilogue.  Each 128-row half of the tile is staged in LDS
// (fp32); a row pass writes the row-major block with 8- or 16-byte vectors and a
// column pass writes the mirrored block of an off-diagonal tile.
//   Gram:   A' = xs²·acc − d·I   (xs = inv at t = 0, whose operands are B; else 1)
//   square: B' = (b + 2cd)·A' + c·acc   (acc = A'·A'ᵀ = A'² since A' is symmetric)
template <typename T, int PH>
__device__ __forceinline__ void sym_epilogue(const DevProblem& P, const LaunchScalars& s,
                                             f32x16_t (&acc)[4][2], char* smem, int slice, int ti,
                                             int tj, int row0, int col0, float d, float xs) {
  const int tid = threadIdx.x;
  const int m = P.m, ldm = P.ld_m;
  T* dst = (T*)(PH == PH_GRAM ? P.ap : P.bp) + (int64_t)slice * m * ldm;
  T* dstT = ti != tj ? dst : nullptr;
  const T* aprime = (const T*)P.ap + (int64_t)slice * m * ldm;
  const float lin = s.b + 2.f * s.c * d;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3, h = lane >> 5, r32 = lane & 31;
#pragma unroll 1
  for (int hf = 0; hf < 2; ++hf) {
    // (1) the four waves holding rows [128·hf, 128·hf + 128) stage their accumulators
    if (wr == hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
            const int cc = wc * 64 + j * 32 + r32;
            *(float*)(smem + stage_off(rr, cc)) = acc[i][j][r];
          }
    }
    __syncthreads();
    // (2) row pass: 128 rows × 64 chunks of 4 columns, in two batches of 8 chunks
    // per thread; each batch issues all its global loads before any store, since
    // loads and stores share one in-order completion counter.
#pragma unroll 1
    for (int kb = 0; kb < 16; kb += 8) {
      float4 xin[8];
      uint2 ain[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int id = tid + kGemmThreads * (kb + q);
        const int rr = id >> 6, cq = id & 63;
        const int gr = row0 + hf * 128 + rr, gc = col0 + 4 * cq;
        xin[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        ain[q] = make_uint2(0u, 0u);
        if (PH == PH_SQUARE && gr < m && gc < ldm) {
          if (sizeof(T) == 2) ain[q] = *(const uint2*)(aprime + (int64_t)gr * ldm + gc);
          else xin[q] = *(const float4*)(aprime + (int64_t)gr * ldm + gc);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int id = tid + kGemmThreads * (kb + q);
        const int rr = id >> 6, cq = id & 63;
        float* sp = (float*)(smem + rr * 1024 + ((cq ^ ((rr >> 3) & 15)) << 4));
        const float4 a4 = *(const float4*)sp;
        float v[4] = {a4.x, a4.y, a4.z, a4.w};
        const int gr = row0 + hf * 128 + rr, gc = col0 + 4 * cq;
        const bool rok = gr < m;
        if (PH == PH_GRAM) {
          const float gsc = xs * xs;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] *= gsc;
            if (gr == gc + e && rok) v[e] -= d;
          }
        } else {
          float ap[4];
          if (sizeof(T) == 2) {
            ap[0] = __uint_as_float(ain[q].x << 16); ap[1] = __uint_as_float(ain[q].x & 0xffff0000u);
            ap[2] = __uint_as_float(ain[q].y << 16); ap[3] = __uint_as_float(ain[q].y & 0xffff0000u);
          } else {
            ap[0] = xin[q].x; ap[1] = xin[q].y; ap[2] = xin[q].z; ap[3] = xin[q].w;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(lin, ap[e], s.c * v[e]);
        }
        if (rok && gc < ldm) store4(dst + (int64_t)gr * ldm + gc, v[0], v[1], v[2], v[3]);
        if (dstT) *(float4*)sp = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
    // (3) column pass: rows of the mirrored block = tile columns
    if (dstT) {
      constexpr int RPC = 16 / (int)sizeof(T);          // rows per 16-byte chunk
      constexpr int CPC = 128 / RPC;                    // chunks per column (this half)
#pragma unroll 2
      for (int k = 0; k < (256 * CPC) / kGemmThreads; ++k) {
        const int id = tid + kGemmThreads * k;
        const int cc = id / CPC, rg = id % CPC;
        const int trow = col0 + cc;
        const int tcol = row0 + hf * 128 + rg * RPC;
        if (trow >= m || tcol >= ldm) continue;
        float v[RPC];
#pragma unroll
        for (int e = 0; e < RPC; ++e) v[e] = *(const float*)(smem + stage_off(rg * RPC + e, cc));
        store_row16(dstT + (int64_t)trow * ldm + tcol, v);
      }
    }
    __syncthreads();
  }
}

// ---- square epilogue on the bf16 path: B' = (b + 2cd)·A' + c·acc, as in
// sym_epilogue, but the row pass takes 8 columns per lane and chunk (16-byte
// loads of A' and 16-byte stores of B'), and each half's A' values are loaded
// one step early (the first half's before its staging, the second half's after
// the first half's row pass), so their latency overlaps the staging, the column
// pass and the barriers instead of stalling the row pass.
template <typename T>
__device__ __forceinline__ void square_epilogue(const DevProblem& P, const LaunchScalars& s,
                                                f32x16_t (&acc)[4][2], char* smem, int slice, int ti,
                                                int tj, int row0, int col0, float d) {
  static_assert(sizeof(T) == 2, "bf16 path");
  const int tid = threadIdx.x;
  const int m = P.m, ldm = P.ld_m;
  T* dst = (T*)P.bp + (int64_t)slice * m * ldm;
  T* dstT = ti != tj ? dst : nullptr;
  const T* aprime = (const T*)P.ap + (int64_t)slice * m * ldm;
  const float lin = s.b + 2.f * s.c * d;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3, h = lane >> 5, r32 = lane & 31;
  // row pass: 128 rows × 32 chunks of 8 columns per half, 8 chunks per thread;
  // chunk q of this thread: row (tid + 512q) / 32, columns 8·((tid + 512q) % 32)
  constexpr int kQ = 8;
  u32x4_t ain[kQ];
  auto load_ap = [&](int hf) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int id = tid + kGemmThreads * q;
      const int gr = row0 + hf * 128 + (id >> 5), gc = col0 + 8 * (id & 31);
      ain[q] = gr < m && gc < ldm ? __builtin_nontemporal_load((const u32x4_t*)(aprime + (int64_t)gr * ldm + gc))  // last read of A'
                                  : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  load_ap(0);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    // (1) the four waves holding rows [128·hf, 128·hf + 128) stage their accumulators
    if (wr == hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
            const int cc = wc * 64 + j * 32 + r32;
            *(float*)(smem + stage_off8(rr, cc)) = acc[i][j][r];
          }
    }
    __syncthreads();
    // (2) row pass
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int id = tid + kGemmThreads * q;
      const int rr = id >> 5, c8 = id & 31;
      float* sp0 = (float*)(smem + stage_off8(rr, 8 * c8));
      float* sp1 = (float*)(smem + stage_off8(rr, 8 * c8 + 4));
      const float4 a0 = *(const float4*)sp0, a1 = *(const float4*)sp1;
      const float c_[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const uint32_t w[4] = {ain[q].x, ain[q].y, ain[q].z, ain[q].w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = fmaf(lin, __uint_as_float(w[e] << 16), s.c * c_[2 * e]);
        v[2 * e + 1] = fmaf(lin, __uint_as_float(w[e] & 0xffff0000u), s.c * c_[2 * e + 1]);
      }
      const int gr = row0 + hf * 128 + rr, gc = col0 + 8 * c8;
      if (gr < m && gc < ldm) store_row16(dst + (int64_t)gr * ldm + gc, v);
      if (dstT) {
        *(float4*)sp0 = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)sp1 = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
    if (hf == 0) load_ap(1);
    __syncthreads();
    // (3) column pass: rows of the mirrored block = tile columns
    if (dstT) {
      constexpr int RPC = 8;                            // rows per 16-byte chunk
      constexpr int CPC = 128 / RPC;                    // chunks per column (this half)
#pragma unroll 2
      for (int k = 0; k < (256 * CPC) / kGemmThreads; ++k) {
        const int id = tid + kGemmThreads * k;
        const int cc = id / CPC, rg = id % CPC;
        const int trow = col0 + cc;
        const int tcol = row0 + hf * 128 + rg * RPC;
        if (trow >= m || tcol >= ldm) continue;
        float v[RPC];
#pragma unroll
        for (int e = 0; e < RPC; ++e) v[e] = *(const float*)(smem + stage_off8(rg * RPC + e, cc));
        store_row16(dstT + (int64_t)trow * ldm + tcol, v);
      }
    }
    __syncthreads();
  }
}

// value of the neighbouring lane (lane ^ 1)
__device__ __forceinline__ float swap_adjacent(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// ---- apply epilogue, in the accumulator layout.
// Lane (h, r32) of wave (wr, wc) holds, for block (i, j) and register r = 4·rq + e,
// the element at tile row 128·wr + 32·i + 8·rq + 4·h + e and tile column
// 64·wc + 32·j + r32.  Per block:
//   X' = xs·(α·X + acc), α = a + b·d + c·d² (xs = 0 for columns past the
//        matrix, whose accumulators hold finite values read past a row's end).
//        fp32 path: at t = 0 X is read from the unscaled source x0 (B, storage
//        layout, 4-byte accesses: each wave instruction covers two 128-byte row
//        segments) and xs = inv; later xs = 1 and X is the stored fp32 iterate,
//        kept in the order of the registers (16-byte pieces per lane, 1 KiB
//        contiguous per wave instruction, 4 loads and 4 stores per block).
//        bf16 path: X = hi + lo with hi its bf16 operand copy.  The contraction
//        already added α·hi (diagonal MFMAs, see DiagTerm), so the epilogue adds
//        α·lo: at t = 0 lo = x0 − bf16(x0) from the fp32 source; later lo is
//        stored in register order as 16 signed bytes per lane and block (one
//        16-byte load and store) with a shared exponent byte (enc_lo).
//        Traffic touched once per phase (the iterate, the copy, the master
//        weight) uses the nontemporal cache policy.
//   t < k−1: the storage-layout operand copy (fp32 path: also the transposed
//        copy); Σ X'² partial
//   last:  W ← (1 − lr·wd)·W − lr·X', optional copy of X' to the output and
//        bf16 copy of W (two columns per dword: even lanes take rows e = 0, 2
//        from their odd neighbour, odd lanes rows 1, 3).
// The bf16 copy of X' goes out through LDS (free once the contraction is done):
// during the block loop each lane writes its values as 16-bit bf16 into a
// row-swizzled 256×256 tile; after the Σ X'² reduction the tile is stored as
// 16-byte pieces of whole rows.  The bf16 path keeps only this storage-layout copy: every
// bf16 contraction reads it row-major or K-major.  The fp32 path (no K-major
// reads) stores the row-major and the transposed copy directly.
template <typename T, bool LAST, bool FROM0>
struct ApplyEpilogue {
  static constexpr unsigned E = sizeof(T);
  static constexpr int kAhead = LAST ? 2 : 4;
  // blocks loaded before the contraction (live across it: two of the fp32 start
  // blocks on the bf16 path's first iteration, whose contraction also holds the
  // diagonal term's registers)
  static constexpr int kPre = LAST ? 1 : (FROM0 && E == 2 ? 2 : 3);
  // registers per loaded block: 16 fp32 values (the fp32 start X₀ = inv·B at
  // t = 0, or the fp32 iterate), or q (4 dwords) + exponent on the bf16 path
  static constexpr int kIn = FROM0 || E != 2 ? 16 : 5;
  // fp32 path: the iterate in fp32, 4 dwords per 4 values.  bf16 path: the
  // iterate is its bf16 operand copy hi (storage layout) plus lo = X − hi in
  // register order, 16 signed bytes per lane and block with one shared
  // exponent byte: kTile² bytes of q, then kTile²/16 exponent bytes per tile
  static constexpr int kXWords = 4;
  static constexpr unsigned kLoBytes = (unsigned)(kTile * kTile);
  static constexpr int64_t kTileIterBytes = E == 2 ? (int64_t)kTile * kTile * 17 / 16 : (int64_t)kTile * kTile * 4;

  __amdgpu_buffer_rsrc_t rx, ri, rw, ro, rd, rt, rp;
  unsigned xi[2], wo[2], dofs[2], tofs[2], po[2];
  unsigned xb, xe, ldi, ld_s, ld_t, cols;
  unsigned lr0;
  int row0, col0;
  bool odd, pub_pairs;
  static constexpr bool from0 = FROM0;
  bool colok[2];                         // the lane's column of block j lies inside the matrix
  bool has_w, has_out, has_pub;          // last apply: which outputs exist (workgroup-uniform)
  float xin[kAhead][kIn];
  float win[LAST ? kAhead : 1][16];

  __device__ __forceinline__ ApplyEpilogue(const DevProblem& P, const LaunchScalars& s, int slice, int u,
                                           int row0_, int col0_) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 2, wc = wave & 3, h = lane >> 5, r32 = lane & 31;
    const int rows = P.rows;
    row0 = row0_;
    col0 = col0_;
    cols = (unsigned)P.cols;
    const int trows = rows - row0 < kTile ? rows - row0 : kTile;
    const int tcols = P.cols - col0 < kTile ? P.cols - col0 : kTile;
    lr0 = (unsigned)(wr * 128 + h * 4);                 // tile row of register e = 0 (i = rq = 0)
    const int lc0 = wc * 64 + r32;                      // tile column of block j = 0
    odd = (lane & 1) != 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) colok[j] = lc0 + 32 * j < tcols;

    // the iterate's tile: fp32 byte (((wave·8 + blk)·4 + rq)·64 + lane)·16; bf16
    // path q at ((wave·8 + blk)·64 + lane)·16, exponent at kLoBytes + (wave·8 + blk)·64 + lane
    rx = range_rsrc((const char*)P.xf + ((int64_t)slice * P.apply_tr * P.apply_tc + u) * kTileIterBytes,
                    kTileIterBytes);
    xb = (unsigned)((wave * 8 * (E == 2 ? 1 : kXWords) * 64 + lane) * 16);
    xe = kLoBytes + (unsigned)(wave * 8 * 64 + lane);
    // the X₀ read at t = 0: the unscaled source in storage layout
    ldi = (unsigned)P.ld_x0;
    ri = range_rsrc(from0 ? P.x0 + ((int64_t)slice * rows + row0) * ldi : nullptr, (int64_t)trows * ldi * 4);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      xi[j] = lc0 + 32 * j < tcols ? (lr0 * ldi + (unsigned)(col0 + lc0 + 32 * j)) * 4u : kOob;

    rw = ro = rd = rt = rp = rx;
    ld_s = ld_t = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) wo[j] = dofs[j] = tofs[j] = po[j] = 0;
    // published bf16 copy: two columns per dword when rows hold an even number of
    // columns (a pair never straddles rows), else one 16-bit store per element
    pub_pairs = (P.cols & 1) == 0;
    has_w = __builtin_amdgcn_readfirstlane(s.write_master ? 1 : 0) != 0;
    has_out = __builtin_amdgcn_readfirstlane(P.out ? 1 : 0) != 0;
    has_pub = __builtin_amdgcn_readfirstlane(s.write_master && P.pub ? 1 : 0) != 0;
    if (LAST) {
      const int64_t first = ((int64_t)slice * rows + row0) * P.cols, bytes = (int64_t)trows * P.cols * 4;
      rw = range_rsrc(s.write_master ? P.master + first : nullptr, bytes);
      ro = range_rsrc(P.out ? P.out + first : nullptr, bytes);
      rp = range_rsrc(s.write_master && P.pub ? P.pub + first : nullptr, (int64_t)trows * P.cols * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        wo[j] = lc0 + 32 * j < tcols ? (lr0 * cols + (unsigned)(col0 + lc0 + 32 * j)) * 4u : kOob;
        const unsigned gc = (unsigned)(col0 + lc0 + 32 * j);
        po[j] = lc0 + 32 * j < tcols
                    ? (pub_pairs ? ((lr0 + (odd ? 1u : 0u)) * cols + (gc & ~1u)) * 2u : (lr0 * cols + gc) * 2u)
                    : kOob;
      }
    } else {
      ld_s = (unsigned)(P.wide ? P.ld_n : P.ld_m);
      ld_t = (unsigned)(P.wide ? P.ld_m : P.ld_n);
      // bf16: the next storage-layout copy; fp32: the row-major and transposed copies
      void* xa_next = (s.t & 1) ? P.xa0 : P.xa1;
      const T* dst = (const T*)(E == 2 ? P.xs[(s.t + 1) & 1] : (P.wide ? P.xg : xa_next)) +
                     (int64_t)slice * rows * ld_s;
      rd = range_rsrc(dst + (int64_t)row0 * ld_s, (int64_t)trows * ld_s * E);
      if (E != 2) {
        const T* dstT = (const T*)(P.wide ? xa_next : P.xg) + (int64_t)slice * P.cols * ld_t;
        rt = range_rsrc(dstT + (int64_t)col0 * ld_t, (int64_t)tcols * ld_t * E);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // row-major copy: the lane's dword starts at an even column
        const unsigned gc = (unsigned)(col0 + lc0 + 32 * j);
        const unsigned gce = E == 2 ? (gc & ~1u) : gc;
        dofs[j] = gce < ld_s ? ((lr0 + (E == 2 && odd ? 1u : 0u)) * ld_s + gce) * E : kOob;
        // transposed copy: row (lc0 + 32 j) of the range, columns from row0 + lr0
        tofs[j] = ((unsigned)(lc0 + 32 * j) * ld_t + (unsigned)row0 + lr0) * E;
      }
    }
  }

  // byte offset of 16-byte piece q of block blk in the iterate's tile
  __device__ __forceinline__ unsigned xq(int blk, int q) const {
    return xb + (unsigned)((blk * (E == 2 ? 1 : kXWords) + q) * 64 * 16);
  }

  // bf16 path: lo = X − hi of the lane's 16 values in a block, as signed bytes
  // q with one shared exponent byte eb (0: all zero).  With mx = max |lo| and
  // eb its biased fp32 exponent, q = rint(lo · 2^(133 − eb)) has |q| ≤ 127 and
  // lo = q · 2^(eb − 133) to within 2^(eb − 134) ≤ mx · 2⁻⁸; since |lo| is at most
  // half a bf16 ulp of X, the stored X keeps about 16 significant bits of the
  // block's largest value.
  static __device__ __forceinline__ void enc_lo(const float (&lo)[16], u32x4_t& q, uint32_t& eb) {
    float mx = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(lo[r]));
    const uint32_t e = (__float_as_uint(mx) >> 23) & 0xFFu;
    eb = e < 8u ? 0u : e;
    const float sc = eb ? __uint_as_float((260u - eb) << 23) : 0.f;
    uint32_t w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t acc = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int qi = (int)__builtin_rintf(fminf(fmaxf(lo[4 * g + b] * sc, -127.f), 127.f));
        acc |= ((uint32_t)qi & 0xFFu) << (8 * b);
      }
      w[g] = acc;
    }
    q = u32x4_t{w[0], w[1], w[2], w[3]};
  }
  static __device__ __forceinline__ void dec_lo(const float (&in)[kIn], float (&lo)[16]) {
    const uint32_t eb = __float_as_uint(in[4]);
    const float sc = eb ? __uint_as_float((eb - 6u) << 23) : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = __builtin_amdgcn_sbfe((int)__float_as_uint(in[r >> 2]), 8 * (r & 3), 8);
      lo[r] = (float)qi * sc;
    }
  }

  __device__ __forceinline__ void load_blk(int blk, int slot) {
    const int i = blk >> 1, j = blk & 1;
    if constexpr (FROM0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned rr = (unsigned)(32 * i + 8 * (r >> 2) + (r & 3));
        xin[slot][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ri, (int)(xi[j] + rr * ldi * 4u), 0, 2));  // nt
      }
    } else if constexpr (E == 2) {
      const f32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)xq(blk, 0), 0, 2);     // nontemporal
      xin[slot][0] = w.x; xin[slot][1] = w.y; xin[slot][2] = w.z; xin[slot][3] = w.w;
      xin[slot][4] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
          rx, (int)(xe + (unsigned)(blk * 64)), 0, 2));
    } else {
#pragma unroll
      for (int q = 0; q < kXWords; ++q) {
        const f32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)xq(blk, q), 0, 2);   // nontemporal
        xin[slot][4 * q] = w.x; xin[slot][4 * q + 1] = w.y;
        xin[slot][4 * q + 2] = w.z; xin[slot][4 * q + 3] = w.w;
      }
    }
    if (LAST && has_w) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned rr = (unsigned)(32 * i + 8 * (r >> 2) + (r & 3));
        // the master weight is read and written once per step: nontemporal
        win[LAST ? slot : 0][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, (int)(wo[j] + rr * cols * 4u), 0, 2));
      }
    }
  }

  __device__ __forceinline__ void prefetch() {
#pragma unroll
    for (int b = 0; b < kPre; ++b) load_blk(b, b);
  }

  // 16-byte-piece swizzle of the LDS-staged row-major tile: the four rows one
  // dword store instruction writes (r, r + 1, r + 4, r + 5 for r ≡ 0 or 2 mod 8)
  // land in four different bank quarters
  static __device__ __forceinline__ unsigned row_swz(unsigned r) {
    return ((r & 1u) | ((r >> 1) & 2u)) << 2;
  }

  __device__ __forceinline__ void finish(const DevProblem& P, const LaunchScalars& s, f32x16_t (&acc)[4][2],
                                         int slice, int u, float d, float xs, char* smem, float* red) {
    constexpr bool kStage = E == 2 && !LAST;
    // bf16 copy (storage layout): each block's dwords (two columns of one row)
    // go into a row-major 256×256 bf16 tile in LDS (free since the contraction's
    // last barrier), whose 16-byte pieces are XOR-swizzled by row_swz; whole rows
    // go out after the block loop
    const unsigned lc0 = (unsigned)(((threadIdx.x >> 6) & 3) * 64 + (threadIdx.x & 31));
    const float alpha = s.a + s.b * d + s.c * d * d;
    // the value's scale, zero for columns past the matrix (their accumulators
    // hold finite values read past a row's end: the next row or padding)
    const float xsj[2] = {colok[0] ? xs : 0.f, colok[1] ? xs : 0.f};
    float sq = 0.f;
#pragma unroll
    for (int b = kPre; b < kAhead; ++b) load_blk(b, b);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int slot = blk % kAhead;
      const int i = blk >> 1, j = blk & 1;
      float v[16];
      if constexpr (E == 2) {
        // the accumulator already holds α·hi (diagonal MFMAs); add α·lo, with
        // lo = X₀ − bf16(X₀) at t = 0 (the operand was bf16 of the fp32 start)
        if constexpr (FROM0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = xin[slot][r] - bf16_to_f32(f32_to_bf16(xin[slot][r]));
        } else {
          dec_lo(xin[slot], v);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = xin[slot][r % kIn];
      }
      // columns past the matrix are zero: a K-major operand can feed them values
      // read past a row's end, which must not reach Σ X'² or any store
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = xsj[j] * fmaf(alpha, v[r], acc[i][j][r]);
      if (LAST) {
        float w[16];
        if (has_out) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned rr = (unsigned)(32 * i + 8 * (r >> 2) + (r & 3));
            buf_st(ro, wo[j] + rr * cols * 4u, v[r]);
          }
        }
        if (has_w) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned rr = (unsigned)(32 * i + 8 * (r >> 2) + (r & 3));
            w[r] = fmaf(-s.lr, v[r], s.decay * win[LAST ? slot : 0][r]);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(w[r]), rw, (int)(wo[j] + rr * cols * 4u), 0, 2);
          }
        }
        if (!has_pub) {
        } else if (pub_pairs) {
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
#pragma unroll
            for (int pe = 0; pe < 2; ++pe) {
              const float w0 = w[4 * rq + 2 * pe], w1 = w[4 * rq + 2 * pe + 1];
              const float got = swap_adjacent(odd ? w0 : w1);
              const unsigned rr = (unsigned)(32 * i + 8 * rq + 2 * pe);
              buf_st(rp, po[j] + rr * cols * 2u, odd ? pack_bf16x2(got, w1) : pack_bf16x2(w0, got));
            }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned rr = (unsigned)(32 * i + 8 * (r >> 2) + (r & 3));
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(w[r]), rp, (int)(po[j] + rr * cols * 2u), 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sq = fmaf(v[r], v[r], sq);
        if constexpr (E == 2) {
          // hi = bf16(X') goes into the LDS-staged copy; v keeps lo = X' − hi
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
#pragma unroll
            for (int e = 0; e < 4; ++e) {           // one 16-bit value per row
              const unsigned cb = (lc0 + 32u * (unsigned)j) * 2u;            // byte of the column in its row
              const unsigned r = lr0 + 32u * (unsigned)i + 8u * (unsigned)rq + (unsigned)e;
              const uint16_t hb = f32_to_bf16(v[4 * rq + e]);
              *(__attribute__((address_space(3))) uint16_t*)(smem + r * 512u + ((((cb >> 4) ^ row_swz(r)) << 4) | (cb & 15u))) = hb;
              v[4 * rq + e] -= bf16_to_f32(hb);
            }
          u32x4_t q;
          uint32_t eb;
          enc_lo(v, q, eb);
          // nontemporal (cache policy 2): read again only by the next apply
          __builtin_amdgcn_raw_buffer_store_b128(q, rx, (int)xq(blk, 0), 0, 2);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)eb, rx, (int)(xe + (unsigned)(blk * 64)), 0, 2);
        } else {
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            __builtin_amdgcn_raw_buffer_store_b128(
                f32x4_t{v[4 * rq], v[4 * rq + 1], v[4 * rq + 2], v[4 * rq + 3]}, rx, (int)xq(blk, rq), 0, 0);
        }
        // fp32 path: the transposed copy, four consecutive rows of one column
        if constexpr (E != 2) {
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const unsigned rr = (unsigned)(32 * i + 8 * rq);
            const unsigned o = (unsigned)row0 + lr0 + rr < ld_t ? tofs[j] + rr * E : kOob;
            const u32x4_t w4 = {__float_as_uint(v[4 * rq]), __float_as_uint(v[4 * rq + 1]),
                                __float_as_uint(v[4 * rq + 2]), __float_as_uint(v[4 * rq + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(w4, rt, (int)o, 0, 0);
          }
        }
        // fp32 path: the row-major copy (the bf16 copy went into LDS above)
        if constexpr (E != 2) {
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const unsigned rr = (unsigned)(32 * i + 8 * rq + e);
              buf_st(rd, dofs[j] + rr * ld_s * E, v[4 * rq + e]);
            }
        }
      }
      if (blk + kAhead < 8) load_blk(blk + kAhead, slot);
    }
    if (!LAST) {
      const float tot = block_sum<kGemmWaves>(sq, red);
      if (threadIdx.x == 0) P.part_apply[(int64_t)slice * P.apply_tr * P.apply_tc + u] = tot;
    }
    if constexpr (kStage) {
      // the staged copy: 16-byte pieces of whole rows go out
      __syncthreads();
#pragma unroll 4
      for (int k = 0; k < 16; ++k) {
        const unsigned id = threadIdx.x + (unsigned)kGemmThreads * k;
        const unsigned r = id >> 5, q = id & 31;
        const u32x4_t p = *(const __attribute__((address_space(3))) u32x4_t*)(smem + r * 512u + ((q ^ row_swz(r)) << 4));
        const unsigned c = (unsigned)col0 + 8u * q;
        const unsigned o = c < ld_s ? (r * ld_s + c) * 2u : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(p, rd, (int)o, 0, 2);   // nontemporal
      }
    }
  }
};

template <typename T, int PH, bool LAST, bool FROM0 = false>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(LaunchTable tab, LaunchScalars s) {
  extern __shared__ __align__(16) char smem[];
  __shared__ float red[kGemmWaves];
  constexpr int kElemsPerRow = kRowBytes / (int)sizeof(T);
  constexpr bool kKmaj = sizeof(T) == 2;     // bf16: one storage-layout copy of X, K-major reads
  const int bid = xcd_logical_block<PH == PH_APPLY ? 64 : 16>();
  const int p = find_prob(tab.wg_prefix + PH * (tab.n_probs + 1), tab.n_probs, bid);
  const DevProblem& P = tab.probs[p];
  if (P.tag != tab.tag) return;      // the workspace holds another plan's table
  const int local = bid - P.wg0[PH];
  const int m = P.m;

  Operands op;
  op.cola_b = op.colb_b = 0;
  int slice, row0, col0, ti = 0, tj = 0, u;
  if (PH == PH_GRAM || PH == PH_SQUARE) {
    const int T_ = P.tiles_m;
    const int per = T_ * (T_ + 1) / 2;
    slice = local / per;
    u = local % per;
    tri_tile<kTriBand>(u, T_, ti, tj);
    row0 = ti * kTile;
    col0 = tj * kTile;
    const int ld = PH == PH_GRAM ? P.ld_n : P.ld_m;
    const T* base = PH == PH_GRAM ? (const T*)P.xg + (int64_t)slice * m * P.ld_n
                                  : (const T*)P.ap + (int64_t)slice * m * P.ld_m;
    op.a = (const char*)(base + (int64_t)row0 * ld);
    op.b = (const char*)(base + (int64_t)col0 * ld);
    op.lda_b = op.ldb_b = ld * (int)sizeof(T);
    op.rows_a = m - row0;
    op.rows_b = m - col0;
    op.ktiles = ld / kElemsPerRow;
    if constexpr (kKmaj) {
      if (PH == PH_GRAM) {
        // X in storage layout: a wide slice's rows are rows of X (row-major
        // operands), a tall slice's rows are its columns (K-major operands)
        const int ld_s = P.wide ? P.ld_n : P.ld_m;
        const T* xs = (const T*)P.xs[s.t & 1] + (int64_t)slice * P.rows * ld_s;
        op.a = (const char*)(P.wide ? xs + (int64_t)row0 * ld_s : xs);
        op.b = (const char*)(P.wide ? xs + (int64_t)col0 * ld_s : xs);
        op.lda_b = op.ldb_b = ld_s * (int)sizeof(T);
        if (!P.wide) {
          op.rows_a = op.rows_b = P.rows;
          op.cola_b = row0 * (int)sizeof(T);
          op.colb_b = col0 * (int)sizeof(T);
        }
      }
    }
  } else {  // PH_APPLY: bands along the short (m) side, see band_tile
    const int per = P.apply_tr * P.apply_tc;
    slice = local / per;
    u = local % per;
    int tr, tc;
    if (P.wide) band_tile(u, P.apply_tr, P.apply_tc, tr, tc);
    else band_tile(u, P.apply_tc, P.apply_tr, tc, tr);
    u = tr * P.apply_tc + tc;           // partial-sum slot in row-major tile order
    row0 = tr * kTile;
    col0 = tc * kTile;
    const T* bp = (const T*)P.bp + (int64_t)slice * m * P.ld_m;
    op.ktiles = P.ld_m / kElemsPerRow;
    op.lda_b = op.ldb_b = P.ld_m * (int)sizeof(T);
    if constexpr (kKmaj) {
      // wide: B′·X with X K-major (its storage rows are k); tall: S·B′ with the
      // storage rows of S row-major and B′ (symmetric) K-major
      const T* xs = (const T*)P.xs[s.t & 1] + (int64_t)slice * P.rows * (P.wide ? P.ld_n : P.ld_m);
      op.colb_b = col0 * (int)sizeof(T);
      if (P.wide) {
        op.a = (const char*)(bp + (int64_t)row0 * P.ld_m);
        op.b = (const char*)xs;
        op.ldb_b = P.ld_n * (int)sizeof(T);
        op.rows_a = P.rows - row0;
        op.rows_b = P.rows;
      } else {
        op.a = (const char*)(xs + (int64_t)row0 * P.ld_m);
        op.b = (const char*)bp;
        op.rows_a = P.rows - row0;
        op.rows_b = m;
      }
    } else {
      const T* xa = (const T*)((s.t & 1) ? P.xa1 : P.xa0) + (int64_t)slice * P.n * P.ld_m;
      const T* pa = P.wide ? bp : xa;     // rows of the output = storage rows
      const T* pb = P.wide ? xa : bp;     // cols of the output = storage cols
      op.a = (const char*)(pa + (int64_t)row0 * P.ld_m);
      op.b = (const char*)(pb + (int64_t)col0 * P.ld_m);
      op.rows_a = P.rows - row0;
      op.rows_b = P.cols - col0;
    }
  }
  float* scal = tab.scal + (int64_t)(P.slice_base + slice) * kScalStride;

  // d_t: at t = 0 from the norm kernel; later the sum of the previous apply's
  // per-tile Σ X² partials (fixed order, identical in every workgroup).
  float d;
  if (PH == PH_GRAM && s.t > 0) {
    const int cnt = P.apply_tr * P.apply_tc;
    d = sum_partials<kGemmWaves>(P.part_apply + (int64_t)slice * cnt, cnt, red) / (float)m;
    if (u == 0 && threadIdx.x == 0) scal[1 + s.t] = d;
  } else {
    d = scal[1 + s.t];
  }

  // X₀ = inv·B enters through its operands' scale (see the epilogues)
  const float xs = s.t == 0 && PH != PH_SQUARE ? scal[0] : 1.f;

  f32x16_t acc[4][2];
  if constexpr (PH == PH_APPLY) {
    ApplyEpilogue<T, LAST, FROM0> epi(P, s, slice, u, row0, col0);
    epi.prefetch();
    if constexpr (kKmaj) {
      // α·hi on the matrix cores: the diagonal block of the B′ side, A for a
      // wide slice (rows of the tile), B for a tall one (its columns)
      const float alpha = s.a + s.b * d + s.c * d * d;
      DiagTerm dg;
      const uint16_t a1 = f32_to_bf16(alpha);
      dg.a1 = a1;
      dg.a2 = f32_to_bf16(alpha - bf16_to_f32(a1));
      dg.kd0 = (P.wide ? row0 : col0) / 32;
      if (P.wide) gemm_mainloop<T, false, true, 1>(op, smem, acc, dg);
      else gemm_mainloop<T, false, true, 2>(op, smem, acc, dg);
    } else {
      gemm_mainloop<T>(op, smem, acc);
    }
    epi.finish(P, s, acc, slice, u, d, xs, smem, red);
  } else {
    if constexpr (!kKmaj || PH == PH_SQUARE) {
      gemm_mainloop<T>(op, smem, acc);
    } else {
      if (P.wide) gemm_mainloop<T, false, false>(op, smem, acc);
      else gemm_mainloop<T, true, true>(op, smem, acc);
    }
    if constexpr (PH == PH_SQUARE && sizeof(T) == 2) square_epilogue<T>(P, s, acc, smem, slice, ti, tj, row0, col0, d);
    else sym_epilogue<T, PH>(P, s, acc, smem, slice, ti, tj, row0, col0, d, xs);
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
__global__ __launch_bounds__(kGemmThreads) void k_gemm_plain(GemmArgs g) {
  extern __shared__ __align__(16) char smem[];
  const int row0 = (blockIdx.x / g.tiles_n) * kTile;
  const int col0 = (blockIdx.x % g.tiles_n) * kTile;
  Operands op;
  op.a = (const char*)((const T*)g.A + row0 * g.lda);
  op.b = (const char*)((const T*)g.B + col0 * g.ldb);
  op.lda_b = (int)(g.lda * (int64_t)sizeof(T));
  op.ldb_b = (int)(g.ldb * (int64_t)sizeof(T));
  op.rows_a = (int)(g.M - row0);
  op.rows_b = (int)(g.N - col0);
  op.cola_b = op.colb_b = 0;
  op.ktiles = g.ktiles;
  f32x16_t acc[4][2];
  gemm_mainloop<T>(op, smem, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t gc = col0 + acc_col(j);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gr = row0 + acc_row(i, r >> 2) + (r & 3);
        if (gr < g.M && gc < g.N) g.C[gr * g.ldc + gc] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------
// table writer: one workgroup copies one piece of a host-built table from its
// kernel arguments to device memory
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_write_table(TableChunk c) {
  for (int i = threadIdx.x; i < c.n_words; i += kThreads) glob(c.dst)[i] = c.words[i];
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <typename K>
static int set_lds(K kernel) {
  return (int)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
}

// The contraction kernels' dynamic-LDS limit is raised once per device and
// precision (the attribute belongs to the device's copy of the kernel); first
// calls may come from several threads, hence the atomic bit set and the lock.
static std::atomic<uint64_t> g_lds_ready{0};
static std::mutex g_lds_mu;

static int ensure_lds(int f32) {
  int dev = 0;
  int e = (int)hipGetDevice(&dev);
  if (e) return e;
  const uint64_t bit = dev >= 0 && dev < 32 ? (uint64_t)1 << (2 * dev + (f32 ? 1 : 0)) : 0;
  if (bit && (g_lds_ready.load(std::memory_order_acquire) & bit)) return 0;
  std::lock_guard<std::mutex> lk(g_lds_mu);
  if (bit && (g_lds_ready.load(std::memory_order_relaxed) & bit)) return 0;
  if (f32) {
    e |= set_lds(k_gemm<float, PH_GRAM, false>);
    e |= set_lds(k_gemm<float, PH_SQUARE, false>);
    e |= set_lds(k_gemm<float, PH_APPLY, false, false>);
    e |= set_lds(k_gemm<float, PH_APPLY, true, false>);
    e |= set_lds(k_gemm<float, PH_APPLY, false, true>);
    e |= set_lds(k_gemm<float, PH_APPLY, true, true>);
    e |= set_lds(k_gemm_plain<float>);
  } else {
    e |= set_lds(k_gemm<uint16_t, PH_GRAM, false>);
    e |= set_lds(k_gemm<uint16_t, PH_SQUARE, false>);
    e |= set_lds(k_gemm<uint16_t, PH_APPLY, false, false>);
    e |= set_lds(k_gemm<uint16_t, PH_APPLY, true, false>);
    e |= set_lds(k_gemm<uint16_t, PH_APPLY, false, true>);
    e |= set_lds(k_gemm<uint16_t, PH_APPLY, true, true>);
    e |= set_lds(k_gemm_plain<uint16_t>);
  }
  if (e == 0 && bit) g_lds_ready.fetch_or(bit, std::memory_order_release);
  return e;
}

int launch_write_table(void* dst, const void* src, size_t bytes, void* stream) {
  TableChunk c;
  c.pad = 0;
  const uint32_t* w = (const uint32_t*)src;
  const size_t words = bytes / 4;
  for (size_t off = 0; off < words; off += kChunkWords) {
    const size_t n = words - off < (size_t)kChunkWords ? words - off : (size_t)kChunkWords;
    c.dst = (uint32_t*)dst + off;
    c.n_words = (int32_t)n;
    __builtin_memcpy(c.words, w + off, n * 4);
    hipLaunchKernelGGL(k_write_table, dim3(1), dim3(kThreads), 0, (hipStream_t)stream, c);
    const int e = (int)hipGetLastError();
    if (e) return e;
  }
  return 0;
}

int launch_adamw(const AdamwTable& tab, const AdamwScalars& s, void* stream) {
  if (tab.total_wg <= 0) return 0;
  timing_before(PH_ADAMW, stream);
  hipLaunchKernelGGL(k_adamw, dim3(tab.total_wg), dim3(kThreads), 0, (hipStream_t)stream, tab, s);
  const int e = (int)hipGetLastError();
  timing_after(PH_ADAMW, stream);
  return e;
}

int launch_phase(int phase, int prec_f32, const LaunchTable& tab, const LaunchScalars& s, void* stream) {
  if (tab.total_wg <= 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(tab.total_wg), block(kThreads), gblock(kGemmThreads);
  int e = ensure_lds(prec_f32);
  if (e) return e;
  timing_before(phase, stream);
  switch (phase) {
    case PH_INGEST:
      if (prec_f32) hipLaunchKernelGGL(k_ingest<float>, grid, block, 0, st, tab, s);
      else hipLaunchKernelGGL(k_ingest<uint16_t>, grid, block, 0, st, tab, s);
      break;
    case PH_GRAM:
      if (prec_f32) hipLaunchKernelGGL((k_gemm<float, PH_GRAM, false>), grid, gblock, kGemmLds, st, tab, s);
      else hipLaunchKernelGGL((k_gemm<uint16_t, PH_GRAM, false>), grid, gblock, kGemmLds, st, tab, s);
      break;
    case PH_SQUARE:
      if (prec_f32) hipLaunchKernelGGL((k_gemm<float, PH_SQUARE, false>), grid, gblock, kGemmLds, st, tab, s);
      else hipLaunchKernelGGL((k_gemm<uint16_t, PH_SQUARE, false>), grid, gblock, kGemmLds, st, tab, s);
      break;
    case PH_APPLY: {
      // instantiations by (last apply, first iteration: X₀ read from its fp32 source)
      const int v = (s.last ? 1 : 0) | (s.t == 0 ? 2 : 0);
      if (prec_f32) {
        if (v == 0) hipLaunchKernelGGL((k_gemm<float, PH_APPLY, false, false>), grid, gblock, kGemmLds, st, tab, s);
        else if (v == 1) hipLaunchKernelGGL((k_gemm<float, PH_APPLY, true, false>), grid, gblock, kGemmLds, st, tab, s);
        else if (v == 2) hipLaunchKernelGGL((k_gemm<float, PH_APPLY, false, true>), grid, gblock, kGemmLds, st, tab, s);
        else hipLaunchKernelGGL((k_gemm<float, PH_APPLY, true, true>), grid, gblock, kGemmLds, st, tab, s);
      } else {
        if (v == 0) hipLaunchKernelGGL((k_gemm<uint16_t, PH_APPLY, false, false>), grid, gblock, kGemmLds, st, tab, s);
        else if (v == 1) hipLaunchKernelGGL((k_gemm<uint16_t, PH_APPLY, true, false>), grid, gblock, kGemmLds, st, tab, s);
        else if (v == 2) hipLaunchKernelGGL((k_gemm<uint16_t, PH_APPLY, false, true>), grid, gblock, kGemmLds, st, tab, s);
        else hipLaunchKernelGGL((k_gemm<uint16_t, PH_APPLY, true, true>), grid, gblock, kGemmLds, st, tab, s);
      }
      break;
    }
    case PH_UPDATE: hipLaunchKernelGGL(k_update, grid, block, 0, st, tab, s); break;
    case PH_NORM: hipLaunchKernelGGL(k_norm, grid, block, 0, st, tab, s); break;
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
  g.ktiles = (int)(kpad * (f32 ? 4 : 2) / kRowBytes);
  g.tiles_n = (int)cdiv(N, kTile);
  const dim3 grid((unsigned)(cdiv(M, kTile) * g.tiles_n)), block(kGemmThreads);
  hipStream_t st = (hipStream_t)stream;
  timing_before(PH_GEMM, stream);
  if (f32) hipLaunchKernelGGL(k_gemm_plain<float>, grid, block, kGemmLds, st, g);
  else hipLaunchKernelGGL(k_gemm_plain<uint16_t>, grid, block, kGemmLds, st, g);
  e = (int)hipGetLastError();
  timing_after(PH_GEMM, stream);
  return e;
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free step (dmuon_muon_step_noalloc).  Each
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the device
// address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kScratchBytes];

int scratch_region(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  static std::mutex mu;
  static std::vector<void*> by_device;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)by_device.size() <= dev) by_device.resize(dev + 1, nullptr);
  if (!by_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p || ((uintptr_t)p & 255)) return (int)hipErrorInvalidSymbol;
    by_device[dev] = p;
  }
  *ptr = by_device[dev];
  return 0;
}

}  // namespace dmuon
