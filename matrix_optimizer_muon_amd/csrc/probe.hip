// Matrix-core ceiling probe (libdmuon_probe.so): waves that issue only bf16
// MFMAs on register operands, so that a caller timing them for a few seconds
// sees what the matrix cores sustain under the board's power limit with no
// memory traffic.  Not part of the Muon step; the contract is in dmuon_probe.h.
// The build compiles this file with the MFMA accumulators in VGPRs, where the
// step's contraction kernels keep them: one wave per SIMD then issues 16×16×32
// MFMAs at ~94% of the peak rate per clock, against ~71% with them in AGPRs.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "dmuon_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

thread_local std::string g_err;

int fail(int code, const char* msg) {
  g_err = msg;
  return code;
}

// 32-bit integer mixer (C. Wellons' "lowbias32" constants): decorrelates the
// operand bits of neighbouring lanes and registers.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// Eight bf16 operands: random sign and 7-bit mantissa, biased exponent
// 120..133 (magnitudes 2^-7 .. 2^7), or all zero.
__device__ __forceinline__ bf16x8_t operand(uint32_t key, int zero) {
  bf16x8_t v;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = mix32(key * 8u + (uint32_t)i);
    const uint16_t bits = zero ? (uint16_t)0 : (uint16_t)((h & 0x807fu) | ((120u + (h >> 8) % 14u) << 7));
    v[i] = __builtin_bit_cast(__bf16, bits);
  }
  return v;
}

// Each round: 8 (32×32×16) or 16 (16×16×32) independent accumulators, each
// advanced by one MFMA; the four A and four B operand registers rotate so that
// consecutive instructions see different operands.  Rounds come four at a time
// so that the rotation is resolved at compile time.
__global__ __launch_bounds__(kThreads) void k_probe32(float* sink, int iters, int zero) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand(t * 16u + (uint32_t)i, zero);
    b[i] = operand(t * 16u + 8u + (uint32_t)i, zero);
  }
  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], b[(i + u) & 3], acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  sink[t] = s;
}

__global__ __launch_bounds__(kThreads) void k_probe16(float* sink, int iters, int zero) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand(t * 16u + (uint32_t)i, zero);
    b[i] = operand(t * 16u + 8u + (uint32_t)i, zero);
  }
  f32x4_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][r] = 0.f;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 3], b[((i >> 2) + u) & 3], acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[i][r];
  sink[t] = s;
}

}  // namespace

extern "C" {

int dmuon_probe_mfma(int32_t shape, int32_t operands, int32_t blocks, int32_t iters, float* sink, void* stream) {
  g_err.clear();
  if (shape != 16 && shape != 32) return fail(DMUON_E_SHAPE, "shape must be 16 or 32");
  if (operands != DMUON_PROBE_RANDOM && operands != DMUON_PROBE_ZERO)
    return fail(DMUON_E_SHAPE, "operands must be DMUON_PROBE_RANDOM or DMUON_PROBE_ZERO");
  if (blocks < 1 || blocks > 65536) return fail(DMUON_E_SHAPE, "blocks must be in [1, 65536]");
  if (iters < 4 || iters > (1 << 24) || iters % 4) return fail(DMUON_E_SHAPE, "iters must be a multiple of 4 in [4, 2^24]");
  if (!sink) return fail(DMUON_E_NULL, "sink must be set");
  const int zero = operands == DMUON_PROBE_ZERO;
  if (shape == 32)
    hipLaunchKernelGGL(k_probe32, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, sink, iters, zero);
  else
    hipLaunchKernelGGL(k_probe16, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, sink, iters, zero);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DMUON_E_HIP, hipGetErrorString(e));
  return DMUON_OK;
}

const char* dmuon_probe_last_error(void) { return g_err.c_str(); }

}  // extern "C"
