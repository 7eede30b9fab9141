// libmla_attainable: a loop of matrix instructions with no memory traffic, for measuring the
// matrix rate the device sustains (see include/mla_attainable.h).  A measurement aid only.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/mla_attainable.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;               // independent accumulators per wave
constexpr int kMaxLds = 163840;          // one compute unit's LDS

// Integer mixer (xor-shift and odd multipliers) for the operand bits: fixed pseudo-random data,
// so the matrix units switch as they do on real operands.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 of magnitude in [0.5, 1) with a random sign and mantissa: bits s 0111 1110 mmm mmmm.
__device__ __forceinline__ uint16_t rand_bf16(uint32_t h) { return (uint16_t)(0x3F00u | (h & 0x807Fu)); }

// e4m3 of magnitude in [0.5, 1): bits s 0110 mmm (exponent 6, bias 7).
__device__ __forceinline__ uint32_t rand_e4m3x4(uint32_t h) { return 0x30303030u | (h & 0x87878787u); }

// Every accumulator stays finite: |a b| < 1, 16 (bf16) or 64 (fp8) products per element and
// instruction, and at most 2^20 iterations give |acc| < 2^24 (2^26).
__device__ __forceinline__ float chain_sum(const f32x16* acc) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  return s;
}

__global__ void __launch_bounds__(256) loop_bf16_kernel(int iters, float* out) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[k][e] = __builtin_bit_cast(__bf16, rand_bf16(mix32(tid * 64u + 16u * k + e)));
      b[k][e] = __builtin_bit_cast(__bf16, rand_bf16(mix32(tid * 64u + 16u * k + 8u + e + 0x9E3779B9u)));
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], acc[k], 0, 0, 0);
  }
  out[tid] = chain_sum(acc);
}

__global__ void __launch_bounds__(256) loop_fp8_kernel(int iters, float* out) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  i32x8 a[kChains], b[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[k][e] = (int)rand_e4m3x4(mix32(tid * 64u + 16u * k + e));
      b[k][e] = (int)rand_e4m3x4(mix32(tid * 64u + 16u * k + 8u + e + 0x9E3779B9u));
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  const int unit = 127;   // E8M0 exponent 127: scale 1
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k)
      acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[k], b[k], acc[k], 0, 0, 0, unit, 0, unit);
  }
  out[tid] = chain_sum(acc);
}

// The kernels reserve dynamic LDS beyond the default limit: raised once per device (idempotent
// calls; the mark is set only after they succeed).
constexpr int kMaxDev = 64;
std::atomic<int> g_lds_set[kMaxDev];

hipError_t set_lds_limits() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<int>* mark = (dev >= 0 && dev < kMaxDev) ? &g_lds_set[dev] : nullptr;
  if (mark && mark->load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)loop_bf16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)loop_fp8_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
  if (e == hipSuccess && mark) mark->store(1, std::memory_order_release);
  return e;
}

}  // namespace

extern "C" int32_t mla_attainable_mfma_loop(int32_t kind, int32_t workgroups, int32_t iters, int32_t lds_bytes,
                                            float* out, void* stream) {
  if (kind != MLA_LOOP_BF16 && kind != MLA_LOOP_FP8) return -1;
  if (workgroups <= 0 || workgroups > (1 << 20) || iters < 0 || iters > (1 << 20)) return -1;
  if (lds_bytes < 0 || lds_bytes > kMaxLds) return -1;
  if (out == nullptr || (reinterpret_cast<uintptr_t>(out) & 15u)) return -1;
  hipError_t e = set_lds_limits();
  if (e != hipSuccess) return (int32_t)e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == MLA_LOOP_BF16)
    hipLaunchKernelGGL(loop_bf16_kernel, dim3(workgroups), dim3(256), lds_bytes, s, iters, out);
  else
    hipLaunchKernelGGL(loop_fp8_kernel, dim3(workgroups), dim3(256), lds_bytes, s, iters, out);
  return (int32_t)hipGetLastError();
}
