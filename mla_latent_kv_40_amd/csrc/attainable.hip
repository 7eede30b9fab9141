// libmla_attainable: a loop of matrix instructions with no memory traffic, for measuring the
// matrix rate the device sustains, and two read-only streams of a device buffer, for the HBM
// read bandwidth it sustains (see include/mla_attainable.h).  A measurement aid only.
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

// ---- read-only streams.  The buffer is cut into chunks of kChunk bytes (a half page of the
// bf16 decode split: 32 rows of 1152 B); workgroup w reads chunks w*n .. w*n+n-1.  Every 32-bit
// word is read exactly once, by one lane, which adds it to its running sum (wrapping), so the
// sum of all lanes' outputs is the sum of the buffer's words mod 2^32.
constexpr int kChunk = 36864;
constexpr int kChunkLoads = kChunk / 4096;   // 16-byte loads per lane and chunk (one workgroup)
constexpr int kRing = 4;                     // LDS stages of the DMA stream
constexpr int kRingDepth = kRing - 1;        // chunks in flight ahead of the one being read

// s_waitcnt immediate: at most n vector-memory operations outstanding (gfx9 encoding, the other
// counters left alone).
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// Plain vector loads into registers: per chunk, each lane loads nine 16-byte pieces 4 KiB apart
// (256 lanes x 16 B = 4 KiB contiguous per load instruction), all nine issued before the sum.
__global__ void __launch_bounds__(256) read_vgpr_kernel(const uint8_t* __restrict__ buf, int chunks_per_wg,
                                                        uint32_t* out) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint8_t* base = buf + (size_t)blockIdx.x * chunks_per_wg * kChunk + 16 * threadIdx.x;
  uint32_t acc = 0;
  for (int c = 0; c < chunks_per_wg; ++c) {
    u32x4 v[kChunkLoads];
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i)
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (size_t)c * kChunk + 4096 * i));
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i) acc += v[i][0] + v[i][1] + v[i][2] + v[i][3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// The decode split's way in: 1 KiB buffer->LDS loads (each wave nine per chunk) into a ring of
// four LDS stages, three chunks in flight, one barrier per chunk; each lane then reads back the
// nine 16-byte pieces it loaded and sums them.  One workgroup per compute unit (all of its LDS).
__global__ void __launch_bounds__(256, 1) read_lds_kernel(const uint8_t* __restrict__ buf, int chunks_per_wg,
                                                          uint32_t* out) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(256))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint8_t* slice = buf + (size_t)blockIdx.x * chunks_per_wg * kChunk;
  // the descriptor covers this workgroup's slice exactly; the chunk offset goes in soffset
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)slice, 0, chunks_per_wg * kChunk, 0x00020000);
  auto issue = [&](int c) {
    uint8_t* stage = smem + (c % kRing) * kChunk;
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i) {
      const int piece = kChunkLoads * wave + i;   // 1 KiB piece of the chunk
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(stage + 1024 * piece),
                                               16, 1024 * piece + 16 * lane, c * kChunk, 0, 0);
    }
  };
  uint32_t acc = 0;
  for (int c = 0; c < kRingDepth && c < chunks_per_wg; ++c) issue(c);
  for (int c = 0; c < chunks_per_wg; ++c) {
    // this wave's loads of chunk c have landed (those of up to two younger chunks may not),
    // then everyone's; the stage refilled below was last read in the previous iteration
    const int younger = (chunks_per_wg - 1 - c) < (kRingDepth - 1) ? (chunks_per_wg - 1 - c) : (kRingDepth - 1);
    if (younger >= 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kChunkLoads));
    else if (younger == 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kChunkLoads));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (c + kRingDepth < chunks_per_wg) issue(c + kRingDepth);
    // read through an absolute LDS address with a restrict pointer: through the shared array the
    // compiler would wait for every load in flight, which it takes to alias the stage
    const uint32_t stage = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)smem +
                           (uint32_t)((c % kRing) * kChunk);
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i) {
      const __attribute__((address_space(3))) u32x4* __restrict__ q =
          (const __attribute__((address_space(3))) u32x4*)(size_t)(stage + 1024 * (kChunkLoads * wave + i) + 16 * lane);
      const u32x4 v = *q;
      acc += v[0] + v[1] + v[2] + v[3];
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  out[blockIdx.x * 256 + threadIdx.x] = acc;
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
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)read_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
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

extern "C" int32_t mla_attainable_read(int32_t kind, const void* buf, int64_t bytes, int32_t workgroups, uint32_t* out,
                                       void* stream) {
  if (kind != MLA_READ_VGPR && kind != MLA_READ_LDS) return -1;
  if (workgroups <= 0 || workgroups > (1 << 16) || bytes <= 0) return -1;
  if (bytes % ((int64_t)workgroups * kChunk) != 0) return -1;
  const int64_t per = bytes / ((int64_t)workgroups * kChunk);
  if (per > (int64_t)(0x7fffffff / kChunk)) return -1;   // a slice must fit one buffer descriptor
  if (buf == nullptr || out == nullptr) return -1;
  if ((reinterpret_cast<uintptr_t>(buf) & 255u) || (reinterpret_cast<uintptr_t>(out) & 15u)) return -1;
  hipError_t e = set_lds_limits();
  if (e != hipSuccess) return (int32_t)e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  if (kind == MLA_READ_VGPR)
    hipLaunchKernelGGL(read_vgpr_kernel, dim3(workgroups), dim3(256), 0, s, b, (int)per, out);
  else
    hipLaunchKernelGGL(read_lds_kernel, dim3(workgroups), dim3(256), kRing * kChunk, s, b, (int)per, out);
  return (int32_t)hipGetLastError();
}
