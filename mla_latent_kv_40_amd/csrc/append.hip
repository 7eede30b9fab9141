// Cache append: write each new token's row [c ; RoPE(k_R, pos)] into its page.
//
// Only the latent and the positional key are stored (podcast "What Is Multi-head Latent
// Attention ...", the paragraph on what the system caches); RoPE is applied to k_R at
// write time, at the token's position (bembew "Multi-head Latent Attention",
// "Implementation Logic" step 4, and "Decoupling RoPE from Compression").
//
// One wave per token, four tokens per 256-thread workgroup; rotation in fp64, one rounding
// to the cache format.  FP8 rows get one fp32 scale amax/448 and e4m3 codes (value/scale).
// The work is a few KB per step, so the kernel's time is its chain of memory round trips: the
// sequence and position lookups, the page lookup, then the token's row (the compiler keeps
// the row loads behind the checks that may return early).  In a step the appends share a
// launch with the query absorption, whose workgroups take longer.
#include "append_dsv2.h"

#include <cmath>

namespace mla {

// d_c = 512, d_R = 64, bf16 activations: four tokens per workgroup.
template <int CacheFmt>
__global__ void __launch_bounds__(256) append_dsv2_kernel(AppendArgs ap, AppendTheta theta) {
  append_dsv2_token<CacheFmt>(ap, theta, blockIdx.x * 4 + (threadIdx.x >> 6));
}

template <typename ActT, int CacheFmt>
__global__ void __launch_bounds__(256) append_kernel(
    uint8_t* __restrict__ cache, float* __restrict__ cache_scale, int num_blocks,
    const ActT* __restrict__ c_kv, const ActT* __restrict__ k_r, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq_of, const int32_t* __restrict__ block_table, int batch,
    int max_blocks, int n, int d_c, int d_r, float rope_base) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= n) return;
  const int s = seq_of[tok];
  const int p = pos[tok];
  if (s < 0 || s >= batch || p < 0 || p / kBlock >= max_blocks) return;
  const int page = block_table[(size_t)s * max_blocks + p / kBlock];
  if (page < 0 || page >= num_blocks) return;
  const int row = d_c + d_r;
  const size_t slot = (size_t)page * kBlock + (p % kBlock);

  if constexpr (CacheFmt == MLA_F32) {
    float* dst = reinterpret_cast<float*>(cache) + slot * row;
    for (int i = lane; i < d_c; i += 64) dst[i] = load_act(c_kv, (size_t)tok * d_c + i);
    for (int j = lane; j < d_r / 2; j += 64) {
      double y0, y1;
      rope_pair_f64(load_act(k_r, (size_t)tok * d_r + 2 * j), load_act(k_r, (size_t)tok * d_r + 2 * j + 1),
                    p, j, d_r, (double)rope_base, &y0, &y1);
      dst[d_c + 2 * j] = (float)y0;
      dst[d_c + 2 * j + 1] = (float)y1;
    }
  } else if constexpr (CacheFmt == MLA_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(cache) + slot * row;
    for (int i = lane; i < d_c; i += 64)
      dst[i] = (uint16_t)f32_to_bf16_bits(load_act(c_kv, (size_t)tok * d_c + i));
    for (int j = lane; j < d_r / 2; j += 64) {
      double y0, y1;
      rope_pair_f64(load_act(k_r, (size_t)tok * d_r + 2 * j), load_act(k_r, (size_t)tok * d_r + 2 * j + 1),
                    p, j, d_r, (double)rope_base, &y0, &y1);
      dst[d_c + 2 * j] = (uint16_t)f64_to_bf16_bits(y0);
      dst[d_c + 2 * j + 1] = (uint16_t)f64_to_bf16_bits(y1);
    }
  } else {  // FP8 e4m3 with a per-token scale
    // Values of the row in fp32: c exactly, the rotated k_R rounded once from fp64.
    // Lane owns elements lane, lane+64, ... (row <= 1024 -> at most 16 per lane).
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = lane + 64 * k;
      float x = 0.0f;
      if (i < d_c) {
        x = load_act(c_kv, (size_t)tok * d_c + i);
      } else if (i < row) {
        const int r = i - d_c, j = r >> 1;
        double y0, y1;
        rope_pair_f64(load_act(k_r, (size_t)tok * d_r + 2 * j), load_act(k_r, (size_t)tok * d_r + 2 * j + 1),
                      p, j, d_r, (double)rope_base, &y0, &y1);
        x = (float)((r & 1) ? y1 : y0);
      }
      v[k] = x;
      amax = fmaxf(amax, fabsf(x));
    }
    amax = wave_max(amax);
    float scale = amax / 448.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    uint8_t* dst = cache + slot * row;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = lane + 64 * k;
      if (i < row) dst[i] = (uint8_t)f32_to_e4m3(v[k] / scale);
    }
    if (lane == 0) cache_scale[slot] = scale;
  }
}

// Block-scaled fp8 append (the format and the routine are in append_dsv2.h): one wave per batch
// entry, four entries per workgroup.
__global__ void __launch_bounds__(256) append_block_fp8_kernel(AppendArgs ap, AppendTheta theta) {
  append_block_token(ap, theta, blockIdx.x * 4 + (threadIdx.x >> 6));
}

hipError_t launch_append(const mla_config_t& cfg, void* cache, float* cache_scale, int num_blocks,
                         const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* seq_of,
                         const int32_t* block_table, int batch, int max_blocks, int n,
                         hipStream_t stream) {
  dim3 grid((n + 3) / 4), block(256);
  auto* c8 = static_cast<uint8_t*>(cache);
  if (n == 0) return hipSuccess;
  if (cfg.cache_dtype == MLA_FP8_E4M3_B32) {   // DeepSeek-V2 shape, bf16 activations (checked by the caller)
    const AppendArgs ap = append_args(cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table, batch,
                                      max_blocks, n);
    hipLaunchKernelGGL(append_block_fp8_kernel, grid, block, 0, stream, ap, append_theta(cfg));
    return hipGetLastError();
  }
  if (append_dsv2_applies(cfg)) {
    const AppendArgs ap = append_args(cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table, batch,
                                      max_blocks, n);
    const AppendTheta theta = append_theta(cfg);
    if (cfg.cache_dtype == MLA_BF16)
      hipLaunchKernelGGL(append_dsv2_kernel<MLA_BF16>, grid, block, 0, stream, ap, theta);
    else
      hipLaunchKernelGGL(append_dsv2_kernel<MLA_FP8_E4M3>, grid, block, 0, stream, ap, theta);
    return hipGetLastError();
  }
  if (cfg.act_dtype == MLA_F32) {
    auto* c = static_cast<const float*>(c_kv);
    auto* k = static_cast<const float*>(k_r);
    if (cfg.cache_dtype == MLA_F32)
      hipLaunchKernelGGL((append_kernel<float, MLA_F32>), grid, block, 0, stream, c8, cache_scale,
                         num_blocks, c, k, pos, seq_of, block_table, batch, max_blocks, n, cfg.d_c,
                         cfg.d_r, cfg.rope_base);
    else
      return hipErrorInvalidValue;
  } else {
    auto* c = static_cast<const uint16_t*>(c_kv);
    auto* k = static_cast<const uint16_t*>(k_r);
    if (cfg.cache_dtype == MLA_BF16)
      hipLaunchKernelGGL((append_kernel<uint16_t, MLA_BF16>), grid, block, 0, stream, c8,
                         cache_scale, num_blocks, c, k, pos, seq_of, block_table, batch, max_blocks,
                         n, cfg.d_c, cfg.d_r, cfg.rope_base);
    else if (cfg.cache_dtype == MLA_FP8_E4M3)
      hipLaunchKernelGGL((append_kernel<uint16_t, MLA_FP8_E4M3>), grid, block, 0, stream, c8,
                         cache_scale, num_blocks, c, k, pos, seq_of, block_table, batch, max_blocks,
                         n, cfg.d_c, cfg.d_r, cfg.rope_base);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
