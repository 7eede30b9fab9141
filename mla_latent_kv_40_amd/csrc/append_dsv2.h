// Cache append for the DeepSeek-V2 shape (d_c = 512, d_R = 64, bf16 activations), one wave
// per token: shared by the append kernel and the fused append + absorb kernel.
//
// Only the latent and the positional key are stored (podcast "What Is Multi-head Latent
// Attention ...", the paragraph on what the system caches); RoPE is applied to k_R at write
// time, at the token's position (bembew "Multi-head Latent Attention", "Implementation Logic"
// step 4).  The work is a few KB per step, so the time is the chain of memory round trips:
// the token's row loads are issued with its sequence and position lookups, so only the page
// lookup waits on another load.
#pragma once
#include "common.h"

#include <cmath>

namespace mla {

constexpr int kAppDC = 512, kAppDR = 64;

// Inverse frequencies base^(-2j/d_R) of the positional pairs, computed on the host in fp64.
struct AppendTheta {
  double v[kAppDR / 2];
};

struct AppendArgs {
  uint8_t* cache;
  float* cache_scale;
  const uint16_t* c_kv;
  const uint16_t* k_r;
  const int32_t* pos;
  const int32_t* seq_of;
  const int32_t* block_table;
  int num_blocks, batch, max_blocks, n;
};

// d_c = 512, d_R = 64, bf16 activations: token `tok` by one wave.  Lane l holds latent values
// 8l .. 8l+7 (one 16-byte load and store) and, for l < 32, positional pair l.
template <int CacheFmt>
__device__ __forceinline__ void append_dsv2_token(const AppendArgs& ap, const AppendTheta& theta, int tok) {
  const int lane = threadIdx.x & 63;
  if (tok >= ap.n) return;
  uint8_t* __restrict__ cache = ap.cache;
  float* __restrict__ cache_scale = ap.cache_scale;
  const uint16_t* __restrict__ c_kv = ap.c_kv;
  const uint16_t* __restrict__ k_r = ap.k_r;
  const int32_t* __restrict__ pos = ap.pos;
  const int32_t* __restrict__ seq_of = ap.seq_of;
  const int32_t* __restrict__ block_table = ap.block_table;
  const int batch = ap.batch, max_blocks = ap.max_blocks, num_blocks = ap.num_blocks;
  const u32x4 cv = *reinterpret_cast<const u32x4*>(c_kv + (size_t)tok * kAppDC + 8 * lane);
  const int jp = lane & 31;
  const uint32_t kv = *reinterpret_cast<const uint32_t*>(k_r + (size_t)tok * kAppDR + 2 * jp);
  const double th = theta.v[jp];
  const int s = seq_of[tok];
  const int p = pos[tok];
  if (s < 0 || s >= batch || p < 0 || p / kBlock >= max_blocks) return;
  const int page = block_table[(size_t)s * max_blocks + p / kBlock];
  if (page < 0 || page >= num_blocks) return;
  const size_t slot = (size_t)page * kBlock + (p % kBlock);
  // rotation of pair jp in fp64 (lanes 32 .. 63 repeat lanes 0 .. 31 and store nothing)
  double sn, cs;
  sincos((double)p * th, &sn, &cs);
  const double x0 = (double)bf16_bits_to_f32(kv & 0xFFFFu), x1 = (double)bf16_bits_to_f32(kv >> 16);
  const double y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
  if constexpr (CacheFmt == MLA_BF16) {
    uint8_t* dst = cache + slot * (kAppDC + kAppDR) * 2;
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = cv;   // bf16 latent: stored as given
    if (lane < 32)
      *reinterpret_cast<uint32_t*>(dst + 2 * kAppDC + 4 * jp) = f64_to_bf16_bits(y0) | (f64_to_bf16_bits(y1) << 16);
  } else {   // FP8 e4m3 with a per-token scale: values in fp32 (the latent exactly, the rotated k_R
             // rounded once from fp64), scale = amax / 448, codes from value / scale
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_bits_to_f32(cv[k] & 0xFFFFu);
      v[2 * k + 1] = bf16_bits_to_f32(cv[k] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * k]), fabsf(v[2 * k + 1])));
    }
    const float r0 = (float)y0, r1 = (float)y1;
    amax = fmaxf(amax, fmaxf(fabsf(r0), fabsf(r1)));   // lanes 32 .. 63 repeat 0 .. 31
    amax = wave_max(amax);
    float scale = amax / 448.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    uint8_t* dst = cache + slot * (kAppDC + kAppDR);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w0 |= f32_to_e4m3(v[k] / scale) << (8 * k);
      w1 |= f32_to_e4m3(v[4 + k] / scale) << (8 * k);
    }
    *reinterpret_cast<u32x2*>(dst + 8 * lane) = u32x2{w0, w1};
    if (lane < 32)
      *reinterpret_cast<uint16_t*>(dst + kAppDC + 2 * jp) =
          (uint16_t)(f32_to_e4m3(r0 / scale) | (f32_to_e4m3(r1 / scale) << 8));
    if (lane == 0) cache_scale[slot] = scale;
  }
}

inline AppendArgs append_args(void* cache, float* cache_scale, int num_blocks, const void* c_kv, const void* k_r,
                              const int32_t* pos, const int32_t* seq_of, const int32_t* block_table, int batch,
                              int max_blocks, int n) {
  return AppendArgs{static_cast<uint8_t*>(cache), cache_scale, static_cast<const uint16_t*>(c_kv),
                    static_cast<const uint16_t*>(k_r), pos, seq_of, block_table, num_blocks, batch, max_blocks, n};
}

inline AppendTheta append_theta(const mla_config_t& cfg) {
  AppendTheta theta;
  for (int j = 0; j < kAppDR / 2; ++j) theta.v[j] = std::pow((double)cfg.rope_base, -2.0 * j / (double)kAppDR);
  return theta;
}

// The DeepSeek-V2-shaped append applies (bf16 activations into a bf16 or fp8 cache).
inline bool append_dsv2_applies(const mla_config_t& cfg) {
  return cfg.act_dtype == MLA_BF16 && cfg.d_c == kAppDC && cfg.d_r == kAppDR &&
         (cfg.cache_dtype == MLA_BF16 || cfg.cache_dtype == MLA_FP8_E4M3);
}

}  // namespace mla
