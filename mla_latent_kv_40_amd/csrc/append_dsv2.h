// Cache append for the DeepSeek-V2 shape (d_c = 512, d_R = 64, bf16 activations), one wave
// per token (per run of tokens for the block-scaled format): shared by the append kernels and
// the fused append + absorb kernel.
//
// Only the latent and the positional key are stored (podcast "What Is Multi-head Latent
// Attention ...", the paragraph on what the system caches); RoPE is applied to k_R at write
// time, at the token's position (bembew "Multi-head Latent Attention", "Implementation Logic"
// step 4).  The work is a few KB per step, so the time is the chain of memory round trips
// (sequence and position lookups, page, then the row: the compiler keeps the row loads
// behind the checks that may return early).
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

// ---------------------------------------------------------- block-scaled fp8 (32 x 32 tiles)
//
// The rows of a page form two tiles of 32 tokens per 32-column block (18 blocks of the 576-wide
// row); each tile holds one power-of-two scale 2^e (stored as that fp32 value at
// cache_scale[(page * 2 + token half) * 18 + block]) and e4m3 codes of value / 2^e.  A call
// takes, for each tile it writes, the smallest e at which none of the tile's rows saturates,
// the rows written by earlier calls included unless the call writes the tile's first row;
// when e grows, the earlier rows' codes are re-encoded at the new scale (exact unless a code
// falls into the subnormal range).  The katajob interview page ("Compression as architecture
// versus compression as post-processing") names per-block scaling as what a quantised cache
// needs.
//
// One wave per run: the consecutive new tokens of a call that write one tile.  The run's first
// wave does all of it (the other waves of the run return), so a tile's rows are read, rescaled
// and written by one wave.  Lane l holds latent values 8l .. 8l+7 (column block l/4) and, as
// lane l%32, positional pair l%32 (column block 16 + (l%32)/16).
constexpr int kTileRows = 32, kColBlocks = (kAppDC + kAppDR) / 32;

// smallest e with amax <= 448 2^e (amax = m 2^x, m in [0.5, 1): e is x - 9 or x - 8), clamped
// to [-126, 127]
__device__ __forceinline__ int tile_exponent(float amax) {
  if (!(amax > 0.0f)) return -126;
  int x;
  frexpf(amax, &x);
  int e = x - 9;
  if (amax > ldexpf(448.0f, e)) e += 1;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// tile of batch entry `tok`: page * 2 + token half, or -1 when the entry writes nothing
__device__ __forceinline__ int tile_key(const AppendArgs& ap, int tok) {
  if (tok < 0 || tok >= ap.n) return -1;
  const int s = ap.seq_of[tok], p = ap.pos[tok];
  if (s < 0 || s >= ap.batch || p < 0 || p / kBlock >= ap.max_blocks) return -1;
  const int page = ap.block_table[(size_t)s * ap.max_blocks + p / kBlock];
  if (page < 0 || page >= ap.num_blocks) return -1;
  return 2 * page + (p % kBlock) / kTileRows;
}

// Block-scaled fp8 append of batch entry `tok` by one wave (see above): the wave of a run's
// first entry writes the whole run; the others return.
__device__ __forceinline__ void append_block_token(const AppendArgs& ap, const AppendTheta& theta, int tok) {
  const int lane = threadIdx.x & 63;
  const int key = tile_key(ap, tok);
  if (key < 0 || tile_key(ap, tok - 1) == key) return;   // writes nothing, or not the run's first entry
  // run length: the following entries (at most 31) that write the same tile
  const int other = (lane >= 1 && lane < kTileRows) ? tile_key(ap, tok + lane) : -2;
  const unsigned long long differ = __ballot(lane >= 1 && lane < kTileRows && other != key) | (1ull << kTileRows);
  const int len = __builtin_ctzll(differ >> 1) + 1;
  const int page = key >> 1, half = key & 1;
  const int r0 = ap.pos[tok] % kTileRows;                 // tile row of the run's first token
  const bool fresh = r0 == 0;
  uint8_t* __restrict__ tile = ap.cache + ((size_t)page * kBlock + half * kTileRows) * (kAppDC + kAppDR);
  float* __restrict__ tscale = ap.cache_scale + (size_t)key * kColBlocks;
  const int jp = lane & 31;
  const double th = theta.v[jp];
  // the run's row u in fp32: latent values (exact) and the rotated positional pair (rounded once)
  auto row = [&](int u, float* v, float* r) {
    const int t = tok + u;
    const u32x4 cv = *reinterpret_cast<const u32x4*>(ap.c_kv + (size_t)t * kAppDC + 8 * lane);
    const uint32_t kv = *reinterpret_cast<const uint32_t*>(ap.k_r + (size_t)t * kAppDR + 2 * jp);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_bits_to_f32(cv[k] & 0xFFFFu);
      v[2 * k + 1] = bf16_bits_to_f32(cv[k] >> 16);
    }
    double sn, cs;
    sincos((double)ap.pos[t] * th, &sn, &cs);
    const double x0 = (double)bf16_bits_to_f32(kv & 0xFFFFu), x1 = (double)bf16_bits_to_f32(kv >> 16);
    r[0] = (float)(x0 * cs - x1 * sn);
    r[1] = (float)(x0 * sn + x1 * cs);
  };
  // exponents the run needs: largest magnitude per column block over its rows
  float m_lat = 0.0f, m_pos = 0.0f;
  for (int u = 0; u < len; ++u) {
    float v[8], r[2];
    row(u, v, r);
#pragma unroll
    for (int k = 0; k < 8; ++k) m_lat = fmaxf(m_lat, fabsf(v[k]));
    m_pos = fmaxf(m_pos, fmaxf(fabsf(r[0]), fabsf(r[1])));
  }
  m_lat = fmaxf(m_lat, __shfl_xor(m_lat, 1));
  m_lat = fmaxf(m_lat, __shfl_xor(m_lat, 2));          // the four lanes of a latent block
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m_pos = fmaxf(m_pos, __shfl_xor(m_pos, d));   // 16 pairs of a block
  int e_lat = tile_exponent(m_lat), e_pos = tile_exponent(m_pos);
  if (!fresh) {
    // the tile's earlier rows 0 .. r0-1: their exponent takes part, and their codes move to the
    // new scale when it grew (scales are normal powers of two: the exponent is bits 23..30)
    const int o_lat = (int)((__float_as_uint(tscale[lane >> 2]) >> 23) & 0xFF) - 127;
    const int o_pos = (int)((__float_as_uint(tscale[16 + (jp >> 4)]) >> 23) & 0xFF) - 127;
    e_lat = e_lat > o_lat ? e_lat : o_lat;
    e_pos = e_pos > o_pos ? e_pos : o_pos;
    for (int rr = 0; rr < r0; ++rr) {
      uint8_t* dst = tile + (size_t)rr * (kAppDC + kAppDR);
      if (e_lat > o_lat) {
        const u32x2 c = *reinterpret_cast<const u32x2*>(dst + 8 * lane);
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float x = ldexpf(e4m3_to_f32((c[k >> 2] >> (8 * (k & 3))) & 0xFFu), o_lat - e_lat);
          w[k >> 2] |= f32_to_e4m3(x) << (8 * (k & 3));
        }
        *reinterpret_cast<u32x2*>(dst + 8 * lane) = u32x2{w[0], w[1]};
      }
      if (lane < 32 && e_pos > o_pos) {
        const uint32_t c = *reinterpret_cast<const uint16_t*>(dst + kAppDC + 2 * jp);
        const float x0 = ldexpf(e4m3_to_f32(c & 0xFFu), o_pos - e_pos);
        const float x1 = ldexpf(e4m3_to_f32(c >> 8), o_pos - e_pos);
        *reinterpret_cast<uint16_t*>(dst + kAppDC + 2 * jp) = (uint16_t)(f32_to_e4m3(x0) | (f32_to_e4m3(x1) << 8));
      }
    }
  }
  // the run's rows at the tile's scale
  for (int u = 0; u < len; ++u) {
    float v[8], r[2];
    row(u, v, r);
    // the token's own tile row (its key matched, so the row is inside the tile)
    uint8_t* dst = tile + (size_t)(ap.pos[tok + u] % kTileRows) * (kAppDC + kAppDR);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w0 |= f32_to_e4m3(ldexpf(v[k], -e_lat)) << (8 * k);
      w1 |= f32_to_e4m3(ldexpf(v[4 + k], -e_lat)) << (8 * k);
    }
    *reinterpret_cast<u32x2*>(dst + 8 * lane) = u32x2{w0, w1};
    if (lane < 32)
      *reinterpret_cast<uint16_t*>(dst + kAppDC + 2 * jp) =
          (uint16_t)(f32_to_e4m3(ldexpf(r[0], -e_pos)) | (f32_to_e4m3(ldexpf(r[1], -e_pos)) << 8));
  }
  if ((lane & 3) == 0) tscale[lane >> 2] = ldexpf(1.0f, e_lat);
  if (lane == 0 || lane == 16) tscale[16 + (lane >> 4)] = ldexpf(1.0f, e_pos);
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
