// The two absorption GEMMs.
//
// absorb_q:  q_abs[t,i] = [ q^C_{t,i} W_UK,i^T ; RoPE(q^R_{t,i}, p_t) ]   (query side)
// out_proj:  out[t,i]   = o_lat[t,i] W_UV,i                             (output side)
//
// The key up-projection folds into the query projection and the value up-projection into
// the output projection (katajob interview page, "solid answer" and "Why it is not just
// extra work at decode time").  Both are per-head batched GEMMs with a small M (the query
// rows of one step) and are bound by reading the 16.8 MB weight once.
//
// Matrix-core path (DeepSeek-V2 shape, bf16): v_mfma_f32_32x32x16_bf16, one workgroup per
// (head, 32 query rows), four waves each owning 128 output columns.  32x32 accumulator
// layout: lane l holds column l%32 and rows 8*(k/4) + 4*(l/32) + k%4 for k = 0..15.
#include "common.h"

namespace mla {

// --------------------------------------------------------------- absorb_q, MFMA

constexpr int kAbsH = 128, kAbsDH = 128, kAbsDC = 512, kAbsDR = 64, kAbsRow = 576;
constexpr int kAbsLdsStride = kAbsRow + 4;   // fp32 words per staged row

__global__ void __launch_bounds__(256) absorb_q_mfma_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const int32_t* __restrict__ q_pos, const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_abs, int T,
    float rope_base) {
  __shared__ float stage[32 * kAbsLdsStride];
  const int h = blockIdx.x;
  const int t0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, lg = lane >> 5;

  // A fragments: q_nope rows t0+li, k = 16*ks + 8*lg .. +7 (8 K-steps over d_h = 128).
  bf16x8 af[8];
  {
    const int t = t0 + li;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < T)
        v = *reinterpret_cast<const u32x4*>(q_nope + ((size_t)t * kAbsH + h) * kAbsDH + 16 * ks + 8 * lg);
      af[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int c = 128 * wave + 32 * nt + li;   // output latent column held by this lane
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(w_uk + (size_t)c * (kAbsH * kAbsDH) + h * kAbsDH + 16 * ks + 8 * lg);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], __builtin_bit_cast(bf16x8, v), acc, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 8 * (k >> 2) + 4 * lg + (k & 3);
      stage[r * kAbsLdsStride + c] = acc[k];
    }
  }
  // positional part: 32 rows x 32 pairs, rotated in fp64
  for (int e = threadIdx.x; e < 32 * (kAbsDR / 2); e += 256) {
    const int r = e / (kAbsDR / 2), j = e % (kAbsDR / 2);
    const int t = t0 + r;
    float y0 = 0.f, y1 = 0.f;
    if (t < T) {
      const uint16_t* src = q_rope + ((size_t)t * kAbsH + h) * kAbsDR + 2 * j;
      double d0, d1;
      rope_pair_f64(bf16_bits_to_f32(src[0]), bf16_bits_to_f32(src[1]), q_pos[t], j, kAbsDR,
                    (double)rope_base, &d0, &d1);
      y0 = (float)d0;
      y1 = (float)d1;
    }
    stage[r * kAbsLdsStride + kAbsDC + 2 * j] = y0;
    stage[r * kAbsLdsStride + kAbsDC + 2 * j + 1] = y1;
  }
  __syncthreads();

  // write out: each wave takes 8 rows; each lane 9 consecutive values of a row
  for (int rr = 0; rr < 8; ++rr) {
    const int r = wave * 8 + rr;
    const int t = t0 + r;
    if (t >= T) break;
    const float* src = stage + r * kAbsLdsStride;
    const size_t obase = ((size_t)t * kAbsH + h) * kAbsRow;
    uint16_t* dst = q_abs + obase;
    for (int i = lane; i < kAbsRow; i += 64) dst[i] = (uint16_t)f32_to_bf16_bits(src[i]);
  }
}

// --------------------------------------------------------------- absorb_q, generic (VALU)

template <typename ActT>
__global__ void __launch_bounds__(256) absorb_q_generic_kernel(
    const ActT* __restrict__ q_nope, const ActT* __restrict__ q_rope, const int32_t* __restrict__ q_pos,
    const ActT* __restrict__ w_uk, ActT* __restrict__ q_abs, int T, int H, int d_h, int d_c, int d_r,
    float rope_base) {
  const int row = d_c + d_r;
  const size_t total = (size_t)T * H * row;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int k = (int)(e % row);
    const size_t th = e / row;
    const int h = (int)(th % H);
    const int t = (int)(th / H);
    float out;
    if (k < d_c) {
      float acc = 0.f;
      for (int d = 0; d < d_h; ++d)
        acc += load_act(q_nope, th * d_h + d) * load_act(w_uk, (size_t)k * H * d_h + (size_t)h * d_h + d);
      out = acc;
    } else {
      const int r = k - d_c, j = r >> 1;
      double y0, y1;
      rope_pair_f64(load_act(q_rope, th * d_r + 2 * j), load_act(q_rope, th * d_r + 2 * j + 1), q_pos[t], j,
                    d_r, (double)rope_base, &y0, &y1);
      out = (float)((r & 1) ? y1 : y0);
    }
    if constexpr (sizeof(ActT) == 4) q_abs[e] = out;
    else q_abs[e] = (ActT)f32_to_bf16_bits(out);
  }
}

// --------------------------------------------------------------- out_proj, MFMA

constexpr int kOutDV = 128;

__global__ void __launch_bounds__(256) out_proj_mfma_kernel(
    const float* __restrict__ o_lat, const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
    int T) {
  const int h = blockIdx.x;
  const int t0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, lg = lane >> 5;
  const int t = t0 + li;                  // A row of this lane
  const int v = 32 * wave + li;           // output column of this lane
  const float* arow = o_lat + ((size_t)t * kAbsH + h) * kAbsDC;
  const uint16_t* bcol = w_uv + (size_t)h * kOutDV + v;   // + c * (H*d_v)
  f32x16 acc = {};
#pragma unroll 4
  for (int ks = 0; ks < kAbsDC / 16; ++ks) {
    const int c0 = 16 * ks + 8 * lg;
    u32x4 a = {0u, 0u, 0u, 0u};
    if (t < T) {
      f32x4 x0 = *reinterpret_cast<const f32x4*>(arow + c0);
      f32x4 x1 = *reinterpret_cast<const f32x4*>(arow + c0 + 4);
      a[0] = pack_bf16x2(x0[0], x0[1]);
      a[1] = pack_bf16x2(x0[2], x0[3]);
      a[2] = pack_bf16x2(x1[0], x1[1]);
      a[3] = pack_bf16x2(x1[2], x1[3]);
    }
    u32x4 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = bcol[(size_t)(c0 + 2 * e) * (kAbsH * kOutDV)];
      const uint32_t hi = bcol[(size_t)(c0 + 2 * e + 1) * (kAbsH * kOutDV)];
      b[e] = lo | (hi << 16);
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = t0 + 8 * (k >> 2) + 4 * lg + (k & 3);
    if (r < T) out[((size_t)r * kAbsH + h) * kOutDV + v] = (uint16_t)f32_to_bf16_bits(acc[k]);
  }
}

// --------------------------------------------------------------- out_proj, generic (VALU)

template <typename ActT>
__global__ void __launch_bounds__(256) out_proj_generic_kernel(
    const float* __restrict__ o_lat, const ActT* __restrict__ w_uv, ActT* __restrict__ out, int T, int H,
    int d_c, int d_v) {
  const size_t total = (size_t)T * H * d_v;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int v = (int)(e % d_v);
    const size_t th = e / d_v;
    const int h = (int)(th % H);
    float acc = 0.f;
    for (int c = 0; c < d_c; ++c)
      acc += o_lat[th * d_c + c] * load_act(w_uv, (size_t)c * H * d_v + (size_t)h * d_v + v);
    if constexpr (sizeof(ActT) == 4) out[e] = acc;
    else out[e] = (ActT)f32_to_bf16_bits(acc);
  }
}

// --------------------------------------------------------------- launchers

bool is_dsv2_shape(const mla_config_t& c) {
  return c.num_heads == kAbsH && c.d_h == kAbsDH && c.d_c == kAbsDC && c.d_r == kAbsDR && c.d_v == kOutDV;
}

static unsigned generic_grid(size_t total) {
  size_t g = (total + 255) / 256;
  return (unsigned)(g > 65535 ? 65535 : (g == 0 ? 1 : g));
}

hipError_t launch_absorb_q(const mla_config_t& cfg, const void* q_nope, const void* q_rope,
                           const int32_t* q_pos, const void* w_uk, void* q_abs, int T, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (cfg.act_dtype == MLA_BF16 && is_dsv2_shape(cfg)) {
    dim3 grid(kAbsH, (T + 31) / 32);
    auto* qn = static_cast<const uint16_t*>(q_nope);
    auto* qr = static_cast<const uint16_t*>(q_rope);
    auto* w = static_cast<const uint16_t*>(w_uk);
    hipLaunchKernelGGL(absorb_q_mfma_kernel, grid, dim3(256), 0, stream, qn, qr, q_pos, w,
                       static_cast<uint16_t*>(q_abs), T, cfg.rope_base);
    return hipGetLastError();
  }
  const size_t total = (size_t)T * cfg.num_heads * (cfg.d_c + cfg.d_r);
  if (cfg.act_dtype == MLA_F32)
    hipLaunchKernelGGL(absorb_q_generic_kernel<float>, dim3(generic_grid(total)), dim3(256), 0, stream,
                       static_cast<const float*>(q_nope), static_cast<const float*>(q_rope), q_pos,
                       static_cast<const float*>(w_uk), static_cast<float*>(q_abs), T, cfg.num_heads, cfg.d_h,
                       cfg.d_c, cfg.d_r, cfg.rope_base);
  else
    hipLaunchKernelGGL(absorb_q_generic_kernel<uint16_t>, dim3(generic_grid(total)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope), q_pos,
                       static_cast<const uint16_t*>(w_uk), static_cast<uint16_t*>(q_abs), T, cfg.num_heads,
                       cfg.d_h, cfg.d_c, cfg.d_r, cfg.rope_base);
  return hipGetLastError();
}

hipError_t launch_out_proj(const mla_config_t& cfg, const float* o_lat, const void* w_uv, void* out, int T,
                           hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (cfg.act_dtype == MLA_BF16 && is_dsv2_shape(cfg)) {
    hipLaunchKernelGGL(out_proj_mfma_kernel, dim3(kAbsH, (T + 31) / 32), dim3(256), 0, stream, o_lat,
                       static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out), T);
    return hipGetLastError();
  }
  const size_t total = (size_t)T * cfg.num_heads * cfg.d_v;
  if (cfg.act_dtype == MLA_F32)
    hipLaunchKernelGGL(out_proj_generic_kernel<float>, dim3(generic_grid(total)), dim3(256), 0, stream, o_lat,
                       static_cast<const float*>(w_uv), static_cast<float*>(out), T, cfg.num_heads, cfg.d_c,
                       cfg.d_v);
  else
    hipLaunchKernelGGL(out_proj_generic_kernel<uint16_t>, dim3(generic_grid(total)), dim3(256), 0, stream,
                       o_lat, static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out), T, cfg.num_heads,
                       cfg.d_c, cfg.d_v);
  return hipGetLastError();
}

}  // namespace mla
