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

  // every weight fragment of this wave (4 column tiles x 8 K-steps) and the query fragments
  // are requested together; the positional part runs while they are in flight
  u32x4 wv[4][8];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      wv[nt][ks] = *reinterpret_cast<const u32x4*>(w_uk + (size_t)(128 * wave + 32 * nt + li) * (kAbsH * kAbsDH) +
                                                   h * kAbsDH + 16 * ks + 8 * lg);
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
  // positional part: 32 rows x 32 pairs.  The angle pos * base^(-2j/d_R) and its reduction
  // modulo 2 pi are taken in fp64 (positions reach 2^15, so an fp32 angle would be off by
  // milliradians); cosine and sine of the reduced angle (|r| <= pi) in fp32 are then accurate
  // to a few fp32 ulps, far below the bf16 rounding of the result.
  __shared__ double theta[kAbsDR / 2];
  if (threadIdx.x < kAbsDR / 2) theta[threadIdx.x] = pow((double)rope_base, -2.0 * (double)threadIdx.x / (double)kAbsDR);
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * (kAbsDR / 2); e += 256) {
    const int r = e / (kAbsDR / 2), j = e % (kAbsDR / 2);
    const int t = t0 + r;
    float y0 = 0.f, y1 = 0.f;
    if (t < T) {
      const uint16_t* src = q_rope + ((size_t)t * kAbsH + h) * kAbsDR + 2 * j;
      const double ang = (double)q_pos[t] * theta[j];
      const double k = rint(ang * 0.15915494309189535);                   // ang / (2 pi)
      const double red = fma(-k, 6.283185307179586, ang) - k * 2.4492935982947064e-16;   // 2 pi = hi + lo
      float sn, cs;
      sincosf((float)red, &sn, &cs);
      const float x0 = bf16_bits_to_f32(src[0]), x1 = bf16_bits_to_f32(src[1]);
      y0 = x0 * cs - x1 * sn;
      y1 = x0 * sn + x1 * cs;
    }
    stage[r * kAbsLdsStride + kAbsDC + 2 * j] = y0;
    stage[r * kAbsLdsStride + kAbsDC + 2 * j + 1] = y1;
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int c = 128 * wave + 32 * nt + li;   // output latent column held by this lane
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], __builtin_bit_cast(bf16x8, wv[nt][ks]), acc, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 8 * (k >> 2) + 4 * lg + (k & 3);
      stage[r * kAbsLdsStride + c] = acc[k];
    }
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
    for (int i = lane; i < kAbsRow / 8; i += 64) {   // 16 bytes (8 values) per lane
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + 8 * i);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 8 * i + 4);
      *reinterpret_cast<u32x4*>(dst + 8 * i) = u32x4{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                                                     pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
    }
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

// out^T[v, t] = W_UV,h^T[v, c] . o_lat^T[c, t] for one head h and 32 query rows: the A operand
// (rows v, K = c) comes from a row-major copy of W_UV,h in LDS through transposing reads, so
// the weight is fetched with 16-byte loads along its rows; the B operand (K = c, contiguous
// in o_lat) comes straight from global memory.  Wave w owns output columns 32w .. 32w+31.
// The weight is staged in chunks of 64 rows (double-buffered); the row pitch of 320 bytes
// puts the four rows of one transposing read on four different 64-byte bank groups.
constexpr int kOpRows = 64;
constexpr int kOpPitch = kOutDV * 2 + 64;

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane i gets element i%4
// of the four values read by source lane 4j + i/4, as its element j.
__device__ __forceinline__ bf16x4 op_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(const MLA_LDS uint8_t*)p);
}

__global__ void __launch_bounds__(256) out_proj_mfma_kernel(
    const float* __restrict__ o_lat, const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
    int T) {
  __shared__ __attribute__((aligned(16))) uint8_t wl[2][kOpRows * kOpPitch];
  const int h = blockIdx.x;
  const int t0 = blockIdx.y * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5;                // K group of this lane: c = 16ks + 8g .. +7
  const int t = t0 + (lane & 31);         // B column (query row) of this lane
  const float* orow = o_lat + ((size_t)(t < T ? t : 0) * kAbsH + h) * kAbsDC;
  // A operand: source lane s = 16G + 4j + a reads row 8(G/2) + j (+4 for the high half) at
  // columns 32w + 16(G%2) + 4a .. +3, so that output lane l holds column l%32 of the tile and
  // rows 8(l/32) .. +7 of the K-step, matching B.
  const int G = lane >> 4, jr = (lane >> 2) & 3, ac = lane & 3;
  const int a_off = (8 * (G >> 1) + jr) * kOpPitch + 2 * (32 * wave + 16 * (G & 1) + 4 * ac);
  // staging: piece p = tid + 256i of a chunk is row p/16, bytes 16(p%16) .. of that row
  const uint16_t* wsrc = w_uv + (size_t)h * kOutDV;
  auto fetch = [&](int kc, u32x4* r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i;
      r[i] = *reinterpret_cast<const u32x4*>(wsrc + (size_t)(kOpRows * kc + (p >> 4)) * (kAbsH * kOutDV) + 8 * (p & 15));
    }
  };
  auto put = [&](int buf, const u32x4* r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&wl[buf][(p >> 4) * kOpPitch + 16 * (p & 15)]) = r[i];
    }
  };
  // weight chunks are fetched three ahead and the o_lat fragments one chunk ahead (the loop is
  // unrolled so that the register rings are static)
  auto ofetch = [&](int kc, f32x4* x) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = kOpRows * kc + 16 * ks + 8 * g;
      x[2 * ks] = *reinterpret_cast<const f32x4*>(orow + c0);
      x[2 * ks + 1] = *reinterpret_cast<const f32x4*>(orow + c0 + 4);
    }
  };
  constexpr int kChunks = kAbsDC / kOpRows;
  u32x4 r[3][4];
  f32x4 ox[2][8];
  fetch(0, r[0]);
  fetch(1, r[1]);
  fetch(2, r[2]);
  ofetch(0, ox[0]);
  put(0, r[0]);
  fetch(3, r[0]);
  __syncthreads();
  f32x16 acc = {};
#pragma unroll
  for (int kc = 0; kc < kChunks; ++kc) {
    if (kc + 1 < kChunks) ofetch(kc + 1, ox[(kc + 1) & 1]);
    const uint8_t* wb = wl[kc & 1] + a_off;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x4 x0 = t < T ? ox[kc & 1][2 * ks] : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 x1 = t < T ? ox[kc & 1][2 * ks + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
      const u32x4 bq = u32x4{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]), pack_bf16x2(x1[0], x1[1]),
                             pack_bf16x2(x1[2], x1[3])};
      const bf16x4 lo = op_tr16(wb + 16 * ks * kOpPitch);
      const bf16x4 hi = op_tr16(wb + (16 * ks + 4) * kOpPitch);
      const bf16x8 a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bq), acc, 0, 0, 0);
    }
    // chunk kc+1 (fetched into ring slot (kc+1)%3) goes to the other buffer, whose last
    // reader (chunk kc-1) every wave finished before the previous barrier
    if (kc + 1 < kChunks) put((kc + 1) & 1, r[(kc + 1) % 3]);
    if (kc + 4 < kChunks) fetch(kc + 4, r[(kc + 1) % 3]);
    __syncthreads();
  }
  // acc[i] = out^T[32w + 8(i/4) + 4g + i%4, t]: four consecutive columns per i/4
  if (t < T) {
    uint16_t* orow_out = out + ((size_t)t * kAbsH + h) * kOutDV + 32 * wave + 4 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x2*>(orow_out + 8 * q) =
          u32x2{pack_bf16x2(acc[4 * q], acc[4 * q + 1]), pack_bf16x2(acc[4 * q + 2], acc[4 * q + 3])};
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
