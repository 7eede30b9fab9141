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
// (head, quarter of the output columns, block of 64 query rows), so that each weight byte is
// read by one workgroup per row block and 512 workgroups (at up to 64 rows) keep every compute
// unit busy; every load of a workgroup is issued before the first matrix instruction.  32x32
// accumulator layout: lane l holds column l%32 and rows 8*(k/4) + 4*(l/32) + k%4 for k = 0..15.
#include "append_dsv2.h"

#include <cmath>

namespace mla {

// --------------------------------------------------------------- absorb_q, MFMA

constexpr int kAbsH = 128, kAbsDH = 128, kAbsDC = 512, kAbsDR = 64, kAbsRow = 576;
constexpr int kPassRows = 64;                 // query rows per pass (two 32-row tiles)
constexpr int kAbsPitch = 128 + 8;            // bf16 per staged row (the 16-byte pad spreads rows over banks)

// Inverse frequencies base^(-2j/d_R) of the positional pairs, computed on the host in fp64
// (an fp64 power per workgroup would sit on every workgroup's critical path).
struct RopeTheta {
  double v[kAbsDR / 2];
};

static RopeTheta rope_theta(const mla_config_t& cfg) {
  RopeTheta theta;
  for (int j = 0; j < kAbsDR / 2; ++j) theta.v[j] = std::pow((double)cfg.rope_base, -2.0 * j / (double)kAbsDR);
  return theta;
}

// q_abs[t, h, 128qc + c'] for c' < 128 and the 64 query rows t of block z: wave w computes
// columns 128qc + 32w .. +31; B[k = d, n = c] = W_UK[c, h, d], A[m = t, k = d] = q^C[t, h, d],
// both read from LDS, where they arrive through loads that each cover 4 x 256 contiguous
// bytes (the weight rows of head h are 256 bytes, 32 KB apart; a fragment-shaped read would
// touch 32 rows per instruction).  Quarter qc also rotates the positional part of the rows
// t with t % 4 == qc.  Every load (weights, query rows, positional inputs) is issued before
// anything waits, and the rotation runs while the matrix instructions execute.
constexpr int kRowPitch = 2 * kAbsDH + 16;    // bytes per staged weight / query row (the pad spreads rows over banks)

struct AbsorbArgs {
  const uint16_t* q_nope;
  const uint16_t* q_rope;
  const int32_t* q_pos;
  const uint16_t* w_uk;
  uint16_t* q_abs;
  int T;
};

// Workgroup (h, qc, z) of the absorption; every thread of the workgroup calls it.
__device__ __forceinline__ void absorb_q_block(const AbsorbArgs& aq, const RopeTheta& theta, int h, int qc, int z) {
  __shared__ __attribute__((aligned(16))) uint8_t wst[128 * kRowPitch];           // [c'][d] bf16
  __shared__ __attribute__((aligned(16))) uint8_t qst[kPassRows * kRowPitch];     // [t - t0][d] bf16, then
  static_assert(kPassRows * kAbsPitch * 2 <= sizeof(qst), "result tile fits the query stage");
  uint16_t* stage = reinterpret_cast<uint16_t*>(qst);   // the results [t - t0][c'] (52 KB in all: 3 per CU)
  const uint16_t* __restrict__ q_nope = aq.q_nope;
  const uint16_t* __restrict__ q_rope = aq.q_rope;
  const int32_t* __restrict__ q_pos = aq.q_pos;
  const uint16_t* __restrict__ w_uk = aq.w_uk;
  uint16_t* __restrict__ q_abs = aq.q_abs;
  const int T = aq.T, t0 = kPassRows * z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lg = lane >> 5;

  // weight rows c = 128qc + p/16, bytes 16(p%16) .. for piece p = tid + 256i
  u32x4 wv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = tid + 256 * i;
    wv[i] = *reinterpret_cast<const u32x4*>(w_uk + (size_t)(128 * qc + (p >> 4)) * (kAbsH * kAbsDH) + h * kAbsDH +
                                            8 * (p & 15));
  }
  // Rows past T read row T - 1 (T >= 1 here) and are zeroed or skipped where they are used: with
  // a load or a zero chosen per row, the compiler waits for the loads before the next ones.
  // query rows t0 + p/16 (zeros past T)
  u32x4 qv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i, t = t0 + (p >> 4);
    qv[i] = *reinterpret_cast<const u32x4*>(q_nope + ((size_t)(t < T ? t : T - 1) * kAbsH + h) * kAbsDH +
                                           8 * (p & 15));
  }
  // positional part: rows t0 + 4i + qc (i < 16) x 32 pairs, pair e = tid + 256i' (i' < 2) being
  // row t0 + 4(e/32) + qc, pair e%32 = tid%32 (rows past T are not rotated)
  const int jp = tid & 31;
  const double th = theta.v[jp];
  uint32_t rx[2];
  int rpos[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 4 * ((tid + 256 * i) >> 5) + qc, tc = t < T ? t : T - 1;
    rx[i] = *reinterpret_cast<const uint32_t*>(q_rope + ((size_t)tc * kAbsH + h) * kAbsDR + 2 * jp);
    rpos[i] = q_pos[tc];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = tid + 256 * i;
    *reinterpret_cast<u32x4*>(wst + (p >> 4) * kRowPitch + 16 * (p & 15)) = wv[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    *reinterpret_cast<u32x4*>(qst + (p >> 4) * kRowPitch + 16 * (p & 15)) =
        t0 + (p >> 4) < T ? qv[i] : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // A fragments: rows 32rt + li, d = 16ks + 8lg .. +7; B fragments: weight row 32w + li, same d
  f32x16 acc[2] = {};
  const uint8_t* wb = wst + (32 * wave + li) * kRowPitch + 16 * lg;
  const uint8_t* qb = qst + li * kRowPitch + 16 * lg;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wb + 32 * ks));
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qb + 32 * rt * kRowPitch + 32 * ks));
      acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[rt], 0, 0, 0);
    }
  }
  // The angle pos * base^(-2j/d_R) and its reduction modulo 2 pi are taken in fp64 (positions
  // reach 2^15, so an fp32 angle would be off by milliradians); cosine and sine of the reduced
  // angle (|r| <= pi) in fp32 are then accurate to a few fp32 ulps, far below the bf16 rounding
  // of the result.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 4 * ((tid + 256 * i) >> 5) + qc;
    if (t < T) {
      const double ang = (double)rpos[i] * th;
      const double k = rint(ang * 0.15915494309189535);                   // ang / (2 pi)
      const double red = fma(-k, 6.283185307179586, ang) - k * 2.4492935982947064e-16;   // 2 pi = hi + lo
      float sn, cs;
      sincosf((float)red, &sn, &cs);
      const float x0 = bf16_bits_to_f32(rx[i] & 0xFFFFu), x1 = bf16_bits_to_f32(rx[i] >> 16);
      *reinterpret_cast<uint32_t*>(q_abs + ((size_t)t * kAbsH + h) * kAbsRow + kAbsDC + 2 * jp) =
          pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
    }
  }
  // 32x32 accumulator layout: lane l holds column l%32 and rows 8(k/4) + 4(l/32) + k%4
  __syncthreads();   // every wave's query-fragment reads are done before the results overwrite them
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 32 * rt + 8 * (k >> 2) + 4 * lg + (k & 3);
      stage[r * kAbsPitch + 32 * wave + li] = (uint16_t)f32_to_bf16_bits(acc[rt][k]);
    }
  __syncthreads();
  // 64 rows x 256 bytes: piece p = tid + 256i is row p/16, bytes 16(p%16) ..
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i, r = p >> 4;
    const int t = t0 + r;
    if (t < T)
      *reinterpret_cast<u32x4*>(q_abs + ((size_t)t * kAbsH + h) * kAbsRow + 128 * qc + 8 * (p & 15)) =
          *reinterpret_cast<const u32x4*>(stage + r * kAbsPitch + 8 * (p & 15));
  }
}

__global__ void __launch_bounds__(256) absorb_q_mfma_kernel(AbsorbArgs aq, RopeTheta theta) {
  absorb_q_block(aq, theta, blockIdx.x, blockIdx.y, blockIdx.z);
}

// One launch for a step's cache append and query absorption (independent work): the first
// n_append workgroups append four tokens each and go out first, the rest are the absorption's
// (h, qc, z).  At three workgroups per CU (the absorption's 52 KB of LDS) up to 256 append
// workgroups and 512 absorption workgroups all run at once.
template <int CacheFmt>
__global__ void __launch_bounds__(256) append_absorb_kernel(AppendArgs ap, AppendTheta ath, AbsorbArgs aq,
                                                            RopeTheta theta, int n_append) {
  const int bid = blockIdx.x;
  if (bid < n_append) {
    if constexpr (CacheFmt == MLA_FP8_E4M3_B32)
      append_block_token(ap, ath, bid * 4 + (threadIdx.x >> 6));
    else
      append_dsv2_token<CacheFmt>(ap, ath, bid * 4 + (threadIdx.x >> 6));
  } else {
    const int a = bid - n_append;
    absorb_q_block(aq, theta, a % kAbsH, (a / kAbsH) % (kAbsDC / 128), a / (kAbsH * (kAbsDC / 128)));
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
      // unrolled so that several iterations' loads are in flight at once (the sum keeps its order)
#pragma unroll 8
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

// out^T[v, t] = W_UV,h^T[v, c] . o_lat^T[c, t] for one head h, output columns
// v = 64qv .. 64qv+63 and the 64 query rows of block z, by eight waves: wave w takes the
// contraction quarter c = 128(w%4) .. +127 of the 32 columns 64qv + 32(w/4) .. +31, and the four
// quarters' partial tiles are summed through LDS.  The weight slice W_UV[:, h, 64qv .. +63]
// (512 rows of 128 bytes, one whole cache line per row) is copied to LDS once, as two planes of
// 32 columns (64-byte rows); the A operand (rows v, K = c) comes from a plane through transposing
// reads, with the 64-byte pitch putting the four rows of one read on four different 64-byte bank
// groups.  o_lat is read with each load instruction covering 1 KB of one row and reaches the B
// operand (K = c, N = t) through an LDS stage in bf16, 32 rows at a time.  (Against 32 columns
// per four-wave workgroup: half the o_lat reads through L2, and whole lines of W_UV per row.)

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane i gets element i%4
// of the four values read by source lane 4j + i/4, as its element j.
__device__ __forceinline__ bf16x4 op_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(const MLA_LDS uint8_t*)p);
}

constexpr int kOutCols = 64;                   // output columns per workgroup
constexpr int kOutThreads = 512;               // 8 waves: 4 contraction quarters x 2 column halves

__global__ void __launch_bounds__(kOutThreads) out_proj_mfma_kernel(
    const float* __restrict__ o_lat, const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
    int T) {
  // [column half][c][32 v] bf16, then the reduction [quarter][half][v/4 in the half][t] of f32x4
  __shared__ __attribute__((aligned(16))) uint8_t wl[2 * kAbsDC * 64];
  // [32 t][512 c] bf16; the 16-byte chunk k of row t sits at chunk k ^ (t % 16), so that the 16
  // rows one B-operand read touches fall on different banks
  __shared__ __attribute__((aligned(16))) uint8_t ost[32 * kAbsDC * 2];
  f32x4 (*red)[2][8][kPassRows] = reinterpret_cast<f32x4 (*)[2][8][kPassRows]>(wl);
  static_assert(sizeof(f32x4) * 4 * 2 * 8 * kPassRows <= sizeof(wl), "reduction tile fits the weight stage");
  const int h = blockIdx.x, qv = blockIdx.y, t0 = kPassRows * blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kw = wave & 3, ch = wave >> 2;   // contraction quarter, column half
  const int g = lane >> 5;                   // K group of this lane: c = 16ks + 8g .. +7
  // weight slice: piece p = tid + 512i is row p/8, bytes 16(p%8) .. of the row's 128
  u32x4 r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = tid + kOutThreads * i;
    r[i] = *reinterpret_cast<const u32x4*>(w_uv + (size_t)(p >> 3) * (kAbsH * kOutDV) + h * kOutDV +
                                           kOutCols * qv + 8 * (p & 7));
  }
  // o_lat rows t0 .. t0+63 of head h: piece p = tid + 512i is row p/128 (= 4i + tid/128), floats
  // 4(p%128) .. +3.  Rows past T read row T - 1 (T >= 1 here) and are staged as zeros: with a load
  // or a zero chosen per row, the compiler waits for the loads before the next ones.
  f32x4 ov[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = tid + kOutThreads * i, t = t0 + (p >> 7);
    ov[i] = *reinterpret_cast<const f32x4*>(o_lat + ((size_t)(t < T ? t : T - 1) * kAbsH + h) * kAbsDC +
                                           4 * (p & 127));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = tid + kOutThreads * i, pc = p & 7;
    *reinterpret_cast<u32x4*>(wl + ((pc >> 2) * kAbsDC + (p >> 3)) * 64 + 16 * (pc & 3)) = r[i];
  }
  // A operand: source lane s = 16G + 4j + a reads row 128kw + 16ks + 8(G/2) + j (+4 for the high
  // half) at columns 16(G%2) + 4a .. +3 of its plane, so that output lane l holds column l%32 of
  // the tile and rows 8(l/32) .. +7 of the K-step, matching B.
  const int G = lane >> 4, jr = (lane >> 2) & 3, ac = lane & 3;
  const uint8_t* wb = wl + (ch * kAbsDC + 128 * kw + 8 * (G >> 1) + jr) * 64 + 2 * (16 * (G & 1) + 4 * ac);
  // B operand: lane l reads staged row l%32, chunk 16kw + 2ks + g (columns 128kw + 16ks + 8g .. +7)
  const int orow = lane & 31;
  const uint8_t* ob = ost + orow * (kAbsDC * 2);
  f32x16 acc[2] = {};
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    // stage rows 32rt .. 32rt+31 (pieces i = 8rt .. 8rt+7)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + kOutThreads * i, row = p >> 7, k = (p & 127) >> 1;
      const f32x4 x = t0 + 32 * rt + row < T ? ov[8 * rt + i] : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<u32x2*>(ost + row * (kAbsDC * 2) + 16 * (k ^ (row & 15)) + 8 * (p & 1)) =
          u32x2{cvt_pk_bf16(x[0], x[1]), cvt_pk_bf16(x[2], x[3])};
    }
    __syncthreads();   // weight slice and stage written
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x4 lo = op_tr16(wb + 16 * ks * 64);
      const bf16x4 hi = op_tr16(wb + (16 * ks + 4) * 64);
      const bf16x8 a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 b =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ob + 16 * ((16 * kw + 2 * ks + g) ^ (orow & 15))));
      acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[rt], 0, 0, 0);
    }
    __syncthreads();   // stage and weight reads done before they are rewritten (or reused for the reduction)
  }
  // acc[rt][4m + i] = partial out^T[v = 32ch + 8m + 4g + i, t = 32rt + lane%32]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      red[kw][ch][2 * m + g][32 * rt + (lane & 31)] =
          f32x4{acc[rt][4 * m], acc[rt][4 * m + 1], acc[rt][4 * m + 2], acc[rt][4 * m + 3]};
  __syncthreads();
  // thread tid: row t0 + tid/8, columns 64qv + 8(tid%8) .. +7 (half vh = tid%8/4)
  {
    const int rr = tid >> 3, vq = tid & 7, vh = vq >> 2, vc = vq & 3;
    f32x4 s0 = red[0][vh][2 * vc][rr], s1 = red[0][vh][2 * vc + 1][rr];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      s0 += red[w][vh][2 * vc][rr];
      s1 += red[w][vh][2 * vc + 1][rr];
    }
    const int t = t0 + rr;
    if (t < T)
      *reinterpret_cast<u32x4*>(out + ((size_t)t * kAbsH + h) * kOutDV + kOutCols * qv + 8 * vq) =
          u32x4{pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]), pack_bf16x2(s1[0], s1[1]),
                pack_bf16x2(s1[2], s1[3])};
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
    // unrolled so that several iterations' loads are in flight at once (the sum keeps its order)
#pragma unroll 8
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
    dim3 grid(kAbsH, kAbsDC / 128, (T + kPassRows - 1) / kPassRows);
    const AbsorbArgs aq{static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope), q_pos,
                        static_cast<const uint16_t*>(w_uk), static_cast<uint16_t*>(q_abs), T};
    hipLaunchKernelGGL(absorb_q_mfma_kernel, grid, dim3(256), 0, stream, aq, rope_theta(cfg));
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
    hipLaunchKernelGGL(out_proj_mfma_kernel, dim3(kAbsH, kOutDV / kOutCols, (T + kPassRows - 1) / kPassRows),
                       dim3(kOutThreads), 0, stream, o_lat, static_cast<const uint16_t*>(w_uv),
                       static_cast<uint16_t*>(out), T);
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

hipError_t launch_append(const mla_config_t& cfg, void* cache, float* cache_scale, int num_blocks,
                         const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* seq_of,
                         const int32_t* block_table, int batch, int max_blocks, int n, hipStream_t stream);

// A step's append and absorption: one launch for the DeepSeek-V2 shape with bf16 activations
// (every cache format), else the two launches.
hipError_t launch_append_absorb(const mla_config_t& cfg, void* cache, float* cache_scale, int num_blocks,
                                const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* seq_of,
                                const int32_t* block_table, int batch, int max_blocks, int n, const void* q_nope,
                                const void* q_rope, const int32_t* q_pos, const void* w_uk, void* q_abs, int T,
                                hipStream_t stream) {
  const bool block8 = cfg.cache_dtype == MLA_FP8_E4M3_B32 && cfg.act_dtype == MLA_BF16;
  if (n > 0 && T > 0 && (append_dsv2_applies(cfg) || block8) && is_dsv2_shape(cfg)) {
    const AppendArgs ap = append_args(cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table, batch,
                                      max_blocks, n);
    const AbsorbArgs aq{static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope), q_pos,
                        static_cast<const uint16_t*>(w_uk), static_cast<uint16_t*>(q_abs), T};
    const int n_append = (n + 3) / 4;
    const dim3 grid(n_append + kAbsH * (kAbsDC / 128) * ((T + kPassRows - 1) / kPassRows));
    if (cfg.cache_dtype == MLA_BF16)
      hipLaunchKernelGGL(append_absorb_kernel<MLA_BF16>, grid, dim3(256), 0, stream, ap, append_theta(cfg), aq,
                         rope_theta(cfg), n_append);
    else if (block8)
      hipLaunchKernelGGL(append_absorb_kernel<MLA_FP8_E4M3_B32>, grid, dim3(256), 0, stream, ap, append_theta(cfg),
                         aq, rope_theta(cfg), n_append);
    else
      hipLaunchKernelGGL(append_absorb_kernel<MLA_FP8_E4M3>, grid, dim3(256), 0, stream, ap, append_theta(cfg), aq,
                         rope_theta(cfg), n_append);
    return hipGetLastError();
  }
  hipError_t e = launch_append(cfg, cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table, batch,
                               max_blocks, n, stream);
  if (e != hipSuccess) return e;
  return launch_absorb_q(cfg, q_nope, q_rope, q_pos, w_uk, q_abs, T, stream);
}

}  // namespace mla
