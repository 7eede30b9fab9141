// Latent-space decode attention: split-K flash decoding over the paged cache, then a
// log-sum-exp combine of the split partials.
//
// After the up-projections are folded away the model attends in latent space directly
// (katajob interview page, "Why it is not just extra work at decode time"): every head's
// score is q_abs[i] . [c_t ; k_R,t] and its output is sum_t w_t c_t, so one cached row
// serves all H heads.  Decode streams the whole cache from HBM once per step (zenaique
// "How does DeepSeek's Multi-Latent Attention (MLA) compress the KV cache below GQA?",
// "Concept explanation"), which makes this kernel the step's bandwidth roofline.
//
// Matrix-core kernel (DeepSeek-V2 shape: H=128, d_c=512, d_R=64, bf16 cache)
//   grid      G*Sq*2 workgroups: G token ranges split the batch's pages evenly ("stream-K":
//             a range may span sequence boundaries), times Sq queries, times two head halves.
//             blockIdx is remapped so that the workgroups sharing a range sit on one XCD and
//             read each page through the same L2.
//   block     256 threads = 4 waves (1 per SIMD); wave w owns 16 heads of the workgroup's 64
//             and keeps their folded queries (72 VGPRs) and O^T (128 AGPRs) in registers.
//   per page  (64 tokens = one tile) staged in LDS by 16-byte global->LDS loads, double
//             buffered (2 x 72 KiB), rows XOR-swizzled at 16-byte granularity:
//               S^T[64 tok, 16 heads] = Tile[64, 576] . Qabs^T     v_mfma_f32_16x16x32_bf16
//               online softmax in the exp2 domain (rescale only when the max grows by > 8)
//               O^T[512, 16 heads]   += Tile[:, :512]^T . P^T       (V^T via ds_read_tr16_b64)
//   output    a range that covers a whole sequence writes o_lat/lse directly; otherwise it
//             writes a normalised partial (O/l, lse) to the workspace slot g + b.
#include "common.h"

namespace mla {

constexpr int kH = 128, kDC = 512, kDR = 64, kRow = 576;
constexpr int kChunks = kRow * 2 / 16;            // 72 sixteen-byte chunks per bf16 row
constexpr int kTileBytes = kBlock * kRow * 2;     // 73728

struct DecodeArgs {
  const uint16_t* q_abs;      // [T, H, 576] bf16
  const uint8_t* cache;       // [num_blocks, 64, 576] bf16
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* kv_lens;     // [B]
  float* o_lat;               // [T, H, 512]
  float* lse;                 // [T, H]
  float* part_o;              // [slots*Sq, H, 512]
  float* part_lse;            // [slots*Sq, H]
  int num_blocks, max_blocks, B, Sq, G;
  float scale_log2;           // softmax_scale * log2(e)
};

// tiles (pages) of sequence b that hold tokens, with kv_len clamped to the table width
__device__ __forceinline__ int seq_tiles(const int32_t* kv_lens, int b, int max_blocks, int* L) {
  int len = kv_lens[b];
  len = len < 0 ? 0 : len;
  const int cap = max_blocks * kBlock;
  len = len > cap ? cap : len;
  *L = len;
  return (len + kBlock - 1) / kBlock;
}

// Owner of global tile x when T tiles are split evenly over G ranges [g*T/G, (g+1)*T/G).
__device__ __forceinline__ int range_of_tile(long long x, long long T, int G) {
  return (int)(((x + 1) * (long long)G - 1) / T);
}

// Wave-level scan over the batch: total tiles, and (if want >= 0) the sequence holding
// global tile `want` with that sequence's first tile index.  Every lane gets the results.
__device__ void scan_batch(const int32_t* kv_lens, int B, int max_blocks, long long want, long long* total,
                           int* seq, long long* seq_first) {
  const int lane = threadIdx.x & 63;
  long long run = 0;
  int found_b = -1;
  long long found_s = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    int L;
    const int n = b < B ? seq_tiles(kv_lens, b, max_blocks, &L) : 0;
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int excl = incl - n;
    const bool mine = n > 0 && want >= run + excl && want < run + incl;
    const unsigned long long mask = __ballot(mine);
    if (mask) {
      const int src = __ffsll((long long)mask) - 1;
      found_b = __shfl(b, src, 64);
      found_s = run + __shfl(excl, src, 64);
    }
    run += __shfl(incl, 63, 64);
  }
  *total = run;
  *seq = found_b;
  *seq_first = found_s;
}

// LDS image of one page (73728 B): the 64 latent rows (1024 B each) first, then the 64
// positional rows (128 B each).  Inside a latent row, 16-byte chunk c is stored at chunk
// c ^ key(r) with key(r) = 8(r&1) + ((r>>1)&7); inside a positional row, chunk c is stored at
// c ^ ((r>>1)&7).  With 64 banks (256 B) this makes the two access patterns conflict-free:
// 16 consecutive rows reading one logical chunk (S operand) land on 16 distinct 16-byte bank
// groups, and two rows of opposite parity reading the same 128 B (V operand) land in opposite
// halves of the bank window.  XOR keys below 16 (8 for positional rows) keep chunks in-row.
__device__ __forceinline__ int lat_key(int r) { return ((r & 1) << 3) | ((r >> 1) & 7); }
__device__ __forceinline__ int pos_key(int r) { return (r >> 1) & 7; }
constexpr int kLatBytes = kBlock * kDC * 2;       // 65536: offset of the positional rows

// Wave w loads rows 16w .. 16w+15 of a page: sixteen 1 KiB latent rows (one row per
// instruction, lane l fetches logical chunk l ^ key) and their 128-byte positional rows (two
// instructions, lane l -> row 16w + 8u + l/8).  Rows at or past `nvalid` are fetched from row
// 0 instead (finite data; their scores are masked).
__device__ __forceinline__ void load_tile(uint8_t* lds_buf, const uint8_t* page, int nvalid, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * wave + i;
    const int rs = r < nvalid ? r : 0;
    const uint8_t* src = page + rs * (kRow * 2) + ((lane ^ lat_key(r)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(lds_buf + r * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * wave + 8 * u + (lane >> 3);
    const int rs = r < nvalid ? r : 0;
    const uint8_t* src = page + rs * (kRow * 2) + kDC * 2 + (((lane & 7) ^ pos_key(r)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (MLA_LDS void*)(lds_buf + kLatBytes + (16 * wave + 8 * u) * 128), 16, 0, 0);
  }
}

__device__ __forceinline__ u32x4 lds_read_b128(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 lds_read_b64(const uint8_t* p) { return *reinterpret_cast<const u32x2*>(p); }

// 16x16x32 bf16 MFMA layout (wave64): A lane l holds row l%16 and the 8 K values of K-group
// l/16; B lane l holds column l%16 and the same K-group; the result lane l holds column
// l%16, rows 4*(l/16) + i, i = 0..3.  The order of K inside one instruction is irrelevant as
// long as A and B agree, so P and V may use any common token order.
//
// Token order inside a 16-row M-tile of S^T: result row 4q+i is token 4i+q (q = l/16), so the
// four lane groups of one V read touch rows of alternating parity (opposite bank halves).
__global__ void __launch_bounds__(256, 1) decode_mfma_bf16_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // 2 pages
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;            // 0..3
  const int m = lane & 15, q = lane >> 4;

  // logical (range g, query j, head half hh) of this workgroup.  Consecutive logical ids
  // share a range, and on an 8-XCD part the remap puts consecutive ids on one XCD (blocks
  // are dealt to XCDs round-robin), so the two halves and Sq queries of a range read each
  // page through the same L2.
  const int NG = a.G * a.Sq * 2;
  int lid = blockIdx.x;
  if ((NG & 7) == 0) lid = (blockIdx.x & 7) * (NG >> 3) + (blockIdx.x >> 3);
  const int hh = lid & 1;
  const int g = (lid >> 1) / a.Sq;
  const int j = (lid >> 1) - g * a.Sq;

  long long T_all, s_first;
  int b;
  {
    int dummy_b;
    long long dummy_s;
    scan_batch(a.kv_lens, a.B, a.max_blocks, -1, &T_all, &dummy_b, &dummy_s);
  }
  const long long x0 = (long long)g * T_all / a.G;
  const long long x1 = (long long)(g + 1) * T_all / a.G;
  if (x0 >= x1) return;
  {
    long long tot;
    scan_batch(a.kv_lens, a.B, a.max_blocks, x0, &tot, &b, &s_first);
  }
  if (b < 0) return;                            // unreachable: x0 < T_all lies in some sequence
  int L;
  int nb = seq_tiles(a.kv_lens, b, a.max_blocks, &L);
  int tb = (int)(x0 - s_first);
  int seg_tb0 = tb;

  const int head = 64 * hh + 16 * wave + m;     // head of this lane (N index of S^T and O^T)

  // S^T operand A = tile row 16mt + rho(m), rho(m) = 4(m%4) + m/4, latent chunk 4ks + q for
  // ks < 16, positional chunk 4(ks-16) + q for ks = 16, 17.  key(16mt + rho) == key(rho).
  const int rho = 4 * (m & 3) + (m >> 2);
  const int lk = lat_key(rho), pk = pos_key(rho);
  int s_lat[4];                                 // by ks % 4; ks / 4 adds 256 B, mt adds 16 KiB
#pragma unroll
  for (int u = 0; u < 4; ++u) s_lat[u] = rho * 1024 + (((4 * u + q) ^ lk) << 4);
  const int s_pos0 = kLatBytes + rho * 128 + ((q ^ pk) << 4);
  const int s_pos1 = kLatBytes + rho * 128 + (((4 + q) ^ pk) << 4);
  // O^T operand A = V^T, read with the transposing LDS load: inside each 16-lane group q,
  // output lane i, element jj is element i%4 of the 8 bytes addressed by source lane
  // 4jj + i/4.  Element e = 4h + jj of lane (m, q) must be token 32kk + 16h + 4jj + q (the P^T
  // order) at latent column 16t + m, so source lane (q, 4jj + u) addresses that token's row,
  // columns 16t + 4u .. +3 = logical chunk 2t + u/2, byte 8(u&1).  The row's key is
  // 8(q&1) + ((2jj + q/2)&7) for every kk, h; the chunk XOR splits into a per-lane part
  // (t&7 ^ key/2, 8 variants) and immediates (kk, h, t&24).
  int v_addr[8];
  {
    const int jj = m >> 2, u = m & 3;
    const int key = 8 * (q & 1) + ((2 * jj + (q >> 1)) & 7);
    const int base = (4 * jj + q) * 1024 + 16 * ((u >> 1) ^ (key & 1)) + 8 * (u & 1);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) v_addr[tt] = base + 32 * (tt ^ (key >> 1));
  }

  bf16x8 qf[18];                                // folded query, K-steps 0..17 (32 columns each)
  f32x4 oacc[32];
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_q = [&](int bb) {
    const uint16_t* qp = a.q_abs + ((size_t)(bb * a.Sq + j) * kH + head) * kRow + 8 * q;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * ks));
  };

  int nvalid_cur;
  {
    int pg = a.block_table[(size_t)b * a.max_blocks + tb];
    int nv = L - tb * kBlock;
    nv = nv > kBlock ? kBlock : nv;
    if (pg < 0 || pg >= a.num_blocks) { pg = 0; nv = 0; }
    nvalid_cur = nv;
    load_tile(smem, a.cache + (size_t)pg * kTileBytes, nv > 0 ? nv : 1, wave, lane);
  }
  load_q(b);

  for (long long x = x0; x < x1; ++x) {
    const int buf = (int)((x - x0) & 1);
    int bn = b, tbn = tb + 1, Ln = L, nbn = nb;
    if (x + 1 < x1 && tbn >= nb) {
      bn = b + 1;
      nbn = seq_tiles(a.kv_lens, bn, a.max_blocks, &Ln);
      while (nbn == 0 && bn + 1 < a.B) { ++bn; nbn = seq_tiles(a.kv_lens, bn, a.max_blocks, &Ln); }
      tbn = 0;
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the current page (and q) landed
    __syncthreads();                  // ... and every wave's; the other buffer is free
    int nvalid_next = 0;
    if (x + 1 < x1) {
      int pg = a.block_table[(size_t)bn * a.max_blocks + tbn];
      int nv = Ln - tbn * kBlock;
      nv = nv > kBlock ? kBlock : nv;
      if (pg < 0 || pg >= a.num_blocks) { pg = 0; nv = 0; }
      nvalid_next = nv;
      load_tile(smem + (buf ^ 1) * kTileBytes, a.cache + (size_t)pg * kTileBytes, nv > 0 ? nv : 1, wave, lane);
    }
    const uint8_t* tile = smem + buf * kTileBytes;

    // ---------------------------------------------------------------- S^T = Tile . Q^T
    // K-step ks reads four 16-byte A fragments (one per M-tile); two K-steps stay in flight
    // ahead of the MFMAs that consume them.
    auto s_frag = [&](int ks, int mt) -> u32x4 {
      const uint8_t* base = ks < 16 ? tile + s_lat[ks & 3] + 256 * (ks >> 2) + mt * 16 * 1024
                                    : tile + (ks == 16 ? s_pos0 : s_pos1) + mt * 16 * 128;
      return lds_read_b128(base);
    };
    f32x4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 ring[3][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { ring[0][mt] = s_frag(0, mt); ring[1][mt] = s_frag(1, mt); }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + 2 < 18) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) ring[(ks + 2) % 3][mt] = s_frag(ks + 2, mt);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ring[ks % 3][mt]), qf[ks],
                                                           sacc[mt], 0, 0, 0);
    }

    // first V fragments (independent of P) go out before the softmax
    // step v = 32kk + t: K-step kk (tokens 32kk..32kk+31), M-tile t (latent columns 16t..16t+15)
    auto v_frag = [&](int v) -> bf16x8 {
      const int kk = v >> 5, t = v & 31;
      const uint8_t* p0 = tile + v_addr[t & 7] + 32 * (t & 24) + (32 * kk) * 1024;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + 16 * 1024));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    constexpr int kVDepth = 4;
    bf16x8 vring[kVDepth];
#pragma unroll
    for (int v = 0; v < kVDepth; ++v) vring[v] = v_frag(v);

    // ---------------------------------------------------------------- online softmax
    // sacc[mt][i] is token 16mt + 4i + q of this tile, head `head`
    const int lim = (L - a.Sq + j) - tb * kBlock;   // visible tile rows are r <= lim
    const bool masked = (nvalid_cur <= 0) || (lim < kBlock - 1);
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sv = sacc[mt][i] * a.scale_log2;
        if (masked && (nvalid_cur <= 0 || 16 * mt + 4 * i + q > lim)) sv = -INFINITY;
        sacc[mt][i] = sv;
        tmax = fmaxf(tmax, sv);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (__ballot(tmax > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) oacc[i] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    uint32_t pw[8];                              // pw[2mt + u]: tokens of M-tile mt, pair u
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(sacc[mt][2 * u] - m_use),
                                       __builtin_amdgcn_exp2f(sacc[mt][2 * u + 1] - m_use));
        pw[2 * mt + u] = w;
        l_run += bf16_bits_to_f32(w & 0xFFFFu) + bf16_bits_to_f32(w >> 16);
      }
    }

    // ---------------------------------------------------------------- O^T += V^T . P^T
    // K-step kk covers tokens 32kk .. 32kk+31 = M-tiles 2kk, 2kk+1: P^T fragment pw[4kk..4kk+3].
    bf16x8 pfrag[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 pf = {pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]};
      pfrag[kk] = __builtin_bit_cast(bf16x8, pf);
    }
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      const bf16x8 af = vring[v % kVDepth];
      if (v + kVDepth < 64) vring[v % kVDepth] = v_frag(v + kVDepth);
      oacc[v & 31] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pfrag[v >> 5], oacc[v & 31], 0, 0, 0);
    }

    // ---------------------------------------------------------------- end of a range?
    if ((tb == nb - 1) || (x + 1 == x1)) {
      float l_tot = l_run + __shfl_xor(l_run, 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const bool whole = (seg_tb0 == 0) && (tb == nb - 1);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.0f;
      const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      const size_t row = whole ? (size_t)(b * a.Sq + j) * kH + head : ((size_t)(g + b) * a.Sq + j) * kH + head;
      float* dst_o = (whole ? a.o_lat : a.part_o) + row * kDC;
      // oacc[t][i] is latent column 16t + 4q + i
#pragma unroll
      for (int t = 0; t < 32; ++t) *reinterpret_cast<f32x4*>(dst_o + 16 * t + 4 * q) = oacc[t] * inv;
      if (q == 0) (whole ? a.lse : a.part_lse)[row] = lse_v;
      if (x + 1 < x1) {
        load_q(bn);
#pragma unroll
        for (int i = 0; i < 32; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        seg_tb0 = 0;
      }
    }
    b = bn;
    tb = tbn;
    L = Ln;
    nb = nbn;
    nvalid_cur = nvalid_next;
  }
}

// ------------------------------------------------------------------------ LSE combine

// One workgroup per (query row, 4 heads); 64 threads per head, 8 latent columns each.
__global__ void __launch_bounds__(256) combine_kernel(DecodeArgs a) {
  const int row = blockIdx.x;          // b*Sq + j
  const int b = row / a.Sq, j = row - b * a.Sq;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  long long T_all, S_b;
  int bb;
  scan_batch(a.kv_lens, a.B, a.max_blocks, -1, &T_all, &bb, &S_b);
  // first tile of sequence b: rescan with an exclusive prefix
  long long first = 0;
  for (int base = 0; base < b; base += 64) {
    const int q = base + lane;
    int L;
    const int n = q < b ? seq_tiles(a.kv_lens, q, a.max_blocks, &L) : 0;
    first += wave_sum_i(n);
  }
  int Lb;
  const int nb = seq_tiles(a.kv_lens, b, a.max_blocks, &Lb);
  float* out = a.o_lat + ((size_t)row * kH + h) * kDC + 8 * lane;
  if (nb == 0) {
    *reinterpret_cast<f32x4*>(out) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(out + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane == 0) a.lse[(size_t)row * kH + h] = -INFINITY;
    return;
  }
  const int g_lo = range_of_tile(first, T_all, a.G);
  const int g_hi = range_of_tile(first + nb - 1, T_all, a.G);
  if (g_lo == g_hi) return;            // one range covered the sequence and wrote the result
  // Ranges between g_lo and g_hi that hold no page at all (possible when the batch has fewer
  // pages than ranges) wrote nothing: skip them.
  auto empty = [&](int g) {
    return (long long)g * T_all / a.G == (long long)(g + 1) * T_all / a.G;
  };
  float mx = -INFINITY;
  for (int g = g_lo; g <= g_hi; ++g)
    if (!empty(g)) mx = fmaxf(mx, a.part_lse[((size_t)(g + b) * a.Sq + j) * kH + h]);
  float den = 0.f;
  for (int g = g_lo; g <= g_hi; ++g)
    if (!empty(g) && mx != -INFINITY) den += __expf(a.part_lse[((size_t)(g + b) * a.Sq + j) * kH + h] - mx);
  const float lse = (den > 0.f) ? mx + __logf(den) : -INFINITY;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int g = g_lo; g <= g_hi; ++g) {
    if (empty(g)) continue;
    const size_t prow = ((size_t)(g + b) * a.Sq + j) * kH + h;
    const float ls = a.part_lse[prow];
    const float w = (lse == -INFINITY || ls == -INFINITY) ? 0.f : __expf(ls - lse);
    const float* src = a.part_o + prow * kDC + 8 * lane;
    acc0 += w * *reinterpret_cast<const f32x4*>(src);
    acc1 += w * *reinterpret_cast<const f32x4*>(src + 4);
  }
  *reinterpret_cast<f32x4*>(out) = acc0;
  *reinterpret_cast<f32x4*>(out + 4) = acc1;
  if (lane == 0) a.lse[(size_t)row * kH + h] = lse;
}

// ------------------------------------------------------------------------ generic decode (VALU)

// One workgroup per (query row, head), whole sequence, tokens in chunks of 256: each
// thread scores one token of the chunk, the chunk's max/sum update a running softmax,
// then each thread accumulates its latent columns over the chunk.  For small shapes
// (the fp32 test configuration) where matrix-core tiling does not apply.
template <typename CacheT, typename QT>
__global__ void __launch_bounds__(256) decode_generic_kernel(
    const QT* __restrict__ q_abs, const CacheT* __restrict__ cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ kv_lens, float* __restrict__ o_lat, float* __restrict__ lse, int num_blocks,
    int max_blocks, int Sq, int H, int d_c, int d_r, float scale) {
  __shared__ float qs[1024];
  __shared__ float ps[256];
  __shared__ int prow[256];
  __shared__ float red[8];
  const int row = blockIdx.x, h = blockIdx.y;
  const int b = row / Sq, j = row - b * Sq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int width = d_c + d_r;
  for (int k = tid; k < width; k += 256) qs[k] = load_act(q_abs, ((size_t)row * H + h) * width + k);
  int L;
  seq_tiles(kv_lens, b, max_blocks, &L);
  const int p = L - Sq + j;
  float m_run = -INFINITY, l_run = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};   // columns tid, tid+256, ...
  __syncthreads();
  for (int t0 = 0; t0 <= p && t0 < L; t0 += 256) {
    const int t = t0 + tid;
    float s = -INFINITY;
    int rowidx = -1;
    if (t <= p && t < L) {
      const int pg = block_table[(size_t)b * max_blocks + t / kBlock];
      if (pg >= 0 && pg < num_blocks) {
        rowidx = pg * kBlock + (t % kBlock);
        const CacheT* r = cache + (size_t)rowidx * width;
        float d = 0.f;
        for (int k = 0; k < width; ++k) d += qs[k] * load_act(r, k);
        s = d * scale;
      }
    }
    float cm = wave_max(s);
    if (lane == 0) red[wave] = cm;
    __syncthreads();
    cm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m_run, cm);
    const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    const float pv = (s == -INFINITY) ? 0.f : __expf(s - m_new);
    ps[tid] = pv;
    prow[tid] = rowidx;
    float cs = wave_sum(pv);
    if (lane == 0) red[4 + wave] = cs;
    __syncthreads();
    cs = red[4] + red[5] + red[6] + red[7];
    l_run = l_run * alpha + cs;
    m_run = m_new;
    const int nt = min(256, min(p + 1, L) - t0);
    for (int q = 0; q < 4; ++q) {
      const int c = tid + 256 * q;
      if (c >= d_c) break;
      float v = acc[q] * alpha;
      for (int u = 0; u < nt; ++u)
        if (prow[u] >= 0) v += ps[u] * load_act(cache + (size_t)prow[u] * width, c);
      acc[q] = v;
    }
    __syncthreads();
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  for (int q = 0; q < 4; ++q) {
    const int c = tid + 256 * q;
    if (c < d_c) o_lat[((size_t)row * H + h) * d_c + c] = acc[q] * inv;
  }
  if (tid == 0) lse[(size_t)row * H + h] = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
}

// ------------------------------------------------------------------------ launchers

bool is_dsv2_shape(const mla_config_t& c);

// Token ranges of the split: one workgroup per (range, query, head half) and one workgroup
// per compute unit (each holds 144 KiB of LDS), so G = CUs / (2 Sq), capped by the pages.
int decode_num_ranges(int num_cus, int B, int Sq, int max_blocks) {
  long long cap = (long long)B * max_blocks;
  int G = num_cus / (2 * (Sq > 0 ? Sq : 1));
  if (G < 1) G = 1;
  if (cap < G) G = (int)(cap < 1 ? 1 : cap);
  return G;
}

size_t decode_workspace_bytes(const mla_config_t& cfg, int num_cus, int B, int Sq, int max_blocks) {
  if (!(cfg.cache_dtype != MLA_F32 && is_dsv2_shape(cfg))) return 256;   // generic path: none needed
  const int G = decode_num_ranges(num_cus, B, Sq, max_blocks);
  const size_t slots = (size_t)(G + B - 1) * Sq;
  const size_t o_bytes = slots * kH * kDC * sizeof(float);
  const size_t l_bytes = slots * kH * sizeof(float);
  return ((o_bytes + 255) & ~(size_t)255) + ((l_bytes + 255) & ~(size_t)255);
}

hipError_t launch_decode(const mla_config_t& cfg, int num_cus, const void* q_abs, const float* q_scale,
                         const void* cache, const float* cache_scale, int num_blocks, const int32_t* block_table,
                         int max_blocks, const int32_t* kv_lens, int B, int Sq, void* workspace, float* o_lat,
                         float* lse, hipStream_t stream, int phases) {
  if (B == 0) return hipSuccess;
  const float scale = cfg.softmax_scale;
  if (cfg.cache_dtype == MLA_BF16 && is_dsv2_shape(cfg)) {
    DecodeArgs a;
    a.q_abs = static_cast<const uint16_t*>(q_abs);
    a.cache = static_cast<const uint8_t*>(cache);
    a.block_table = block_table;
    a.kv_lens = kv_lens;
    a.o_lat = o_lat;
    a.lse = lse;
    const int G = decode_num_ranges(num_cus, B, Sq, max_blocks);
    const size_t slots = (size_t)(G + B - 1) * Sq;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                          ((slots * kH * kDC * sizeof(float) + 255) & ~(size_t)255));
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.B = B;
    a.Sq = Sq;
    a.G = G;
    a.scale_log2 = scale * 1.4426950408889634f;
    static bool attr_set = false;   // idempotent; races only repeat the same call
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)decode_mfma_bf16_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kTileBytes);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    if (phases & 1) {
      hipLaunchKernelGGL(decode_mfma_bf16_kernel, dim3(G * Sq * 2), dim3(256), 2 * kTileBytes, stream, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (phases & 2) hipLaunchKernelGGL(combine_kernel, dim3(B * Sq, kH / 4), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (!(phases & 1)) return hipSuccess;   // generic path: one launch does everything
  if (cfg.cache_dtype == MLA_F32 && cfg.act_dtype == MLA_F32) {
    hipLaunchKernelGGL((decode_generic_kernel<float, float>), dim3(B * Sq, cfg.num_heads), dim3(256), 0, stream,
                       static_cast<const float*>(q_abs), static_cast<const float*>(cache), block_table, kv_lens,
                       o_lat, lse, num_blocks, max_blocks, Sq, cfg.num_heads, cfg.d_c, cfg.d_r, scale);
    return hipGetLastError();
  }
  if (cfg.cache_dtype == MLA_BF16 && cfg.act_dtype == MLA_BF16) {
    hipLaunchKernelGGL((decode_generic_kernel<uint16_t, uint16_t>), dim3(B * Sq, cfg.num_heads), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(q_abs), static_cast<const uint16_t*>(cache),
                       block_table, kv_lens, o_lat, lse, num_blocks, max_blocks, Sq, cfg.num_heads, cfg.d_c,
                       cfg.d_r, scale);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
