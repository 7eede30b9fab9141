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
//   grid      G*Sq workgroups: G token ranges split the batch's pages evenly ("stream-K":
//             a range may span sequence boundaries), times Sq queries.  blockIdx is remapped
//             so that the Sq workgroups of one range sit on one XCD and share its L2.
//   block     512 threads = 8 waves (2 per SIMD); all 128 heads of the query live in the
//             workgroup, so every cached row is read from HBM once per query.
//   per step  32 tokens (half a page) staged in LDS by 16-byte global->LDS loads, four
//             stages in flight, rows XOR-swizzled at 16-byte granularity:
//               S^T[32 tok, 16 heads] = Stage[32, 576] . Qabs^T   v_mfma_f32_16x16x32_bf16
//               online softmax in the exp2 domain (rescale only when the max grows by > 8)
//               O^T[256 cols, 32 heads] += Stage[:, :512]^T . P^T (V^T via ds_read_b64_tr_b16)
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

// Read-only kernel inputs are read through the constant address space: with a uniform index
// that is a scalar load, which the compiler may not prove safe through a plain pointer.
__device__ __forceinline__ int ld_const(const int32_t* p, size_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Workgroup barrier without a memory fence: the caller has already waited for its own LDS
// writes (lgkmcnt) and page DMA (vmcnt); the "memory" clobber keeps the compiler from moving
// memory accesses across it.  (A fenced barrier would also wait for the pages in flight.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// tiles (pages) of sequence b that hold tokens, with kv_len clamped to the table width
__device__ __forceinline__ int seq_tiles(const int32_t* kv_lens, int b, int max_blocks, int* L) {
  int len = ld_const(kv_lens, b);
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
  // wave-uniform results: hand them back as scalars
  *total = ((long long)__builtin_amdgcn_readfirstlane((int)(run >> 32)) << 32) |
           (unsigned)__builtin_amdgcn_readfirstlane((int)run);
  *seq = __builtin_amdgcn_readfirstlane(found_b);
  *seq_first = ((long long)__builtin_amdgcn_readfirstlane((int)(found_s >> 32)) << 32) |
               (unsigned)__builtin_amdgcn_readfirstlane((int)found_s);
}

// ---------------------------------------------------------------------------------------
// LDS layout.  The page stream is cut into 32-token half pages; four stages of 36 KiB hold
// the half page being computed and the next three in flight (global->LDS DMA).  One stage:
// 32 latent rows of 1024 B, then 32 positional rows of 128 B.  Inside a latent row, 16-byte
// chunk c is stored at c ^ key(r), key linear over GF(2) in the low four row bits (columns
// 9, 11, 6, 7); inside a positional row at c ^ ((r>>1)&7).  The key was chosen by timing
// the two read patterns on gfx950: 16 rows x one 16-byte chunk per lane group (S operand,
// ds_read_b128) and 4 rows x 32 bytes per 16-lane group (V operand, ds_read_b64_tr_b16) both
// run at the bank-conflict-free rate with it (plain row-parity keys leave one of them 2x
// slower).  XOR keys below 16 (8) keep every chunk inside its row.
// After the stages: one 16-byte P fragment per lane per wave (8 KiB) and a small per-wave
// exchange area (rescale factors, flags, 1/l).
constexpr unsigned long long kLatKeys = 0x3A815CE74DF62B90ull;   // key(r), r = 0..15, one nibble each
constexpr int lat_key_c(int r) { return (int)((kLatKeys >> (4 * (r & 15))) & 15); }
static_assert(lat_key_c(1) == 9 && lat_key_c(2) == 11 && lat_key_c(4) == 6 && lat_key_c(8) == 7 &&
                  lat_key_c(15) == (9 ^ 11 ^ 6 ^ 7),
              "latent-row XOR key is the linear map with columns 9, 11, 6, 7");
__device__ __forceinline__ int lat_key(int r) { return lat_key_c(r); }
__device__ __forceinline__ int pos_key(int r) { return (r >> 1) & 7; }
constexpr int kHalf = 32;                            // tokens per pipeline step
constexpr int kStageLat = kHalf * 1024;              // 32768: offset of the positional rows
constexpr int kStageBytes = kHalf * (1024 + 128);    // 36864
constexpr int kStages = 4;
constexpr int kPBufOff = kStages * kStageBytes;      // 147456
constexpr int kXchOff = kPBufOff + 8 * 64 * 16;      // 155648
constexpr int kXchWave = 256;                        // per wave: alpha[16], inv_l[16], flag
constexpr int kDecodeLds = kXchOff + 8 * kXchWave;   // 157696 bytes (< 160 KiB)

__device__ __forceinline__ u32x4 lds_read_b128(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding and
// leaves the other counters alone (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).  Vector loads complete in order, so vmcnt(n) with n = number of loads issued
// after the ones waited for is sufficient even with stores outstanding.
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// Position in the page stream: sequence b (kv_len L, nb pages), page tb, half h.
struct Cursor {
  int b, tb, h, L, nb;
};

// Wave-uniform values are pinned to scalar registers: table and length lookups then become
// scalar loads, which never wait behind the vector-memory counter of the page DMA.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ void cursor_next(Cursor& c, const int32_t* kv_lens, int B, int max_blocks) {
  if (c.h == 0) {
    c.h = 1;
  } else {
    c.h = 0;
    if (++c.tb >= c.nb) {
      c.tb = 0;
      do {
        if (c.b + 1 >= B) { c.nb = 1; break; }          // past the batch: only reached beyond the range
        ++c.b;
        c.nb = seq_tiles(kv_lens, c.b, max_blocks, &c.L);
      } while (c.nb == 0);
    }
  }
  c.b = uni(c.b); c.tb = uni(c.tb); c.h = uni(c.h); c.L = uni(c.L); c.nb = uni(c.nb);
}

// Valid tokens of the cursor's half page (may be <= 0 for the empty second half of a short
// last page) and its page base; out-of-range page ids read page 0 with no valid token.
__device__ __forceinline__ const uint8_t* half_page(const DecodeArgs& a, const Cursor& c, int* nvalid) {
  int pg = uni(ld_const(a.block_table, (size_t)c.b * a.max_blocks + c.tb));
  int nv = c.L - c.tb * kBlock - c.h * kHalf;
  nv = nv > kHalf ? kHalf : nv;
  if (pg < 0 || pg >= a.num_blocks) { pg = 0; nv = 0; }
  *nvalid = nv;
  return a.cache + (size_t)pg * kTileBytes;
}

// Waves 0..3 each issue nine 1 KiB global->LDS loads per half page: latent rows 8w .. 8w+7
// (lane l fetches logical chunk l ^ key) and the positional rows 8w .. 8w+7 (lane l -> row
// 8w + l/8).  Rows at or past `nvalid` are fetched from the page's row 0 instead (finite
// data, masked scores).
__device__ __forceinline__ void load_half(uint8_t* stage, const uint8_t* page, int h, int nvalid, int wave,
                                          int lane) {
  asm volatile("" : "+v"(lane));   // rebuild the per-lane offsets here rather than keep them live
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * wave + i;
    const int rs = r < nvalid ? kHalf * h + r : 0;
    const uint8_t* src = page + rs * (kRow * 2) + ((lane ^ lat_key(r)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(stage + r * 1024), 16, 0, 0);
  }
  const int r = 8 * wave + (lane >> 3);
  const int rs = r < nvalid ? kHalf * h + r : 0;
  const uint8_t* src = page + rs * (kRow * 2) + kDC * 2 + (((lane & 7) ^ pos_key(r)) << 4);
  __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(stage + kStageLat + 8 * wave * 128), 16, 0, 0);
}

// 16x16x32 bf16 MFMA layout (wave64): A lane l holds row l%16 and the 8 K values of K-group
// l/16; B lane l holds column l%16 and the same K-group; the result lane l holds column
// l%16, rows 4*(l/16) + i, i = 0..3.  The order of K inside one instruction is irrelevant as
// long as A and B agree, so P and V may use any common token order.
//
// Work split (waves w = 0..7, head group hg = w&3 owns heads 32hg .. 32hg+31, sh = w>>2):
//   scores/softmax  wave w: heads 32hg + 16sh + (0..15), all 576 columns, 32 tokens
//                   S^T[32 tok, 16 heads] = Stage[32, 576] . Qabs^T; result row 4q+i of M-tile
//                   mt is token 16mt + 4q + i (q = l/16), which is exactly the P^T operand
//                   order below, so each lane's probabilities are its own B fragment.
//   values          wave w: O^T[256 columns 256sh.., 32 heads of hg] += V^T . P^T with the two
//                   P^T fragments of the pair (hg, hg+4); one transposed V fragment feeds both.
__global__ void __launch_bounds__(512, 1) decode_mfma_bf16_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps row math scalar
  const int m = lane & 15, q = lane >> 4;
  const int hg = wave & 3, sh = wave >> 2;
  const int s_head = 32 * hg + 16 * sh + m;       // scores/softmax head of this lane

  // logical (range g, query j) of this workgroup; consecutive logical ids sit on one XCD
  // (blocks are dealt to the 8 XCDs round-robin), so the Sq queries of a range share L2.
  const int NG = a.G * a.Sq;
  int lid = blockIdx.x;
  if ((NG & 7) == 0) lid = (blockIdx.x & 7) * (NG >> 3) + (blockIdx.x >> 3);
  const int g = lid / a.Sq;
  const int j = lid - g * a.Sq;

  long long T_all, s_first;
  int b0;
  {
    int db;
    long long ds;
    scan_batch(a.kv_lens, a.B, a.max_blocks, -1, &T_all, &db, &ds);
  }
  const long long x0 = (long long)g * T_all / a.G;
  const long long x1 = (long long)(g + 1) * T_all / a.G;
  if (x0 >= x1) return;
  {
    long long tot;
    scan_batch(a.kv_lens, a.B, a.max_blocks, x0, &tot, &b0, &s_first);
  }
  if (b0 < 0) return;                             // unreachable: x0 < T_all lies in some sequence
  const int n_steps = (int)(2 * (x1 - x0));       // half pages of this range

  Cursor cur;
  cur.b = uni(b0);
  cur.nb = uni(seq_tiles(a.kv_lens, cur.b, a.max_blocks, &cur.L));
  cur.L = uni(cur.L);
  cur.tb = uni((int)(x0 - s_first));
  cur.h = 0;
  Cursor pre = cur;                               // prefetch cursor, three half pages ahead
  int seg_tb0 = cur.tb;

  uint8_t* pbuf = smem + kPBufOff;
  uint8_t* xch = smem + kXchOff;
  float* x_alpha = reinterpret_cast<float*>(xch + wave * kXchWave);        // [16]
  float* x_invl = reinterpret_cast<float*>(xch + wave * kXchWave + 64);    // [16]
  int* x_flag = reinterpret_cast<int*>(xch + wave * kXchWave + 128);

  bf16x8 qf[18];
  auto load_q = [&](int bb) {
    const uint16_t* qp = a.q_abs + ((size_t)(bb * a.Sq + j) * kH + s_head) * kRow + 8 * q;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * ks));
  };

  f32x4 oacc[2][16];                              // [N-tile (head half of hg)][M-tile of 16 columns]
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[n][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: half pages 0, 1, 2 of the range in flight
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (k < n_steps) {
      int nv;
      const uint8_t* pg = half_page(a, pre, &nv);
      if (wave < 4) load_half(smem + k * kStageBytes, pg, pre.h, nv, wave, lane);
      cursor_next(pre, a.kv_lens, a.B, a.max_blocks);
    }
  }
  load_q(cur.b);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  for (int y = 0; y < n_steps; ++y) {
    // wait for this wave's loads of half page y (the two younger half pages may stay in flight)
    if (wave < 4) {
      const int younger = min(2, n_steps - 1 - y);
      if (younger >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(18));
      else if (younger == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    lds_barrier();   // every wave's loads landed; stage (y-1)%4 is free
    if (y + 3 < n_steps) {
      int nv;
      const uint8_t* pg = half_page(a, pre, &nv);
      if (wave < 4) load_half(smem + ((y + 3) & 3) * kStageBytes, pg, pre.h, nv, wave, lane);
      cursor_next(pre, a.kv_lens, a.B, a.max_blocks);
    }
    const uint8_t* tile = smem + (y & 3) * kStageBytes;
    // Per-lane LDS addresses, rebuilt each step from an opaque copy of the lane id: cheaper
    // than keeping them live across the loop (the compiler would hoist and spill them).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lm = ln & 15, lq = ln >> 4;
    // S^T operand A: stage row 16mt + m; latent chunk 4ks + q for ks < 16, positional chunk
    // 4(ks-16) + q for ks = 16, 17.  key(16mt + m) == key(m).
    const int rho = lm;
    const int s_row = rho * 1024, s_key = lat_key(rho), p_key = pos_key(rho);
    // V^T operand through the transposing LDS read: inside each 16-lane group q, output lane
    // i, element jj is element i%4 of the 8 bytes addressed by source lane 4jj + i/4.  Element
    // e = 4h + jj of lane (m, q) is token 16h + 4q + jj (the P^T order) at column
    // 256sh + 16t + m, so source lane (q, 4jj + u) addresses that token's row at columns
    // 256sh + 16t + 4u .. +3: logical chunk 32sh + 2t + u/2, byte 8(u&1).  The row key is
    // key(4q + jj) for both h; h adds 16 KiB and t>>3 adds 256 B.
    const int vjj = lm >> 2, vu = lm & 3;
    const int v_key = lat_key(4 * lq + vjj);
    const int v_base = (4 * lq + vjj) * 1024 + 512 * sh + 8 * (vu & 1);
    int nvalid;
    {
      int nv = cur.L - cur.tb * kBlock - cur.h * kHalf;
      nvalid = nv > kHalf ? kHalf : nv;
      const int pg = uni(ld_const(a.block_table, (size_t)cur.b * a.max_blocks + cur.tb));
      if (pg < 0 || pg >= a.num_blocks) nvalid = 0;
    }

    // ---------------------------------------------------------------- S^T = Stage . Q^T
    auto s_frag = [&](int ks, int mt) -> u32x4 {
      return ks < 16 ? lds_read_b128(tile + s_row + (((4 * (ks & 3) + lq) ^ s_key) << 4) + 256 * (ks >> 2) +
                                     mt * 16 * 1024)
                     : lds_read_b128(tile + kStageLat + rho * 128 + (((4 * (ks - 16) + lq) ^ p_key) << 4) +
                                     mt * 16 * 128);
    };
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    u32x4 ring[2][2];
    ring[0][0] = s_frag(0, 0);
    ring[0][1] = s_frag(0, 1);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + 1 < 18) {
        ring[(ks + 1) & 1][0] = s_frag(ks + 1, 0);
        ring[(ks + 1) & 1][1] = s_frag(ks + 1, 1);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ring[ks & 1][mt]), qf[ks],
                                                           sacc[mt], 0, 0, 0);
    }

    // ---------------------------------------------------------------- online softmax (16 heads)
    // sacc[mt][i] is token 16mt + 4q + i of this half page, head s_head
    const int lim = (cur.L - a.Sq + j) - (cur.tb * kBlock + cur.h * kHalf);   // visible rows r <= lim
    const bool masked = (nvalid <= 0) || (lim < kHalf - 1);
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sv = sacc[mt][i] * a.scale_log2;
        if (masked && (nvalid <= 0 || 16 * mt + 4 * q + i > lim)) sv = -INFINITY;
        sacc[mt][i] = sv;
        tmax = fmaxf(tmax, sv);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool rescale = __ballot(tmax > m_run + 8.0f) != 0;   // p stays <= 2^8 otherwise
    if (rescale) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      if (q == 0) x_alpha[m] = alpha;
    }
    if (lane == 0) *x_flag = rescale ? 1 : 0;
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    u32x4 own;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(sacc[mt][2 * u] - m_use),
                                       __builtin_amdgcn_exp2f(sacc[mt][2 * u + 1] - m_use));
        own[2 * mt + u] = w;
        l_run += bf16_bits_to_f32(w & 0xFFFFu) + bf16_bits_to_f32(w >> 16);
      }
    }
    *reinterpret_cast<u32x4*>(pbuf + wave * 1024 + lane * 16) = own;
    lds_barrier();   // P fragments, rescale flags and factors of all eight waves visible

    // ---------------------------------------------------------------- O^T += V^T . P^T
    // N-tile n holds heads 32hg + 16n + (0..15), whose softmax ran on wave hg + 4n.
    u32x4 pf[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int src = hg + 4 * n;
      pf[n] = *reinterpret_cast<const u32x4*>(pbuf + src * 1024 + lane * 16);
      const int flag = *reinterpret_cast<const int*>(xch + src * kXchWave + 128);
      if (flag) {
        const float al = reinterpret_cast<const float*>(xch + src * kXchWave)[m];
#pragma unroll
        for (int t = 0; t < 16; ++t) oacc[n][t] *= al;
      }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint8_t* p0 = tile + v_base + 16 * ((2 * (t & 7) + (vu >> 1)) ^ v_key) + 256 * (t >> 3);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + 16 * 1024));
      const bf16x8 af = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oacc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, pf[0]), oacc[0][t], 0, 0, 0);
      oacc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, pf[1]), oacc[1][t], 0, 0, 0);
    }

    // ---------------------------------------------------------------- end of a range segment?
    const bool last_half = cur.h == 1;
    if (last_half && (cur.tb == cur.nb - 1 || y + 1 == n_steps)) {
      float l_tot = l_run + __shfl_xor(l_run, 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const bool whole = (seg_tb0 == 0) && (cur.tb == cur.nb - 1);
      const size_t row_base = whole ? (size_t)(cur.b * a.Sq + j) * kH : ((size_t)(g + cur.b) * a.Sq + j) * kH;
      if (q == 0) {
        const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        (whole ? a.lse : a.part_lse)[row_base + s_head] = lse_v;
        x_invl[m] = l_tot > 0.f ? 1.0f / l_tot : 0.0f;
      }
      lds_barrier();   // 1/l of every head visible
      float* obase = (whole ? a.o_lat : a.part_o) + row_base * kDC;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int src = hg + 4 * n;
        const float inv = reinterpret_cast<const float*>(xch + src * kXchWave + 64)[m];
        float* dst = obase + (size_t)(32 * hg + 16 * n + m) * kDC + 256 * sh + 4 * q;
        // oacc[n][t][i] is column 256sh + 16t + 4q + i of head 32hg + 16n + m
#pragma unroll
        for (int t = 0; t < 16; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t) = oacc[n][t] * inv;
      }
      if (y + 1 < n_steps) {
        Cursor nx = cur;
        cursor_next(nx, a.kv_lens, a.B, a.max_blocks);
        load_q(nx.b);
        // wait here (rare path) so the steady-state loop carries no pending query loads;
        // otherwise every step would wait for the whole page pipeline before its first MFMA
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int t = 0; t < 16; ++t) oacc[n][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        seg_tb0 = 0;
      }
    }
    cursor_next(cur, a.kv_lens, a.B, a.max_blocks);
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

// Token ranges of the split: one workgroup per (range, query) and one workgroup per compute
// unit (each holds 154 KiB of LDS), so G = CUs / Sq, capped by the number of pages.
int decode_num_ranges(int num_cus, int B, int Sq, int max_blocks) {
  long long cap = (long long)B * max_blocks;
  int G = num_cus / (Sq > 0 ? Sq : 1);
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
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kDecodeLds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    if (phases & 1) {
      hipLaunchKernelGGL(decode_mfma_bf16_kernel, dim3(G * Sq), dim3(512), kDecodeLds, stream, a);
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
