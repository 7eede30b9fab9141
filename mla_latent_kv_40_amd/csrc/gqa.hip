// Decode over a standard per-head key/value cache (multi-head or grouped-query attention), the
// layout MLA replaces: every cached token holds a key and a value for each of H_kv heads, and
// the H_q query heads share them in groups of H_q / H_kv (H_kv = H_q is multi-head attention).
// It exists to measure, on the same GPU and workloads, what the latent cache saves: zenaique
// ("What MLA caches versus what MHA and GQA cache": 128 heads of width 128 cache over thirty
// thousand numbers per token and layer, against one latent) and the podcast's grouped-query
// sizing (8 key/value heads of width 128).
//
//   cache      k [num_blocks, H_kv, 64, d], v [num_blocks, H_kv, d, 64] bf16 (one head's 64-token
//              page contiguous; the value page stored transposed, column-major, so that the value
//              product reads its operand with plain loads)
//   query      q [B, H_q, d] bf16 (one query per sequence, already rotated)
//   score      s[t] = softmax_scale * q . k[t];   o = sum_t softmax(s)[t] v[t],  lse
//
// Work split (flash decoding): a wave owns (sequence, key/value head, chunk of kChunkPages pages)
// and all G = H_q / H_kv queries of that head on the matrix cores; its partial (O unnormalised,
// running max m and sum l per query) goes to the workspace and a combine kernel merges the chunks
// of a sequence.  This is bandwidth-bound: a page of one head is 32 KiB of keys and values and
// serves G queries; several waves per SIMD keep several pages in flight.
#include "common.h"

namespace mla {

constexpr int kGqaD = 128;          // head width (queries, keys and values)
constexpr int kChunkPages = 16;     // pages per work item

struct GqaArgs {
  const uint16_t* q;           // [B, H_q, d]
  const uint16_t* k;           // [num_blocks, H_kv, 64, d]
  const uint16_t* v;
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* kv_lens;      // [B]
  const int32_t* item_start;   // [B + 1] first work item of each sequence (prefix over chunks x H_kv)
  float* o;                    // [B, H_q, d]
  float* lse;                  // [B, H_q]
  float* part_o;               // [items, G, d]
  float* part_ml;              // [items, G, 2]
  int num_blocks, max_blocks, B, H_q, H_kv, n_items;
  int QS;                      // query slices per key/value head: a work item takes G = (H_q/H_kv)/QS queries
  float scale_log2;
};

__device__ __forceinline__ int gqa_chunks(const int32_t* kv_lens, int b, int max_blocks) {
  int L = kv_lens[b];
  L = L < 0 ? 0 : (L > 64 * max_blocks ? 64 * max_blocks : L);
  const int pages = (L + 63) / 64;
  return (pages + kChunkPages - 1) / kChunkPages;
}

// item_start[b] = H_kv * QS * (chunks of sequences 0 .. b-1), item_start[B] = the total: one wave,
// an exclusive prefix sum over 64 sequences at a time.
__global__ void gqa_plan_kernel(GqaArgs a, int32_t* item_start) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  int run = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int b = base + lane;
    const int n = b < a.B ? a.H_kv * a.QS * gqa_chunks(a.kv_lens, b, a.max_blocks) : 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (b < a.B) item_start[b] = run + incl - n;
    run += __shfl(incl, 63, 64);
  }
  if (lane == 0) item_start[a.B] = run;
}

// One wave per work item: (sequence, key/value head, chunk of kChunkPages pages) and the group's
// G <= 16 queries, on v_mfma_f32_16x16x32_bf16 (A 16x32: lane l holds row l%16 and K values
// 8(l/16) .. +7; B 32x16: column l%16, the same K values; D 16x16: column l%16, rows 4(l/16) .. +3;
// the order of K inside one instruction is free as long as A and B agree).  Columns past G are
// padding (zero queries) and are not stored.  Per page (h = l/16):
//   scores  S^T[t, q] = K[t, :] . Q^T[:, q] for four groups of 16 tokens x four K-steps of 32: A =
//           the key rows (16 bytes straight from the page), B = the queries (registers); lane l
//           holds query l%16 for tokens 16 tg + 4h + i;
//   softmax per query over the page: the lane's 16 scores, then lanes l^16, l^32 (running max and
//           sum, O rescaled when the max grows);
//   values  O^T[c, q] += V^T[c, t] . P^T[t, q] for 8 tiles of 16 columns x two K-steps of 32
//           tokens: the K-step j takes the tokens the lane's own probabilities belong to,
//           32 j + 4h + i and 32 j + 16 + 4h + i, so P is the B operand as it stands (bf16), and A
//           is read from the value page stored transposed ([c][t]: two 8-byte pieces per lane).
template <int G>
__global__ void __launch_bounds__(256) gqa_split_kernel(GqaArgs a) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.n_items || item >= a.item_start[a.B]) return;   // past this batch's items
  int lo = 0, hi = a.B - 1;                                      // sequence of the item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.item_start[mid] <= item) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int rel = item - a.item_start[b];
  const int hk = rel % a.H_kv, chunk = rel / a.H_kv;
  int L = a.kv_lens[b];
  L = L < 0 ? 0 : (L > 64 * a.max_blocks ? 64 * a.max_blocks : L);
  const int p0 = chunk * kChunkPages;
  const int pages = (L + 63) / 64;
  const int p1 = p0 + kChunkPages < pages ? p0 + kChunkPages : pages;
  const int col = lane & 15, h = lane >> 4;
  // B operand of the scores: query `col` of the group (zero past G), dims 32k + 8h .. +7
  bf16x8 qf[4];
  {
    const int qi = col < G ? col : 0;
    const uint16_t* qp = a.q + ((size_t)b * a.H_q + hk * G + qi) * kGqaD + 8 * h;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qf[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * k));
      if (col >= G) qf[k] = bf16x8{};
    }
  }
  float m = -INFINITY, l = 0.f;   // running max (exp2 domain) and sum of query `col`
  f32x4v o[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4v{0.f, 0.f, 0.f, 0.f};
  for (int p = p0; p < p1; ++p) {
    const int pg = a.block_table[(size_t)b * a.max_blocks + p];
    const bool ok = pg >= 0 && pg < a.num_blocks;
    const size_t off = ((size_t)(ok ? pg : 0) * a.H_kv + hk) * 64 * kGqaD;
    // key rows 16 tg + col, dims 32k + 8h: all 16 pieces first, then the value pieces
    u32x4 kf[4][4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        kf[tg][k] = *reinterpret_cast<const u32x4*>(a.k + off + (size_t)(16 * tg + col) * kGqaD + 32 * k + 8 * h);
    // value page transposed: row c = 16 ct + col, tokens 32 j + 4h .. +3 and 32 j + 16 + 4h .. +3
    u32x2 vf[8][2][2];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          vf[ct][j][u] = *reinterpret_cast<const u32x2*>(a.v + off + (size_t)(16 * ct + col) * 64 + 32 * j + 16 * u +
                                                         4 * h);
    f32x4v sc[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      sc[tg] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        sc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[tg][k]), qf[k], sc[tg], 0, 0, 0);
    }
    // softmax of query `col` over this page's tokens 16 tg + 4h + i (masked past the length)
    const int nv = ok ? L - 64 * p : 0;
    float mx = -INFINITY;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tg + 4 * h + i;
        sc[tg][i] = t < nv ? sc[tg][i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[tg][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_use);
    float ps = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 pv = (__bf16)__builtin_amdgcn_exp2f(sc[2 * j + u][i] - m_use);
          pf[j][4 * u + i] = pv;
          ps += (float)pv;   // the sum of the rounded values that enter the product
        }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      o[ct] *= alpha;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{vf[ct][j][0][0], vf[ct][j][0][1], vf[ct][j][1][0],
                                                          vf[ct][j][1][1]});
        o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[j], o[ct], 0, 0, 0);
      }
    }
  }
  // partial of this item (an empty chunk leaves m = -inf, l = 0): O^T rows 16 ct + 4h + i of column col
  if (col < G) {
    float* po = a.part_o + ((size_t)item * G + col) * kGqaD;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<f32x4v*>(po + 16 * ct + 4 * h) = o[ct];
    if (h == 0) *reinterpret_cast<float2*>(a.part_ml + ((size_t)item * G + col) * 2) = float2{m, l};
  }
}

// One wave per (sequence, query head): merge the chunks of its slice.
template <int G>
__global__ void __launch_bounds__(256) gqa_combine_kernel(GqaArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // b * H_q + h
  if (row >= a.B * a.H_q) return;
  const int b = row / a.H_q, h = row % a.H_q;
  const int grp = G * a.QS;                               // queries per key/value head
  const int hq = (h / grp) * a.QS + (h % grp) / G, g = h % G;
  const int chunks = gqa_chunks(a.kv_lens, b, a.max_blocks);
  const int base = a.item_start[b], per = a.H_kv * a.QS;
  float M = -INFINITY;
  for (int c = 0; c < chunks; ++c) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + ((size_t)(base + c * per + hq) * G + g) * 2);
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  float Ls = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < chunks; ++c) {
      const size_t it = (size_t)(base + c * per + hq) * G + g;
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + it * 2);
      if (!(ml.y > 0.f)) continue;
      const float w = __builtin_amdgcn_exp2f(ml.x - M);
      Ls += w * ml.y;
      const float2 po = *reinterpret_cast<const float2*>(a.part_o + it * kGqaD + 2 * lane);
      o0 += w * po.x;
      o1 += w * po.y;
    }
  }
  const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
  *reinterpret_cast<float2*>(a.o + (size_t)row * kGqaD + 2 * lane) = float2{o0 * inv, o1 * inv};
  if (lane == 0) a.lse[row] = Ls > 0.f ? (M + __log2f(Ls)) * 0.69314718055994531f : -INFINITY;
}

// queries per work item and slices per key/value head
static void gqa_slices(int H_q, int H_kv, int* G, int* QS) {
  *G = H_q / H_kv;   // one work item takes the whole group (at most 16 queries: one MFMA tile)
  *QS = 1;
}

// Most work items one launch may take (four per workgroup); larger batches are refused.
constexpr size_t kMaxItems = (size_t)1 << 25;

// Workspace: item starts, then partials for the most items the batch can have (0: refused).
size_t gqa_workspace_bytes(int B, int H_q, int H_kv, int max_blocks) {
  int G, QS;
  gqa_slices(H_q, H_kv, &G, &QS);
  const size_t items = (size_t)B * H_kv * QS * ((max_blocks + kChunkPages - 1) / kChunkPages);
  if (items > kMaxItems) return 0;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)(B + 1) * 4) + al(items * G * kGqaD * 4) + al(items * G * 2 * 4);
}

bool gqa_supported(int H_q, int H_kv, int d) {
  if (d != kGqaD || H_kv <= 0 || H_q % H_kv != 0) return false;
  const int grp = H_q / H_kv;
  return grp == 1 || grp == 2 || grp == 4 || grp == 8 || grp == 16;
}

hipError_t launch_gqa_decode(int H_q, int H_kv, float softmax_scale, const void* q, const void* k, const void* v,
                             int num_blocks, const int32_t* block_table, int max_blocks, const int32_t* kv_lens,
                             int B, void* workspace, float* o, float* lse, hipStream_t stream) {
  int G, QS;
  gqa_slices(H_q, H_kv, &G, &QS);
  const size_t items_max = (size_t)B * H_kv * QS * ((max_blocks + kChunkPages - 1) / kChunkPages);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  uint8_t* w = static_cast<uint8_t*>(workspace);
  GqaArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  int32_t* item_start = reinterpret_cast<int32_t*>(w);
  a.item_start = item_start;
  a.part_o = reinterpret_cast<float*>(w + al((size_t)(B + 1) * 4));
  a.part_ml = reinterpret_cast<float*>(w + al((size_t)(B + 1) * 4) + al(items_max * G * kGqaD * 4));
  a.o = o;
  a.lse = lse;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.B = B;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.QS = QS;
  a.n_items = (int)items_max;   // the batch's own count (item_start[B]) is read on the device
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(gqa_plan_kernel, dim3(1), dim3(64), 0, stream, a, item_start);
  const dim3 grid((unsigned)((items_max + 3) / 4)), block(256);
  const dim3 cgrid((unsigned)(((size_t)B * H_q + 3) / 4));
#define MLA_GQA_CASE(GG)                                                             \
  case GG:                                                                           \
    hipLaunchKernelGGL(gqa_split_kernel<GG>, grid, block, 0, stream, a);             \
    hipLaunchKernelGGL(gqa_combine_kernel<GG>, cgrid, block, 0, stream, a);          \
    break;
  switch (G) {
    MLA_GQA_CASE(1)
    MLA_GQA_CASE(2)
    MLA_GQA_CASE(4)
    MLA_GQA_CASE(8)
    MLA_GQA_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MLA_GQA_CASE
  return hipGetLastError();
}

}  // namespace mla
