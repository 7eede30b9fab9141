// Decode over a standard per-head key/value cache (multi-head or grouped-query attention), the
// layout MLA replaces: every cached token holds a key and a value for each of H_kv heads, and
// the H_q query heads share them in groups of H_q / H_kv (H_kv = H_q is multi-head attention).
// It exists to measure, on the same GPU and workloads, what the latent cache saves: zenaique
// ("What MLA caches versus what MHA and GQA cache": 128 heads of width 128 cache over thirty
// thousand numbers per token and layer, against one latent) and the podcast's grouped-query
// sizing (8 key/value heads of width 128).
//
//   cache      k, v [num_blocks, H_kv, 64, d] bf16 (one 64-token page per head is contiguous)
//   query      q [B, H_q, d] bf16 (one query per sequence, already rotated)
//   score      s[t] = softmax_scale * q . k[t];   o = sum_t softmax(s)[t] v[t],  lse
//
// Work split (flash decoding): a wave owns (sequence, key/value head, chunk of kChunkPages pages)
// and all G = H_q / H_kv queries of that head, with lane = token for the scores and lane =
// column pair for the values; its partial (O unnormalised, running max m and sum l per query)
// goes to the workspace and a combine kernel merges the chunks of a sequence.  This is
// bandwidth-bound: a page of one head is 32 KiB of keys and values and serves G queries; two or
// more waves per SIMD keep several pages in flight.
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

// item_start[b] = H_kv * QS * (chunks of sequences 0 .. b-1): one thread, a serial scan (B is small
// next to the split kernel's work).
__global__ void gqa_plan_kernel(GqaArgs a, int32_t* item_start) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int acc = 0;
  for (int b = 0; b < a.B; ++b) {
    item_start[b] = acc;
    acc += a.H_kv * a.QS * gqa_chunks(a.kv_lens, b, a.max_blocks);
  }
  item_start[a.B] = acc;
}

// G queries per work item (a slice of one key/value head's group); G * 2 value accumulators per
// lane (columns 2 lane, 2 lane + 1).  Groups of 16 queries run as two slices of 8 (the second read
// of a page comes from cache), which keeps the registers of a wave at two or more waves per SIMD.
template <int G>
__global__ void __launch_bounds__(256) gqa_split_kernel(GqaArgs a) {
  __shared__ float qs[4][G][kGqaD];   // this wave's queries, fp32 (read as broadcasts)
  __shared__ float ps[4][G][64];      // this page's probabilities
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.n_items || item >= a.item_start[a.B]) return;   // past this batch's items
  // sequence of the item: binary search over item_start
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.item_start[mid] <= item) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int rel = item - a.item_start[b];
  const int hq = rel % (a.H_kv * a.QS), chunk = rel / (a.H_kv * a.QS);
  const int hk = hq / a.QS, q0 = (hq % a.QS) * G;   // key/value head, first query of the slice
  int L = a.kv_lens[b];
  L = L < 0 ? 0 : (L > 64 * a.max_blocks ? 64 * a.max_blocks : L);
  const int p0 = chunk * kChunkPages;
  const int pages = (L + 63) / 64;
  const int p1 = p0 + kChunkPages < pages ? p0 + kChunkPages : pages;
  // queries of this head group
  for (int e = lane; e < G * kGqaD; e += 64) {
    const int g = e / kGqaD, d = e % kGqaD;
    qs[wave][g][d] = bf16_bits_to_f32(a.q[((size_t)b * a.H_q + hk * G * a.QS + q0 + g) * kGqaD + d]);
  }
  // running max and sum per query are wave-uniform (scalar registers); the value accumulators
  // hold columns 2 lane, 2 lane + 1
  float m[G], l[G], acc0[G], acc1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
    acc0[g] = 0.f;
    acc1[g] = 0.f;
  }
  auto page_id = [&](int p) -> int {
    const int pg = a.block_table[(size_t)b * a.max_blocks + p];
    return (pg >= 0 && pg < a.num_blocks) ? pg : -1;
  };
  for (int p = p0; p < p1; ++p) {
    const int pid = page_id(p);
    const size_t off = ((size_t)(pid < 0 ? 0 : pid) * a.H_kv + hk) * 64 * kGqaD;
    const uint16_t* kp = a.k + off + lane * kGqaD;         // this lane's key row (token = lane)
    const uint16_t* vp = a.v + off + 2 * lane;             // columns 2 lane, 2 lane + 1 of each token
    // the key row and the first 16 tokens' values are requested before anything waits
    u32x4 kc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kc[i] = *reinterpret_cast<const u32x4*>(kp + 8 * i);
    uint32_t vv[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) vv[t] = *reinterpret_cast<const uint32_t*>(vp + t * kGqaD);
    const bool live = pid >= 0 && lane < L - 64 * p;
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      float kv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[2 * e] = bf16_bits_to_f32(kc[i][e] & 0xFFFFu);
        kv[2 * e + 1] = bf16_bits_to_f32(kc[i][e] >> 16);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(&qs[wave][g][8 * i]);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(&qs[wave][g][8 * i + 4]);
        float d = s[g];
        d = __builtin_fmaf(q0[0], kv[0], d);
        d = __builtin_fmaf(q0[1], kv[1], d);
        d = __builtin_fmaf(q0[2], kv[2], d);
        d = __builtin_fmaf(q0[3], kv[3], d);
        d = __builtin_fmaf(q1[0], kv[4], d);
        d = __builtin_fmaf(q1[1], kv[5], d);
        d = __builtin_fmaf(q1[2], kv[6], d);
        d = __builtin_fmaf(q1[3], kv[7], d);
        s[g] = d;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sg = live ? s[g] * a.scale_log2 : -INFINITY;
      const float m_new = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(fmaxf(m[g], wave_max(sg)))));
      const float pg = live ? __builtin_amdgcn_exp2f(sg - m_new) : 0.f;
      const float alpha = m[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[g] - m_new);
      l[g] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(l[g] * alpha + wave_sum(pg))));
      acc0[g] *= alpha;
      acc1[g] *= alpha;
      m[g] = m_new;
      ps[wave][g][lane] = pg;
    }
    // values, 16 tokens at a time (the next group's values in flight)
#pragma unroll 1
    for (int tg = 0; tg < 4; ++tg) {
      uint32_t vn[16];
      if (tg < 3) {
#pragma unroll
        for (int t = 0; t < 16; ++t) vn[t] = *reinterpret_cast<const uint32_t*>(vp + (16 * (tg + 1) + t) * kGqaD);
      }
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(&ps[wave][g][16 * tg + 4 * t4]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t x = vv[4 * t4 + u];
            acc0[g] = __builtin_fmaf(w[u], bf16_bits_to_f32(x & 0xFFFFu), acc0[g]);
            acc1[g] = __builtin_fmaf(w[u], bf16_bits_to_f32(x >> 16), acc1[g]);
          }
        }
      }
      if (tg < 3) {
#pragma unroll
        for (int t = 0; t < 16; ++t) vv[t] = vn[t];
      }
    }
  }
  // partial of this item (an empty chunk leaves m = -inf, l = 0)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    *reinterpret_cast<float2*>(a.part_o + ((size_t)item * G + g) * kGqaD + 2 * lane) = float2{acc0[g], acc1[g]};
    if (lane == 0) *reinterpret_cast<float2*>(a.part_ml + ((size_t)item * G + g) * 2) = float2{m[g], l[g]};
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
  const int grp = H_q / H_kv;
  *G = grp > 8 ? 8 : grp;
  *QS = grp / *G;
}

// Workspace: item starts, then partials for the most items the batch can have.
size_t gqa_workspace_bytes(int B, int H_q, int H_kv, int max_blocks) {
  int G, QS;
  gqa_slices(H_q, H_kv, &G, &QS);
  const size_t items = (size_t)B * H_kv * QS * ((max_blocks + kChunkPages - 1) / kChunkPages);
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
    default:
      return hipErrorInvalidValue;
  }
#undef MLA_GQA_CASE
  return hipGetLastError();
}

}  // namespace mla
