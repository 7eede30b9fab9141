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
//   block     256 threads = 4 waves, one per SIMD; wave w owns heads 32w .. 32w+31, so all
//             128 heads of the query live in the workgroup and every cached row is read from
//             HBM once per query.
//   per step  32 tokens (half a page) staged in LDS by 16-byte buffer->LDS loads, four
//             stages in flight, rows XOR-swizzled at 16-byte granularity:
//               S^T[32 tok, 32 heads] = Stage[32, 576] . Qabs^T   v_mfma_f32_32x32x16_bf16
//               softmax in the exp2 domain against a fixed per-segment reference
//               O^T[512 cols, 32 heads] += Stage[:, :512]^T . P^T (V^T via ds_read_b64_tr_b16),
//               O held in the accumulation registers for the whole segment
//   output    each segment (one sequence's part of a range) writes its unnormalised O and
//             (m, l) per head to workspace slot g + b; the combine normalises.
#include "common.h"

#include <atomic>
#include <cstdlib>
#include <type_traits>

namespace mla {

constexpr int kH = 128, kDC = 512, kDR = 64, kRow = 576;
constexpr int kChunks = kRow * 2 / 16;            // 72 sixteen-byte chunks per bf16 row
constexpr int kTileBytes = kBlock * kRow * 2;     // 73728

struct DecodeArgs {
  const uint16_t* q_abs;      // [T, H, 576] bf16
  const uint8_t* cache;       // [num_blocks, 64, 576] bf16 (e4m3 codes for an fp8 cache)
  const float* cache_scale;   // fp8 only: [num_blocks, 64] per token, or [num_blocks, 2, 18] per
                              // tile of 32 tokens x 32 columns (block8): row value = code * scale
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* kv_lens;     // [B]
  float* o_lat;               // [T, H, 512]
  float* lse;                 // [T, H]
  uint16_t* part_o;           // [slots*Sq] x 128 KiB unnormalised segment outputs, bf16 (register order)
  float* part_ml;             // [slots*Sq, H, 2]   (reference max m in log2 units, l)
  int num_blocks, max_blocks, B, Sq, G;
  float scale_log2;           // softmax_scale * log2(e)
  int fp8;                    // cache and queries are e4m3 codes with scales
  int block8;                 // fp8 cache with tile scales (powers of two) instead of token scales
  int seg_w;                  // per-segment overhead in pages, for cutting the ranges
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

// Ranges are cut in cost units rather than pages.  A sequence with n > 0 pages costs w + n
// units: w units of per-segment overhead (a segment's partial output stores, the query reload
// of the next segment, its ragged last page, a reference maximum), then one per page.  Page x
// of the r-th non-empty sequence (r = 0, 1, ..) sits at cost position c(x) = x + w (r + 1), and
// range g owns the pages with floor(g C / G) <= c(x) < floor((g+1) C / G), C the total cost.
// With w = 0 this is the even split of pages.  A range whose interval holds only overhead
// units or is empty owns no page.

// Owner of cost position c when C units are split over G ranges.
__device__ __forceinline__ int range_of_tile(long long c, long long C, int G) {
  return (int)(((c + 1) * (long long)G - 1) / C);
}

// Page a cost boundary maps to (the first page at or after it), with its sequence.
struct CostHit {
  long long page;      // page index; the total page count when the boundary is at or past the end
  int seq;             // sequence of that page (-1 past the end)
  long long seq_first; // first page of that sequence
};

// Wave-level scan over the batch: total cost and pages, and (for each boundary >= 0) the page
// it maps to.  Every lane gets the results.
__device__ void scan_batch(const int32_t* kv_lens, int B, int max_blocks, int w, long long want0, long long want1,
                           long long* cost_total, long long* page_total, CostHit* h0, CostHit* h1) {
  const int lane = threadIdx.x & 63;
  long long run_c = 0, run_n = 0;
  CostHit hit[2] = {{-1, -1, 0}, {-1, -1, 0}};
  const long long want[2] = {want0, want1};
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    int L;
    const int n = b < B ? seq_tiles(kv_lens, b, max_blocks, &L) : 0;
    const int c = n > 0 ? n + w : 0;
    int incl_n = n, incl_c = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int yn = __shfl_up(incl_n, o, 64), yc = __shfl_up(incl_c, o, 64);
      if (lane >= o) {
        incl_n += yn;
        incl_c += yc;
      }
    }
    const int excl_n = incl_n - n, excl_c = incl_c - c;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool mine = n > 0 && want[k] >= run_c + excl_c && want[k] < run_c + incl_c;
      const unsigned long long mask = __ballot(mine);
      if (mask) {
        const int src = __ffsll((long long)mask) - 1;
        const long long cstart = run_c + __shfl(excl_c, src, 64);
        const long long first = run_n + __shfl(excl_n, src, 64);
        const long long off = want[k] - cstart - w;
        hit[k] = CostHit{first + (off > 0 ? off : 0), __shfl(b, src, 64), first};
      }
    }
    run_n += __shfl(incl_n, 63, 64);
    run_c += __shfl(incl_c, 63, 64);
  }
  // wave-uniform results: hand them back as scalars
  auto uni64 = [](long long v) {
    return ((long long)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
           (unsigned)__builtin_amdgcn_readfirstlane((int)v);
  };
  *cost_total = uni64(run_c);
  *page_total = uni64(run_n);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    CostHit* h = k == 0 ? h0 : h1;
    if (h == nullptr) continue;
    if (hit[k].seq < 0) hit[k].page = run_n;   // at or past the end (or want < 0)
    *h = CostHit{uni64(hit[k].page), __builtin_amdgcn_readfirstlane(hit[k].seq), uni64(hit[k].seq_first)};
  }
}

// Pages [x0, x1) of range g and the sequence b0 (first page s_first) holding x0; false when the
// range owns no page.
__device__ bool range_pages(const DecodeArgs& a, int g, long long* x0, long long* x1, int* b0, long long* s_first) {
  long long C_all, T_all;
  scan_batch(a.kv_lens, a.B, a.max_blocks, a.seg_w, -1, -1, &C_all, &T_all, nullptr, nullptr);
  const long long c0 = (long long)g * C_all / a.G;
  const long long c1 = (long long)(g + 1) * C_all / a.G;
  if (c0 >= c1) return false;
  CostHit h0, h1;
  scan_batch(a.kv_lens, a.B, a.max_blocks, a.seg_w, c0, c1, &C_all, &T_all, &h0, &h1);
  *x0 = h0.page;
  *x1 = h1.seq < 0 ? T_all : h1.page;
  *b0 = h0.seq;
  *s_first = h0.seq_first;
  return *x0 < *x1 && h0.seq >= 0;
}

// ---------------------------------------------------------------------------------------
// LDS layout.  The page stream is cut into 32-token half pages; four stages of 36 KiB hold
// the half page whose values are being accumulated, the one whose scores are being computed
// and the next two in flight (global->LDS DMA).  One stage: 32 latent rows of 1024 B, then
// 32 positional rows of 128 B.  Inside a latent row, 16-byte chunk c is stored at c ^ key(r)
// with key(r) = 4(r&3) + ((r>>2)&3); inside a positional row at c ^ ((r>>1)&7).
//
// On gfx950 the LDS has 64 four-byte banks.  A ds_read_b128 serves, per cycle, the 16 lanes
// that agree on lane bit 5 and on the parity of lane bits 2..4; a ds_read_b64_tr_b16 serves
// a half wave per cycle (both fitted to timings of 170 access patterns).  Under that model
// the key makes both reads below conflict-free:
//   scores  lane l reads row l&31, chunk 2s + (l>>5): within a cycle's 16 lanes the rows
//           differ in a way the key maps to 16 distinct bank groups;
//   values  a half wave reads 4 rows x 4 consecutive chunks: the rows' keys differ in bits
//           2-3, so the four 64-byte blocks land on different banks.
// XOR keys below 16 (8) keep every chunk inside its row.
__device__ __forceinline__ int lat_key(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int pos_key(int r) { return (r >> 1) & 7; }
constexpr int kHalf = 32;                            // tokens per pipeline step
constexpr int kStageLat = kHalf * 1024;              // 32768: offset of the positional rows
constexpr int kStageBytes = kHalf * (1024 + 128);    // 36864
constexpr int kStages = 4;
constexpr int kTabOff = kStages * kStageBytes;       // 147456: the range's page table
constexpr int kTabCap = 1024;                        // entries of 16 bytes: pages per range
constexpr int kDecodeLds = kTabOff + 16 * kTabCap;   // 163840 bytes (all of a CU's LDS)
constexpr int kFirst = 1, kLast = 2;                 // page table flags
constexpr int kWaves = 4;                            // one per SIMD, 32 heads each

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding and
// leaves the other counters alone (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).  Vector loads complete in order.
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// Wave-uniform values are pinned to scalar registers: table and length lookups then become
// scalar loads, which never wait behind the vector-memory counter of the page DMA.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Each of the four waves issues nine 1 KiB global->LDS loads per half page: latent rows
// 8w .. 8w+7 (lane l fetches logical chunk l ^ key) and the positional rows 8w .. 8w+7
// (lane l -> row 8w + l/8).  The loads go through a buffer descriptor that starts at the half
// page's first row and ends after its last valid row: rows past it are out of range and the
// load writes zeros for them (finite data, masked scores), and the per-lane offsets are the
// same for every half page.  Unlike the flat-encoded global->LDS form, buffer loads let the
// compiler keep counting LDS reads precisely while page loads are in flight (a pending flat
// access forces every LDS wait to zero).  Aux is the cache policy: non-temporal when no other
// workgroup reads the page, so that the stream does not evict the queries and partial outputs
// from L2.
struct PageLoad {
  __amdgpu_buffer_rsrc_t rsrc;   // rows 0 .. nvalid-1 of the half page
  uint8_t* stage;
};
__device__ __forceinline__ PageLoad page_load(uint8_t* stage, const uint8_t* cache, int pg, int h, int nvalid) {
  const uint8_t* half = cache + (size_t)(pg < 0 ? 0 : pg) * kTileBytes + (size_t)h * (kHalf * kRow * 2);
  const int nv = nvalid < 0 ? 0 : (nvalid > kHalf ? kHalf : nvalid);
  return PageLoad{__builtin_amdgcn_make_buffer_rsrc((void*)half, 0, nv * kRow * 2, 0x00020000), stage};
}
// Source offset (within the half page) of the 16 bytes lane `lane` of row load i fetches.
__device__ __forceinline__ int half_src(int wave, int i, int lane) {
  if (i < 8) {
    const int r = 8 * wave + i;
    return r * (kRow * 2) + ((lane ^ lat_key(r)) << 4);
  }
  const int r = 8 * wave + (lane >> 3);
  return r * (kRow * 2) + kDC * 2 + (((lane & 7) ^ pos_key(r)) << 4);
}
// Row load i of this wave (i < 8: latent row 8w + i; i == 8: positional rows 8w .. 8w+7).
template <int Aux>
__device__ __forceinline__ void load_row(const PageLoad& p, int i, int wave, int src) {
  if (i < 8)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rsrc, (MLA_LDS void*)(p.stage + (8 * wave + i) * 1024), 16, src, 0,
                                             0, Aux);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rsrc, (MLA_LDS void*)(p.stage + kStageLat + 8 * wave * 128), 16, src,
                                             0, 0, Aux);
}

// LDS reads at absolute LDS byte addresses (the callers fold the array base in once).  The
// restrict qualifier tells the compiler that the stage read is not written behind its back,
// which is true (page loads only ever target another stage, and every read of a stage follows
// the explicit wait and barrier for its loads); without it the compiler waits for all page
// loads in flight before the first transposing read of every step.
__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) {
  const MLA_LDS u32x4* __restrict__ p = (const MLA_LDS u32x4*)(size_t)addr;
  return *p;
}
__device__ __forceinline__ uint32_t lds_u32(uint32_t addr) {
  const MLA_LDS uint32_t* __restrict__ p = (const MLA_LDS uint32_t*)(size_t)addr;
  return *p;
}
__device__ __forceinline__ uint32_t lds_u16(uint32_t addr) {
  const MLA_LDS uint16_t* __restrict__ p = (const MLA_LDS uint16_t*)(size_t)addr;
  return *p;
}
__device__ __forceinline__ bf16x4 lds_tr16(const uint8_t* __restrict__ base, uint32_t off) {
  const MLA_LDS uint8_t* __restrict__ lb = (const MLA_LDS uint8_t*)base;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(lb + off));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const MLA_LDS uint8_t*)p;
}

// Value of lane l and lane l^32 of x, combined: max or sum (v_permlane32_swap).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The output tiles accumulate in the accumulation registers (AGPRs) through inline MFMAs, so
// that the folded queries and the score accumulator keep the 256 architectural VGPRs.  No
// vector ALU instruction ever reads or writes them: they are zeroed by an MFMA (0 . 0 + 0) and
// stored straight from the AGPRs at the end of a segment (the combine normalises).  With all
// 256 AGPRs in use, any vector access would make the compiler move them through VGPRs and
// spill.
// The compiler does not see these MFMAs, so their hazards are resolved here: two wait states
// before each (a vector write of an operand just before), none between chained accumulations
// into the same registers, and a fence tying all tiles before any other access of O (results
// of an 8-pass XDL op need 11 wait states, a WAR on src C 15).
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_zero(f32x16& acc, const bf16x8& z) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}
template <int N>
__device__ __forceinline__ void o_fence(f32x16* o) {
  static_assert(N > 0 && N <= 32, "wait states");
  if constexpr (N > 16)
    asm volatile("s_nop 15\n\ts_nop %16"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]),
                   "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15])
                 : "i"(N - 17));
  else
    asm volatile("s_nop %16"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]),
                   "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15])
                 : "i"(N - 1));
}

// A segment's unnormalised O in bf16 (fp32 range, relative rounding 2^-9; the segments of a
// sequence are summed in fp32 by the combine), in register order: lane l's oacc[ct][8qp .. +7]
// (columns 32ct + 8(2qp) + 4hl + 0..3 and 32ct + 8(2qp + 1) + 4hl + 0..3 of its head) goes to
// 1 KiB block 2ct + qp at 16 bytes per lane, so every store writes 1 KiB contiguously.
__device__ __forceinline__ f32x16 read_acc(const f32x16& x) {   // accumulation registers -> VGPRs
  f32x16 r;
  asm volatile("v_accvgpr_read_b32 %0, %16\n\tv_accvgpr_read_b32 %1, %17\n\tv_accvgpr_read_b32 %2, %18\n\t"
               "v_accvgpr_read_b32 %3, %19\n\tv_accvgpr_read_b32 %4, %20\n\tv_accvgpr_read_b32 %5, %21\n\t"
               "v_accvgpr_read_b32 %6, %22\n\tv_accvgpr_read_b32 %7, %23\n\tv_accvgpr_read_b32 %8, %24\n\t"
               "v_accvgpr_read_b32 %9, %25\n\tv_accvgpr_read_b32 %10, %26\n\tv_accvgpr_read_b32 %11, %27\n\t"
               "v_accvgpr_read_b32 %12, %28\n\tv_accvgpr_read_b32 %13, %29\n\tv_accvgpr_read_b32 %14, %30\n\t"
               "v_accvgpr_read_b32 %15, %31"
               : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]),
                 "=v"(r[8]), "=v"(r[9]), "=v"(r[10]), "=v"(r[11]), "=v"(r[12]), "=v"(r[13]), "=v"(r[14]), "=v"(r[15])
               : "a"(x[0]), "a"(x[1]), "a"(x[2]), "a"(x[3]), "a"(x[4]), "a"(x[5]), "a"(x[6]), "a"(x[7]), "a"(x[8]),
                 "a"(x[9]), "a"(x[10]), "a"(x[11]), "a"(x[12]), "a"(x[13]), "a"(x[14]), "a"(x[15]));
  return r;
}
__device__ __forceinline__ void store_partial(uint16_t* so, const f32x16* oacc) {
#pragma unroll
  for (int ct = 0; ct < 16; ++ct) {
    __builtin_amdgcn_sched_barrier(0);   // one column tile at a time: few registers in flight
    const f32x16 o = read_acc(oacc[ct]);
#pragma unroll
    for (int qp = 0; qp < 2; ++qp)
      *reinterpret_cast<u32x4*>(so + 512 * (2 * ct + qp)) =
          u32x4{cvt_pk_bf16(o[8 * qp], o[8 * qp + 1]), cvt_pk_bf16(o[8 * qp + 2], o[8 * qp + 3]),
                cvt_pk_bf16(o[8 * qp + 4], o[8 * qp + 5]), cvt_pk_bf16(o[8 * qp + 6], o[8 * qp + 7])};
  }
  __builtin_amdgcn_sched_barrier(0);
}

// ---- page table of the range, built once in LDS: entry k describes range page k
//   pg     page id in the cache (out-of-range ids are treated as holding no valid token)
//   r      tokens from the page's first row to the end of its sequence (kv_len - 64 tb)
//   b      sequence
//   flags  kFirst: first page of its segment in this range, kLast: last page of it
// One thread per sequence (256 at a time) finds where its pages start in the range; each
// sequence marks its first page, a prefix maximum over the marks gives every page its
// sequence, and one gather per page fetches the ids.  The step loop then needs no cursor
// walking and no scalar loads.
// `scratch` (LDS not in use yet) holds 3 KiB of per-sequence arrays, then 4 KiB of page marks.
// Every thread of the workgroup calls it; n_pages <= 1024.  The barriers wait only for LDS
// traffic, so page loads already in flight keep going.
__device__ void build_page_table(const DecodeArgs& a, uint8_t* scratch, int4* tab, int n_pages, long long x0,
                                 int b0, long long s_first) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int* s_start = reinterpret_cast<int*>(scratch);       // [256]
  int* s_len = s_start + 256;                           // [256]
  int* s_nb = s_start + 512;                            // [256]
  int* s_wsum = s_start + 768;                          // [4]
  int* s_mark = s_start + 1024;                         // [kTabCap]
  const int t = threadIdx.x;
  long long chunk_b = b0;
  long long rel_base = -(x0 - s_first);                 // start of sequence chunk_b in range pages
  int k_done = 0;
  while (true) {
    const long long bl = chunk_b + t;
    int L = 0;
    const int nb = bl < a.B ? seq_tiles(a.kv_lens, (int)bl, a.max_blocks, &L) : 0;
    // block-wide exclusive scan of nb
    int incl = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    lds_barrier();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int ws = s_wsum[w];
      before += w < wave ? ws : 0;
      total += ws;
    }
    const long long start = rel_base + before + incl - nb;
    s_start[t] = (int)(start < -(1ll << 30) ? -(1 << 30) : start);
    s_len[t] = L;
    s_nb[t] = nb;
    const long long k_end_ll = rel_base + total;       // range pages covered by this chunk
    const int k_end = (int)(k_end_ll < n_pages ? k_end_ll : n_pages);
    for (int k = k_done + t; k < k_end; k += 256) s_mark[k] = -1;
    lds_barrier();
    if (nb > 0 && start >= k_done && start < k_end) s_mark[start] = t;   // sequence t starts at page start
    lds_barrier();
    // pages k_done .. k_end-1: sequence = last mark at or before k (page k_done may continue
    // the sequence of the previous chunk's last page, or of chunk_b itself at the range start)
    {
      // parallel prefix maximum: thread t owns pages k_done + 4t .. +3 (k_end - k_done <= 1024)
      int m4[4];
      int run = -1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k_done + 4 * t + i;
        const int v = k < k_end ? s_mark[k] : -1;
        run = v > run ? v : run;
        m4[i] = run;
      }
      int inc = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        if (lane >= o) inc = v > inc ? v : inc;
      }
      lds_barrier();                                   // everyone has read its marks
      if (lane == 63) s_wsum[wave] = inc;
      lds_barrier();
      int prev = __shfl_up(inc, 1, 64);
      if (lane == 0) prev = -1;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (w < wave) prev = s_wsum[w] > prev ? s_wsum[w] : prev;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k_done + 4 * t + i;
        const int r = m4[i] > prev ? m4[i] : prev;
        if (k < k_end) s_mark[k] = r < 0 ? 0 : r;        // no mark yet: sequence chunk_b
      }
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {                       // k_end - k_done <= 1024
      const int k = k_done + t + 256 * i;
      if (k < k_end) {
        const int st = s_mark[k];
        const int tb = k - s_start[st];
        const int bk = (int)(chunk_b + st);
        const int pg = a.block_table[(size_t)bk * a.max_blocks + tb];
        const int flags = ((k == 0 || tb == 0) ? kFirst : 0) | ((k == n_pages - 1 || tb == s_nb[st] - 1) ? kLast : 0);
        tab[k] = int4{pg, s_len[st] - kBlock * tb, bk, flags};
      }
    }
    k_done = k_end;
    lds_barrier();
    if (k_done >= n_pages || chunk_b + 256 >= a.B) break;
    chunk_b += 256;
    rel_base += total;
  }
}

// Softmax reference.  Probabilities are taken against a fixed per-segment reference m (the
// first visible score maximum) instead of the running maximum: bf16 and fp32 keep their
// relative precision at any magnitude, and scores below m merely underflow, which is exact to
// fp32 precision relative to the final maximum.  A segment whose scores exceed m by more than
// a safe margin (p could overflow) is marked (l = -1) and the combine recomputes its heads
// exactly; O is therefore never rescaled in the page loop.  The bf16 kernel tests the running
// sum of p (kOverflowSum, 2^80: then every p and O stay far below the fp32 range; an infinite
// or NaN sum fails the test too), the fp8 kernel the page maximum (kRescaleLog2).
constexpr float kRescaleLog2 = 64.0f;
constexpr float kOverflowSum = 0x1p80f;

// 32x32x16 bf16 MFMA layout (wave64): A lane l holds row l%32 and the 8 K values of K-group
// l/32; B lane l holds column l%32 and the same K-group; the result lane l holds column l%32,
// rows 8(i/4) + 4(l/32) + i%4, i = 0..15.  The order of K inside one instruction is free as
// long as A and B agree.
//
// Wave w owns heads 32w .. 32w+31; lane l works for head 32w + l%32 throughout:
//   scores  S^T[32 tok, 32 heads] = Stage[32, 576] . Qabs^T, 36 K-steps; step s takes
//           chunks 2s, 2s+1 (lane halves).  Lane l ends up with its head's scores for tokens
//           8(i/4) + 4(l/32) + i%4.
//   values  O^T[512, 32 heads] += V^T . P^T, 16 column tiles x 2 token steps.  The B operand
//           of token step k is the lane's own probabilities i = 8k .. 8k+7, i.e. tokens
//           16k + 8(e/4) + 4(l/32) + e%4; the transposing reads deliver V^T in that order.
// The page loop is software-pipelined by one half page: step y computes the scores of half
// page y+1, with the probabilities of half page y (from the raw scores of the step before)
// worked out between those score MFMAs, then accumulates the values of half page y.
// Every segment (the part of one sequence inside the range) ends with its unnormalised O and
// (m, l) per head in workspace slot g + b.
template <int Aux>
__global__ void __launch_bounds__(256, 1) decode_mfma_bf16_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(256))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;
  const int head = 32 * wave + (lane & 31);

  // logical (range g, query j) of this workgroup; consecutive logical ids sit on one XCD
  // (blocks are dealt to the 8 XCDs round-robin), so the Sq queries of a range share L2.
  const int NG = a.G * a.Sq;
  int lid = blockIdx.x;
  if ((NG & 7) == 0) lid = (blockIdx.x & 7) * (NG >> 3) + (blockIdx.x >> 3);
  const int g = lid / a.Sq;
  const int j = lid - g * a.Sq;

  long long x0, x1, s_first;
  int b0;
  if (!range_pages(a, g, &x0, &x1, &b0, &s_first)) return;

  // the host sizes the ranges to fit the table; the clamp only keeps LDS accesses in bounds
  const int n_pages = (int)(x1 - x0 < kTabCap ? x1 - x0 : kTabCap);
  const int n_steps = 2 * n_pages;               // half pages of this range

  bf16x8 qf[36];
  auto load_q = [&](int bb) {
    const uint16_t* qp = a.q_abs + ((size_t)(bb * a.Sq + j) * kH + head) * kRow + 8 * hl;
#pragma unroll
    for (int s = 0; s < 36; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * s));
  };
  // this lane's part of workspace slot (g + b, j): O row of its head, columns 4hl + 8q4 + 32ct
  // this lane's part of workspace slot (g + b, j), stored in register order: wave block of
  // 64 KiB, then (column tile ct, quad q4) blocks of 1 KiB, then 16 bytes per lane, so that
  // every store instruction writes 1 KiB contiguously
  auto slot_o = [&](int bb) -> uint16_t* {
    return a.part_o + ((size_t)(g + bb) * a.Sq + j) * (kH * kDC) + (size_t)wave * (32 * kDC) + 8 * lane;
  };

  f32x16 oacc[16];
  const bf16x8 zero8 = {};
#pragma unroll
  for (int t = 0; t < 16; ++t) mfma_zero(oacc[t], zero8);
  float m_ref = -INFINITY, l_run = 0.f;
  bool over = false;                              // a score left the reference's safe range
  bool m_set = false;                             // the segment's reference is set (uniform)

  // ---- S^T of the half page in `tile` (36 chained K-steps)
  // this lane's LDS read bases inside a stage (kept live: one add per stage and step)
  const uint32_t lat = (uint32_t)((lane & 31) * 1024) | (uint32_t)(16 * (lat_key(lane & 31) ^ hl));
  const uint32_t pos = (uint32_t)(kStageLat + (lane & 31) * 128) | (uint32_t)(16 * (pos_key(lane & 31) ^ hl));
  // transposing reads: source lane (gg, 4jj + uu) reads row 4hh + jj (+8E +16k), chunk
  // 4ct + 2(gg&1) + uu/2, byte 8(uu&1)
  const uint32_t vb = (uint32_t)((4 * hl + ((lane & 15) >> 2)) * 1024 + 8 * (lane & 1)) |
                      (uint32_t)(16 * ((2 * ((lane >> 4) & 1) + ((lane >> 1) & 1)) ^ (4 * ((lane & 15) >> 2)) ^ hl));
  uint32_t vbx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) vbx[e] = vb ^ (64u * (e & 3) ^ 32u * (e >> 2));
  auto scores = [&](const uint8_t* tile, auto hook) -> f32x16 {
    // the eight swizzle variants of this lane's row address, stage offset included once (the
    // XOR touches bits 5..7 only and stages start at multiples of 256); the rest of each
    // address is the read's immediate offset
    const uint32_t T = lds_addr(tile);   // 256-byte aligned
    uint32_t xs[8], xp[4];
#pragma unroll
    for (int d = 0; d < 8; ++d) xs[d] = (lat + T) ^ (32u * d);
#pragma unroll
    for (int d = 0; d < 4; ++d) xp[d] = (pos + T) ^ (32u * d);
    auto koff = [&](int st) -> uint32_t { return st < 32 ? xs[st & 7] + 256u * (st >> 3) : xp[st - 32]; };
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    // K fragments four steps ahead, each read issued before the MFMA it runs under (the
    // scheduling barriers keep the compiler from hoisting all 36 reads, 144 VGPRs, to the top)
    constexpr int D = 4;
    u32x4 kr[D + 1];
#pragma unroll
    for (int d = 0; d < D; ++d) kr[d] = lds_b128(koff(d));
#pragma unroll
    for (int st = 0; st < 36; ++st) {
      if (st + D < 36) kr[(st + D) % (D + 1)] = lds_b128(koff(st + D));
      __builtin_amdgcn_sched_barrier(0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[st % (D + 1)]), qf[st], acc, 0, 0, 0);
      hook(st);
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };

  // ---- softmax of one half page: raw scores sv -> bf16 probabilities against the segment
  // reference (log2 units).  `fresh` starts a new segment.  The softmax scale rides in the
  // FMA that feeds exp2; l sums the bf16-rounded probabilities (dot2 with ones), the same
  // values that enter P.V.  soft_begin masks the tail and, when the segment's reference is not
  // yet set, takes the maximum (a block); the eight probability pairs (soft_pair) then run
  // between the score MFMAs of the next half page, and soft_end collects them.
  struct Soft {
    float m_new, l_new, m_use;
    bool over_new, m_set_new;
    bf16x2 pk[8];
    bf16x8 p0, p1;
  };
  auto soft_begin = [&](f32x16& sv, int vis, bool fresh, Soft& st) {
    if (vis < kHalf - 1) {   // partial half page (sequence end, causal limit): mask the tail
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * hl + (i & 3) > vis) sv[i] = -INFINITY;
    }
    const float c = a.scale_log2;
    const float m_in = fresh ? -INFINITY : m_ref;
    st.m_set_new = (fresh ? false : m_set) || vis >= 0;   // wave-uniform
    if (fresh || !m_set) {   // the first visible scores of the segment fix the reference
      float mx = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sv[i]), sv[i + 1]);
      mx = fmaxf(mx, sv[15]);
      st.m_new = pair_max(mx) * c;
    } else {
      st.m_new = m_in;
    }
    st.m_use = (st.m_new == -INFINITY) ? 0.0f : st.m_new;
    st.l_new = fresh ? 0.0f : l_run;
    st.over_new = fresh ? false : over;
  };
  auto soft_pair = [&](const f32x16& sv, int u, Soft& st) {
    const float c = a.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    st.pk[u] = bf16x2{(__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * u], c, -st.m_use)),
                      (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * u + 1], c, -st.m_use))};
    st.l_new = __builtin_amdgcn_fdot2_f32_bf16(st.pk[u], ones, st.l_new, false);
  };
  auto soft_end = [&](Soft& st) {
    st.over_new = st.over_new || !(st.l_new < kOverflowSum);   // also catches inf and NaN
    const bf16x2* pk = st.pk;
    st.p0 = bf16x8{pk[0][0], pk[0][1], pk[1][0], pk[1][1], pk[2][0], pk[2][1], pk[3][0], pk[3][1]};
    st.p1 = bf16x8{pk[4][0], pk[4][1], pk[5][0], pk[5][1], pk[6][0], pk[6][1], pk[7][0], pk[7][1]};
  };

  // ---- O^T += V^T . P^T for the half page in `tile`
  auto values = [&](const uint8_t* tile, const bf16x8* pf) {
    o_fence<3>(oacc);   // MFMA writes of O settled
    // eight swizzle variants (column tile mod 4, token half E): the stage offset T is a multiple
    // of 256 and the XOR touches bits 5..7 only, so (vb + T) ^ c = (vb ^ c) + T with vb ^ c
    // loop-invariant
    const uint8_t* xv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = tile + vbx[e];
    auto vfrag = [&](int it) -> bf16x8 {
      const int k = it >> 4, ct = it & 15;
      const bf16x4 lo = lds_tr16(xv[ct & 3], 16384u * k + 256u * (ct >> 2));
      const bf16x4 hi = lds_tr16(xv[4 + (ct & 3)], 16384u * k + 8192u + 256u * (ct >> 2));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    constexpr int D = 3;
    bf16x8 vr[D + 1];
#pragma unroll
    for (int d = 0; d < D; ++d) vr[d] = vfrag(d);
#pragma unroll
    for (int it = 0; it < 32; ++it) {
      if (it + D < 32) vr[(it + D) % (D + 1)] = vfrag(it + D);
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc(oacc[it & 15], vr[it % (D + 1)], pf[it >> 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // (the next accumulation into the same tiles needs no wait; the segment-end stores fence)
  };

  bf16x8 pf[2];
  Soft sm;
  auto soft_commit = [&](const Soft& st) {
    m_ref = st.m_new;
    l_run = st.l_new;
    over = st.over_new;
    m_set = st.m_set_new;
    pf[0] = st.p0;
    pf[1] = st.p1;
  };

  // One page load per stage is issued every step, also past the end of the range (then it
  // reads row 0 of page 0 and holds no valid token), so that every step issues the same nine
  // vector-memory operations and the wait at the top of a step is always "all but the nine
  // youngest".
  auto load_for = [&](int stage, int pg, int nv, int h) {
    return page_load(smem + stage * kStageBytes, a.cache, nv > 0 ? pg : 0, h, nv);
  };
  int src[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) src[i] = half_src(wave, i, lane);
  auto issue = [&](const PageLoad& pl) {
#pragma unroll
    for (int i = 0; i < 9; ++i) load_row<Aux>(pl, i, wave, src[i]);
  };
  // table entry of half page z (wave-uniform); past the range: no valid token
  // (read through an absolute LDS address: through a pointer into the shared array the
  // compiler would wait for the page loads in flight, which may alias it)
  const uint32_t tab_addr = lds_addr(smem + kTabOff);
  auto entry_raw = [&](int z) -> u32x4 {   // z clamped to the table
    return lds_b128(tab_addr + 16u * (uint32_t)((z < n_steps ? z : n_steps - 1) >> 1));
  };
  auto entry_of = [&](const u32x4& e, int z) -> int4 {
    if (z >= n_steps) return int4{-1, 0, 0, 0};
    return int4{uni((int)e[0]), uni((int)e[1]), uni((int)e[2]), uni((int)e[3])};
  };
  auto entry = [&](int z) -> int4 { return entry_of(entry_raw(z), z); };
  auto valid_page = [&](const int4& e) { return e.x >= 0 && e.x < a.num_blocks; };
  // valid tokens of half page z (<= 0 for an empty second half); 0 for an invalid page
  auto nvalid = [&](const int4& e, int z) {
    const int nv = e.y - kHalf * (z & 1);
    return valid_page(e) ? (nv < kHalf ? nv : kHalf) : 0;
  };
  // last visible row of half page z for query j (causal: position kv_len - Sq + j)
  auto last_visible = [&](const int4& e, int z) {
    const int v = e.y - kHalf * (z & 1) - a.Sq + j;
    return valid_page(e) ? (v < kHalf - 1 ? v : kHalf - 1) : -1;
  };

  // prologue: the range's page table (built in stage 3, not yet in use) comes first, so that
  // its own loads wait for nothing else (vector loads complete in order); then the queries and
  // half pages 0..2 are requested, and the scores and probabilities of half page 0 wait only
  // for the queries and that half page.
  build_page_table(a, smem + 3 * kStageBytes, reinterpret_cast<int4*>(smem + kTabOff), n_pages, x0, b0, s_first);
  // e0..e3: table entries of half pages y .. y+3
  int4 e0 = entry(0), e1 = entry(1), e2 = entry(2), e3;
  // the entry of half page y+3 is read during step y-1 and made scalar at its end, so the
  // page-table read never waits
  int4 e3_next = entry(3);
  load_q(b0);
  issue(load_for(0, e0.x, nvalid(e0, 0), 0));
  issue(load_for(1, e1.x, nvalid(e1, 1), 1));
  issue(load_for(2, e2.x, nvalid(e2, 2), 0));
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(18));
  lds_barrier();
  // raw scores of half page 0; its softmax runs under the score MFMAs of half page 1
  f32x16 s_cur = scores(smem, [](int) {});
  bool fresh_cur = true;   // half page y starts a segment

  // one step; P = y & 1 (a compile-time constant: the loop below runs two steps per page)
  auto step = [&](int y, auto par) {
    constexpr int P = decltype(par)::value;
    const bool has_next = y + 1 < n_steps;
    // this wave's loads of half page y+1 landed (only the nine loads of half page y+2 may
    // stay in flight), then everyone's
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
    lds_barrier();   // stage (y+3)%4 == (y-1)%4 is no longer read by anyone
    e3 = e3_next;
    const u32x4 e4_raw = entry_raw(y + 4);
    // the nine page loads of half page y+3 go out one after every fourth score MFMA, so that
    // their issue (which may wait for queue space) overlaps matrix work
    const PageLoad pl = load_for((y + 3) & 3, e3.x, nvalid(e3, y + 3), 1 - P);
    const bool seg_end = (P == 1 && (e0.w & kLast)) || !has_next;
    if (seg_end && has_next) {
      // the next half page starts another sequence: its queries replace this one's before its
      // scores (waiting here keeps the steady-state loop free of pending query loads)
      load_q(e1.z);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    // scores of half page y+1, with the probabilities of half page y computed between its
    // matrix instructions (one pair of tokens after every fourth, between the page loads)
    soft_begin(s_cur, last_visible(e0, y), fresh_cur, sm);
    f32x16 sv = scores(smem + ((y + 1) & 3) * kStageBytes, [&](int st) {   // stale data if !has_next
      if ((st & 3) == 0) load_row<Aux>(pl, st >> 2, wave, src[st >> 2]);
      if ((st & 3) == 2) soft_pair(s_cur, st >> 2, sm);
    });
    soft_end(sm);
    soft_commit(sm);
    // values of half page y
    values(smem + (y & 3) * kStageBytes, pf);
    if (seg_end) {
      // unnormalised O and (m, l) of this segment into its slot; the combine normalises
      const float l_tot = pair_sum(l_run);
      const bool over_seg = pair_sum(over ? 1.0f : 0.0f) > 0.0f;   // either half of the head
      const size_t row = ((size_t)(g + e0.z) * a.Sq + j) * kH + head;
      if (hl == 0) reinterpret_cast<float2*>(a.part_ml)[row] = float2{m_ref, over_seg ? -1.0f : l_tot};
      uint16_t* so = slot_o(e0.z);
      o_fence<20>(oacc);   // results of the last accumulation settled before the stores
      store_partial(so, oacc);
      if (has_next) {
#pragma unroll
        for (int t = 0; t < 16; ++t) mfma_zero(oacc[t], zero8);
      }
    }
    s_cur = sv;
    fresh_cur = seg_end;
    // all four words stay live until here (a word the compiler finds unused would otherwise
    // have its register recycled while the read is still in flight, which forces a wait)
    asm volatile("" ::"v"(e4_raw));
    e3_next = entry_of(e4_raw, y + 4);
    e0 = e1;
    e1 = e2;
    e2 = e3;
  };
  for (int y = 0; y < n_steps; y += 2) {   // n_steps is even: two half pages per page
    step(y, std::integral_constant<int, 0>{});
    step(y + 1, std::integral_constant<int, 1>{});
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no page load may land after the workgroup ends
}

// ------------------------------------------------------------------------ fp8 cache

// An fp8 cache holds OCP e4m3 codes with one fp32 scale per token (value = code * scale), so
// a page of codes is 36,864 B, the size of a bf16 half page.  The kernel below keeps the bf16
// kernel's structure (ranges, LDS page table, four stages, one barrier per step, O in the
// accumulation registers) with one whole page per step and the scaled fp8 matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4:
//   scores  S^T[64 tok, 32 heads] = Codes[64, 576] . (Qhi + Qlo/16)^T, 2 token blocks x 9
//           K-steps of 64 x 2 query terms: the bf16 folded query is split into two e4m3 terms
//           per segment, so the query keeps about 8 bits; the token scale, the query scale and
//           the softmax scale multiply the fp32 result;
//   values  O^T[512, 32 heads] += Codes[:, :512]^T . Pt^T, one 64-token K-step per column
//           tile.  Pt = p * token scale * 2^-e is rounded to e4m3 and the instruction's E8M0
//           block scale of the B operand multiplies 2^e back in; e (per head and page) keeps
//           every Pt of the page at or below 256.
// Scaled 32x32x64 fp8 operands (measured on gfx950): lane l of A (of B) holds row (column)
// l%32; its bytes 0..15 belong to K-block 0 and bytes 16..31 to K-block 1, and byte j of lane
// l meets byte j of the other operand's lane with the same l/32.  The block scale of row
// (column) r and K-block k is byte 0 of lane r + 32k's scale register.  Results use the 32x32
// layout of the bf16 instruction.
constexpr int kPage8 = kBlock * kRow;                // 36864: one page of codes
constexpr int kStage8 = kPage8 + kWaves * 256;       // + one copy of the page's 64 scales per wave
constexpr int kTabOff8 = kStages * kStage8;          // 151552
constexpr int kTabCap8 = 512;
constexpr int kSrcTab8 = kTabOff8 + 16 * kTabCap8;   // 159744: per-lane source offsets of the row loads
constexpr int kDecodeLds8 = kSrcTab8 + 2 * 9 * 64 * 2;   // 162048
constexpr int kE8M0One = 127;                        // E8M0 code of 1.0
constexpr int kTileCols = kRow / 32;                 // 18 column blocks of a row (tile scales)

// LDS layout of a page of codes: row r (576 B = 36 chunks of 16 B) at 576r, chunk c stored at
// c ^ key8(r), which flips only the two low chunk bits (every chunk stays in its 64-byte group).
//   scores  ds_read_b128 of chunks 4s + h and 4s + 2 + h (h = l/32) of row l%32 (+32): in one
//           cycle's 16 lanes the two low row bits pick the bank quarter (the pitch is 36
//           chunks) and key8 of the three next row bits the 16-byte slot in it;
//   values  ds_read_b64_tr_b8: a half wave reads 8 rows x 4 eight-byte columns; key8 moves the
//           rows that the pitch would put on the same banks to different 16-byte slots.
__device__ __forceinline__ int key8(int r) { return 2 * (((r >> 3) ^ (r >> 4)) & 1) + (((r >> 2) ^ (r >> 4)) & 1); }

// Transposing 8-bit LDS read (gfx950): output lane l, byte j = byte l%8 of the 8 bytes at the
// address of source lane 16(l/16) + 2j + (l/8)%2 (measured).
__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* __restrict__ base, uint32_t off) {
  const MLA_LDS uint8_t* __restrict__ lb = (const MLA_LDS uint8_t*)base;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(lb + off));
}

// e4m3 codes of 16a and 16b packed into half Hi of `old`, the codes v_cvt_pk_fp8_f32 gives for 16a
// and 16b: v_cvt_scalef32_pk_fp8_f32 with scale 2^-4 (it divides by the power of two of its
// scale) saves the two multiplications.  The two matched bit for bit on 2^20 pairs of arbitrary
// and of residual-range inputs on gfx950.
template <bool Hi>
__device__ __forceinline__ int cvt_pk_fp8_x16(float a, float b, int old) {
  typedef short v2i16 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(
      int, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2i16, old), a, b, 0.0625f, Hi));
}

// O tile += A . B on fp8 operands in the accumulation registers (hazards as for mfma_acc; the
// 16-pass instruction needs 19 wait states before its results are read, see o_fence<20>).
__device__ __forceinline__ void mfma8_acc(f32x16& acc, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// Page loads of the fp8 kernel: each wave moves 9 KiB of codes (LDS bytes 9216w .. +9215 of the
// stage, lane l of load i writing bytes 1024(9w + i) + 16l) and the page's 64 scales into its
// own 256-byte copy.  Both descriptors end at the page's last valid token: rows past it are
// out of range and the load writes zeros for them (codes and scales 0: finite, and masked).
struct PageLoad8 {
  __amdgpu_buffer_rsrc_t rows, scales;
  uint8_t* stage;
};
// With tile scales (Block) the page's 36 scales (token half h, column block c at 18h + c) take
// the first 144 bytes of the copy, and the second half's 18 are in range only when the page has
// a valid row in that half (else they read as zeros: scale byte 0, codes 0).
template <bool Block>
__device__ __forceinline__ PageLoad8 page_load8(uint8_t* stage, const uint8_t* cache, const float* cache_scale,
                                                int pg, int nvalid) {
  const size_t p = (size_t)(pg < 0 ? 0 : pg);
  const int nv = nvalid < 0 ? 0 : nvalid;
  const float* sc = Block ? cache_scale + p * (2 * kTileCols) : cache_scale + p * kBlock;
  const int sbytes = Block ? 4 * kTileCols * (nv > 32 ? 2 : (nv > 0 ? 1 : 0)) : nv * 4;
  return PageLoad8{__builtin_amdgcn_make_buffer_rsrc((void*)(cache + p * kPage8), 0, nv * kRow, 0x00020000),
                   __builtin_amdgcn_make_buffer_rsrc((void*)sc, 0, sbytes, 0x00020000), stage};
}
// source offset in the page of the 16 bytes that lane `lane` of load i (of wave `wave`) writes
__device__ __forceinline__ int page8_src(int wave, int i, int lane) {
  const int ch = 64 * (9 * wave + i) + lane;     // LDS chunk of the stage, 0 .. 2303
  const int r = ch / 36, pos = ch - 36 * r;
  return r * kRow + 16 * (pos ^ key8(r));
}
// Wave w's nine row loads cover rows 16w .. 16w+15 (9 x 64 chunks = 16 rows of 36), so their
// source offsets are 16w rows (the scalar offset) plus a per-lane part that depends on w only
// through the parity of w (row bit 4 enters key8).  That part, below 9216, is computed once per
// workgroup into an LDS table [w%2][i][lane] of 16-bit entries; a load then reads its entry
// (one LDS read) instead of recomputing the division and the key.
__device__ __forceinline__ int page8_src_lane(int par, int i, int lane) {
  return page8_src(par, i, lane) - 16 * par * kRow;
}
template <int Aux>
__device__ __forceinline__ void load_row8(const PageLoad8& p, int i, int wave, int lane, int off) {
  if (i < 9) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rows, (MLA_LDS void*)(p.stage + 1024 * (9 * wave + i)), 16, off,
                                             16 * kRow * wave, 0, Aux);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p.scales, (MLA_LDS void*)(p.stage + kPage8 + 256 * wave), 4, 4 * lane,
                                             0, 0, Aux);
  }
}

// Wave w owns heads 32w .. 32w+31 and lane l works for head 32w + l%32, as in the bf16 kernel.
//   scores  token block tb (rows 32tb ..), K-step s: A = chunks 4s + l/32 and 4s + 2 + l/32 of
//           row 32tb + l%32, B = the same 32 columns of the head's query terms.  Lane l ends
//           up with its head's scores for tokens 32tb + 8(i/4) + 4(l/32) + i%4, i = 0..15.
//   values  B byte j of lane l = Pt of that lane's own score i = j%16 of block tb = j/16, i.e.
//           token T(l/32, j) = 32(j/16) + 8((j%16)/4) + 4(l/32) + j%4.  The A operand of
//           column tile ct must hold Codes[T(l/32, j), 32ct + l%32] in byte j: four
//           transposing reads (bytes 8q .. 8q+7) whose source lane σ points at token
//           16q + 8((σ>>3)&1) + 4(σ>>5) + ((σ>>1)&3), columns 32ct + 8(2((σ>>4)&1) + (σ&1)).
template <int Aux, bool Block>
__global__ void __launch_bounds__(256, 1) decode_mfma_fp8_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(256))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;
  const int head = 32 * wave + (lane & 31);

  const int NG = a.G * a.Sq;
  int lid = blockIdx.x;
  if ((NG & 7) == 0) lid = (blockIdx.x & 7) * (NG >> 3) + (blockIdx.x >> 3);
  const int g = lid / a.Sq;
  const int j = lid - g * a.Sq;

  long long x0, x1, s_first;
  int b0;
  if (!range_pages(a, g, &x0, &x1, &b0, &s_first)) return;
  const int n_steps = (int)(x1 - x0 < kTabCap8 ? x1 - x0 : kTabCap8);   // pages of this range
  {
    uint16_t* st = reinterpret_cast<uint16_t*>(smem + kSrcTab8);
    for (int e = threadIdx.x; e < 2 * 9 * 64; e += 256) st[e] = (uint16_t)page8_src_lane(e / 576, (e / 64) % 9, e % 64);
  }
  // (the table build's barriers also publish the source-offset table)
  build_page_table(a, smem, reinterpret_cast<int4*>(smem + kTabOff8), n_steps, x0, b0, s_first);   // stage 0 scratch

  // The folded query (bf16) becomes two e4m3 operands per K-step: with s = amax/448 over the
  // head's 576 values and x = q/s, hi = e4m3(x) and lo = e4m3(16 (x - hi)), so that
  // q = s (hi + lo/16) to about 2^-8 relative.  The lo products enter the same accumulator
  // with the B block scale 2^-4.  Lane l holds, for K-step k, the values 64k + 16(l/32) + 0..15
  // (bytes 0..15) and 64k + 32 + 16(l/32) + 0..15 (bytes 16..31) of its head.
  i32x8 qhi[9], qlo[9];
  float kq = 0.f;   // s * softmax scale * log2(e) of this lane's head
  auto load_q = [&](int bb) {
    const size_t row = (size_t)(bb * a.Sq + j) * kH + head;
    const uint16_t* qp = a.q_abs + row * kRow + 16 * hl;
    auto qword = [&](int k, int v) {   // values 64k + 32(v/2) + 16hl + 8(v%2) .. +7
      return *reinterpret_cast<const u32x4*>(qp + 64 * k + 32 * (v >> 1) + 8 * (v & 1));
    };
    // two passes over the (cached) query: its maximum first, then the split, one K-step at a
    // time so that only one step's raw values are live next to the finished terms
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 9; ++k)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4 r = qword(k, v);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(r[e] & 0xFFFFu)), fabsf(bf16_bits_to_f32(r[e] >> 16))));
      }
    amax = pair_max(amax);
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    kq = (amax > 0.f ? amax / 448.0f : 1.0f) * a.scale_log2;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 raw[4] = {qword(k, 0), qword(k, 1), qword(k, 2), qword(k, 3)};
      int hw[8], lw[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {   // dword d: values 4d .. 4d+3 of the 32
        const u32x4& r = raw[d >> 1];
        const uint32_t w0 = r[2 * (d & 1)], w1 = r[2 * (d & 1) + 1];
        const float x0 = bf16_bits_to_f32(w0 & 0xFFFFu) * inv, x1 = bf16_bits_to_f32(w0 >> 16) * inv;
        const float x2 = bf16_bits_to_f32(w1 & 0xFFFFu) * inv, x3 = bf16_bits_to_f32(w1 >> 16) * inv;
        int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
        const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false), h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
        int l = cvt_pk_fp8_x16<false>(x0 - h01[0], x1 - h01[1], 0);
        l = cvt_pk_fp8_x16<true>(x2 - h23[0], x3 - h23[1], l);
        hw[d] = h;
        lw[d] = l;
      }
      qhi[k] = i32x8{hw[0], hw[1], hw[2], hw[3], hw[4], hw[5], hw[6], hw[7]};
      qlo[k] = i32x8{lw[0], lw[1], lw[2], lw[3], lw[4], lw[5], lw[6], lw[7]};
    }
  };
  auto slot_o = [&](int bb) -> uint16_t* {
    return a.part_o + ((size_t)(g + bb) * a.Sq + j) * (kH * kDC) + (size_t)wave * (32 * kDC) + 8 * lane;
  };

  f32x16 oacc[16];
  const bf16x8 zero8 = {};
#pragma unroll
  for (int t = 0; t < 16; ++t) mfma_zero(oacc[t], zero8);
  float m_ref = -INFINITY, l_run = 0.f;
  bool over = false;
  const int one = kE8M0One;

  // ---- raw S^T of the page in `tile`: per K-step, the hi and the lo query terms of both token
  // blocks (36 MFMAs; the accumulators alternate)
  const int lo_scale = kE8M0One - 4;   // 2^-4
  auto scores = [&](const uint8_t* tile, auto hook, f32x16& s0, f32x16& s1) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int rr = ln & 31, hh = ln >> 5, key = key8(rr);
    const uint32_t T = lds_addr(tile);
    const uint32_t a0 = T + (uint32_t)(rr * kRow + 16 * (hh ^ key));
    const uint32_t a1 = T + (uint32_t)(rr * kRow + 16 * ((2 + hh) ^ key));
    // tile scales: the codes of K-step k, token block tb, K-block hh are columns 64k + 32hh ..,
    // block 2k + hh of token half tb; the exponent field of the stored power of two is the
    // E8M0 operand scale
    const uint32_t sa_addr = T + (uint32_t)(kPage8 + 256 * wave + 4 * hh);
    auto kscale = [&](int f) -> int {
      if constexpr (Block) return (int)(lds_u32(sa_addr + 4u * (uint32_t)(kTileCols * (f & 1) + 2 * (f >> 1))) >> 23);
      else return one;
    };
    auto kfrag = [&](int f) -> i32x8 {   // K-step f/2, token block f%2
      const uint32_t o = 64u * (f >> 1) + (uint32_t)(32 * kRow) * (f & 1);
      const u32x4 lo = lds_b128(a0 + o), hi = lds_b128(a1 + o);
      return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
    // fragment f = (K-step f/2, token block f%2) feeds two consecutive MFMAs (hi, lo); the next
    // two fragments are read ahead
    constexpr int D = 1;
    i32x8 kr[D + 1];
    int ks[D + 1];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      kr[d] = kfrag(d);
      ks[d] = kscale(d);
    }
#pragma unroll
    for (int f = 0; f < 18; ++f) {
      if (f + D < 18) {
        kr[(f + D) % (D + 1)] = kfrag(f + D);
        ks[(f + D) % (D + 1)] = kscale(f + D);
      }
      const int k = f >> 1;
      f32x16& acc = (f & 1) ? s1 : s0;
      const int sa = ks[f % (D + 1)];
      __builtin_amdgcn_sched_barrier(0);
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr[f % (D + 1)], qhi[k], acc, 0, 0, 0, sa, 0, one);
      hook(2 * f);
      __builtin_amdgcn_sched_barrier(0);
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr[f % (D + 1)], qlo[k], acc, 0, 0, 0, sa, 0, lo_scale);
      hook(2 * f + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- softmax of one page: raw scores -> e4m3 Pt and the B block scale, against the segment
  // reference (log2 units).  y = raw * token scale; log2-domain score = kq * y.  It runs in
  // pieces -1 .. 22: -1 .. 5 scale the scores and find the page maximum and the block-scale
  // exponent as one block; 6 .. 21 each turn two scores into probabilities and e4m3 Pt, and in
  // the steps piece 6 + c follows value MFMA c of the previous page, so that their vector
  // instructions issue in the shadow of the 16-pass matrix instructions (about ten per MFMA
  // cost a fraction of what they cost as one block); 22 finishes.  Scales are read one piece
  // ahead of their use.
  struct Soft {
    float m_new, l_new;
    bool over_new;
    i32x8 p, plo;   // Pt ~ hi + lo/16, two e4m3 terms
    int sb;
  };
  struct SoftState {
    uint32_t cmu;   // largest token scale of the page (non-negative floats order as integers)
    float mx;       // largest y of this lane's tokens
    float neg;      // -(reference + e)
    int e;          // block-scale exponent of Pt
    float lsum;
    f32x4 c[2];     // scales: in use / in flight
    int w, wl;      // first half of a block's packed Pt terms
    int pk[8], pl[8];
  };
  auto soft_piece = [&](int p, f32x16& s0, f32x16& s1, const uint8_t* tile, int vis, bool fresh, SoftState& q,
                        Soft& st) {
    const uint32_t sbase = lds_addr(tile) + kPage8 + 256 * wave + 16 * hl;
    // scales of tokens 32tb + 8u + 4hl + 0..3 (block d = 4tb + u)
    auto scales = [&](int d) {
      if constexpr (Block) return f32x4{1.0f, 1.0f, 1.0f, 1.0f};   // the scales ride in the matrix instructions
      else return __builtin_bit_cast(f32x4, lds_b128(sbase + 128 * (d >> 2) + 32 * (d & 3)));
    };
    auto umax = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
    if (p == -1) {
      q.c[0] = scales(0);
      q.c[1] = scales(1);
      q.cmu = 0;
    } else if (p < 4) {   // y of blocks 2p, 2p+1 (elements 8(p&1) .. +7 of s0 or s1)
      f32x16& sv = p < 2 ? s0 : s1;
      const f32x4 ca = q.c[0], cb = q.c[1];
      if (p < 3) {
        q.c[0] = scales(2 * p + 2);
        q.c[1] = scales(2 * p + 3);
      }
      const int i0 = 8 * (p & 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        sv[i0 + k] *= ca[k];
        sv[i0 + 4 + k] *= cb[k];
      }
      uint32_t m = q.cmu;
#pragma unroll
      for (int k = 0; k < 4; ++k) m = umax(m, umax(__float_as_uint(ca[k]), __float_as_uint(cb[k])));
      q.cmu = m;
    } else if (p == 4) {
      if (vis < kBlock - 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = 8 * (i >> 2) + 4 * hl + (i & 3);
          if (t > vis) s0[i] = -INFINITY;
          if (t + 32 > vis) s1[i] = -INFINITY;
        }
      }
      float mx = s0[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
      q.mx = mx;
    } else if (p == 5) {
      float mx = q.mx;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
      const float tmax = pair_max(mx) * kq;
      const float cm = pair_max(__uint_as_float(q.cmu));
      const float m_in = fresh ? -INFINITY : m_ref;
      st.m_new = (m_in == -INFINITY) ? tmax : m_in;
      st.over_new = (fresh ? false : over) || (tmax > st.m_new + kRescaleLog2);
      const float m_use = (st.m_new == -INFINITY) ? 0.0f : st.m_new;
      // largest Pt of the page <= 2^(tmax - m) * max scale < 2^frexp_exp(...): shift it to <= 256
      int e = __builtin_amdgcn_frexp_expf(__builtin_amdgcn_exp2f(tmax - m_use) * cm) - 8;
      e = e < -120 ? -120 : (e > 120 ? 120 : e);
      q.e = e;
      q.neg = -(m_use + (float)e);
      q.lsum = 0.f;
      q.c[1] = scales(0);
    } else if (p < 22) {   // tokens 2h, 2h+1 of block d = h/2 (h = p - 6)
      const int h = p - 6, d = h >> 1, k0 = 2 * (h & 1);
      const f32x16& sv = (d < 4) ? s0 : s1;
      if ((h & 1) == 0) {
        q.c[0] = q.c[1];
        if (d + 1 < 8) q.c[1] = scales(d + 1);
      }
      const f32x4 c4 = q.c[0];
      const float u0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * (d & 3) + k0], kq, q.neg));
      const float u1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * (d & 3) + k0 + 1], kq, q.neg));
      q.lsum += u0;
      q.lsum += u1;
      // Pt = hi + lo/16: hi = e4m3(Pt), lo = e4m3(16 (Pt - hi)), so Pt keeps about 8 bits
      // (one e4m3 term alone moved the output of a few dominant tokens by up to 2^-4 of a
      // token's weight).  The empty asm statements pin the piece between its MFMAs (otherwise
      // the compiler sinks this arithmetic below the loop, next to the first use of its results)
      const float t0 = u0 * c4[k0], t1 = u1 * c4[k0 + 1];
      if ((h & 1) == 0) {   // low 16 bits of the block's packed words
        q.w = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
        const auto hv = __builtin_amdgcn_cvt_pk_f32_fp8(q.w, false);
        q.wl = cvt_pk_fp8_x16<false>(t0 - hv[0], t1 - hv[1], 0);
        asm volatile("" : "+v"(q.lsum), "+v"(q.w), "+v"(q.wl));
      } else {              // high 16 bits
        q.pk[d] = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, q.w, true);
        const auto hv = __builtin_amdgcn_cvt_pk_f32_fp8(q.pk[d], true);
        q.pl[d] = cvt_pk_fp8_x16<true>(t0 - hv[0], t1 - hv[1], q.wl);
        asm volatile("" : "+v"(q.lsum), "+v"(q.pk[d]), "+v"(q.pl[d]));
      }
    } else if (p == 22) {
      st.l_new = (fresh ? 0.0f : l_run) + __builtin_ldexpf(q.lsum, q.e);
      st.p = i32x8{q.pk[0], q.pk[1], q.pk[2], q.pk[3], q.pk[4], q.pk[5], q.pk[6], q.pk[7]};
      st.plo = i32x8{q.pl[0], q.pl[1], q.pl[2], q.pl[3], q.pl[4], q.pl[5], q.pl[6], q.pl[7]};
      st.sb = q.e + kE8M0One;
    }
  };

  // ---- O^T += Codes^T . Pt^T for the page in `tile`
  auto values = [&](const uint8_t* tile, const i32x8& pf, const i32x8& pfl, int sb, auto hook) {
    o_fence<3>(oacc);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int rl = 8 * ((ln >> 3) & 1) + 4 * (ln >> 5) + ((ln >> 1) & 3);
    const int h4 = (ln >> 4) & 1;
    const uint32_t T = (uint32_t)(tile - smem);
    const uint8_t* xv[4];   // [2 * (q & 1) + (ct & 1)]
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * (e >> 1) + rl;
      xv[e] = smem + T + (uint32_t)(r * kRow + 16 * ((2 * (e & 1) + h4) ^ key8(r)) + 8 * (ln & 1));
    }
    auto vfrag = [&](int ct) -> i32x8 {
      const uint32_t o = 64u * (ct >> 1);
      const i32x2 t0 = lds_tr8(xv[ct & 1], o);
      const i32x2 t1 = lds_tr8(xv[2 + (ct & 1)], o);
      const i32x2 t2 = lds_tr8(xv[ct & 1], o + 32 * kRow);
      const i32x2 t3 = lds_tr8(xv[2 + (ct & 1)], o + 32 * kRow);
      return i32x8{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
    };
    // tile scales: column tile ct is column block ct; K-block hl of the operand is token half hl
    const uint32_t va_addr = lds_addr(tile) + (uint32_t)(kPage8 + 256 * wave + 4 * kTileCols * (ln >> 5));
    auto vscale = [&](int ct) -> int {
      if constexpr (Block) return (int)(lds_u32(va_addr + 4u * (uint32_t)ct) >> 23);
      else return one;
    };
    constexpr int D = 1;
    i32x8 vr[D + 1];
    int vs[D + 1];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      vr[d] = vfrag(d);
      vs[d] = vscale(d);
    }
    hook(-1);
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
      if (ct + D < 16) {
        vr[(ct + D) % (D + 1)] = vfrag(ct + D);
        vs[(ct + D) % (D + 1)] = vscale(ct + D);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma8_acc(oacc[ct], vr[ct % (D + 1)], pf, vs[ct % (D + 1)], sb);
      mfma8_acc(oacc[ct], vr[ct % (D + 1)], pfl, vs[ct % (D + 1)], sb - 4);   // lo term: block scale 2^(e-4)
      hook(ct);
      __builtin_amdgcn_sched_barrier(0);
    }
    o_fence<20>(oacc);
  };

  i32x8 pf, pfl;
  int psb = kE8M0One;
  Soft sm;
  auto soft_commit = [&](const Soft& st) {
    m_ref = st.m_new;
    l_run = st.l_new;
    over = st.over_new;
    pf = st.p;
    pfl = st.plo;
    psb = st.sb;
  };
  auto load_for = [&](int stage, int pg, int nv) {
    return page_load8<Block>(smem + stage * kStage8, a.cache, a.cache_scale, nv > 0 ? pg : 0, nv);
  };
  // this lane's entry of row load i in the source-offset table
  const uint32_t src_addr = lds_addr(smem + kSrcTab8) + (uint32_t)(1152 * (wave & 1) + 2 * lane);
  auto src_off = [&](int i) -> int { return (int)lds_u16(src_addr + 128u * (uint32_t)i); };
  auto issue = [&](const PageLoad8& pl) {
    int off[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) off[i] = src_off(i);
#pragma unroll
    for (int i = 0; i < 10; ++i) load_row8<Aux>(pl, i, wave, lane, i < 9 ? off[i] : 0);
  };
  const uint32_t tab_addr = lds_addr(smem + kTabOff8);
  auto entry = [&](int z) -> int4 {
    if (z >= n_steps) return int4{-1, 0, 0, 0};
    const u32x4 e = lds_b128(tab_addr + 16u * (uint32_t)z);
    return int4{uni((int)e[0]), uni((int)e[1]), uni((int)e[2]), uni((int)e[3])};
  };
  auto valid_page = [&](const int4& e) { return e.x >= 0 && e.x < a.num_blocks; };
  auto nvalid = [&](const int4& e) { return valid_page(e) ? (e.y < kBlock ? e.y : kBlock) : 0; };
  auto last_visible = [&](const int4& e) {
    const int v = e.y - a.Sq + j;
    return valid_page(e) ? (v < kBlock - 1 ? v : kBlock - 1) : -1;
  };

  int4 e0 = entry(0), e1 = entry(1), e2 = entry(2), e3;
  // pages 0..2 are requested first: they land while the queries are split
  issue(load_for(0, e0.x, nvalid(e0)));
  issue(load_for(1, e1.x, nvalid(e1)));
  issue(load_for(2, e2.x, nvalid(e2)));
  load_q(e0.z);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();
  {
    f32x16 s0, s1;
    scores(smem, [](int) {}, s0, s1);
    SoftState ss;
#pragma unroll
    for (int p = -1; p < 23; ++p) soft_piece(p, s0, s1, smem, last_visible(e0), true, ss, sm);
    soft_commit(sm);
  }

  for (int y = 0; y < n_steps; ++y) {
    const bool has_next = y + 1 < n_steps;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(10));   // page y+1 landed (page y+2 may be in flight)
    lds_barrier();                                 // stage (y+3)%4 is no longer read by anyone
    e3 = entry(y + 3);
    const PageLoad8 pl = load_for((y + 3) & 3, e3.x, nvalid(e3));
    const bool seg_end = (e0.w & kLast) || !has_next;
    if (seg_end && has_next) {
      load_q(e1.z);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    // scores of page y+1, then the values of page y with the softmax of page y+1 spread over
    // its MFMAs
    const uint8_t* next = smem + ((y + 1) & 3) * kStage8;
    f32x16 s0, s1;
    // row load k goes out after score MFMA 4k, its table entry having been read one load ahead
    int off_next = src_off(0);
    scores(next, [&](int st) {   // stale data if !has_next
      if ((st & 3) == 0) {   // st = 0, 4, .., 32
        const int k = st >> 2, off = off_next;
        if (k + 1 < 9) off_next = src_off(k + 1);
        load_row8<Aux>(pl, k, wave, lane, off);
      }
      if (st == 34) load_row8<Aux>(pl, 9, wave, lane, 0);
    }, s0, s1);
    const float m_old = m_ref, l_old = l_run;
    const bool over_old = over;
    const int vis = last_visible(e1);
    SoftState ss;
#pragma unroll
    for (int p = -1; p < 6; ++p) soft_piece(p, s0, s1, next, vis, seg_end, ss, sm);
    values(smem + (y & 3) * kStage8, pf, pfl, psb, [&](int c) {
      if (c >= 0) soft_piece(c + 6, s0, s1, next, vis, seg_end, ss, sm);
    });
    soft_piece(22, s0, s1, next, vis, seg_end, ss, sm);

    if (seg_end) {
      const float l_tot = pair_sum(l_old);
      const size_t row = ((size_t)(g + e0.z) * a.Sq + j) * kH + head;
      if (hl == 0) reinterpret_cast<float2*>(a.part_ml)[row] = float2{m_old, over_old ? -1.0f : l_tot};
      uint16_t* so = slot_o(e0.z);
      store_partial(so, oacc);
      if (has_next) {
#pragma unroll
        for (int t = 0; t < 16; ++t) mfma_zero(oacc[t], zero8);
      }
    }
    soft_commit(sm);
    e0 = e1;
    e1 = e2;
    e2 = e3;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// ------------------------------------------------------------------------ LSE combine

// Exact attention of one (query row, head) by one wave, two passes over the visible tokens in
// fp32 (scores in the exp2 domain).  Used by the combine for heads whose fast-path segments
// were marked (a score far above the segment's reference); slow, but right for any input.
// Lane l handles columns 9l .. 9l+8 of the score and c0 + 2l, c0 + 2l + 1 of the output (one
// quarter of the latent row); the log-sum-exp is written when `with_lse`.
__device__ void exact_head(const DecodeArgs& a, int b, int j, int h, int L, int c0, bool with_lse) {
  const int lane = threadIdx.x & 63;
  const int row = b * a.Sq + j;
  const int last = L - a.Sq + j;                     // last visible position
  const int n = last + 1 < L ? last + 1 : L;
  const size_t qrow = (size_t)row * kH + h;
  float qv[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) qv[i] = bf16_bits_to_f32(a.q_abs[qrow * kRow + 9 * lane + i]);
  // cache slot of token t, or -1 when its page id is out of range
  auto slot = [&](int t) -> long long {
    const int pg = a.block_table[(size_t)b * a.max_blocks + t / kBlock];
    if (pg < 0 || pg >= a.num_blocks) return -1;
    return (long long)pg * kBlock + t % kBlock;
  };
  // value of column c of slot sl (tile scales: the page's tile of token half (sl % 64) / 32 and
  // column block c / 32; token scales multiply whole scores and weights below)
  auto elem = [&](long long sl, int c) -> float {
    if (!a.fp8) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.cache)[sl * kRow + c]);
    const float v = e4m3_to_f32(a.cache[sl * kRow + c]);
    if (!a.block8) return v;
    return v * a.cache_scale[((sl / kBlock) * 2 + (sl % kBlock) / 32) * kTileCols + c / 32];
  };
  auto token_scale = [&](long long sl) { return (a.fp8 && !a.block8) ? a.cache_scale[sl] : 1.0f; };
  auto score = [&](long long sl) {
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 9; ++i) d += qv[i] * elem(sl, 9 * lane + i);
    return wave_sum(d) * token_scale(sl) * a.scale_log2;
  };
  float mx = -INFINITY;
  for (int t = 0; t < n; ++t) {
    const long long sl = slot(t);
    if (sl >= 0) mx = fmaxf(mx, score(sl));
  }
  float l = 0.f;
  float acc0 = 0.f, acc1 = 0.f;
  const int col = c0 + 2 * lane;
  if (mx != -INFINITY) {
    for (int t = 0; t < n; ++t) {
      const long long sl = slot(t);
      if (sl < 0) continue;
      const float w = __builtin_amdgcn_exp2f(score(sl) - mx);
      l += w;
      const float wc = w * token_scale(sl);
      acc0 += wc * elem(sl, col);
      acc1 += wc * elem(sl, col + 1);
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.0f;
  *reinterpret_cast<float2*>(a.o_lat + qrow * kDC + col) = float2{acc0 * inv, acc1 * inv};
  if (with_lse && lane == 0) a.lse[qrow] = l > 0.f ? (mx + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}


// One workgroup per (query row, group of 32 heads, quarter of the latent columns).  Every
// segment left its unnormalised O_g (in register order) and (m_g, l_g) per head in slot g + b;
// with M = max m_g over the non-empty ones and w_g = 2^(m_g - M):  o = sum w_g O_g / sum w_g l_g,
// lse = ln 2 * (M + log2 sum w_g l_g).  The partials are bf16 (summed here in fp32).  Quarter c
// of a group's 32 KiB block is its 1 KiB blocks 8c .. 8c+7 (column tiles 4c .. 4c+3, so columns
// 128c .. 128c+127), contiguous in every slot: thread t reads its 16-byte pieces t + 256i
// (i < 2, eight values each), all of head 32w + t%32, so each thread needs one head's
// weights.  The pieces and (m, l) of KB slots are requested together, so a sequence's slots
// cost about one memory latency rather than one each; KB = 8 where sequences span many
// ranges (G >= 3B), 4 where G >= B, else 2 (the batch's unused slots still load a slot, so a
// smaller batch reads less where rows have one or two slots, as in a prefill's single range;
// fewer registers also allow more workgroups per CU).  The result goes
// through LDS so that each head's 128 columns are written contiguously.  Heads marked by the
// fast path (or whose sums are not finite) are then recomputed exactly, quarter by quarter.
constexpr int kCombinePitch = 128 + 4;   // fp32 words per head in the LDS tile (spreads heads over banks)

template <int KB>
__global__ void __launch_bounds__(256) combine_kernel(DecodeArgs a) {
  constexpr int kCombineBatch = KB;
  __shared__ __attribute__((aligned(16))) float tile[32 * kCombinePitch];   // [32 heads][128 columns]
  __shared__ int redo_mask;                                                 // heads to recompute
  const int row = blockIdx.x;          // b*Sq + j
  const int b = row / a.Sq, j = row - b * a.Sq;
  const int w = blockIdx.y;            // heads 32w .. 32w+31
  const int c = blockIdx.z;            // columns 128c .. 128c+127
  const int t = threadIdx.x, lane = t & 63;
  const int hh = t & 31, h = 32 * w + hh, hl = (t >> 5) & 1;
  // One pass over the lengths: the batch's total cost, and the pages and non-empty sequences
  // before b (the same units the split's cut uses).
  long long C_all = 0;
  long long first = 0;                 // first page of sequence b
  int rank = 0;                        // non-empty sequences before b
  for (int base = 0; base < a.B; base += 64) {
    const int q = base + lane;
    int L;
    const int n = q < a.B ? seq_tiles(a.kv_lens, q, a.max_blocks, &L) : 0;
    C_all += wave_sum_i(n > 0 ? n + a.seg_w : 0);
    first += wave_sum_i(q < b ? n : 0);
    rank += wave_sum_i(q < b && n > 0 ? 1 : 0);
  }
  const long long cfirst = first + (long long)a.seg_w * (rank + 1);   // cost position of that page
  int Lb;
  const int nb = seq_tiles(a.kv_lens, b, a.max_blocks, &Lb);
  if (t == 0) redo_mask = 0;
  __syncthreads();
  // head 32w + k of this row starts at out_base + k * kDC
  float* out_base = a.o_lat + ((size_t)row * kH + 32 * w) * kDC + 128 * c;
  if (nb == 0) {
    for (int i = t; i < 32 * 32; i += 256)
      *reinterpret_cast<f32x4*>(out_base + (i >> 5) * kDC + 4 * (i & 31)) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c == 0 && t < 32) a.lse[(size_t)row * kH + 32 * w + t] = -INFINITY;
    return;
  }
  const int g_lo = range_of_tile(cfirst, C_all, a.G);
  const int g_hi = range_of_tile(cfirst + nb - 1, C_all, a.G);
  // Walk of the ranges g_lo, g_lo + 1, ..: range g's cost interval starts at floor(g C / G), and
  // with g C = floor(g C / G) G + rem, the next start is floor(g C / G) + C/G + carry (carry = 1
  // when rem + C%G >= G).  A range whose interval is empty (possible when the batch costs fewer
  // units than there are ranges) wrote nothing: it is skipped.  One division per sequence.
  const long long cq = C_all / a.G, cr = C_all % a.G;
  long long rem = ((long long)g_lo * C_all) % a.G;
  auto walk_empty = [&]() {   // is the next range of the walk empty?  (advances the walk)
    const bool e = cq == 0 && rem + cr < a.G;
    rem += cr;
    if (rem >= a.G) rem -= a.G;
    return e;
  };
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  auto slot = [&](int g) { return ((size_t)(g + b) * a.Sq + j); };
  // partials (bf16) and (m, l) of the slots g .. g + kCombineBatch - 1.  Every load is issued
  // (a slot that is past g_hi or empty reads slot g_hi, which the range holding the sequence's
  // last page wrote, and is then given weight 0), so the loads of a batch share one memory
  // latency; the flags are wave-uniform.
  const size_t piece = (size_t)w * (32 * kDC) + (size_t)c * (8 * 512) + 8 * t;
  u32x4 v[kCombineBatch][2];
  float2 mv[kCombineBatch];
  bool use[kCombineBatch];
  auto fetch = [&](int g) {
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int gk = g + k;
      use[k] = gk <= g_hi && !walk_empty();
      const size_t sl = slot(use[k] ? gk : g_hi);
      const uint16_t* src = a.part_o + sl * (kH * kDC) + piece;
#pragma unroll
      for (int i = 0; i < 2; ++i) v[k][i] = *reinterpret_cast<const u32x4*>(src + 2048 * i);
      mv[k] = ml[sl * kH + h];
    }
  };
  // Running maximum over the batches: acc and L are rescaled when a batch raises it (a
  // sequence's slots mostly fit one batch, and then nothing is rescaled).  A segment with
  // nothing visible (l = 0) holds zeros and gets weight 0; one marked by the fast path (l < 0)
  // sends the head to the exact recomputation.
  float M = -INFINITY;
  bool redo = false;
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int g = g_lo; g <= g_hi; g += kCombineBatch) {
    fetch(g);
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      if (use[k] && mv[k].y < 0.f) redo = true;
      if (use[k] && mv[k].y > 0.f) Mb = fmaxf(Mb, mv[k].x);
    }
    if (Mb > M) {
      const float r = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mb);
      L *= r;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= r;
      M = Mb;
    }
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const bool live = use[k] && mv[k].y > 0.f;
      const float wg = live ? __builtin_amdgcn_exp2f(mv[k].x - M) : 0.0f;
      L += live ? wg * mv[k].y : 0.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * i + (e >> 1)][2 * (e & 1)] += wg * __uint_as_float(v[k][i][e] << 16);
          acc[2 * i + (e >> 1)][2 * (e & 1) + 1] += wg * __uint_as_float(v[k][i][e] & 0xFFFF0000u);
        }
    }
  }
  if (redo || M == -INFINITY) {   // as before: nothing summed for a redone head; no token: zeros
    L = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool fin = __builtin_isfinite(L);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    fin = fin && __builtin_isfinite(acc[i][0]) && __builtin_isfinite(acc[i][1]) && __builtin_isfinite(acc[i][2]) &&
          __builtin_isfinite(acc[i][3]);
  redo = redo || !fin;
  const float inv = L > 0.f ? 1.0f / L : 0.0f;
  // piece t + 256i is 1 KiB block 8c + bq, bq = t/64 + 4i = 2ct + qp (column tile 4c + ct):
  // acc[2i] holds columns 128c + 32ct + 16qp + 4hl .. +3 of head hh, acc[2i+1] the same + 8
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int bq = (t >> 6) + 4 * i, col = 32 * (bq >> 1) + 16 * (bq & 1) + 4 * hl;
    *reinterpret_cast<f32x4*>(tile + hh * kCombinePitch + col) = acc[2 * i] * inv;
    *reinterpret_cast<f32x4*>(tile + hh * kCombinePitch + col + 8) = acc[2 * i + 1] * inv;
  }
  if (redo) atomicOr(&redo_mask, 1 << hh);
  __syncthreads();
  for (int i = t; i < 32 * 32; i += 256)
    *reinterpret_cast<f32x4*>(out_base + (i >> 5) * kDC + 4 * (i & 31)) =
        *reinterpret_cast<const f32x4*>(tile + (i >> 5) * kCombinePitch + 4 * (i & 31));
  if (c == 0 && t < 32) a.lse[(size_t)row * kH + h] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
  const int mask = redo_mask;
  if (mask) {
    __syncthreads();   // the plain results are written before any exact row replaces them
    for (int k = t >> 6; k < 32; k += 4)
      if (mask & (1 << k)) exact_head(a, b, j, 32 * w + k, Lb, 128 * c, c == 0);
  }
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
        rowidx = pg * kBlock + (t % kBlock);   // pages < 2^24: fits an int
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
// unit (each holds all 160 KiB of LDS), so G = CUs / Sq, capped by the number of pages, and
// raised where needed so that no range exceeds the LDS page table (kTabCap pages for bf16,
// kTabCap8 for fp8: the pages of the batch are at most B * max_blocks).
// Per-segment overhead in pages for cutting the ranges, fitted to measured workgroup times (a
// range with one more segment ran ~20K cycles longer: ~3 bf16 pages, ~2 fp8 pages).
constexpr int kSegCost = 3, kSegCost8 = 2;

// Test-only overrides of the range count, read at every call (so a workspace size and the
// decode calls that use it must see the same values), applied within the same limits as the
// default (the page table's capacity, at most one range per page):
//   MLA_FORCE_SPLITS = G > 0   G ranges;
//   MLA_SPLIT_TOKENS = n > 0   ranges of about n tokens of the block tables' capacity,
//                              G = ceil(64 B max_blocks / n) (ignored when MLA_FORCE_SPLITS is set).
// The result is the same attention for any count, up to the rounding of the probabilities and
// partials that a different cut changes.  Unset, empty or malformed values are ignored.
long long env_positive(const char* name, long long max) {
  const char* v = std::getenv(name);
  if (v == nullptr || *v == 0) return 0;
  char* end = nullptr;
  const long long x = std::strtoll(v, &end, 10);
  if (end == v || *end != 0 || x <= 0 || x > max) return 0;
  return x;
}
int forced_ranges() { return (int)env_positive("MLA_FORCE_SPLITS", 1LL << 24); }
long long forced_split_tokens() { return env_positive("MLA_SPLIT_TOKENS", 1LL << 40); }

// Small batches: at least this many pages (of the block tables' capacity) per range.  A range
// costs a fixed ~20K cycles (page table, queries, segment end) and a 128 KiB partial that the
// combine reads back; at B = 16 x 4096 tokens split + combine took 54.6 us with 128 ranges,
// 51.4 with 160, 50.0 with 192, 50.5 with 224 and 51.5 with 256.
constexpr int kMinRangePages = 5;

// Most split workgroups (ranges x queries per sequence) a plan may launch; wider plans are refused.
constexpr long long kMaxSplitGrid = 1LL << 23;

long long decode_num_ranges(int num_cus, int B, int Sq, int max_blocks, bool fp8) {
  const long long cap = (long long)B * max_blocks;
  const int tab = fp8 ? kTabCap8 : kTabCap;
  long long G = num_cus / (Sq > 0 ? Sq : 1);
  if (G > cap / kMinRangePages) G = cap / kMinRangePages;
  if (G < 1) G = 1;
  if (const int f = forced_ranges()) G = f;
  else if (const long long n = forced_split_tokens()) G = (cap * kBlock + n - 1) / n;
  // a range owns at most ceil(C / G) pages, C <= B (max_blocks + w) the total cost
  const long long need = ((long long)B * ((long long)max_blocks + (fp8 ? kSegCost8 : kSegCost)) + tab - 1) / tab;
  if (G < need) G = need;
  if (cap < G) G = cap < 1 ? 1 : cap;
  return G;
}

size_t decode_workspace_bytes(const mla_config_t& cfg, int num_cus, int B, int Sq, int max_blocks) {
  if (!(cfg.cache_dtype != MLA_F32 && is_dsv2_shape(cfg))) return 256;   // generic path: none needed
  const long long G = decode_num_ranges(num_cus, B, Sq, max_blocks,
                                        cfg.cache_dtype == MLA_FP8_E4M3 || cfg.cache_dtype == MLA_FP8_E4M3_B32);
  if (G > kMaxSplitGrid / (Sq > 0 ? Sq : 1)) return 0;   // refused: too many workgroups
  const size_t slots = (size_t)(G + B - 1) * Sq;
  const size_t o_bytes = slots * kH * kDC * sizeof(uint16_t);
  const size_t l_bytes = slots * kH * 2 * sizeof(float);
  return ((o_bytes + 255) & ~(size_t)255) + ((l_bytes + 255) & ~(size_t)255);
}

// The split kernels take all of a compute unit's LDS, above the default dynamic limit, so the
// limit is raised once per device before their first launch.  Several host threads may get
// here at once: each one that finds the device not yet marked repeats the same (idempotent)
// attribute calls, and the mark is an atomic with release/acquire ordering, so no thread
// launches before some thread's calls have returned successfully.  A failed call is returned
// and leaves the device unmarked.
constexpr int kMaxDev = 64;
std::atomic<int> g_lds_set[kMaxDev];

hipError_t set_decode_lds_limits() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<int>* mark = (dev >= 0 && dev < kMaxDev) ? &g_lds_set[dev] : nullptr;
  if (mark && mark->load(std::memory_order_acquire)) return hipSuccess;
  const void* kernels[6] = {(const void*)decode_mfma_bf16_kernel<0>,       (const void*)decode_mfma_bf16_kernel<2>,
                            (const void*)decode_mfma_fp8_kernel<0, false>, (const void*)decode_mfma_fp8_kernel<2, false>,
                            (const void*)decode_mfma_fp8_kernel<0, true>,  (const void*)decode_mfma_fp8_kernel<2, true>};
  for (int k = 0; k < 6; ++k) {
    e = hipFuncSetAttribute(kernels[k], hipFuncAttributeMaxDynamicSharedMemorySize, k < 2 ? kDecodeLds : kDecodeLds8);
    if (e != hipSuccess) return e;
  }
  if (mark) mark->store(1, std::memory_order_release);
  return hipSuccess;
}

hipError_t launch_decode(const mla_config_t& cfg, int num_cus, const void* q_abs, const void* cache, const float* cache_scale, int num_blocks, const int32_t* block_table,
                         int max_blocks, const int32_t* kv_lens, int B, int Sq, void* workspace, float* o_lat,
                         float* lse, hipStream_t stream, int phases) {
  if (B == 0) return hipSuccess;
  const float scale = cfg.softmax_scale;
  const bool block8 = cfg.cache_dtype == MLA_FP8_E4M3_B32;
  const bool fp8 = cfg.cache_dtype == MLA_FP8_E4M3 || block8;
  if ((cfg.cache_dtype == MLA_BF16 || fp8) && is_dsv2_shape(cfg)) {
    DecodeArgs a;
    a.q_abs = static_cast<const uint16_t*>(q_abs);
    a.cache = static_cast<const uint8_t*>(cache);
    a.cache_scale = cache_scale;
    a.block_table = block_table;
    a.kv_lens = kv_lens;
    a.o_lat = o_lat;
    a.lse = lse;
    // the caller has checked the plan against kMaxSplitGrid (a zero workspace size)
    const int G = (int)decode_num_ranges(num_cus, B, Sq, max_blocks, fp8);
    const size_t slots = (size_t)(G + B - 1) * Sq;
    a.part_o = static_cast<uint16_t*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                          ((slots * kH * kDC * sizeof(uint16_t) + 255) & ~(size_t)255));
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.B = B;
    a.Sq = Sq;
    a.G = G;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.fp8 = fp8 ? 1 : 0;
    a.block8 = block8 ? 1 : 0;
    a.seg_w = fp8 ? kSegCost8 : kSegCost;
    {
      hipError_t e = set_decode_lds_limits();
      if (e != hipSuccess) return e;
    }
    if (phases & 1) {
      // non-temporal page loads when no other workgroup reads the same pages (one query)
      const dim3 grid(G * Sq), block(64 * kWaves);
      if (block8) {
        if (Sq == 1)
          hipLaunchKernelGGL((decode_mfma_fp8_kernel<2, true>), grid, block, kDecodeLds8, stream, a);
        else
          hipLaunchKernelGGL((decode_mfma_fp8_kernel<0, true>), grid, block, kDecodeLds8, stream, a);
      } else if (fp8) {
        if (Sq == 1)
          hipLaunchKernelGGL((decode_mfma_fp8_kernel<2, false>), grid, block, kDecodeLds8, stream, a);
        else
          hipLaunchKernelGGL((decode_mfma_fp8_kernel<0, false>), grid, block, kDecodeLds8, stream, a);
      } else {
        if (Sq == 1)
          hipLaunchKernelGGL(decode_mfma_bf16_kernel<2>, grid, block, kDecodeLds, stream, a);
        else
          hipLaunchKernelGGL(decode_mfma_bf16_kernel<0>, grid, block, kDecodeLds, stream, a);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (phases & 2) {
      // a sequence spans about G / B + 1 ranges
      if (G >= 3 * B)
        hipLaunchKernelGGL(combine_kernel<8>, dim3(B * Sq, kH / 32, 4), dim3(256), 0, stream, a);
      else if (G >= B)
        hipLaunchKernelGGL(combine_kernel<4>, dim3(B * Sq, kH / 32, 4), dim3(256), 0, stream, a);
      else   // fewer ranges than sequences (prefill: one range): mostly one slot per row
        hipLaunchKernelGGL(combine_kernel<2>, dim3(B * Sq, kH / 32, 4), dim3(256), 0, stream, a);
    }
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

// ------------------------------------------------------------------------ fixed scratch

// For callers that cannot allocate (code under graph capture, serving loops that forbid it):
// mla_decode_attn_noalloc puts the split-K partials in this file-scope device array instead of
// a caller workspace.  Every device the library runs on holds its own copy until the process
// ends.  In host code the array's name is only a stand-in, so the device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and kept; kernels get that
// address.  The decode kernels write every partial before reading it, so the array needs no
// clearing; calls on one device share it, so calls that overlap in time on one device race.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDev];

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev].store(p, std::memory_order_release);   // every thread finds the same address
  }
  *out = p;
  return hipSuccess;
}

}  // namespace mla
