// Projections from and to the model width, on either side of the latent-space decode:
//
//   upstream    [c ; k_R raw] = h [W_down | W_KR]     the latent and the positional key of each new
//               [q^C ; q^R]   = h [W_Q | W_QR]        token, and the two query parts (katajob
//                                                     interview page, "code": latent = x @ W_down;
//                                                     bembew "Multi-head Latent Attention",
//                                                     "Implementation Logic", steps 1, 3 and 4)
//   downstream  out = sum_i o_lat_i W_O'_i            the value up-projection folded into the output
//               W_O'_i = W_UV,i W_O,i  [d_c, d_model]  projection (katajob "solid answer")
//
// All are row GEMMs Y[t, n] = sum_k X[t, k] W[k, n] with few rows t (the step's tokens) and a large
// weight, so they are bound by reading the weight once.  The weight is taken transposed, Wt[n, k]
// (each output's weights contiguous, the layout of a linear layer's weight matrix), so that both
// matrix operands are 16-byte row loads: A = Wt rows (32 outputs x 8 consecutive k per lane), B = X
// rows (32 tokens x 8 consecutive k), D = Y^T on v_mfma_f32_32x32x16_bf16.
//
// A workgroup owns 256 outputs x 64 rows and a slice of the contraction (each wave 64 outputs);
// weights and X reach LDS by buffer->LDS loads, three chunks deep.  With one slice the workgroup
// writes the result;
// with S slices each writes fp32 partials and a second kernel adds the S partials in a fixed order
// (deterministic) and writes the result.
#include "common.h"

#include <atomic>
#include <cmath>

namespace mla {

constexpr int kPjT = 64;       // rows per workgroup
constexpr int kPjChunk = 64;   // contraction elements per chunk (four MFMA K-steps)

// Result routing: output n < split goes to dst0[t * ld0 + n], the rest to dst1[t * ld1 + n - split]
// (the latent and the positional key, or the content and the positional query, are separate
// arrays of the next call).
struct PjOut {
  void* dst0;
  void* dst1;
  long long ld0, ld1;
  int split;
};

template <typename OutT>
__device__ __forceinline__ void pj_store(const PjOut& o, int t, int n, float v) {
  OutT* d;
  size_t i;
  if (n < o.split) {
    d = static_cast<OutT*>(o.dst0);
    i = (size_t)t * o.ld0 + n;
  } else {
    d = static_cast<OutT*>(o.dst1);
    i = (size_t)t * o.ld1 + (n - o.split);
  }
  if constexpr (sizeof(OutT) == 4) d[i] = v;
  else d[i] = (OutT)f32_to_bf16_bits(v);
}

// Workgroup (output group of 256, slice s, row block z): wave w owns outputs n0 + 64w .. +63 (two
// 32-row A tiles) and all 64 rows (two 32-column B tiles), over the slice's chunks of 64
// contraction elements.  Every chunk is moved into LDS by buffer->LDS loads (no registers in
// flight): the wave's own 64 weight rows (8 KiB) and a share of the rows' X block (bf16: 8 KiB,
// fp32: 16 KiB, converted to bf16 when read), three stages, two chunks in flight while one is
// multiplied, one barrier per chunk.  Rows are XOR-swizzled at 16-byte granularity so that the
// fragment reads (32 rows, one 16-byte chunk each) spread over the banks.
// X [T, K] (ldx), Wt [N, K] bf16; K % 64 == 0.  part == nullptr: write through `o` (bf16);
// else fp32 partials part[s][t][n].
constexpr int kPjGroup = 256;    // outputs per workgroup
constexpr int kPjA = 256 * 128;  // A stage bytes: 256 rows x 64 bf16

template <typename XT>
constexpr int pj_stage_bytes() { return kPjA + kPjT * kPjChunk * (int)sizeof(XT); }

__device__ __forceinline__ int pj_key(int r) { return (r >> 1) & 7; }   // bf16 rows: 8 chunks of 16 B

// s_waitcnt that lets at most n vector-memory operations stay outstanding (gfx9 encoding; other
// counters untouched)
constexpr int pj_waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// One row GEMM of a launch.  A launch runs up to two of them (the latent and the query
// projections of a step share one grid): workgroups wg0 .. wg0 + groups_n * S * row blocks - 1
// belong to this one, as (output group, slice, row block) with the output group fastest.
template <typename XT>
struct PjGemm {
  const XT* X;
  long long ldx;
  const uint16_t* Wt;
  PjOut o;
  float* part;   // S > 1: fp32 partials [S][T][N]
  int T, N, K, S, groups_n, wg0;
};
template <typename XT>
struct PjJob {
  PjGemm<XT> g[2];
  int np;
};

template <typename XT>
__global__ void __launch_bounds__(256) rows_gemm_kernel(PjJob<XT> job) {
  extern __shared__ __attribute__((aligned(256))) uint8_t pj_smem[];
  constexpr int SB = pj_stage_bytes<XT>();
  constexpr bool kF32 = sizeof(XT) == 4;
  constexpr int NX = kF32 ? 4 : 2;   // X loads per wave per chunk (1 KiB each)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  const PjGemm<XT> P = (job.np > 1 && bid >= job.g[1].wg0) ? job.g[1] : job.g[0];
  const XT* __restrict__ X = P.X;
  const uint16_t* __restrict__ Wt = P.Wt;
  float* __restrict__ part = P.part;
  const long long ldx = P.ldx;
  const int T = P.T, N = P.N, K = P.K, S = P.S;
  const int local = bid - P.wg0, xg = local % P.groups_n, rest = local / P.groups_n;
  const int n_base = kPjGroup * xg, s = rest % S, t0 = kPjT * (rest / S);
  const int r = lane & 31, g = lane >> 5;
  const int n_chunks = K / kPjChunk;
  const int c0 = (int)((long long)s * n_chunks / S), c1 = (int)((long long)(s + 1) * n_chunks / S);
  // weight rows n_base .. N-1 and X rows t0 .. T-1 of this workgroup (loads past them read zeros)
  const int a_rows = N - n_base < kPjGroup ? N - n_base : kPjGroup;
  const int x_rows = T - t0 < kPjT ? T - t0 : kPjT;
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Wt + (size_t)n_base * K), 0, a_rows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + (size_t)t0 * ldx), 0, (int)(((x_rows - 1) * ldx + K) * (long long)sizeof(XT)), 0x00020000);
  // per-lane source offsets: A load i writes LDS rows 64w + 8i + lane/8 (position lane%8); X load i
  // writes rows (bf16) 8(2w + i) + lane/8 or (fp32) 4(4w + i) + lane/16.  x_off has room for
  // the larger count (an array bound that depends on XT does not compile in the host pass).
  int a_off[8], x_off[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = 64 * wave + 8 * i + (lane >> 3);
    a_off[i] = rr * K * 2 + 16 * ((lane & 7) ^ pj_key(rr));
  }
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    if constexpr (kF32) {
      const int xrw = 4 * (4 * wave + i) + (lane >> 4);
      x_off[i] = (int)(xrw * ldx * 4) + 16 * ((lane & 15) ^ (xrw & 15));
    } else {
      const int xrw = 8 * (2 * wave + i) + (lane >> 3);
      x_off[i] = (int)(xrw * ldx * 2) + 16 * ((lane & 7) ^ pj_key(xrw));
    }
  }
  const int x_chunk_bytes = kPjChunk * (int)sizeof(XT);
  auto issue = [&](int c, int stage) {
    uint8_t* st = pj_smem + stage * SB;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (MLA_LDS void*)(st + (8 * wave + i) * 1024), 16, a_off[i],
                                               c * kPjChunk * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < NX; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (MLA_LDS void*)(st + kPjA + (NX * wave + i) * 1024), 16, x_off[i],
                                               c * x_chunk_bytes, 0, 0);
  };
  f32x16 acc[4];   // [n tile][t tile]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  if (c0 < c1) issue(c0, 0);
  if (c0 + 1 < c1) issue(c0 + 1, 1);
  for (int c = c0; c < c1; ++c) {
    const int stage = (c - c0) % 3;
    if (c + 1 < c1) __builtin_amdgcn_s_waitcnt(pj_waitcnt_vm(8 + NX));   // chunk c landed (c+1 may not)
    else __builtin_amdgcn_s_waitcnt(pj_waitcnt_vm(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // everyone's loads of c, and stage (c+2)%3 free
    if (c + 2 < c1) issue(c + 2, (c - c0 + 2) % 3);
    const uint8_t* st = pj_smem + stage * SB;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int rr = 64 * wave + 32 * nt + r;
        av[nt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + rr * 128 + 16 * ((2 * q + g) ^ pj_key(rr))));
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 32 * tt + r;
        if constexpr (kF32) {
          const uint8_t* xb = st + kPjA + t * 256;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(xb + 16 * ((4 * q + 2 * g) ^ (t & 15)));
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(xb + 16 * ((4 * q + 2 * g + 1) ^ (t & 15)));
          bv[tt] = __builtin_bit_cast(bf16x8, u32x4{cvt_pk_bf16(x0[0], x0[1]), cvt_pk_bf16(x0[2], x0[3]),
                                                   cvt_pk_bf16(x1[0], x1[1]), cvt_pk_bf16(x1[2], x1[3])});
        } else {
          bv[tt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + kPjA + t * 128 +
                                                                                16 * ((2 * q + g) ^ pj_key(t))));
        }
      }
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[0], bv[0], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[0], bv[1], acc[1], 0, 0, 0);
      acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[1], bv[0], acc[2], 0, 0, 0);
      acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[1], bv[1], acc[3], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(pj_waitcnt_vm(0));   // no load may land after the workgroup ends
  // acc[2 nt + tt][i] = Y^T[n = n_base + 64w + 32 nt + 8(i/4) + 4g + i%4, t = t0 + 32 tt + r]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nt = i >> 1, tt = i & 1;
    const int t = t0 + 32 * tt + r;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int n = n_base + 64 * wave + 32 * nt + 8 * (e >> 2) + 4 * g + (e & 3);
      if (n < N && t < T) {
        if (S > 1) part[((size_t)s * T + t) * N + n] = acc[i][e];
        else pj_store<uint16_t>(P.o, t, n, acc[i][e]);
      }
    }
  }
}

// Y = sum over the S slices of part[s][t][n], in slice order, written through `o`, for every
// GEMM of the job with S > 1 (their elements one after the other).
template <typename XT>
__global__ void __launch_bounds__(256) rows_reduce_kernel(PjJob<XT> job) {
  for (int p = 0; p < job.np; ++p) {   // uniform: each GEMM's fields stay scalar
    const PjGemm<XT> P = p == 0 ? job.g[0] : job.g[1];
    if (P.S <= 1) continue;
    const size_t total = (size_t)P.T * P.N;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
      float v = 0.f;
      for (int s = 0; s < P.S; ++s) v += P.part[(size_t)s * total + e];
      pj_store<uint16_t>(P.o, (int)(e / P.N), (int)(e % P.N), v);
    }
  }
}

// Generic (fp32 or bf16, any K): one thread per output element, fp32 accumulation.
template <typename XT, typename WT, typename OutT>
__global__ void __launch_bounds__(256) rows_gemm_generic_kernel(const XT* __restrict__ X, long long ldx,
                                                                const WT* __restrict__ Wt, int T, int N, int K,
                                                                PjOut o) {
  const size_t total = (size_t)T * N;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int t = (int)(e / N), n = (int)(e % N);
    float acc = 0.f;
#pragma unroll 8   // several iterations' loads in flight at once (the sum keeps its order)
    for (int k = 0; k < K; ++k) acc += load_act(X, (size_t)t * ldx + k) * load_act(Wt, (size_t)n * K + k);
    pj_store<OutT>(o, t, n, acc);
  }
}

// Slices of the contraction for the row GEMMs of one launch (one S for all of them).  One
// workgroup fits a compute unit (its LDS), so the launch runs in rounds of num_cus workgroups: S
// minimises the modelled time, rounds x (chunks per slice + 3 chunks of pipeline fill) chunk loads
// per compute unit, plus the fp32 partials written and read back once (S x T x N x 8 bytes, spread
// over the whole chip).  Each slice keeps at least four chunks.
struct PjShape {
  int T, N, K;
};
int rows_gemm_slices(int num_cus, const PjShape* sh, int np) {
  long long groups = 0, outputs = 0;
  int chunks = 0;
  for (int i = 0; i < np; ++i) {
    groups += (long long)((sh[i].N + kPjGroup - 1) / kPjGroup) * ((sh[i].T + kPjT - 1) / kPjT);
    outputs += (long long)sh[i].T * sh[i].N;
    if (sh[i].K / kPjChunk > chunks) chunks = sh[i].K / kPjChunk;
  }
  if (groups <= 0 || num_cus <= 0) return 1;   // nothing to compute
  int min_chunks = chunks;
  for (int i = 0; i < np; ++i)
    if (sh[i].K / kPjChunk < min_chunks) min_chunks = sh[i].K / kPjChunk;
  const long long S_max = min_chunks / 4 > 0 ? min_chunks / 4 : 1;
  const double chunk_bytes = (double)(kPjA + kPjT * kPjChunk * 2);
  long long best_S = 1;
  double best = -1.0;
  for (long long S = 1; S <= S_max; ++S) {
    const long long rounds = (groups * S + num_cus - 1) / num_cus;
    const long long per = (chunks + S - 1) / S;
    const double cost = (double)rounds * (double)(per + 3) * chunk_bytes * num_cus +
                        (S > 1 ? (double)S * outputs * 8.0 : 0.0);
    if (best < 0.0 || cost < best) { best = cost; best_S = S; }
  }
  return (int)best_S;
}

// Partials of the GEMMs of one launch, each in its own 256-byte aligned block.
size_t rows_gemm_workspace(int num_cus, const PjShape* sh, int np) {
  const int S = rows_gemm_slices(num_cus, sh, np);
  if (S <= 1) return 0;
  size_t ws = 0;
  for (int i = 0; i < np; ++i) ws += (((size_t)S * sh[i].T * sh[i].N * sizeof(float)) + 255) & ~(size_t)255;
  return ws;
}

// The row GEMM takes more LDS than the default dynamic limit, raised once per device (an atomic
// mark per device; racing threads repeat the same idempotent calls).
constexpr int kPjMaxDev = 64;
std::atomic<int> g_pj_lds_set[kPjMaxDev];

hipError_t set_rows_gemm_lds_limits() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<int>* mark = (dev >= 0 && dev < kPjMaxDev) ? &g_pj_lds_set[dev] : nullptr;
  if (mark && mark->load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)rows_gemm_kernel<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          3 * pj_stage_bytes<uint16_t>());
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)rows_gemm_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          3 * pj_stage_bytes<float>());
  if (e != hipSuccess) return e;
  if (mark) mark->store(1, std::memory_order_release);
  return hipSuccess;
}

template <typename XT, typename WT, typename OutT>
hipError_t launch_rows_gemm_generic(const XT* X, long long ldx, const WT* Wt, int T, int N, int K, const PjOut& o,
                                    hipStream_t stream);

// The MFMA kernel addresses one workgroup's weight rows and X rows with 32-bit buffer offsets.
template <typename XT>
bool rows_gemm_offsets_fit(long long ldx, int K) {
  return (long long)kPjGroup * K * 2 < (1ll << 31) && (long long)kPjT * ldx * (long long)sizeof(XT) < (1ll << 31);
}

// One row GEMM's operands: Y = X . Wt^T through `o` (X [T, K] with row stride ldx, Wt [N, K] bf16).
template <typename XT>
struct PjArgs {
  const XT* X;
  long long ldx;
  const uint16_t* Wt;
  int T, N, K;
  PjOut o;
};

// The row GEMMs in `a` (one or two, K % 64 == 0, every T > 0), bf16 MFMA path, in one launch
// (plus one launch adding the slices' partials when S > 1).
template <typename XT>
hipError_t launch_rows_gemm(int num_cus, const PjArgs<XT>* a, int np, void* workspace, hipStream_t stream) {
  for (int i = 0; i < np; ++i)
    if (!rows_gemm_offsets_fit<XT>(a[i].ldx, a[i].K)) {   // too large for 32-bit buffer offsets
      for (int j = 0; j < np; ++j) {
        const hipError_t e =
            launch_rows_gemm_generic<XT, uint16_t, uint16_t>(a[j].X, a[j].ldx, a[j].Wt, a[j].T, a[j].N, a[j].K, a[j].o,
                                                             stream);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  PjShape sh[2];
  for (int i = 0; i < np; ++i) sh[i] = PjShape{a[i].T, a[i].N, a[i].K};
  const int S = rows_gemm_slices(num_cus, sh, np);
  PjJob<XT> job{};
  job.np = np;
  int wgs = 0;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  for (int i = 0; i < np; ++i) {
    const int groups_n = (a[i].N + kPjGroup - 1) / kPjGroup;
    job.g[i] = PjGemm<XT>{a[i].X, a[i].ldx, a[i].Wt, a[i].o, S > 1 ? reinterpret_cast<float*>(ws) : nullptr,
                          a[i].T, a[i].N, a[i].K, S, groups_n, wgs};
    wgs += groups_n * S * ((a[i].T + kPjT - 1) / kPjT);
    if (S > 1) ws += (((size_t)S * a[i].T * a[i].N * sizeof(float)) + 255) & ~(size_t)255;
  }
  hipError_t e0 = set_rows_gemm_lds_limits();
  if (e0 != hipSuccess) return e0;
  hipLaunchKernelGGL(rows_gemm_kernel<XT>, dim3(wgs), dim3(256), 3 * pj_stage_bytes<XT>(), stream, job);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  size_t total = 0;
  for (int i = 0; i < np; ++i) total += (size_t)a[i].T * a[i].N;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(rows_reduce_kernel<XT>, dim3(blocks), dim3(256), 0, stream, job);
  return hipGetLastError();
}

template <typename XT, typename WT, typename OutT>
hipError_t launch_rows_gemm_generic(const XT* X, long long ldx, const WT* Wt, int T, int N, int K, const PjOut& o,
                                    hipStream_t stream) {
  const size_t total = (size_t)T * N;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  hipLaunchKernelGGL((rows_gemm_generic_kernel<XT, WT, OutT>), dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     X, ldx, Wt, T, N, K, o);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fold of W_UV into W_O

// W_O'^T[n, i*d_c + c] = sum_v W_UV[c, i*d_v + v] W_O[i*d_v + v, n]: one thread per element, fp32
// sums of the products, one rounding to the output format.  Weight preparation, run once.
template <typename T>
__global__ void __launch_bounds__(256) fold_wo_kernel(const T* __restrict__ w_uv, const T* __restrict__ w_o,
                                                      T* __restrict__ w_fold_t, int H, int d_c, int d_v,
                                                      int d_model) {
  const size_t total = (size_t)d_model * H * d_c;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int c = (int)(e % d_c);
    const size_t rest = e / d_c;
    const int i = (int)(rest % H);
    const int n = (int)(rest / H);
    float acc = 0.f;
#pragma unroll 8   // several iterations' loads in flight at once (the sum keeps its order)
    for (int v = 0; v < d_v; ++v)
      acc += load_act(w_uv, (size_t)c * H * d_v + (size_t)i * d_v + v) * load_act(w_o, ((size_t)i * d_v + v) * d_model + n);
    if constexpr (sizeof(T) == 4) w_fold_t[e] = acc;
    else w_fold_t[e] = (T)f32_to_bf16_bits(acc);
  }
}

// ------------------------------------------------------------------ launchers (host)

bool is_dsv2_shape(const mla_config_t& c);

// The upstream projections of one step: latent rows (c, k_R raw) of the n new tokens into
// kv_c [n, d_c] / kv_r [n, d_R], and the queries of the T query rows into q_nope [T, H*d_h] /
// q_rope [T, H*d_R], all in the activation format.
hipError_t launch_project_hidden(const mla_config_t& cfg, int num_cus, int d_model, const void* h_kv,
                                 const void* w_dkv_t, int n, const void* h_q, const void* w_q_t, int T, void* kv_c,
                                 void* kv_r, void* q_nope, void* q_rope, void* gemm_ws, hipStream_t stream) {
  const int H = cfg.num_heads, d_c = cfg.d_c, d_r = cfg.d_r, d_h = cfg.d_h;
  const PjOut okv{kv_c, kv_r, d_c, d_r, d_c};
  const PjOut oq{q_nope, q_rope, (long long)H * d_h, (long long)H * d_r, H * d_h};
  const int Nkv = d_c + d_r, Nq = H * (d_h + d_r);
  hipError_t e = hipSuccess;
  if (cfg.act_dtype == MLA_BF16 && d_model % kPjChunk == 0) {
    // both projections in one launch
    PjArgs<uint16_t> a[2];
    int np = 0;
    if (n > 0)
      a[np++] = PjArgs<uint16_t>{static_cast<const uint16_t*>(h_kv), d_model, static_cast<const uint16_t*>(w_dkv_t), n,
                                 Nkv, d_model, okv};
    if (T > 0)
      a[np++] = PjArgs<uint16_t>{static_cast<const uint16_t*>(h_q), d_model, static_cast<const uint16_t*>(w_q_t), T,
                                 Nq, d_model, oq};
    return np > 0 ? launch_rows_gemm(num_cus, a, np, gemm_ws, stream) : hipSuccess;
  }
  if (cfg.act_dtype == MLA_BF16) {
    if (n > 0)
      e = launch_rows_gemm_generic<uint16_t, uint16_t, uint16_t>(static_cast<const uint16_t*>(h_kv), d_model,
                                                                static_cast<const uint16_t*>(w_dkv_t), n, Nkv,
                                                                d_model, okv, stream);
    if (e == hipSuccess && T > 0)
      e = launch_rows_gemm_generic<uint16_t, uint16_t, uint16_t>(static_cast<const uint16_t*>(h_q), d_model,
                                                                static_cast<const uint16_t*>(w_q_t), T, Nq, d_model,
                                                                oq, stream);
    return e;
  }
  if (n > 0)
    e = launch_rows_gemm_generic<float, float, float>(static_cast<const float*>(h_kv), d_model,
                                                      static_cast<const float*>(w_dkv_t), n, Nkv, d_model, okv,
                                                      stream);
  if (e == hipSuccess && T > 0)
    e = launch_rows_gemm_generic<float, float, float>(static_cast<const float*>(h_q), d_model,
                                                      static_cast<const float*>(w_q_t), T, Nq, d_model, oq, stream);
  return e;
}

// Workspace of launch_project_hidden: the two projections' outputs plus the GEMM partials.
size_t project_hidden_workspace(const mla_config_t& cfg, int num_cus, int d_model, int n, int T) {
  const size_t el = cfg.act_dtype == MLA_F32 ? 4 : 2;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  size_t ws = al((size_t)n * cfg.d_c * el) + al((size_t)n * cfg.d_r * el) +
              al((size_t)T * cfg.num_heads * cfg.d_h * el) + al((size_t)T * cfg.num_heads * cfg.d_r * el);
  if (cfg.act_dtype == MLA_BF16 && d_model % kPjChunk == 0) {
    PjShape sh[2];
    int np = 0;
    if (n > 0) sh[np++] = PjShape{n, cfg.d_c + cfg.d_r, d_model};
    if (T > 0) sh[np++] = PjShape{T, cfg.num_heads * (cfg.d_h + cfg.d_r), d_model};
    ws += rows_gemm_workspace(num_cus, sh, np);
  }
  return ws;
}

// out [T, d_model] = o_lat [T, H*d_c] . W_O'  (W_O' given transposed: w_fold_t [d_model, H*d_c]).
hipError_t launch_out_proj_folded(const mla_config_t& cfg, int num_cus, int d_model, const float* o_lat,
                                  const void* w_fold_t, void* out, int T, void* workspace, hipStream_t stream) {
  const int K = cfg.num_heads * cfg.d_c;
  const PjOut o{out, out, d_model, d_model, d_model};
  if (cfg.act_dtype == MLA_BF16 && K % kPjChunk == 0) {
    const PjArgs<float> a{o_lat, (long long)K, static_cast<const uint16_t*>(w_fold_t), T, d_model, K, o};
    return T > 0 ? launch_rows_gemm(num_cus, &a, 1, workspace, stream) : hipSuccess;
  }
  if (cfg.act_dtype == MLA_BF16)
    return launch_rows_gemm_generic<float, uint16_t, uint16_t>(o_lat, K, static_cast<const uint16_t*>(w_fold_t), T,
                                                               d_model, K, o, stream);
  return launch_rows_gemm_generic<float, float, float>(o_lat, K, static_cast<const float*>(w_fold_t), T, d_model, K,
                                                       o, stream);
}

size_t out_proj_folded_workspace(const mla_config_t& cfg, int num_cus, int d_model, int T) {
  const int K = cfg.num_heads * cfg.d_c;
  if (cfg.act_dtype == MLA_BF16 && K % kPjChunk == 0) {
    const PjShape sh{T, d_model, K};
    return rows_gemm_workspace(num_cus, &sh, 1);
  }
  return 0;
}

hipError_t launch_fold_wo(const mla_config_t& cfg, int d_model, const void* w_uv, const void* w_o, void* w_fold_t,
                          hipStream_t stream) {
  const size_t total = (size_t)d_model * cfg.num_heads * cfg.d_c;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (cfg.act_dtype == MLA_F32)
    hipLaunchKernelGGL(fold_wo_kernel<float>, dim3(blocks), dim3(256), 0, stream, static_cast<const float*>(w_uv),
                       static_cast<const float*>(w_o), static_cast<float*>(w_fold_t), cfg.num_heads, cfg.d_c, cfg.d_v,
                       d_model);
  else
    hipLaunchKernelGGL(fold_wo_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w_uv), static_cast<const uint16_t*>(w_o),
                       static_cast<uint16_t*>(w_fold_t), cfg.num_heads, cfg.d_c, cfg.d_v, d_model);
  return hipGetLastError();
}

}  // namespace mla
