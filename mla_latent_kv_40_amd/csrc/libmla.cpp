// libmla host side: argument validation and kernel dispatch for the C ABI in include/mla.h.
// Every entry point validates before it touches the HIP runtime, so argument errors are
// reported (and testable) on machines without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/mla.h"

namespace mla {
hipError_t launch_append(const mla_config_t&, void*, float*, int, const void*, const void*, const int32_t*,
                         const int32_t*, const int32_t*, int, int, int, hipStream_t);
hipError_t launch_absorb_q(const mla_config_t&, const void*, const void*, const int32_t*, const void*, void*, int,
                           hipStream_t);
hipError_t launch_append_absorb(const mla_config_t&, void*, float*, int, const void*, const void*, const int32_t*,
                                const int32_t*, const int32_t*, int, int, int, const void*, const void*,
                                const int32_t*, const void*, void*, int, hipStream_t);
hipError_t launch_out_proj(const mla_config_t&, const float*, const void*, void*, int, hipStream_t);
hipError_t launch_decode(const mla_config_t&, int, const void*, const void*, const float*, int,
                         const int32_t*, int, const int32_t*, int, int, void*, float*, float*, hipStream_t,
                         int phases);
size_t decode_workspace_bytes(const mla_config_t&, int, int, int, int);
size_t static_scratch_bytes();
hipError_t static_scratch(void** out);
bool is_dsv2_shape(const mla_config_t&);
hipError_t launch_project_hidden(const mla_config_t&, int, int, const void*, const void*, int, const void*,
                                 const void*, int, void*, void*, void*, void*, void*, hipStream_t);
size_t project_hidden_workspace(const mla_config_t&, int, int, int, int);
hipError_t launch_out_proj_folded(const mla_config_t&, int, int, const float*, const void*, void*, int, void*,
                                  hipStream_t);
size_t out_proj_folded_workspace(const mla_config_t&, int, int, int);
hipError_t launch_fold_wo(const mla_config_t&, int, const void*, const void*, void*, hipStream_t);
size_t gqa_workspace_bytes(int B, int H_q, int H_kv, int max_blocks);
bool gqa_supported(int H_q, int H_kv, int d);
hipError_t launch_gqa_decode(int H_q, int H_kv, float softmax_scale, const void* q, const void* k, const void* v,
                             int num_blocks, const int32_t* block_table, int max_blocks, const int32_t* kv_lens,
                             int B, void* workspace, float* o, float* lse, hipStream_t stream);
}  // namespace mla

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not yet queried

// Compute units of the current device (cached per device); 256 if it cannot be queried.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Size limits checked before anything is launched.  Within them every row, token-slot and page
// index fits the kernels' 32-bit arithmetic and every launch keeps far below the 2^32
// work-items one grid dimension can hold.
constexpr int32_t kMaxRows = 1 << 20;    // query rows (B*Sq, T), appended tokens, batch entries
constexpr int32_t kMaxPages = 1 << 24;   // pages in the pool, and in one block-table row
constexpr long long kMaxKvPairs = 1LL << 24;   // (sequence, query head) pairs of a per-head decode

bool rows_ok(long long r) { return r >= 0 && r <= kMaxRows; }
bool pages_ok(int32_t p) { return p > 0 && p <= kMaxPages; }


// Shape and format checks shared by every call.
mla_status_t check_cfg(const mla_config_t* c) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->num_heads <= 0 || c->d_c <= 0 || c->d_r <= 0 || c->d_h <= 0 || c->d_v <= 0) return MLA_ERR_INVALID_ARG;
  if (c->d_c % 16 || c->d_r % 16 || c->d_h % 16 || c->d_v % 16) return MLA_ERR_INVALID_ARG;
  if (c->block_size != 64) return MLA_ERR_INVALID_ARG;
  if (!(c->softmax_scale > 0.0f) || !(c->rope_base > 0.0f)) return MLA_ERR_INVALID_ARG;
  const bool f32 = c->cache_dtype == MLA_F32 && c->act_dtype == MLA_F32;
  const bool bf16 = c->cache_dtype == MLA_BF16 && c->act_dtype == MLA_BF16;
  const bool fp8 = (c->cache_dtype == MLA_FP8_E4M3 || c->cache_dtype == MLA_FP8_E4M3_B32) && c->act_dtype == MLA_BF16;
  if (c->cache_dtype < 0 || c->cache_dtype > 3 || c->act_dtype < 0 || c->act_dtype > 1) return MLA_ERR_INVALID_ARG;
  if (!(f32 || bf16 || fp8)) return MLA_ERR_UNSUPPORTED;
  if (fp8 && !mla::is_dsv2_shape(*c)) return MLA_ERR_UNSUPPORTED;
  if (!mla::is_dsv2_shape(*c)) {
    if (c->num_heads > 128 || c->d_c + c->d_r > 1024 || c->d_h > 256 || c->d_v > 256) return MLA_ERR_UNSUPPORTED;
  }
  return MLA_OK;
}

mla_status_t from_hip(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return 8; }

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: format or shape not supported";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
  }
  return "MLA_ERR_UNKNOWN";
}

static mla_status_t check_append(const mla_config_t* cfg, void* cache, float* cache_scale, int32_t num_blocks,
                                 const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* seq_of,
                                 const int32_t* block_table, int32_t batch, int32_t max_blocks, int32_t n) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (!rows_ok(n) || !pages_ok(num_blocks) || batch <= 0 || !rows_ok(batch) || !pages_ok(max_blocks))
    return MLA_ERR_INVALID_ARG;
  if (!cache || !block_table) return MLA_ERR_INVALID_ARG;
  if (n > 0 && (!c_kv || !k_r || !pos || !seq_of)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(cache) || !aligned16(block_table)) return MLA_ERR_INVALID_ARG;
  if (n > 0 && (!aligned16(c_kv) || !aligned16(k_r) || !aligned16(pos) || !aligned16(seq_of)))
    return MLA_ERR_INVALID_ARG;
  const bool fp8 = cfg->cache_dtype == MLA_FP8_E4M3 || cfg->cache_dtype == MLA_FP8_E4M3_B32;
  if (fp8 != (cache_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (cache_scale && !aligned16(cache_scale)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

static mla_status_t check_absorb(const mla_config_t* cfg, const void* q_nope, const void* q_rope,
                                 const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t T) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (!rows_ok(T)) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!q_nope || !q_rope || !q_pos || !w_uk || !q_abs) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(q_pos) || !aligned16(w_uk) || !aligned16(q_abs))
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status_t mla_cache_append(const mla_config_t* cfg, void* cache, float* cache_scale, int32_t num_blocks,
                              const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* seq_of,
                              const int32_t* block_table, int32_t batch, int32_t max_blocks, int32_t n,
                              void* stream) {
  mla_status_t st = check_append(cfg, cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table, batch,
                                 max_blocks, n);
  if (st != MLA_OK) return st;
  if (n == 0) return MLA_OK;
  return from_hip(mla::launch_append(*cfg, cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table,
                                     batch, max_blocks, n, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_absorb_q(const mla_config_t* cfg, const void* q_nope, const void* q_rope, const int32_t* q_pos,
                          const void* w_uk, void* q_abs, int32_t T, void* stream) {
  mla_status_t st = check_absorb(cfg, q_nope, q_rope, q_pos, w_uk, q_abs, T);
  if (st != MLA_OK) return st;
  if (T == 0) return MLA_OK;
  return from_hip(mla::launch_absorb_q(*cfg, q_nope, q_rope, q_pos, w_uk, q_abs, T,
                                       static_cast<hipStream_t>(stream)));
}

mla_status_t mla_append_absorb(const mla_config_t* cfg, void* cache, float* cache_scale, int32_t num_blocks,
                               const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* seq_of,
                               const int32_t* block_table, int32_t batch, int32_t max_blocks, int32_t n,
                               const void* q_nope, const void* q_rope, const int32_t* q_pos, const void* w_uk,
                               void* q_abs, int32_t T, void* stream) {
  mla_status_t st = check_append(cfg, cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table, batch,
                                 max_blocks, n);
  if (st != MLA_OK) return st;
  st = check_absorb(cfg, q_nope, q_rope, q_pos, w_uk, q_abs, T);
  if (st != MLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n == 0 && T == 0) return MLA_OK;
  if (T == 0)
    return from_hip(mla::launch_append(*cfg, cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of, block_table,
                                       batch, max_blocks, n, s));
  if (n == 0) return from_hip(mla::launch_absorb_q(*cfg, q_nope, q_rope, q_pos, w_uk, q_abs, T, s));
  return from_hip(mla::launch_append_absorb(*cfg, cache, cache_scale, num_blocks, c_kv, k_r, pos, seq_of,
                                            block_table, batch, max_blocks, n, q_nope, q_rope, q_pos, w_uk, q_abs,
                                            T, s));
}

size_t mla_decode_workspace_size(const mla_config_t* cfg, int32_t B, int32_t Sq, int32_t max_blocks) {
  if (check_cfg(cfg) != MLA_OK || B <= 0 || Sq <= 0 || !rows_ok((long long)B * Sq) || !pages_ok(max_blocks))
    return 0;
  return mla::decode_workspace_bytes(*cfg, current_cu_count(), B, Sq, max_blocks);
}

// use_static: the partials go to the library's fixed device scratch (workspace arguments unused)
static mla_status_t decode_common(const mla_config_t* cfg, const void* q_abs, const void* cache, const float* cache_scale, int32_t num_blocks,
                                  const int32_t* block_table, int32_t max_blocks, const int32_t* kv_lens, int32_t B,
                                  int32_t Sq, void* workspace, size_t ws_bytes, float* o_lat, float* lse,
                                  void* stream, int phases, bool use_static = false) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (B < 0 || Sq <= 0 || !rows_ok((long long)B * Sq) || !pages_ok(num_blocks) || !pages_ok(max_blocks))
    return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!q_abs || !cache || !block_table || !kv_lens || !o_lat || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_abs) || !aligned16(cache) || !aligned16(o_lat) || !aligned16(lse) || !aligned16(kv_lens) ||
      !aligned16(block_table))
    return MLA_ERR_INVALID_ARG;
  const bool fp8 = cfg->cache_dtype == MLA_FP8_E4M3 || cfg->cache_dtype == MLA_FP8_E4M3_B32;
  if (fp8 != (cache_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (cache_scale && !aligned16(cache_scale)) return MLA_ERR_INVALID_ARG;
  const int cus = current_cu_count();
  const size_t need = mla::decode_workspace_bytes(*cfg, cus, B, Sq, max_blocks);
  if (need == 0) return MLA_ERR_UNSUPPORTED;   // the split plan needs too many workgroups
  if (use_static) {   // mla_decode_attn_noalloc
    if (need > mla::static_scratch_bytes()) return MLA_ERR_WORKSPACE;
    if (mla::static_scratch(&workspace) != hipSuccess) return MLA_ERR_HIP;
    ws_bytes = mla::static_scratch_bytes();
  }
  if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MLA_ERR_WORKSPACE;
  return from_hip(mla::launch_decode(*cfg, cus, q_abs, cache, cache_scale, num_blocks, block_table,
                                     max_blocks, kv_lens, B, Sq, workspace, o_lat, lse,
                                     static_cast<hipStream_t>(stream), phases));
}

mla_status_t mla_decode_attn(const mla_config_t* cfg, const void* q_abs, const void* cache,
                             const float* cache_scale, int32_t num_blocks, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* kv_lens, int32_t B, int32_t Sq, void* workspace,
                             size_t ws_bytes, float* o_lat, float* lse, void* stream) {
  return decode_common(cfg, q_abs, cache, cache_scale, num_blocks, block_table, max_blocks, kv_lens, B, Sq,
                       workspace, ws_bytes, o_lat, lse, stream, 3);
}

mla_status_t mla_decode_split(const mla_config_t* cfg, const void* q_abs, const void* cache,
                              const float* cache_scale, int32_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* kv_lens, int32_t B, int32_t Sq, void* workspace,
                              size_t ws_bytes, float* o_lat, float* lse, void* stream) {
  return decode_common(cfg, q_abs, cache, cache_scale, num_blocks, block_table, max_blocks, kv_lens, B, Sq,
                       workspace, ws_bytes, o_lat, lse, stream, 1);
}

mla_status_t mla_decode_combine(const mla_config_t* cfg, const void* q_abs, const void* cache,
                                const float* cache_scale, int32_t num_blocks, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* kv_lens, int32_t B, int32_t Sq, void* workspace,
                                size_t ws_bytes, float* o_lat, float* lse, void* stream) {
  return decode_common(cfg, q_abs, cache, cache_scale, num_blocks, block_table, max_blocks, kv_lens, B, Sq,
                       workspace, ws_bytes, o_lat, lse, stream, 2);
}

mla_status_t mla_decode_attn_noalloc(const mla_config_t* cfg, const void* q_abs, const void* cache,
                                     const float* cache_scale, int32_t num_blocks, const int32_t* block_table,
                                     int32_t max_blocks, const int32_t* kv_lens, int32_t B, int32_t Sq,
                                     float* o_lat, float* lse, void* stream) {
  return decode_common(cfg, q_abs, cache, cache_scale, num_blocks, block_table, max_blocks, kv_lens, B, Sq,
                       nullptr, 0, o_lat, lse, stream, 3, true);
}

// ---------------------------------------------------------------- from and to the model width

static bool d_model_ok(int32_t d_model) { return d_model > 0 && d_model % 16 == 0 && d_model <= (1 << 20); }

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t mla_hidden_workspace_size(const mla_config_t* cfg, int32_t d_model, int32_t n, int32_t T) {
  if (check_cfg(cfg) != MLA_OK || !d_model_ok(d_model) || !rows_ok(n) || !rows_ok(T)) return 0;
  return mla::project_hidden_workspace(*cfg, current_cu_count(), d_model, n, T) + 256;
}

mla_status_t mla_append_absorb_hidden(const mla_config_t* cfg, int32_t d_model, const void* h_kv,
                                      const void* w_dkv_t, void* cache, float* cache_scale, int32_t num_blocks,
                                      const int32_t* pos, const int32_t* seq_of, const int32_t* block_table,
                                      int32_t batch, int32_t max_blocks, int32_t n, const void* h_q,
                                      const void* w_q_t, const int32_t* q_pos, const void* w_uk, void* q_abs,
                                      int32_t T, void* workspace, size_t ws_bytes, void* stream) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (!d_model_ok(d_model) || !rows_ok(n) || !rows_ok(T)) return MLA_ERR_INVALID_ARG;
  if (n > 0 && (!h_kv || !w_dkv_t || !aligned16(h_kv) || !aligned16(w_dkv_t))) return MLA_ERR_INVALID_ARG;
  if (T > 0 && (!h_q || !w_q_t || !aligned16(h_q) || !aligned16(w_q_t))) return MLA_ERR_INVALID_ARG;
  if (n == 0 && T == 0) return MLA_OK;
  const int cus = current_cu_count();
  const size_t need = mla::project_hidden_workspace(*cfg, cus, d_model, n, T);
  if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MLA_ERR_WORKSPACE;
  // the projections' outputs, laid out as mla_cache_append and mla_absorb_q take them
  const size_t el = cfg->act_dtype == MLA_F32 ? 4 : 2;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  void* kv_c = w;
  w += align256((size_t)n * cfg->d_c * el);
  void* kv_r = w;
  w += align256((size_t)n * cfg->d_r * el);
  void* q_nope = w;
  w += align256((size_t)T * cfg->num_heads * cfg->d_h * el);
  void* q_rope = w;
  w += align256((size_t)T * cfg->num_heads * cfg->d_r * el);
  // validate the append and absorption halves (as mla_append_absorb will) with the arrays they
  // will receive, before anything is launched
  st = check_append(cfg, cache, cache_scale, num_blocks, kv_c, kv_r, pos, seq_of, block_table, batch, max_blocks, n);
  if (st != MLA_OK) return st;
  st = check_absorb(cfg, q_nope, q_rope, q_pos, w_uk, q_abs, T);
  if (st != MLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mla::launch_project_hidden(*cfg, cus, d_model, h_kv, w_dkv_t, n, h_q, w_q_t, T, kv_c, kv_r, q_nope,
                                            q_rope, w, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return mla_append_absorb(cfg, cache, cache_scale, num_blocks, kv_c, kv_r, pos, seq_of, block_table, batch,
                           max_blocks, n, q_nope, q_rope, q_pos, w_uk, q_abs, T, stream);
}

mla_status_t mla_fold_output_weights(const mla_config_t* cfg, int32_t d_model, const void* w_uv, const void* w_o,
                                     void* w_fold_t, void* stream) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (!d_model_ok(d_model)) return MLA_ERR_INVALID_ARG;
  if (!w_uv || !w_o || !w_fold_t || !aligned16(w_uv) || !aligned16(w_o) || !aligned16(w_fold_t))
    return MLA_ERR_INVALID_ARG;
  return from_hip(mla::launch_fold_wo(*cfg, d_model, w_uv, w_o, w_fold_t, static_cast<hipStream_t>(stream)));
}

size_t mla_out_proj_folded_workspace_size(const mla_config_t* cfg, int32_t d_model, int32_t T) {
  if (check_cfg(cfg) != MLA_OK || !d_model_ok(d_model) || !rows_ok(T)) return 0;
  return mla::out_proj_folded_workspace(*cfg, current_cu_count(), d_model, T) + 256;
}

mla_status_t mla_out_proj_folded(const mla_config_t* cfg, int32_t d_model, const float* o_lat, const void* w_fold_t,
                                 void* out, int32_t T, void* workspace, size_t ws_bytes, void* stream) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (!d_model_ok(d_model) || !rows_ok(T)) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_fold_t || !out || !aligned16(o_lat) || !aligned16(w_fold_t) || !aligned16(out))
    return MLA_ERR_INVALID_ARG;
  const int cus = current_cu_count();
  const size_t need = mla::out_proj_folded_workspace(*cfg, cus, d_model, T);
  if (need > 0 && (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return MLA_ERR_WORKSPACE;
  return from_hip(mla::launch_out_proj_folded(*cfg, cus, d_model, o_lat, w_fold_t, out, T, workspace,
                                              static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- per-head key/value cache (comparison)

static mla_status_t check_kv_cfg(const mla_config_t* cfg, int32_t num_kv_heads) {
  if (!cfg) return MLA_ERR_INVALID_ARG;
  if (cfg->num_heads <= 0 || num_kv_heads <= 0 || cfg->d_h <= 0 || !(cfg->softmax_scale > 0.0f)) return MLA_ERR_INVALID_ARG;
  if (cfg->block_size != 64 || cfg->num_heads % num_kv_heads != 0) return MLA_ERR_INVALID_ARG;
  if (cfg->cache_dtype != MLA_BF16 || cfg->act_dtype != MLA_BF16 || cfg->d_v != cfg->d_h) return MLA_ERR_UNSUPPORTED;
  if (!mla::gqa_supported(cfg->num_heads, num_kv_heads, cfg->d_h)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

size_t mla_kv_decode_workspace_size(const mla_config_t* cfg, int32_t num_kv_heads, int32_t B, int32_t max_blocks) {
  if (check_kv_cfg(cfg, num_kv_heads) != MLA_OK || B <= 0 || !rows_ok(B) || !pages_ok(max_blocks)) return 0;
  if ((long long)B * cfg->num_heads > kMaxKvPairs) return 0;
  return mla::gqa_workspace_bytes(B, cfg->num_heads, num_kv_heads, max_blocks);
}

mla_status_t mla_kv_decode_attn(const mla_config_t* cfg, int32_t num_kv_heads, const void* q, const void* k_cache,
                                const void* v_cache, int32_t num_blocks, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* kv_lens, int32_t B, void* workspace,
                                size_t ws_bytes, float* o, float* lse, void* stream) {
  mla_status_t st = check_kv_cfg(cfg, num_kv_heads);
  if (st != MLA_OK) return st;
  if (!rows_ok(B) || !pages_ok(num_blocks) || !pages_ok(max_blocks)) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if ((long long)B * cfg->num_heads > kMaxKvPairs) return MLA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !block_table || !kv_lens || !o || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(block_table) || !aligned16(kv_lens) ||
      !aligned16(o) || !aligned16(lse))
    return MLA_ERR_INVALID_ARG;
  const size_t need = mla::gqa_workspace_bytes(B, cfg->num_heads, num_kv_heads, max_blocks);
  if (need == 0) return MLA_ERR_UNSUPPORTED;   // more work items than one launch takes
  if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MLA_ERR_WORKSPACE;
  return from_hip(mla::launch_gqa_decode(cfg->num_heads, num_kv_heads, cfg->softmax_scale, q, k_cache, v_cache,
                                         num_blocks, block_table, max_blocks, kv_lens, B, workspace, o, lse,
                                         static_cast<hipStream_t>(stream)));
}

mla_status_t mla_out_proj(const mla_config_t* cfg, const float* o_lat, const void* w_uv, void* out, int32_t T,
                          void* stream) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (!rows_ok(T)) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  return from_hip(mla::launch_out_proj(*cfg, o_lat, w_uv, out, T, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
