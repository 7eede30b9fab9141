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
bool is_dsv2_shape(const mla_config_t&);
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


// Shape and format checks shared by every call.
mla_status_t check_cfg(const mla_config_t* c) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->num_heads <= 0 || c->d_c <= 0 || c->d_r <= 0 || c->d_h <= 0 || c->d_v <= 0) return MLA_ERR_INVALID_ARG;
  if (c->d_c % 16 || c->d_r % 16 || c->d_h % 16 || c->d_v % 16) return MLA_ERR_INVALID_ARG;
  if (c->block_size != 64) return MLA_ERR_INVALID_ARG;
  if (!(c->softmax_scale > 0.0f) || !(c->rope_base > 0.0f)) return MLA_ERR_INVALID_ARG;
  const bool f32 = c->cache_dtype == MLA_F32 && c->act_dtype == MLA_F32;
  const bool bf16 = c->cache_dtype == MLA_BF16 && c->act_dtype == MLA_BF16;
  const bool fp8 = c->cache_dtype == MLA_FP8_E4M3 && c->act_dtype == MLA_BF16;
  if (c->cache_dtype < 0 || c->cache_dtype > 2 || c->act_dtype < 0 || c->act_dtype > 1) return MLA_ERR_INVALID_ARG;
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

int32_t mla_abi_version(void) { return 3; }

const char* mla_status_string(mla_status_t s) {
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
  if (n < 0 || num_blocks <= 0 || batch <= 0 || max_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (!cache || !block_table) return MLA_ERR_INVALID_ARG;
  if (n > 0 && (!c_kv || !k_r || !pos || !seq_of)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(cache) || (n > 0 && (!aligned16(c_kv) || !aligned16(k_r)))) return MLA_ERR_INVALID_ARG;
  const bool fp8 = cfg->cache_dtype == MLA_FP8_E4M3;
  if (fp8 != (cache_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

static mla_status_t check_absorb(const mla_config_t* cfg, const void* q_nope, const void* q_rope,
                                 const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t T) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (T < 0) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!q_nope || !q_rope || !q_pos || !w_uk || !q_abs) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(q_abs)) return MLA_ERR_INVALID_ARG;
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
  if (check_cfg(cfg) != MLA_OK || B <= 0 || Sq <= 0 || max_blocks <= 0) return 0;
  return mla::decode_workspace_bytes(*cfg, current_cu_count(), B, Sq, max_blocks);
}

static mla_status_t decode_common(const mla_config_t* cfg, const void* q_abs, const void* cache, const float* cache_scale, int32_t num_blocks,
                                  const int32_t* block_table, int32_t max_blocks, const int32_t* kv_lens, int32_t B,
                                  int32_t Sq, void* workspace, size_t ws_bytes, float* o_lat, float* lse,
                                  void* stream, int phases) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (B < 0 || Sq <= 0 || num_blocks <= 0 || max_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if ((long long)B * Sq > (1LL << 30)) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!q_abs || !cache || !block_table || !kv_lens || !o_lat || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_abs) || !aligned16(cache) || !aligned16(o_lat)) return MLA_ERR_INVALID_ARG;
  const bool fp8 = cfg->cache_dtype == MLA_FP8_E4M3;
  if (fp8 != (cache_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  const int cus = current_cu_count();
  const size_t need = mla::decode_workspace_bytes(*cfg, cus, B, Sq, max_blocks);
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

mla_status_t mla_out_proj(const mla_config_t* cfg, const float* o_lat, const void* w_uv, void* out, int32_t T,
                          void* stream) {
  mla_status_t st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (T < 0) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  return from_hip(mla::launch_out_proj(*cfg, o_lat, w_uv, out, T, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
