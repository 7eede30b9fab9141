/*
 * libmla -- Multi-head Latent Attention (MLA) decode over a paged latent cache, for AMD
 * Instinct MI355X (gfx950).  Plain C ABI: pointers and sizes only.
 *
 * The method (katajob interview page "What does Multi-head Latent Attention compress ...",
 * sections "The mechanism" and "Why it is not just extra work at decode time"; zenaique
 * "How does DeepSeek's Multi-Latent Attention (MLA) compress the KV cache below GQA?",
 * "What MLA caches versus what MHA and GQA cache"):
 *   - each token is cached only as a latent c_t (d_c values) plus a small positional key
 *     k_R,t (d_R values, RoPE applied) that is shared by all heads;
 *   - the per-head key up-projection W_UK is folded into the query, and the value
 *     up-projection W_UV is applied to the output once per query, so attention runs
 *     directly against the cached rows [c_t ; k_R,t] and per-head K and V never exist.
 *
 * One decode step is four calls on one stream:
 *   mla_cache_append  write the step's new tokens into the paged cache (RoPE on k_R here)
 *   mla_absorb_q      q_abs[t,i] = [ q^C_{t,i} W_UK,i^T ; RoPE(q^R_{t,i}, p_t) ]
 *   mla_decode_attn   o_lat[t,i] = sum_s softmax_s(scale * q_abs[t,i] . row_s) c_s,  lse[t,i]
 *   mla_out_proj      out[t,i]   = o_lat[t,i] W_UV,i
 *
 * Conventions shared by every call
 *   Vectors are rows and weights are stored [in, out] with head-major output columns, as
 *   in the katajob numpy snippet (keys = (latent @ W_up_k).reshape(seq, n_heads, d_head)):
 *   head i of W_UK owns columns i*d_h .. i*d_h+d_h-1.  All arrays are row-major, contiguous,
 *   device memory owned by the caller, 16-byte aligned.  Nothing is allocated or freed by
 *   the library.  Every call validates its arguments before touching the device: on error
 *   it returns a status and launches nothing.  Launches are asynchronous on `stream`
 *   (a hipStream_t; NULL is the default stream); a launch failure returns MLA_ERR_HIP.
 *   Calls on the same device may run from several host threads; calls that write the
 *   same buffers must be ordered by the caller (same stream or events).
 *
 * Size limits (MLA_ERR_INVALID_ARG beyond them; a workspace-size query returns 0)
 *   At most 2^20 query rows per call (B*Sq, T), 2^20 appended tokens (n) and batch entries,
 *   and 2^24 pages in the pool (num_blocks) or in a block-table row (max_blocks): a sequence
 *   holds up to 2^30 tokens.  A decode whose split plan would need more than 2^23 workgroups
 *   (very wide block tables) returns MLA_ERR_UNSUPPORTED and a workspace size of 0; so does a
 *   per-head cache decode past 2^24 (sequence, query head) pairs or 2^25 work items.
 *
 * Positions and the causal mask
 *   Sequence b holds kv_len[b] tokens at positions 0 .. kv_len[b]-1; token t lives at
 *   page block_table[b*max_blocks + t/64], slot t%64.  A step has Sq new query tokens per
 *   sequence (rows t = b*Sq + j of the query arrays, j = 0..Sq-1); query j sits at
 *   position p = kv_len[b] - Sq + j and attends to tokens 0..p.
 *
 * Number formats (mla_config_t.cache_dtype / act_dtype)
 *   F32 cache with F32 activations   any head shape within the generic limits below
 *   BF16 cache with BF16 activations DeepSeek-V2 shape (H=128, d_h=128, d_R=64, d_c=512,
 *                                    d_v=128) on matrix cores; other shapes on the generic path
 *   FP8_E4M3 cache with BF16 activ.  DeepSeek-V2 shape only.  Each cached row (all d_c+d_R
 *                                    values of a token) is stored as OCP e4m3fn codes with
 *                                    one fp32 scale = amax(row)/448 (1.0 for a zero row);
 *                                    value = code * scale.  Queries, weights and outputs
 *                                    stay bf16.
 *   Generic limits: num_heads <= 128, d_c + d_R <= 1024, d_h <= 256, d_v <= 256.
 *   All shapes: d_c, d_R, d_h, d_v multiples of 16, d_R even, block_size == 64.
 */
#ifndef LIBMLA_MLA_H
#define LIBMLA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or shape */
  MLA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (format/shape combination) */
  MLA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than mla_decode_workspace_size */
  MLA_ERR_HIP = 4            /* the HIP runtime reported an error (device query or launch) */
} mla_status_t;

/*
 * Cache formats.  MLA_FP8_E4M3: e4m3 codes with one fp32 scale per token.  MLA_FP8_E4M3_B32:
 * e4m3 codes with one power-of-two scale per tile of 32 tokens x 32 columns (katajob, section
 * "Compression as architecture versus compression as post-processing": quantised caches depend
 * on per-block scales, and a low-precision latent composes with MLA); DeepSeek-V2 shape only.
 */
typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2, MLA_FP8_E4M3_B32 = 3 } mla_dtype_t;

typedef struct {
  int32_t num_heads;     /* H */
  int32_t d_c;           /* latent width (512 in DeepSeek-V2, talentme card "Core Definition") */
  int32_t d_r;           /* decoupled RoPE key width */
  int32_t d_h;           /* per-head content query/key width */
  int32_t d_v;           /* per-head value width */
  int32_t block_size;    /* tokens per cache page; must be 64 */
  float softmax_scale;   /* multiplies q.k; 1/sqrt(d_h + d_r) for concatenated keys */
  float rope_base;       /* RoPE frequency base (10000) */
  int32_t cache_dtype;   /* mla_dtype_t of the cache rows */
  int32_t act_dtype;     /* mla_dtype_t of q_nope, q_rope, c_kv, k_r, weights and out */
} mla_config_t;

/*
 * mla_cache_append -- write n new tokens into the paged latent cache.
 *
 * Only the latent and the positional key are stored (podcast "What Is Multi-head Latent
 * Attention ...": the system caches the compact latent and the positional part; zenaique:
 * the latent is the only thing written to the cache).  RoPE is applied to k_R here, at the
 * token's own position, because rotation does not commute with the absorbed up-projection
 * (katajob, end of "Why it is not just extra work at decode time"; bembew "Multi-head
 * Latent Attention", "Decoupling RoPE from Compression"; bembew "Implementation Logic",
 * step 4).
 *
 *   cache        [num_blocks, 64, d_c + d_R] in cache_dtype; row = [c ; RoPE(k_R, pos)]
 *   cache_scale  FP8_E4M3: [num_blocks, 64] fp32, one per token; FP8_E4M3_B32: [num_blocks, 2, 18]
 *                fp32, one power of two 2^e per tile (token half, 32-column block); NULL for
 *                other formats
 *   c_kv         [n, d_c]  act_dtype      k_r [n, d_R] act_dtype, before RoPE
 *   pos          [n] int32 (device)       position of each token within its sequence
 *   seq_of       [n] int32 (device)       sequence of each token, 0 .. batch-1
 *   block_table  [batch, max_blocks] int32 (device) physical page ids
 * RoPE: the pair (2j, 2j+1) of k_R is rotated by pos * rope_base^(-2j/d_R); the angle
 * and its cosine/sine are evaluated in fp64.
 * A token whose sequence, page slot or page id is out of range is skipped (not written).
 * FP8: scale = amax/448 in fp32, code = e4m3(value / scale), nearest-even, saturating.
 * FP8_E4M3_B32: for every tile the call writes, e = the smallest integer with amax <= 448 * 2^e
 * (amax over the tile's rows, those written by earlier calls included unless this call writes
 * the tile's first row), clamped to [-126, 127]; codes = e4m3(value * 2^-e); when e grows,
 * the earlier rows' codes are re-encoded as e4m3(code * 2^(e_old - e)).  Preconditions: the
 * positions of a sequence are appended in order, each once, and the tokens of one call that
 * fall into one tile are consecutive in the call (true for one token per sequence and for
 * chunks of consecutive positions); otherwise the tile's contents are undefined.
 */
mla_status_t mla_cache_append(const mla_config_t* cfg, void* cache, float* cache_scale,
                              int32_t num_blocks, const void* c_kv, const void* k_r,
                              const int32_t* pos, const int32_t* seq_of,
                              const int32_t* block_table, int32_t batch, int32_t max_blocks,
                              int32_t n, void* stream);

/*
 * mla_absorb_q -- fold W_UK into the query and rotate the positional query.
 *
 * q_abs[t,i] = [ q_nope[t,i] W_UK,i^T ; RoPE(q_rope[t,i], q_pos[t]) ], W_UK,i = columns
 * i*d_h .. i*d_h+d_h-1 of w_uk.  Since k^C = c W_UK,i, the content score q^C . k^C equals
 * (q^C W_UK,i^T) . c (katajob "solid answer": the up-projections fold into the query and
 * output projections; "Why it is not just extra work at decode time").
 *
 *   q_nope  [T, H, d_h] act_dtype      q_rope [T, H, d_R] act_dtype (before RoPE)
 *   q_pos   [T] int32 (device)         w_uk [d_c, H*d_h] act_dtype
 *   q_abs   [T, H, d_c + d_R] act_dtype (for every cache format)
 * Matrix-core path: bf16 products, fp32 accumulation, one rounding to the output format.
 */
mla_status_t mla_absorb_q(const mla_config_t* cfg, const void* q_nope, const void* q_rope,
                          const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t T, void* stream);

/*
 * mla_append_absorb -- mla_cache_append and mla_absorb_q of one decode step in a single
 * launch (the two are independent: the append writes cache rows, the absorption reads the
 * step's queries and writes q_abs).  Arguments, layouts and results are exactly those of the
 * two calls (see their passages above); validation is theirs, and on any error nothing is
 * launched.  For the DeepSeek-V2 shape with bf16 activations one kernel does both; otherwise
 * the two kernels are launched in order.  n = 0 or T = 0 skips that half.
 */
mla_status_t mla_append_absorb(const mla_config_t* cfg, void* cache, float* cache_scale, int32_t num_blocks,
                               const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* seq_of,
                               const int32_t* block_table, int32_t batch, int32_t max_blocks, int32_t n,
                               const void* q_nope, const void* q_rope, const int32_t* q_pos, const void* w_uk,
                               void* q_abs, int32_t T, void* stream);

/*
 * mla_decode_workspace_size -- bytes of scratch mla_decode_attn needs for batch B,
 * Sq queries per sequence and block tables of width max_blocks on the current device.
 * Returns 0 for invalid arguments or sizes past the limits above.  The value depends only
 * on these arguments, the device's compute-unit count and the test-only environment
 * overrides MLA_FORCE_SPLITS (a number of token ranges) and MLA_SPLIT_TOKENS (tokens per
 * range, counted over the block tables' capacity; MLA_FORCE_SPLITS wins when both are set);
 * they must be the same here and in the decode calls that use the workspace.  It bounds the
 * split-K partial results.
 */
size_t mla_decode_workspace_size(const mla_config_t* cfg, int32_t B, int32_t Sq,
                                 int32_t max_blocks);

/*
 * mla_decode_attn -- attention in latent space (katajob, "Why it is not just extra work at
 * decode time": once folded, attention runs on the latent itself, with no per-head keys or
 * values built; zenaique: decode streams the whole cache from HBM, so the
 * bytes per cached token set the ceiling).
 *
 * For every query row t = b*Sq + j and head i, over tokens s = 0 .. p (p = kv_len[b]-Sq+j):
 *   score[s] = softmax_scale * (q_abs[t,i] . cache_row[s])       (content + positional)
 *   o_lat[t,i] = sum_s softmax(score)[s] * c_s                   ([T, H, d_c] fp32)
 *   lse[t,i]   = log sum_s exp(score[s])                         ([T, H] fp32, natural log)
 * FP8: row values are code*cache_scale (FP8_E4M3_B32: code * the tile's 2^e, which the matrix
 * instructions take as their E8M0 operand block scales).  The matrix instructions take e4m3 operands: each
 * head's query becomes two e4m3 terms (hi + lo/16 with one fp32 scale, about 8 significant
 * bits), and so do the probabilities (hi + lo/16 per token, with a power-of-two block scale).
 * The token range is split across workgroups (split-K); partial results go to `workspace`
 * and are merged by a log-sum-exp combine.  A query row that sees no token gives o_lat = 0 and
 * lse = -inf: every row of a sequence with kv_len <= 0, and row j of a sequence with
 * kv_len < Sq when its position p = kv_len - Sq + j is negative (the rows with p >= 0 attend
 * to tokens 0 .. p as usual).  kv_len[b] <= 64*max_blocks (longer lengths are clamped to the
 * table); pages in [0, num_blocks) (tokens on other pages are skipped).  Lengths live in
 * device memory and are not read on the host, so these cases are results, not errors.
 *
 *   q_abs       [T, H, d_c + d_R] act_dtype (mla_absorb_q output)
 *   cache       [num_blocks, 64, d_c + d_R]                 cache_scale as for mla_cache_append
 *   block_table [B, max_blocks] int32 (device)              kv_lens [B] int32 (device)
 *   workspace   >= mla_decode_workspace_size(cfg, B, Sq, max_blocks) bytes, 256-byte aligned;
 *               contents need no initialisation and are not preserved.
 */
mla_status_t mla_decode_attn(const mla_config_t* cfg, const void* q_abs,
                             const void* cache, const float* cache_scale, int32_t num_blocks,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* kv_lens, int32_t B, int32_t Sq, void* workspace,
                             size_t ws_bytes, float* o_lat, float* lse, void* stream);

/*
 * mla_decode_split / mla_decode_combine -- the two launches of mla_decode_attn, for callers
 * that time or schedule them separately.  Same arguments as mla_decode_attn; calling split
 * then combine on one stream is exactly mla_decode_attn.  split writes o_lat/lse of every
 * sequence that one token range covers whole and workspace partials for the others;
 * combine merges the partials (and writes the kv_len <= 0 results).  On the generic
 * (non-matrix-core) path split does all the work and combine launches nothing.
 */
mla_status_t mla_decode_split(const mla_config_t* cfg, const void* q_abs,
                              const void* cache, const float* cache_scale, int32_t num_blocks,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* kv_lens, int32_t B, int32_t Sq, void* workspace,
                              size_t ws_bytes, float* o_lat, float* lse, void* stream);
mla_status_t mla_decode_combine(const mla_config_t* cfg, const void* q_abs,
                                const void* cache, const float* cache_scale, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* kv_lens, int32_t B, int32_t Sq, void* workspace,
                                size_t ws_bytes, float* o_lat, float* lse, void* stream);

/*
 * mla_decode_attn_noalloc -- mla_decode_attn without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops or harnesses that
 * forbid allocation).  Same arguments (minus workspace and ws_bytes), results and validation as
 * mla_decode_attn; the split-K partials go to a fixed device array inside the library
 * (MLA_NOALLOC_SCRATCH_BYTES = 64 MiB per device, held until the process ends).  A launch whose
 * partials exceed it, i.e. mla_decode_workspace_size(cfg, B, Sq, max_blocks) >
 * MLA_NOALLOC_SCRATCH_BYTES, returns MLA_ERR_WORKSPACE and launches nothing.  Nothing is
 * allocated or freed.  Every call on one device shares that array: calls that can overlap in
 * time on one device (other streams, other host threads) race and must be ordered by the caller.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mla_status_t mla_decode_attn_noalloc(const mla_config_t* cfg, const void* q_abs,
                                     const void* cache, const float* cache_scale, int32_t num_blocks,
                                     const int32_t* block_table, int32_t max_blocks,
                                     const int32_t* kv_lens, int32_t B, int32_t Sq,
                                     float* o_lat, float* lse, void* stream);

/*
 * From the hidden state: the projections upstream of the cache and the query (katajob "code":
 * latent = x @ W_down; bembew "Multi-head Latent Attention", "Implementation Logic", steps 1, 3
 * and 4), fused with the step's append and absorption.
 *
 * mla_append_absorb_hidden -- for the n new tokens, [c ; k_R raw] = h_kv [W_down | W_KR]; for the
 * T query rows, [q^C ; q^R] = h_q [W_Q | W_QR]; then exactly mla_append_absorb with those arrays
 * (RoPE on k_R at pos, the cache write, the fold of W_UK and RoPE on q^R at q_pos).  The
 * projections accumulate in fp32 and are rounded once to the activation format, the format
 * mla_cache_append and mla_absorb_q take.
 *   d_model    model width (a multiple of 16; multiples of 64 take the matrix-core path)
 *   h_kv       [n, d_model] act_dtype     hidden states of the new tokens
 *   w_dkv_t    [d_c + d_R, d_model] act_dtype: the transposed weights, row j holding the weights
 *              of output j: rows 0 .. d_c-1 are W_down^T, rows d_c .. d_c+d_R-1 are W_KR^T
 *   h_q        [T, d_model] act_dtype     hidden states of the query rows
 *   w_q_t      [H*(d_h + d_R), d_model] act_dtype: rows 0 .. H*d_h-1 are W_Q^T (head i's
 *              content query is rows i*d_h ..), then H*d_R rows of W_QR^T (head-major)
 *   workspace  >= mla_hidden_workspace_size(cfg, d_model, n, T) bytes, 256-byte aligned, contents
 *              need no initialisation; it holds the projected rows and GEMM partial sums
 * The other arguments are those of mla_append_absorb, validated the same way before anything is
 * launched.  The weights are taken transposed so that each output's weights are contiguous: the
 * matrix-core kernels then read both operands with 16-byte row loads.
 */
size_t mla_hidden_workspace_size(const mla_config_t* cfg, int32_t d_model, int32_t n, int32_t T);
mla_status_t mla_append_absorb_hidden(const mla_config_t* cfg, int32_t d_model, const void* h_kv,
                                      const void* w_dkv_t, void* cache, float* cache_scale, int32_t num_blocks,
                                      const int32_t* pos, const int32_t* seq_of, const int32_t* block_table,
                                      int32_t batch, int32_t max_blocks, int32_t n, const void* h_q,
                                      const void* w_q_t, const int32_t* q_pos, const void* w_uk, void* q_abs,
                                      int32_t T, void* workspace, size_t ws_bytes, void* stream);

/*
 * To the model width, with W_UV folded into the output projection (katajob "solid answer": the
 * value up-projection folds into the output projection).  With W_O [H*d_v, d_model] the layer's
 * output is concat_i(o_i) W_O = sum_i o_lat_i W_UV,i W_O,i = sum_i o_lat_i W_O'_i.
 *
 * mla_fold_output_weights -- W_O'_i = W_UV,i W_O,i, once, into w_fold_t [d_model, H*d_c]
 *   (transposed: row n holds W_O'[i, c, n] at column i*d_c + c), fp32 sums, one rounding.
 *   w_uv [d_c, H*d_v], w_o [H*d_v, d_model], all act_dtype.
 * mla_out_proj_folded -- out [T, d_model] (act_dtype) = o_lat [T, H*d_c] (fp32; rounded to bf16 on
 *   the matrix-core path) . W_O'.  workspace >= mla_out_proj_folded_workspace_size(cfg, d_model, T)
 *   bytes (GEMM partial sums), 256-byte aligned.
 * At decode batch sizes the folded weight (H*d_c*d_model values) is d_c/d_v times the size of
 * W_O, so applying W_UV with mla_out_proj and then W_O reads fewer bytes; the folded form is the
 * one-GEMM path.
 */
mla_status_t mla_fold_output_weights(const mla_config_t* cfg, int32_t d_model, const void* w_uv, const void* w_o,
                                     void* w_fold_t, void* stream);
size_t mla_out_proj_folded_workspace_size(const mla_config_t* cfg, int32_t d_model, int32_t T);
mla_status_t mla_out_proj_folded(const mla_config_t* cfg, int32_t d_model, const float* o_lat, const void* w_fold_t,
                                 void* out, int32_t T, void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode over a standard per-head key/value cache, for comparison: the cache MLA replaces
 * (zenaique "What MLA caches versus what MHA and GQA cache": every head keeps its own key and
 * value per token; the podcast's grouped-query sizing shares them among groups of query heads).
 * Same paging, lengths and split-K flash decoding as mla_decode_attn, one query per sequence.
 *
 * mla_kv_decode_attn -- for sequence b and query head i (of H = cfg->num_heads), with key/value
 *   head j = i / (H / num_kv_heads):  o[b,i] = sum_t softmax_t(softmax_scale * q[b,i] . k[t,j]) v[t,j]
 *   over t < kv_len[b]; lse[b,i] = log sum_t exp(softmax_scale * q . k).
 *   num_kv_heads = H is multi-head attention.  Head width d = cfg->d_h = cfg->d_v = 128, bf16
 *   cache and activations, H / num_kv_heads in {1, 2, 4, 8, 16}; other fields of cfg are unused.
 *   q       [B, H, d] bf16 (positions already encoded)
 *   k_cache [num_blocks, num_kv_heads, 64, d] bf16 (a head's 64-token page contiguous, token-major)
 *   v_cache [num_blocks, num_kv_heads, d, 64] bf16 (the same pages stored transposed, column-major:
 *           the value product contracts over tokens and reads them contiguously)
 *   block_table [B, max_blocks], kv_lens [B] int32 (device)
 *   o [B, H, d] fp32, lse [B, H] fp32;  workspace >= mla_kv_decode_workspace_size(...) bytes,
 *   256-byte aligned, no initialisation needed.  Sequences with kv_len <= 0 give o = 0, lse = -inf.
 */
size_t mla_kv_decode_workspace_size(const mla_config_t* cfg, int32_t num_kv_heads, int32_t B, int32_t max_blocks);
mla_status_t mla_kv_decode_attn(const mla_config_t* cfg, int32_t num_kv_heads, const void* q, const void* k_cache,
                                const void* v_cache, int32_t num_blocks, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* kv_lens, int32_t B, void* workspace,
                                size_t ws_bytes, float* o, float* lse, void* stream);

/*
 * mla_out_proj -- apply W_UV once per query on the output side:
 * out[t,i] = o_lat[t,i] W_UV,i, W_UV,i = columns i*d_v .. i*d_v+d_v-1 of w_uv
 * (katajob "solid answer": the value up-projection folds into the output projection).
 *   o_lat [T, H, d_c] fp32     w_uv [d_c, H*d_v] act_dtype     out [T, H, d_v] act_dtype
 * Matrix-core path: o_lat rounded to bf16, fp32 accumulation.
 */
mla_status_t mla_out_proj(const mla_config_t* cfg, const float* o_lat, const void* w_uv,
                          void* out, int32_t T, void* stream);

/* Human-readable name of a status code (static storage).  Takes any integer: a value that is not
 * an mla_status_t gives "MLA_ERR_UNKNOWN" (an enum parameter could not hold such values safely). */
const char* mla_status_string(int32_t status);

/* ABI version of this header: 8. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMLA_MLA_H */
