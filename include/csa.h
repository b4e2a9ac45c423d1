/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed sparse attention library (libcsa.so).
 *
 * One attention layer of DeepSeek-V4-style compressed sparse attention (CSA), as
 * described by three web pages:
 *   [P1] "vLLM DeepSeek V4 Support: Efficient Long-context Attention" (agentlenshq.com)
 *   [P2] "vLLM解密：DeepSeek-V4本地部署為何如此困難" (yhxrc.cn)
 *   [P3] blog.hotdry.top, "DeepSeek V4 inference latency optimization" (2026-04-24)
 *
 * The four calls of one decode or prefill-chunk step, in stream order:
 *   csa_compress_insert  (main cache and, for c4a, indexer cache)
 *   csa_index_topk       (c4a only)
 *   csa_attend           (top-k entries + raw sliding window, or dense for c128a; optional fused inverse RoPE)
 *   csa_inv_rope         (standalone inverse RoPE, when not fused)
 *   csa_inv_rope_quant_fp8 (inverse RoPE fused with fp8 quantisation of the output, for an fp8 projection)
 *   csa_attend_quant_fp8 (csa_attend with that fp8 output epilogue fused into the attention kernels)
 * and, upstream of the step, csa_prepare_qk (query norm + RoPE, window-key RoPE + insert).
 *
 * Conventions
 *   - Every pointer is DEVICE memory unless marked [host]. Every call is asynchronous on
 *     `stream`; the library never synchronises, allocates or frees. Its only global state is the
 *     fixed per-GPU scratch array of csa_index_topk_noalloc.
 *   - The caller owns every buffer (pages, block tables, inputs, outputs, workspaces).
 *   - Arguments are validated on the host BEFORE any HIP call; an invalid call returns a
 *     non-zero status and touches nothing. A failed launch returns CSA_ERR_HIP and
 *     csa_last_hip_error() (thread-local) holds the hipError_t.
 *   - Device-side contents (block-table ids, positions, top-k indices) cannot be checked on
 *     the host. Kernels bounds-check every id against n_phys / bt_stride / batch / rope_rows and
 *     skip accesses that would fall outside; such inputs give unspecified but memory-safe results.
 *   - Paging ([P1] "KV Cache Memory Management", [P2] "3.1 顯存"): one logical block is 256 raw
 *     positions for every layer kind. A compressed cache with ratio m holds E = 256/m entries per
 *     block (64 for c4a, 2 for c128a). Entry i of sequence b lives at page row
 *     block_table[b][i / E] * E + i % E; raw position j lives at row block_table[b][j / 256] * 256 + j % 256.
 *   - Windows ([P1] "DeepSeek V4 Attention Architecture", [P3] "KV 缓存压缩"): c4a entry i covers raw
 *     positions 4i .. 4i+7 (stride 4, window 8), c128a entry i covers 128i .. 128i+127; the RoPE
 *     anchor is the first position of the window. An entry exists once its whole window exists
 *     and is usable by a query at position p iff its window ends at or before p
 *     ([P3] "注意力计算剪枝").
 *   - RoPE: interleaved pairs (D-R+2j, D-R+2j+1) on the last R dims, angle p * theta^(-2j/R),
 *     read from a caller-owned fp32 table rope_cs[rows][R/2][2] = (cos, sin) (see csa_rope_table).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum, inconsistent descriptor */
  CSA_ERR_UNSUPPORTED = 2, /* valid request with no kernel (dtype combination, head count, dim) */
  CSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the matching *_workspace() size */
  CSA_ERR_HIP = 4,         /* a HIP launch failed; see csa_last_hip_error() */
  CSA_ERR_TOO_LARGE = 5    /* the request needs more than the fixed scratch of a no-allocation entry point */
} csa_status_t;

typedef enum {
  CSA_F32 = 0,
  CSA_BF16 = 1,
  CSA_FP8_E4M3 = 2, /* OCP e4m3fn (max 448), one fp32 scale per row: value = scale * e4m3(code) */
  CSA_FP4_E2M1 = 3  /* OCP MXFP4, compressed caches only (the indexer cache; [P1] "DeepSeek V4 Attention
                       Architecture" and [P2] "一、官方部署 Recipe" name an fp4 indexer cache): a row of D
                       channels is D/2 bytes, channel 2j in the low nibble of byte j; every block of 32
                       channels has one E8M0 byte X+127 and value = 2^X * e2m1.
                       X = floor(log2(block amax)) - 2 (0 for an all-zero block), elements rounded to
                       nearest-even and saturated at 6. D must be a multiple of 32. */
} csa_dtype_t;

typedef enum {
  CSA_SCORE_DOT = 0,  /* s_e = q . k_e (exactly one indexer head) */
  CSA_SCORE_WRELU = 1 /* s_e = sum_h w_h * max(0, q_h . k_e) */
} csa_score_t;

/* One compressed cache: main attention cache (D = 512 or 128) or indexer cache (D = 128 or 32).
 * [P2] "3.2 內核": the indexer K cache and the main K cache are separate compressor instances. */
typedef struct {
  int32_t ratio, window;    /* (4, 8) c4a or (128, 128) c128a; any other pair is CSA_ERR_INVALID_ARG */
  int32_t dim;              /* D in {32, 64, 128, 256, 512} */
  int32_t rope_dims;        /* R, even, 0 <= R <= D; rotated dims are [D-R, D) */
  csa_dtype_t dtype;        /* element type of pages */
  void* pages;              /* [n_phys * E][D] rows, E = 256 / ratio */
  float* scales;            /* fp8: [n_phys * E] per-entry fp32 scales; fp4: cast of a uint8 array
                               [n_phys * E][D / 32] of E8M0 block exponents; NULL otherwise */
  const int32_t* block_table; /* [batch][bt_stride] logical 256-position block -> physical page id */
  int32_t batch, bt_stride; /* rows and columns of block_table */
  int32_t n_phys;           /* physical pages in `pages` */
} csa_cache_t;

/* Raw per-position pages on the same 256-position paging: either the compressor state
 * (roles = window / ratio; raw kv rows plus their role logits, [P2] "3.1 顯存": compressor
 * residual kept as sliding-window KV), or the sliding-window K=V rows used by attention
 * (roles = 0; rows already rotated at their own position). */
typedef struct {
  csa_dtype_t dtype;        /* state: CSA_F32 or CSA_BF16; window: same dtype as the attention cache */
  int32_t dim, roles;
  void* kv_pages;           /* [n_phys * 256][dim] */
  void* logit_pages;        /* [n_phys * 256][roles][dim] (state only, else NULL) */
  float* scales;            /* [n_phys * 256] per-row scales (fp8 window only, else NULL) */
  const int32_t* block_table; /* [batch][bt_stride] */
  int32_t batch, bt_stride, n_phys;
} csa_raw_t;

/* ---------------------------------------------------------------------------------------------
 * csa_compress_insert -- KV compressor fused with RMSNorm, RoPE and cache insertion.
 * [P1] "GPU Compute Saturation" / [P2] "3.2 內核": compressor + RMSNorm + RoPE + cache write as one
 * elementwise-fused step, one instance per cache. Weights ([P1] architecture section): a
 * compressed entry is a weighted sum of its window's raw tokens; here the weight of raw row t of
 * the window for channel c is softmax_t(logit[t][c]) with logit[t] the row's role-(t / ratio)
 * logit vector. Then y = z / sqrt(mean(z^2) + rms_eps) * gamma, RoPE at the anchor, rounding to
 * the cache dtype (fp8: scale = amax/448, code = e4m3_rne(y * (448/amax)), computed in fp32; fp4: the
 * MXFP4 rule of CSA_FP4_E2M1 applied to the fp32 row).
 *
 * Sequence b appends n_b = cu_new[b+1] - cu_new[b] raw tokens at positions start_pos[b] ... to the
 * state pages (rows cu_new[b] .. of kv_new [total_new][D] and logit_new [total_new][roles][D],
 * state dtype), then builds every entry whose window ends inside the new positions. Rows of
 * older positions are read from the state pages: at least the last window-1 positions before
 * start_pos[b] must be present. Earlier positions may be unmapped.
 *   max_new_per_seq [host] >= max_b n_b (sizes the grid).
 *   out_slots [batch][max_entries_out] receives the page row of each entry written, in entry
 *   order, -1 padded (may be NULL); out_new_entries [batch] receives the entry counts (may be NULL).
 *   max_entries_out must be >= ceil(max_new_per_seq / ratio) when out_slots is given.
 *   rope_rows [host] = rows of rope_cs; anchors must be < rope_rows.
 * ------------------------------------------------------------------------------------------- */
csa_status_t csa_compress_insert(const csa_cache_t* cache, const csa_raw_t* state, int32_t batch,
                                 const int32_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                 int32_t max_new_per_seq, const void* kv_new, const void* logit_new,
                                 const float* gamma, float rms_eps, const float* rope_cs,
                                 int32_t rope_rows, int32_t* out_slots, int32_t max_entries_out,
                                 int32_t* out_new_entries, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_compress_insert_pair -- csa_compress_insert of two caches that take the same new tokens (a c4a
 * layer's main cache a and indexer cache b: [P2] "3.2 內核" keeps one compressor instance per cache) in one
 * call. Each cache's arguments mean what they mean for csa_compress_insert (kv_a / logit_a / gamma_a /
 * rope_cs_a belong to cache_a, and so on); batch, start_pos, cu_new, total_new, max_new_per_seq and rms_eps
 * are shared; no slot or count outputs. Results are those of the two separate calls. A c4a bf16 / fp8 main
 * cache of dim 512 with an indexer cache of dim 128 of the same dtype (or an fp4 indexer cache beside an fp8
 * main cache) and bf16 inputs runs as one kernel launch whose blocks
 * each work for one of the two caches (each with its own per-dim code); any other pair runs as two launches.
 * Validation: both argument sets as for csa_compress_insert, before any HIP call.
 * ------------------------------------------------------------------------------------------- */
csa_status_t csa_compress_insert_pair(const csa_cache_t* cache_a, const csa_raw_t* state_a, const void* kv_a,
                                      const void* logit_a, const float* gamma_a, const float* rope_cs_a,
                                      int32_t rope_rows_a, const csa_cache_t* cache_b, const csa_raw_t* state_b,
                                      const void* kv_b, const void* logit_b, const float* gamma_b,
                                      const float* rope_cs_b, int32_t rope_rows_b, int32_t batch,
                                      const int32_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                      int32_t max_new_per_seq, float rms_eps, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_index_topk -- indexer score over eligible entries and top-k selection (c4a layers).
 * [P1] architecture section / [P2] "二、注意力機制為什么這么麻煩": DeepSeek Sparse Attention keeps the
 * top-k compressed entries (k = 512 on c4a). [P2] "3.2 內核": the indexer pipeline has its own
 * compressed cache and stream. The score formula is an input choice (csa_score_t).
 *
 * Query q belongs to sequence q_seq[q] (a block-table row) at position q_pos[q]; its candidates
 * are entries 0 .. n_elig-1 with n_elig = csa_num_eligible(q_pos[q]), clamped to max_elig [host]
 * (max_elig <= 2^31-1).
 * q_idx is [n_q][n_heads][D] in q_dtype (CSA_F32 for an fp32 cache, CSA_BF16 otherwise);
 * head_w [n_q][n_heads] fp32 for WRELU, NULL for DOT. fp8 keys score as scale_e * (q . code_e); fp4
 * keys are dequantised exactly (2^X_b * e2m1) and score as q . k_e. An fp4 cache is scored for WRELU on
 * c4a pages of dim 128 with 16, 32, 48 or 64 heads and CSA_BF16 q; other fp4 requests are
 * CSA_ERR_UNSUPPORTED.
 * Order: score descending, ties to the lower entry index, -0 == +0, NaN below every number.
 * Output out_idx [n_q][k]: the min(k, n_elig) chosen entries in ascending index order, -1 padded;
 * out_count [n_q] (may be NULL); out_scores [n_q][k] fp32 scores in the same order, NaN padded
 * (may be NULL). k in [1, 2048]. k > n_elig is not an error. The chosen set is unique, so the
 * result does not depend on work distribution.
 *
 * Workspace: csa_index_topk_workspace(n_q, max_elig, k, n_heads) bytes, 256-byte aligned, owned by
 * the caller. Its leading histogram region must be zero when a score pass starts: zero-fill the
 * workspace once after allocating it (or call csa_index_workspace_clear); every select pass leaves
 * that region zero again, so a workspace reused with the same n_q needs no further clearing. Calls
 * that share a workspace must not overlap.
 *
 * csa_index_topk = csa_index_score followed by csa_index_select (same arguments). The two halves
 * are exported so a caller can place them on streams or time them separately; a score pass must be
 * followed by the select pass on the same workspace before the next score pass.
 * ------------------------------------------------------------------------------------------- */
size_t csa_index_topk_workspace(int32_t n_q, int64_t max_elig, int32_t k, int32_t n_heads);
csa_status_t csa_index_workspace_clear(void* workspace, size_t workspace_bytes, int32_t n_q, hipStream_t stream);
csa_status_t csa_index_topk(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq,
                            const int32_t* q_pos, int64_t max_elig, const void* q_idx,
                            csa_dtype_t q_dtype, int32_t n_heads, const float* head_w,
                            csa_score_t mode, int32_t k, int32_t* out_idx, int32_t* out_count,
                            float* out_scores, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
csa_status_t csa_index_score(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq,
                             const int32_t* q_pos, int64_t max_elig, const void* q_idx,
                             csa_dtype_t q_dtype, int32_t n_heads, const float* head_w,
                             csa_score_t mode, int32_t k, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);
csa_status_t csa_index_select(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq,
                              const int32_t* q_pos, int64_t max_elig, int32_t k, int32_t* out_idx,
                              int32_t* out_count, float* out_scores, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_compress_index_score -- a c4a decode step's csa_compress_insert_pair (main cache a, indexer cache b)
 * followed by csa_index_score over cache b, in one launch where the configuration allows.
 * [P1] "GPU Compute Saturation" (the small kernels of a decode step fused so each launch's fixed latency is
 * paid once) / [P2] "3.2 內核": the indexer-cache compressor feeds the indexer, and the decode step's
 * latency is the sum of its launches. Arguments: those of csa_compress_insert_pair, then those of
 * csa_index_score with idx_cache = cache_b. Decode form only: every sequence appends exactly one token
 * (total_new == batch, max_new_per_seq == 1) and query q is sequence q's new token (n_q == batch, and on
 * the device q_seq[q] == q, q_pos[q] == start_pos[q]); otherwise CSA_ERR_INVALID_ARG for the host-checked
 * parts, and unspecified (memory-safe) results for the device-side part. Results are those of the two calls
 * in turn. A c4a main cache of dim 512 (bf16 or fp8) with an indexer cache of dim 128 (bf16, fp8 or MXFP4,
 * with the main cache's dtype or an fp8 main cache), bf16 inputs and a WRELU score of 64 heads over fewer
 * than 256 queries runs as one launch: the workgroup that scores query q's last page first runs sequence q's
 * compress units (main and indexer, append and entry), so the entry the query's own token completes is in
 * that page before it is read; anything else runs as the two launches. Validation: both argument sets as for
 * the two calls, before any HIP call. The workspace rules are those of csa_index_score.
 * ------------------------------------------------------------------------------------------- */
csa_status_t csa_compress_index_score(const csa_cache_t* cache_a, const csa_raw_t* state_a, const void* kv_a,
                                      const void* logit_a, const float* gamma_a, const float* rope_cs_a,
                                      int32_t rope_rows_a, const csa_cache_t* cache_b, const csa_raw_t* state_b,
                                      const void* kv_b, const void* logit_b, const float* gamma_b,
                                      const float* rope_cs_b, int32_t rope_rows_b, int32_t batch,
                                      const int32_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                      int32_t max_new_per_seq, float rms_eps, int32_t n_q, const int32_t* q_seq,
                                      const int32_t* q_pos, int64_t max_elig, const void* q_idx,
                                      csa_dtype_t q_dtype, int32_t n_heads, const float* head_w,
                                      csa_score_t mode, int32_t k, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_index_topk_noalloc -- csa_index_topk for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, meaning and
 * results as csa_index_topk, without the workspace: the score keys, histograms, candidate list and
 * bitmap live in a library-owned static device array of CSA_NOALLOC_SCRATCH_BYTES (64 MiB), one per
 * GPU the library runs on, held until the process ends. No call allocates or frees anything.
 *   - A request whose csa_index_topk_workspace(n_q, max_elig, k, n_heads) exceeds CSA_NOALLOC_SCRATCH_BYTES
 *     returns CSA_ERR_TOO_LARGE before any HIP call (e.g. 32 queries of 32767 entries need 13.7 MB, 4 of
 *     262143 need 12.7 MB; a 4096-query prefill chunk does not fit).
 *   - Each call first zero-fills the histogram region it uses (a fill kernel on `stream`), then runs the
 *     score and select launches of csa_index_topk on the scratch.
 *   - All calls on one GPU share that GPU's scratch and it keeps the last call's contents: calls that
 *     overlap on one GPU (on different streams, or from different threads without ordering) race and
 *     give undefined results. Order them on one stream or with events.
 *   - The first call on a device (the current device) looks up that device's copy of the array
 *     (hipGetSymbolAddress); a failed lookup returns CSA_ERR_HIP.
 * ------------------------------------------------------------------------------------------- */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
csa_status_t csa_index_topk_noalloc(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq,
                                    const int32_t* q_pos, int64_t max_elig, const void* q_idx,
                                    csa_dtype_t q_dtype, int32_t n_heads, const float* head_w,
                                    csa_score_t mode, int32_t k, int32_t* out_idx, int32_t* out_count,
                                    float* out_scores, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_attend -- shared-K=V attention over selected compressed entries plus the raw sliding window.
 * [P1] architecture section: K and V are one shared vector; DSA top-k entries; a 128-token sliding
 * window of uncompressed tokens; inverse RoPE on the output. [P2] attention section: c128a (HCA)
 * layers attend densely. [P2] "3.2 內核": inverse RoPE is fused after attention.
 *
 * Keys of query q: entries topk_idx[q][0..k) that are >= 0 (must be < n_elig), or, with
 * topk_idx == NULL, every eligible entry (n_elig clamped to max_elig [host]); plus window rows
 * at positions max(0, p - swa_window + 1) .. p read from `swa`. One joint softmax over all keys:
 * o_h = sum_s softmax_s(softmax_scale * q_h . k_s) k_s over all D dims, in fp32.
 * q [n_q][n_heads][D] in q_dtype (CSA_F32 for fp32 caches, CSA_BF16 otherwise); an fp4 cache is
 * CSA_ERR_UNSUPPORTED (fp4 is the indexer cache's format);
 * out [n_q][n_heads][D] fp32; out_lse [n_q][n_heads] natural-log sum of exp of the scaled
 * logits (may be NULL). fuse_inv_rope = 1 applies the inverse rotation at q_pos to out.
 * swa_window in [0, 1024]; n_heads in [1, 128]; k in [1, 2048] when topk_idx != NULL.
 * Workspace: csa_attend_workspace(n_q, n_heads, dim, max_keys) bytes, 16-byte aligned, with
 * max_keys = (topk_idx ? k : max_elig) + swa_window. It is non-zero only for dim 512 with a multiple
 * of 64 heads and few enough queries that each query's keys are split over several workgroups
 * (partial softmax states are merged by a second kernel); 0 means workspace may be NULL.
 * ------------------------------------------------------------------------------------------- */
size_t csa_attend_workspace(int32_t n_q, int32_t n_heads, int32_t dim, int32_t max_keys);
csa_status_t csa_attend(const csa_cache_t* kv_cache, const csa_raw_t* swa, int32_t swa_window,
                        int32_t n_q, const int32_t* q_seq, const int32_t* q_pos, const void* q,
                        csa_dtype_t q_dtype, int32_t n_heads, const int32_t* topk_idx, int32_t k,
                        int64_t max_elig, float softmax_scale, int32_t fuse_inv_rope,
                        const float* rope_cs, int32_t rope_rows, float* out, float* out_lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_attend_quant_fp8 -- csa_attend with the output epilogue of an fp8 output projection fused in.
 * [P1] "GPU Compute Saturation" (kernel fusions) / [P2] "3.2 內核": the attention output goes through the
 * inverse RoPE and into the fp8 batched matmul of the o_lora projection, and the two steps are fused so the
 * output skips an HBM round trip. Same arguments and attention as csa_attend with fuse_inv_rope = 1; instead of
 * an fp32 output, each (query, head) row of the inverse-rotated output is written as groups of `group`
 * consecutive channels in OCP e4m3fn with one fp32 scale per group, by the rule of csa_inv_rope_quant_fp8
 * (amax = max|y|, code = e4m3_rne(y * (448 / amax)), scale = amax / 448, computed in fp32; zero codes and scale
 * 1 for an all-zero group). The fp32 output never reaches memory.
 *   out_codes  [n_q][n_heads][D] uint8 (8-byte aligned); out_scales [n_q][n_heads][D / group] fp32;
 *   out_lse    as for csa_attend (may be NULL).
 *   group in {16, 32, 64, 128}. Supported for D = 512 with bf16 / fp8 caches and a multiple of 16 heads (the
 *   MFMA attention kernels); other shapes return CSA_ERR_UNSUPPORTED (use csa_attend + csa_inv_rope_quant_fp8).
 *   Workspace: as for csa_attend (csa_attend_workspace).
 * ------------------------------------------------------------------------------------------- */
csa_status_t csa_attend_quant_fp8(const csa_cache_t* kv_cache, const csa_raw_t* swa, int32_t swa_window,
                                  int32_t n_q, const int32_t* q_seq, const int32_t* q_pos, const void* q,
                                  csa_dtype_t q_dtype, int32_t n_heads, const int32_t* topk_idx, int32_t k,
                                  int64_t max_elig, float softmax_scale, const float* rope_cs, int32_t rope_rows,
                                  int32_t group, uint8_t* out_codes, float* out_scales, float* out_lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_inv_rope -- inverse rotation (u, v) -> (u c + v s, -u s + v c) of the last rope_dims dims of
 * io [n_q][n_heads][dim] (fp32, in place) at each query's position q_pos[q] < rope_rows.
 * [P1] architecture section: the inverse RoPE restores translation invariance of the shared-K=V output.
 * ------------------------------------------------------------------------------------------- */
csa_status_t csa_inv_rope(int32_t n_q, int32_t n_heads, int32_t dim, int32_t rope_dims,
                          const int32_t* q_pos, const float* rope_cs, int32_t rope_rows, float* io,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_prepare_qk -- query norm + query RoPE and window-key RoPE + window-key insert, fused.
 * [P1] "GPU Compute Saturation" (kernel fusions) / [P2] "3.2 內核": the elementwise work on the query
 * heads and on the uncompressed sliding-window key in front of the main attention runs as one
 * horizontally fused kernel, each wavefront statically assigned to a query head or to the key.
 * For every new token t (position tok_pos[t] < rope_rows of sequence tok_seq[t]):
 *   q_out[t][h] = RoPE_p(RMSNorm(q_in[t][h]) * q_gamma), RMSNorm over the D channels of each head with
 *     eps rms_eps and one weight vector q_gamma [D] for all heads, rounded once to q_dtype;
 *   the window row of position p in `swa` (roles 0) = RoPE_p(kv_in[t]), rounded to the window pages'
 *     type (fp8: code = e4m3_rne(y * 448/amax), scale = amax/448 per row, zeros and scale 1 for a zero row);
 *     a position whose block is unmapped is skipped.
 *   q_in, q_out [n_tok][n_heads][D] and kv_in [n_tok][D] in q_dtype; D = swa->dim. Type pairs:
 *   (CSA_F32 q, CSA_F32 window) or (CSA_BF16 q, CSA_BF16 or CSA_FP8_E4M3 window). n_heads in [1, 128].
 *   q_out must not alias q_in and must be 16-byte aligned (CSA_ERR_INVALID_ARG otherwise). Caller-owned
 *   buffers; nothing is allocated.
 * ------------------------------------------------------------------------------------------- */
csa_status_t csa_prepare_qk(int32_t n_tok, int32_t n_heads, const int32_t* tok_seq, const int32_t* tok_pos,
                            const void* q_in, csa_dtype_t q_dtype, const float* q_gamma, float rms_eps,
                            const void* kv_in, const csa_raw_t* swa, int32_t rope_dims,
                            const float* rope_cs, int32_t rope_rows, void* q_out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_inv_rope_quant_fp8 -- inverse RoPE fused with fp8 quantisation of the attention output.
 * [P1] "GPU Compute Saturation" (kernel fusions) / [P2] "3.2 內核": the main attention output goes
 * through the inverse RoPE and into the fp8 batched matmul of the o_lora projection; fusing the two
 * saves one HBM round trip of the output. The pages give no quantisation granularity; here every
 * (query, head) row is cut into groups of `group` consecutive channels, each stored as OCP e4m3fn
 * codes with one fp32 scale by the rule of the fp8 caches, computed in fp32 after the rotation:
 * amax = max|y|, code = e4m3_rne(y * (448 / amax)), scale = amax / 448 (zero codes and scale 1 for an
 * all-zero group).
 *   in          [n_q][n_heads][dim] fp32, the output of csa_attend with fuse_inv_rope = 0 (16-byte aligned)
 *   out_codes   [n_q][n_heads][dim] uint8 (8-byte aligned); out_scales [n_q][n_heads][dim / group] fp32
 *   dim in {32, 64, 128, 256, 512}; rope_dims even, <= dim (the rotated dims are the last rope_dims);
 *   group a power of two in [8, 512] dividing dim; n_heads in [1, 128]; positions q_pos[q] < rope_rows
 *   (a position outside the table leaves that query unrotated). Caller-owned buffers; nothing is allocated.
 * ------------------------------------------------------------------------------------------- */
csa_status_t csa_inv_rope_quant_fp8(int32_t n_q, int32_t n_heads, int32_t dim, int32_t rope_dims,
                                    const int32_t* q_pos, const float* rope_cs, int32_t rope_rows,
                                    const float* in, int32_t group, uint8_t* out_codes, float* out_scales,
                                    hipStream_t stream);

/* csa_rope_table -- fill rope_cs [rows][rope_dims/2][2] with (cos, sin) of p * theta^(-2j/R),
 * evaluated in fp64 and rounded to the nearest fp32. */
csa_status_t csa_rope_table(int32_t rows, int32_t rope_dims, double theta, float* rope_cs,
                            hipStream_t stream);

/* ----------------------------- [host]-only helpers: no device access, no HIP call ------------ */
int64_t csa_num_entries(int64_t n_raw, int32_t ratio, int32_t window);  /* entries of n_raw raw tokens; -1 if bad shape */
int64_t csa_num_eligible(int64_t q_pos, int32_t ratio, int32_t window); /* = csa_num_entries(q_pos + 1) */
int64_t csa_entry_slot(const int32_t* bt_row /*[host]*/, int64_t entry, int32_t ratio); /* page row of entry */
int64_t csa_raw_slot(const int32_t* bt_row /*[host]*/, int64_t pos);                    /* page row of raw position */
const char* csa_status_string(csa_status_t status);
int32_t csa_last_hip_error(void); /* hipError_t of this thread's last failed launch, 0 if none */
int32_t csa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
