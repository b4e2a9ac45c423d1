// C ABI of libcsa: host-side argument validation (before any HIP call), workspace sizing and
// dispatch to the kernel launchers. Declarations and semantics: include/csa.h.
#include <math.h>

#include <mutex>

#include "csa_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_shape(int ratio, int window) { return (ratio == 4 && window == 8) || (ratio == 128 && window == 128); }
bool valid_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256 || d == 512; }
bool valid_dtype(csa_dtype_t t) { return t == CSA_F32 || t == CSA_BF16 || t == CSA_FP8_E4M3; }
bool valid_cache_dtype(csa_dtype_t t) { return valid_dtype(t) || t == CSA_FP4_E2M1; }

bool valid_cache(const csa_cache_t* c) {
  if (!c) return false;
  if (!valid_shape(c->ratio, c->window) || !valid_dim(c->dim)) return false;
  if (c->rope_dims < 0 || c->rope_dims > c->dim || (c->rope_dims & 1)) return false;
  if (!valid_cache_dtype(c->dtype) || !c->pages || !aligned(c->pages, 16)) return false;
  if ((c->dtype == CSA_FP8_E4M3 || c->dtype == CSA_FP4_E2M1) && !c->scales) return false;
  if (c->dtype == CSA_FP4_E2M1 && (c->dim % 32 != 0 || !aligned(c->scales, 4))) return false;
  if (!c->block_table || c->batch < 1 || c->bt_stride < 1 || c->n_phys < 1) return false;
  return true;
}

bool valid_raw_common(const csa_raw_t* r, int dim) {
  if (!r || r->dim != dim || !valid_dtype(r->dtype) || !r->kv_pages || !aligned(r->kv_pages, 16)) return false;
  if (!r->block_table || r->batch < 1 || r->bt_stride < 1 || r->n_phys < 1) return false;
  return true;
}

csa_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return CSA_OK;
  g_last_hip_error = int32_t(e);
  return CSA_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t csa_version(void) { return 1; }

const char* csa_status_string(csa_status_t s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_HIP: return "HIP launch failed";
    case CSA_ERR_TOO_LARGE: return "request exceeds the fixed scratch of a no-allocation entry point";
    default: return "unknown status";
  }
}

int32_t csa_last_hip_error(void) { return g_last_hip_error; }

int64_t csa_num_entries(int64_t n_raw, int32_t ratio, int32_t window) {
  if (!valid_shape(ratio, window)) return -1;
  return n_raw >= window ? (n_raw - window) / ratio + 1 : 0;
}

int64_t csa_num_eligible(int64_t q_pos, int32_t ratio, int32_t window) {
  return csa_num_entries(q_pos + 1, ratio, window);
}

int64_t csa_entry_slot(const int32_t* bt_row, int64_t entry, int32_t ratio) {
  if (!bt_row || entry < 0 || (ratio != 4 && ratio != 128)) return -1;
  const int64_t e = csa::kBlock / ratio;
  return int64_t(bt_row[entry / e]) * e + entry % e;
}

int64_t csa_raw_slot(const int32_t* bt_row, int64_t pos) {
  if (!bt_row || pos < 0) return -1;
  return int64_t(bt_row[pos / csa::kBlock]) * csa::kBlock + pos % csa::kBlock;
}

}  // extern "C"

namespace {

// Host validation of one compress_insert (every check made before any HIP call); fills *out on CSA_OK.
csa_status_t compress_args(const csa_cache_t* cache, const csa_raw_t* state, int32_t batch, const int32_t* start_pos,
                           const int32_t* cu_new, int32_t total_new, int32_t max_new_per_seq, const void* kv_new,
                           const void* logit_new, const float* gamma, float rms_eps, const float* rope_cs,
                           int32_t rope_rows, int32_t* out_slots, int32_t max_entries_out, int32_t* out_new_entries,
                           csa::CompressArgs* out) {
  if (!valid_cache(cache) || !valid_raw_common(state, cache ? cache->dim : -1)) return CSA_ERR_INVALID_ARG;
  if (state->dtype != CSA_F32 && state->dtype != CSA_BF16) return CSA_ERR_INVALID_ARG;
  if (state->roles != cache->window / cache->ratio || !state->logit_pages || !aligned(state->logit_pages, 16))
    return CSA_ERR_INVALID_ARG;
  if (batch < 0 || total_new < 0 || max_new_per_seq < 0) return CSA_ERR_INVALID_ARG;
  if (batch > 0 && (!start_pos || !cu_new || batch > cache->batch || batch > state->batch)) return CSA_ERR_INVALID_ARG;
  if (total_new > 0 && (!kv_new || !logit_new || !aligned(kv_new, 16) || !aligned(logit_new, 16)))
    return CSA_ERR_INVALID_ARG;
  if (!gamma || !(rms_eps >= 0.f) || !isfinite(rms_eps)) return CSA_ERR_INVALID_ARG;
  if (cache->rope_dims > 0 && (!rope_cs || rope_rows < 1)) return CSA_ERR_INVALID_ARG;
  const int bound = (max_new_per_seq + cache->ratio - 1) / cache->ratio;
  if (out_slots && max_entries_out < bound) return CSA_ERR_INVALID_ARG;
  *out = csa::CompressArgs{*cache, *state, batch, start_pos, cu_new, total_new, max_new_per_seq, bound,
                           kv_new, logit_new, gamma, rms_eps, rope_cs, rope_rows, out_slots,
                           out_slots ? max_entries_out : 0, out_new_entries};
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status_t csa_compress_insert(const csa_cache_t* cache, const csa_raw_t* state, int32_t batch,
                                 const int32_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                 int32_t max_new_per_seq, const void* kv_new, const void* logit_new,
                                 const float* gamma, float rms_eps, const float* rope_cs, int32_t rope_rows,
                                 int32_t* out_slots, int32_t max_entries_out, int32_t* out_new_entries,
                                 hipStream_t stream) {
  csa::CompressArgs a;
  const csa_status_t st = compress_args(cache, state, batch, start_pos, cu_new, total_new, max_new_per_seq, kv_new,
                                        logit_new, gamma, rms_eps, rope_cs, rope_rows, out_slots, max_entries_out,
                                        out_new_entries, &a);
  if (st != CSA_OK || batch == 0) return st;
  return hip_status(csa::launch_compress(a, stream));
}

csa_status_t csa_compress_insert_pair(const csa_cache_t* cache_a, const csa_raw_t* state_a, const void* kv_a,
                                      const void* logit_a, const float* gamma_a, const float* rope_cs_a,
                                      int32_t rope_rows_a, const csa_cache_t* cache_b, const csa_raw_t* state_b,
                                      const void* kv_b, const void* logit_b, const float* gamma_b,
                                      const float* rope_cs_b, int32_t rope_rows_b, int32_t batch,
                                      const int32_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                      int32_t max_new_per_seq, float rms_eps, hipStream_t stream) {
  csa::CompressArgs a, b;
  csa_status_t st = compress_args(cache_a, state_a, batch, start_pos, cu_new, total_new, max_new_per_seq, kv_a,
                                  logit_a, gamma_a, rms_eps, rope_cs_a, rope_rows_a, nullptr, 0, nullptr, &a);
  if (st != CSA_OK) return st;
  st = compress_args(cache_b, state_b, batch, start_pos, cu_new, total_new, max_new_per_seq, kv_b, logit_b, gamma_b,
                     rms_eps, rope_cs_b, rope_rows_b, nullptr, 0, nullptr, &b);
  if (st != CSA_OK || batch == 0) return st;
  return hip_status(csa::launch_compress_pair(a, b, stream));
}

size_t csa_index_topk_workspace(int32_t n_q, int64_t max_elig, int32_t k, int32_t n_heads) {
  (void)n_heads;
  if (n_q < 0 || max_elig < 0 || k < 1) return 0;
  return csa::index_workspace(n_q, max_elig, k);
}

}  // extern "C"

namespace {

csa_status_t index_check(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq, const int32_t* q_pos,
                         int64_t max_elig, int32_t k, void* workspace, size_t workspace_bytes) {
  if (!valid_cache(idx_cache) || n_q < 0 || max_elig < 0 || max_elig > 0x7FFFFFFF) return CSA_ERR_INVALID_ARG;
  if (k < 1 || k > csa::kMaxK) return CSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q_seq || !q_pos)) return CSA_ERR_INVALID_ARG;
  const size_t need = csa::index_workspace(n_q, max_elig, k);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return CSA_ERR_WORKSPACE;
  return CSA_OK;
}

csa_status_t score_check(const csa_cache_t* idx_cache, int32_t n_q, const void* q_idx, csa_dtype_t q_dtype,
                         int32_t n_heads, const float* head_w, csa_score_t mode) {
  if (n_heads < 1 || n_heads > 128) return CSA_ERR_INVALID_ARG;
  if (mode != CSA_SCORE_DOT && mode != CSA_SCORE_WRELU) return CSA_ERR_INVALID_ARG;
  if (mode == CSA_SCORE_DOT && n_heads != 1) return CSA_ERR_INVALID_ARG;
  if (q_dtype != CSA_F32 && q_dtype != CSA_BF16) return CSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q_idx || !aligned(q_idx, 16))) return CSA_ERR_INVALID_ARG;
  if (n_q > 0 && mode == CSA_SCORE_WRELU && !head_w) return CSA_ERR_INVALID_ARG;
  if (!csa::index_supported(*idx_cache, q_dtype, n_heads, mode)) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status_t csa_index_workspace_clear(void* workspace, size_t workspace_bytes, int32_t n_q, hipStream_t stream) {
  if (n_q < 0) return CSA_ERR_INVALID_ARG;
  if (n_q == 0) return CSA_OK;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < csa::index_clean_bytes(n_q)) return CSA_ERR_WORKSPACE;
  return hip_status(csa::launch_index_clear(workspace, n_q, stream));
}

csa_status_t csa_index_score(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq, const int32_t* q_pos,
                             int64_t max_elig, const void* q_idx, csa_dtype_t q_dtype, int32_t n_heads,
                             const float* head_w, csa_score_t mode, int32_t k, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  csa_status_t st = index_check(idx_cache, n_q, q_seq, q_pos, max_elig, k, workspace, workspace_bytes);
  if (st != CSA_OK) return st;
  st = score_check(idx_cache, n_q, q_idx, q_dtype, n_heads, head_w, mode);
  if (st != CSA_OK || n_q == 0) return st;
  csa::IndexArgs a{*idx_cache, n_q, q_seq, q_pos, max_elig, q_idx, q_dtype, n_heads, head_w, mode, k,
                   nullptr, nullptr, nullptr, workspace};
  return hip_status(csa::launch_index_score(a, stream));
}

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
                                      hipStream_t stream) {
  csa::CompressArgs a, b;
  csa_status_t st = compress_args(cache_a, state_a, batch, start_pos, cu_new, total_new, max_new_per_seq, kv_a,
                                  logit_a, gamma_a, rms_eps, rope_cs_a, rope_rows_a, nullptr, 0, nullptr, &a);
  if (st != CSA_OK) return st;
  st = compress_args(cache_b, state_b, batch, start_pos, cu_new, total_new, max_new_per_seq, kv_b, logit_b, gamma_b,
                     rms_eps, rope_cs_b, rope_rows_b, nullptr, 0, nullptr, &b);
  if (st != CSA_OK) return st;
  st = index_check(cache_b, n_q, q_seq, q_pos, max_elig, k, workspace, workspace_bytes);
  if (st != CSA_OK) return st;
  st = score_check(cache_b, n_q, q_idx, q_dtype, n_heads, head_w, mode);
  if (st != CSA_OK) return st;
  // the decode form: one new token per sequence, query q = sequence q's token
  if (n_q != batch || total_new != batch || (batch > 0 && max_new_per_seq != 1)) return CSA_ERR_INVALID_ARG;
  if (batch == 0) return CSA_OK;
  csa::IndexArgs ia{*cache_b, n_q, q_seq, q_pos, max_elig, q_idx, q_dtype, n_heads, head_w, mode, k,
                    nullptr, nullptr, nullptr, workspace};
  return hip_status(csa::launch_compress_index_score(a, b, ia, stream));
}

csa_status_t csa_index_select(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq, const int32_t* q_pos,
                              int64_t max_elig, int32_t k, int32_t* out_idx, int32_t* out_count, float* out_scores,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  csa_status_t st = index_check(idx_cache, n_q, q_seq, q_pos, max_elig, k, workspace, workspace_bytes);
  if (st != CSA_OK) return st;
  if (n_q > 0 && !out_idx) return CSA_ERR_INVALID_ARG;
  if (n_q == 0) return CSA_OK;
  csa::IndexArgs a{*idx_cache, n_q, q_seq, q_pos, max_elig, nullptr, CSA_BF16, 1, nullptr, CSA_SCORE_DOT, k,
                   out_idx, out_count, out_scores, workspace};
  return hip_status(csa::launch_index_select(a, stream));
}

csa_status_t csa_index_topk(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq, const int32_t* q_pos,
                            int64_t max_elig, const void* q_idx, csa_dtype_t q_dtype, int32_t n_heads,
                            const float* head_w, csa_score_t mode, int32_t k, int32_t* out_idx, int32_t* out_count,
                            float* out_scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  csa_status_t st = index_check(idx_cache, n_q, q_seq, q_pos, max_elig, k, workspace, workspace_bytes);
  if (st != CSA_OK) return st;
  st = score_check(idx_cache, n_q, q_idx, q_dtype, n_heads, head_w, mode);
  if (st != CSA_OK) return st;
  if (n_q > 0 && !out_idx) return CSA_ERR_INVALID_ARG;
  if (n_q == 0) return CSA_OK;
  csa::IndexArgs a{*idx_cache, n_q, q_seq, q_pos, max_elig, q_idx, q_dtype, n_heads, head_w, mode, k,
                   out_idx, out_count, out_scores, workspace};
  hipError_t e = csa::launch_index_score(a, stream);
  if (e == hipSuccess) e = csa::launch_index_select(a, stream);
  return hip_status(e);
}

}  // extern "C"

namespace {

// Scratch of csa_index_topk_noalloc: a static device array, one copy per GPU (each device's copy is created
// when the library's code object is loaded on it). Host code never passes the array's name to a kernel: in
// host code it is a stand-in, not a device address. Its device address is looked up once per device with
// hipGetSymbolAddress and kept here.
__device__ __align__(256) static uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

csa_status_t csa_index_topk_noalloc(const csa_cache_t* idx_cache, int32_t n_q, const int32_t* q_seq,
                                    const int32_t* q_pos, int64_t max_elig, const void* q_idx, csa_dtype_t q_dtype,
                                    int32_t n_heads, const float* head_w, csa_score_t mode, int32_t k,
                                    int32_t* out_idx, int32_t* out_count, float* out_scores, hipStream_t stream) {
  if (!valid_cache(idx_cache) || n_q < 0 || max_elig < 0 || max_elig > 0x7FFFFFFF) return CSA_ERR_INVALID_ARG;
  if (k < 1 || k > csa::kMaxK) return CSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q_seq || !q_pos)) return CSA_ERR_INVALID_ARG;
  csa_status_t st = score_check(idx_cache, n_q, q_idx, q_dtype, n_heads, head_w, mode);
  if (st != CSA_OK) return st;
  if (n_q > 0 && !out_idx) return CSA_ERR_INVALID_ARG;
  if (csa::index_workspace(n_q, max_elig, k) > CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_TOO_LARGE;
  if (n_q == 0) return CSA_OK;
  void* ws = nullptr;
  hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return hip_status(e);
  csa::IndexArgs a{*idx_cache, n_q, q_seq, q_pos, max_elig, q_idx, q_dtype, n_heads, head_w, mode, k,
                   out_idx, out_count, out_scores, ws};
  // the scratch keeps whatever the previous call on this device left: zero the histogram region first
  e = csa::launch_index_clear(ws, n_q, stream);
  if (e == hipSuccess) e = csa::launch_index_score(a, stream);
  if (e == hipSuccess) e = csa::launch_index_select(a, stream);
  return hip_status(e);
}

size_t csa_attend_workspace(int32_t n_q, int32_t n_heads, int32_t dim, int32_t max_keys) {
  if (n_q < 0 || n_heads < 1 || max_keys < 0) return 0;
  return csa::attend_workspace(n_q, n_heads, dim, max_keys);
}

}  // extern "C"

namespace {

// Validation shared by csa_attend and csa_attend_quant_fp8 (everything but the output buffers); fills *a.
csa_status_t attend_args(const csa_cache_t* kv_cache, const csa_raw_t* swa, int32_t swa_window, int32_t n_q,
                         const int32_t* q_seq, const int32_t* q_pos, const void* q, csa_dtype_t q_dtype,
                         int32_t n_heads, const int32_t* topk_idx, int32_t k, int64_t max_elig, float softmax_scale,
                         int32_t fuse_inv_rope, const float* rope_cs, int32_t rope_rows, void* workspace,
                         size_t workspace_bytes, csa::AttendArgs* a) {
  if (!valid_cache(kv_cache) || !valid_raw_common(swa, kv_cache ? kv_cache->dim : -1)) return CSA_ERR_INVALID_ARG;
  if (kv_cache->dtype == CSA_FP4_E2M1) return CSA_ERR_UNSUPPORTED;  // fp4 is the indexer cache's format
  if (swa->dtype != kv_cache->dtype || swa->roles != 0) return CSA_ERR_INVALID_ARG;
  if (swa->dtype == CSA_FP8_E4M3 && !swa->scales) return CSA_ERR_INVALID_ARG;
  if (swa_window < 0 || swa_window > 1024 || n_q < 0 || n_heads < 1 || n_heads > 128) return CSA_ERR_INVALID_ARG;
  if (topk_idx && (k < 1 || k > csa::kMaxK)) return CSA_ERR_INVALID_ARG;
  if (max_elig < 0 || !isfinite(softmax_scale) || (fuse_inv_rope != 0 && fuse_inv_rope != 1)) return CSA_ERR_INVALID_ARG;
  if (q_dtype != CSA_F32 && q_dtype != CSA_BF16) return CSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q_seq || !q_pos || !q || !aligned(q, 16))) return CSA_ERR_INVALID_ARG;
  if (fuse_inv_rope && kv_cache->rope_dims > 0 && (!rope_cs || rope_rows < 1)) return CSA_ERR_INVALID_ARG;
  if (!csa::attend_supported(*kv_cache, q_dtype, n_heads)) return CSA_ERR_UNSUPPORTED;
  if (int64_t(swa->n_phys) * csa::kBlock > 0x7FFFFFFF) return CSA_ERR_UNSUPPORTED;  // window rows are 32-bit
  const int64_t max_keys = (topk_idx ? int64_t(k) : max_elig) + swa_window;
  const size_t need = max_keys <= 0x7FFFFFFF ? csa::attend_workspace(n_q, n_heads, kv_cache->dim, max_keys) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return CSA_ERR_WORKSPACE;
  *a = csa::AttendArgs{*kv_cache, *swa, swa_window, n_q, q_seq, q_pos, q, q_dtype, n_heads, topk_idx,
                       topk_idx ? k : 0, max_elig, softmax_scale, fuse_inv_rope, rope_cs, rope_rows, nullptr, nullptr,
                       nullptr, nullptr, 0};
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status_t csa_attend(const csa_cache_t* kv_cache, const csa_raw_t* swa, int32_t swa_window, int32_t n_q,
                        const int32_t* q_seq, const int32_t* q_pos, const void* q, csa_dtype_t q_dtype,
                        int32_t n_heads, const int32_t* topk_idx, int32_t k, int64_t max_elig, float softmax_scale,
                        int32_t fuse_inv_rope, const float* rope_cs, int32_t rope_rows, float* out, float* out_lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n_q > 0 && !out) return CSA_ERR_INVALID_ARG;
  csa::AttendArgs a;
  const csa_status_t st = attend_args(kv_cache, swa, swa_window, n_q, q_seq, q_pos, q, q_dtype, n_heads, topk_idx, k,
                                      max_elig, softmax_scale, fuse_inv_rope, rope_cs, rope_rows, workspace,
                                      workspace_bytes, &a);
  if (st != CSA_OK || n_q == 0) return st;
  a.out = out;
  a.out_lse = out_lse;
  return hip_status(csa::launch_attend(a, workspace, workspace_bytes, stream));
}

csa_status_t csa_attend_quant_fp8(const csa_cache_t* kv_cache, const csa_raw_t* swa, int32_t swa_window, int32_t n_q,
                                  const int32_t* q_seq, const int32_t* q_pos, const void* q, csa_dtype_t q_dtype,
                                  int32_t n_heads, const int32_t* topk_idx, int32_t k, int64_t max_elig,
                                  float softmax_scale, const float* rope_cs, int32_t rope_rows, int32_t group,
                                  uint8_t* out_codes, float* out_scales, float* out_lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (group != 16 && group != 32 && group != 64 && group != 128) return CSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!out_codes || !out_scales || !aligned(out_codes, 8) || !aligned(out_scales, 4)))
    return CSA_ERR_INVALID_ARG;
  csa::AttendArgs a;
  csa_status_t st = attend_args(kv_cache, swa, swa_window, n_q, q_seq, q_pos, q, q_dtype, n_heads, topk_idx, k,
                                max_elig, softmax_scale, 1, rope_cs, rope_rows, workspace, workspace_bytes, &a);
  if (st != CSA_OK) return st;
  if (!csa::attend_quant_supported(*kv_cache, q_dtype, n_heads, group)) return CSA_ERR_UNSUPPORTED;
  if (n_q == 0) return CSA_OK;
  a.out_lse = out_lse;
  a.out_codes = out_codes;
  a.out_scales = out_scales;
  a.group = group;
  return hip_status(csa::launch_attend(a, workspace, workspace_bytes, stream));
}

csa_status_t csa_inv_rope(int32_t n_q, int32_t n_heads, int32_t dim, int32_t rope_dims, const int32_t* q_pos,
                          const float* rope_cs, int32_t rope_rows, float* io, hipStream_t stream) {
  if (n_q < 0 || n_heads < 1 || dim < 2 || rope_dims < 0 || rope_dims > dim || (rope_dims & 1)) return CSA_ERR_INVALID_ARG;
  if (n_q > 0 && rope_dims > 0 && (!q_pos || !rope_cs || !io || rope_rows < 1)) return CSA_ERR_INVALID_ARG;
  if (n_q == 0 || rope_dims == 0) return CSA_OK;
  return hip_status(csa::launch_inv_rope(n_q, n_heads, dim, rope_dims, q_pos, rope_cs, rope_rows, io, stream));
}

csa_status_t csa_inv_rope_quant_fp8(int32_t n_q, int32_t n_heads, int32_t dim, int32_t rope_dims,
                                    const int32_t* q_pos, const float* rope_cs, int32_t rope_rows, const float* in,
                                    int32_t group, uint8_t* out_codes, float* out_scales, hipStream_t stream) {
  if (n_q < 0 || n_heads < 1 || n_heads > 128 || !valid_dim(dim)) return CSA_ERR_INVALID_ARG;
  if (rope_dims < 0 || rope_dims > dim || (rope_dims & 1)) return CSA_ERR_INVALID_ARG;
  if (group < 8 || group > 512 || (group & (group - 1)) || dim % group) return CSA_ERR_INVALID_ARG;
  if (n_q == 0) return CSA_OK;
  if (!q_pos || !in || !out_codes || !out_scales || !aligned(in, 16) || !aligned(out_codes, 8) || !aligned(out_scales, 4))
    return CSA_ERR_INVALID_ARG;
  if (rope_dims > 0 && (!rope_cs || rope_rows < 1)) return CSA_ERR_INVALID_ARG;
  return hip_status(csa::launch_inv_rope_quant(n_q, n_heads, dim, rope_dims, q_pos, rope_cs, rope_rows, in, group,
                                               out_codes, out_scales, stream));
}

csa_status_t csa_prepare_qk(int32_t n_tok, int32_t n_heads, const int32_t* tok_seq, const int32_t* tok_pos,
                            const void* q_in, csa_dtype_t q_dtype, const float* q_gamma, float rms_eps,
                            const void* kv_in, const csa_raw_t* swa, int32_t rope_dims, const float* rope_cs,
                            int32_t rope_rows, void* q_out, hipStream_t stream) {
  if (n_tok < 0 || n_heads < 1 || n_heads > 128 || !swa || !valid_dim(swa->dim)) return CSA_ERR_INVALID_ARG;
  if (!valid_raw_common(swa, swa->dim) || swa->roles != 0) return CSA_ERR_INVALID_ARG;
  const bool combo = (q_dtype == CSA_F32 && swa->dtype == CSA_F32) ||
                     (q_dtype == CSA_BF16 && (swa->dtype == CSA_BF16 || swa->dtype == CSA_FP8_E4M3));
  if (!combo) return CSA_ERR_INVALID_ARG;
  if (swa->dtype == CSA_FP8_E4M3 && !swa->scales) return CSA_ERR_INVALID_ARG;
  if (rope_dims < 0 || rope_dims > swa->dim || (rope_dims & 1)) return CSA_ERR_INVALID_ARG;
  if (rope_dims > 0 && (!rope_cs || rope_rows < 1)) return CSA_ERR_INVALID_ARG;
  if (!(rms_eps >= 0.f) || !isfinite(rms_eps)) return CSA_ERR_INVALID_ARG;
  if (n_tok == 0) return CSA_OK;
  if (!tok_seq || !tok_pos || !q_in || !q_out || !q_gamma || !kv_in || !aligned(q_out, 16)) return CSA_ERR_INVALID_ARG;
  csa::PrepareArgs a{n_tok, n_heads, tok_seq, tok_pos, q_in, q_out, q_gamma, rms_eps, kv_in, *swa, rope_dims,
                     rope_cs, rope_rows};
  return hip_status(csa::launch_prepare_qk(a, q_dtype, stream));
}

csa_status_t csa_rope_table(int32_t rows, int32_t rope_dims, double theta, float* rope_cs, hipStream_t stream) {
  if (rows < 0 || rope_dims < 2 || (rope_dims & 1) || !(theta > 0.0) || !isfinite(theta)) return CSA_ERR_INVALID_ARG;
  if (rows > 0 && !rope_cs) return CSA_ERR_INVALID_ARG;
  if (rows == 0) return CSA_OK;
  return hip_status(csa::launch_rope_table(rows, rope_dims, theta, rope_cs, stream));
}

}  // extern "C"
