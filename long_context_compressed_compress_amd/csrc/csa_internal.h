// Internal declarations and device helpers of libcsa (gfx950 only).
//
// Element codecs (bf16 round-to-nearest-even, OCP e4m3fn), order-preserving score keys,
// paging arithmetic, and the launchers each kernel file exports to the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int kBlock = 256;      // raw positions per logical block
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kHistBits = 12;    // first radix digit of the top-k select (bits 31..20 of the key)
constexpr int kHistBins = 1 << kHistBits;
constexpr int kMaxK = 2048;

// ------------------------------------------------------------------ synchronisation
// Workgroup barrier that orders LDS only. __syncthreads() also fences global memory, which on gfx950
// waits for every outstanding vector load (vmcnt(0)) and so drains prefetches issued before it; kernels
// whose waves share nothing but LDS across a barrier use this instead. The "memory" clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ element codecs
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// OCP e4m3fn: bias 7, 3 mantissa bits, S.1111.111 = NaN, max 448, subnormal step 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 0x7u;
  if (e == 0xFu && m == 0x7u) return __uint_as_float(0x7FC00000u | s);
  if (e == 0) return __uint_as_float(s | __float_as_uint(float(m) * 0.001953125f));  // m * 2^-9, exact
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// Round-to-nearest-even into e4m3fn with saturation at +-448 (input finite).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t s = (u >> 24) & 0x80u;
  float a = fabsf(f);
  if (!(a < 464.0f)) return s | 0x7Eu;  // >= 464 rounds above 448 -> saturate (also NaN -> 448; never produced here)
  if (a < 0.015625f) {                   // below 2^-6: subnormal grid m * 2^-9, m in 0..8
    const float m = rintf(a * 512.0f);   // exact scaling, rintf = ties to even
    return s | uint32_t(m);              // m == 8 encodes 2^-6 (exponent 1, mantissa 0): 8 = 0b0001000
  }
  uint32_t au = __float_as_uint(a);
  // keep 3 mantissa bits with round-to-nearest-even on the dropped 20 bits
  au += 0x7FFFFu + ((au >> 20) & 1u);
  const uint32_t e = (au >> 23) - 120u;  // biased e4m3 exponent (>= 1 here)
  const uint32_t m = (au >> 20) & 0x7u;
  uint32_t code = (e << 3) | m;
  if (code > 0x7Eu) code = 0x7Eu;
  return s | code;
}

// Nearest e2m1 code (ties to the code with mantissa bit 0, saturation at 6) of a finite value; bit 3 is
// the sign, set for every negative input. Magnitudes by code: 0, 0.5, 1, 1.5, 2, 3, 4, 6; each comparison
// below is against a midpoint, strict where the lower code is the even one of the tie.
__device__ __forceinline__ uint32_t f32_to_e2m1_rne(float f) {
  const float a = fabsf(f);
  const uint32_t m = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                     uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
  return m | (f < 0.f ? 8u : 0u);
}

// Order-preserving 32-bit key of an fp32 score: larger score -> larger key.
// -0 is folded onto +0 and every NaN maps to 0 (below -inf).
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ------------------------------------------------------------------ paging
// Entries eligible at position p (window end <= p).
__host__ __device__ __forceinline__ int64_t num_eligible(int64_t p, int ratio, int window) {
  const int64_t n = p + 1;
  return n >= window ? (n - window) / ratio + 1 : 0;
}

// Page row of entry i of block-table row `bt`, or -1 when the table does not map it. The table load is
// unconditional (index clamped into the row, which is at least one block wide), so it can be issued early and
// overlap other loads: a load inside a branch is waited for before the branch closes.
__device__ __forceinline__ int64_t entry_row(const int32_t* bt, int bt_stride, int n_phys, int64_t i, int per_block) {
  const int64_t blk = i / per_block;
  const bool in = i >= 0 && blk < bt_stride;
  const int32_t phys = bt[in ? blk : 0];
  return (in && phys >= 0 && phys < n_phys) ? int64_t(phys) * per_block + (i - blk * per_block) : -1;
}

__device__ __forceinline__ int64_t raw_row(const int32_t* bt, int bt_stride, int n_phys, int64_t pos) {
  return entry_row(bt, bt_stride, n_phys, pos, kBlock);
}

__host__ __device__ __forceinline__ int elem_bytes(csa_dtype_t t) { return t == CSA_F32 ? 4 : (t == CSA_BF16 ? 2 : 1); }

// ------------------------------------------------------------------ launchers (one per kernel file)
struct CompressArgs {
  csa_cache_t cache;
  csa_raw_t state;
  int batch;
  const int32_t* start_pos;
  const int32_t* cu_new;
  int total_new, max_new_per_seq, max_entries_bound;
  const void* kv_new;
  const void* logit_new;
  const float* gamma;
  float eps;
  const float* rope_cs;
  int rope_rows;
  int32_t* out_slots;
  int max_entries_out;
  int32_t* out_new_entries;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);
hipError_t launch_compress_pair(const CompressArgs& a, const CompressArgs& b, hipStream_t stream);

struct IndexArgs {
  csa_cache_t cache;
  int n_q;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int64_t max_elig;
  const void* q;
  csa_dtype_t q_dtype;
  int n_heads;
  const float* head_w;
  csa_score_t mode;
  int k;
  int32_t* out_idx;
  int32_t* out_count;
  float* out_scores;
  void* ws;
};
size_t index_workspace(int n_q, int64_t max_elig, int k);
size_t index_clean_bytes(int n_q);
bool index_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads, csa_score_t mode);
hipError_t launch_index_clear(void* ws, int n_q, hipStream_t stream);
hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream);
hipError_t launch_index_select(const IndexArgs& a, hipStream_t stream);
// The decode step's compress_insert of a c4a main cache and its indexer cache, done inside the index-score launch
// where the configuration allows (else the two launches in turn); one new token per sequence, query q = sequence q.
struct FusedCompress {
  CompressArgs main, idx;
};
hipError_t launch_compress_index_score(const CompressArgs& main, const CompressArgs& idx, const IndexArgs& a,
                                       hipStream_t stream);

struct AttendArgs {
  csa_cache_t cache;
  csa_raw_t swa;
  int swa_window;
  int n_q;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const void* q;
  csa_dtype_t q_dtype;
  int n_heads;
  const int32_t* topk;
  int k;
  int64_t max_elig;
  float scale;
  int fuse_inv_rope;
  const float* rope_cs;
  int rope_rows;
  float* out;
  float* out_lse;
  // fp8 output (out == nullptr): inverse-rotated rows stored as grouped e4m3 codes [n_q][H][D] and one fp32 scale
  // per `group` channels [n_q][H][D / group]
  uint8_t* out_codes;
  float* out_scales;
  int group;
};
bool attend_quant_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads, int group);
bool attend_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads);
size_t attend_workspace(int n_q, int n_heads, int dim, int64_t max_keys);
hipError_t launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);

hipError_t launch_inv_rope(int n_q, int n_heads, int dim, int rope_dims, const int32_t* q_pos, const float* rope_cs,
                           int rope_rows, float* io, hipStream_t stream);
hipError_t launch_rope_table(int rows, int rope_dims, double theta, float* out, hipStream_t stream);
struct PrepareArgs {
  int n_tok, n_heads;
  const int32_t* tok_seq;
  const int32_t* tok_pos;
  const void* q_in;
  void* q_out;
  const float* gamma;
  float eps;
  const void* kv_in;
  csa_raw_t swa;
  int rope_dims;
  const float* rope_cs;
  int rope_rows;
};
hipError_t launch_prepare_qk(const PrepareArgs& a, csa_dtype_t q_dtype, hipStream_t stream);
hipError_t launch_inv_rope_quant(int n_q, int n_heads, int dim, int rope_dims, const int32_t* q_pos,
                                 const float* rope_cs, int rope_rows, const float* in, int group, uint8_t* codes,
                                 float* scales, hipStream_t stream);

}  // namespace csa
