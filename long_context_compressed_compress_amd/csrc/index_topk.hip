// csa_index_topk kernels: indexer score over the eligible compressed entries of each query,
// then an exact radix top-k select with ties to the lower entry index.
//
// [P1] "DeepSeek V4 Attention Architecture" and [P2] "二、注意力機制為什么這么麻煩": DeepSeek Sparse
// Attention attends only to the top-k compressed entries (k = 512 on c4a layers). [P2] "3.2 內核": the
// indexer pipeline (its own compressor instance, score, top-k) is separate from the main cache.
//
// Two launches on the caller's stream (csa_index_score, then csa_index_select):
//   1. score     -- one workgroup per (query, run of pages). WRELU with 16*HT heads over dim-128
//                   bf16 / fp8 / MXFP4 keys runs on MFMA (v_mfma_f32_16x16x32_bf16: heads x 16 entries x 32
//                   dims per instruction; fp8 and fp4 codes widened exactly to bf16, fp4 with its block's
//                   power-of-two scale folded in); bf16 / fp8 pages are loaded 1 KiB per instruction and
//                   transposed through LDS (score_lt_kernel), fp4 pages straight into operand layout
//                   (score_mfma_kernel), a prefill launch shares pages among 8 queries (score_shared_kernel);
//                   other shapes run on a VALU path (not for fp4).
//                   Each score becomes an order-preserving 32-bit key; a 4096-bin LDS histogram of
//                   the top 12 key bits is flushed into the query's global histogram.
//   2. select    -- one 1024-thread workgroup per query: find the histogram bin that holds the k-th
//                   largest key; in one pass over the query's keys mark the keys above it in a bitmap of
//                   chosen entries and list the keys inside it (candidates) with a second histogram of
//                   their next 12 bits; resolve the last 8 bits and exact ties (ascending index) over the
//                   candidates, read the bitmap in word order for an index-sorted output, then re-zero
//                   the query's histogram. The workspace's histogram region therefore only needs zeroing
//                   once (csa_index_workspace_clear).
// The chosen set is unique (score order plus index order is total), so the result does not depend
// on how work is split or on the order of atomics.
#include "compress_unit.h"

namespace csa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;


struct Workspace {
  uint32_t* hist;   // [n_q][kHistBins]: score histogram of key bits 31..20
  uint32_t* hist2;  // [n_q][kHistBins]: bits 19..8 of the boundary-bin candidates (pre-marked selects)
  uint32_t* ncand;  // [n_q]: candidates listed by the mark pass (pre-marked selects)
  uint32_t* keys;   // [n_q][key_stride]: order-preserving score keys (rows 256-byte aligned)
  uint2* cand;      // [n_q][max_elig] (key, index): candidates beyond the LDS list
  uint32_t* bits;   // [n_q][bits_stride]: chosen-entry bitmap (long queries, pre-marked selects)
  int64_t bits_stride;
  int64_t key_stride;  // max_elig rounded up to a multiple of 64
};

__host__ __device__ inline int64_t key_stride_of(int64_t max_elig) { return (max_elig + 63) / 64 * 64; }

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline size_t clean_bytes(int n_q) {
  return 2 * align256(size_t(n_q) * kHistBins * 4) + align256(size_t(n_q) * 4);
}

// Layout: [hist][hist2][ncand] (the region that must be zero between calls), then [keys][cand][bits].
__host__ __device__ inline Workspace carve(void* base, int n_q, int64_t max_elig) {
  char* p = static_cast<char*>(base);
  Workspace w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(n_q) * kHistBins * 4);
  w.hist2 = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(n_q) * kHistBins * 4);
  w.ncand = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(n_q) * 4);
  w.keys = reinterpret_cast<uint32_t*>(p);
  w.key_stride = key_stride_of(max_elig);
  p += align256(size_t(n_q) * size_t(w.key_stride) * 4);
  w.cand = reinterpret_cast<uint2*>(p);
  p += align256(size_t(n_q) * size_t(max_elig) * 8);
  w.bits_stride = (max_elig + 31) / 32;
  w.bits = reinterpret_cast<uint32_t*>(p);
  return w;
}

__device__ __forceinline__ int64_t query_elig(const IndexArgs& a, int q, int* seq_out) {
  const int seq = a.q_seq[q];
  *seq_out = seq;
  if (seq < 0 || seq >= a.cache.batch) return 0;
  int64_t n = num_eligible(a.q_pos[q], a.cache.ratio, a.cache.window);
  if (n > a.max_elig) n = a.max_elig;
  if (n < 0) n = 0;
  return n;
}

__global__ void clear_kernel(uint32_t* clean, int64_t n_words) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words; i += int64_t(gridDim.x) * blockDim.x)
    clean[i] = 0u;
}

__device__ __forceinline__ void flush_hist(uint32_t* hist_s, uint32_t* hist_q) {
  __syncthreads();
  for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) {
    const uint32_t v = hist_s[b];
    if (v) atomicAdd(hist_q + b, v);
  }
}

// ------------------------------------------------------------------ MFMA score (WRELU, dim 128, c4a pages)
// Work unit: one 64-entry page (bf16: 16 KiB, fp8: 8 KiB, contiguous). A wavefront walks its pages with the
// next page's loads in flight while the current page runs through MFMA. Lane l feeds MFMA column l%16 of
// each 16-entry tile with dims (l/16)*8 .. +8 of every 32-dim k-step; after the head reduction all four lane
// groups hold the 16 scores of a tile, and lane l keeps the score of entry l of the page, so each page ends
// in one coalesced 256-byte key store.
constexpr int kPagesPerBlock = 32;
constexpr int kQueryFastMin = 256;  // queries per launch from which workgroups share pages among queries

// Key formats of the MFMA score: 0 bf16, 1 fp8 e4m3 (per-entry scale), 2 MXFP4 (per-32-channel E8M0 scale).
// bf16 and fp8 lanes feed dims ks*32 + kg*8 .. +8 of k-step ks; an fp4 lane feeds dims kg*32 + ks*8 .. +8,
// so its four k-steps are one contiguous 32-channel block (16 B, one scale) and the query fragments follow
// the same permutation (a dot product does not depend on the order of its terms).
template <int KF>
struct PageBuf;
template <>
struct PageBuf<0> { uint4 v[4][4]; };  // [tile][k-step] 16 B
template <>
struct PageBuf<1> { uint2 v[4][4]; float sc[4]; };  // 8 B codes + per-tile-column scale
template <>
struct PageBuf<2> { uint4 v[4]; float sc[4]; };  // [tile] 32 codes of the lane's block + that block's 2^X

// E8M0 byte -> 2^(e-127) as fp32 (e = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

template <int KF>
__device__ __forceinline__ void load_page(PageBuf<KF>& b, const void* pages, const float* scales, int64_t row0,
                                          int col, int kg) {
  constexpr int DIM = 128;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t row = row0 + u * 16 + col;
    if constexpr (KF == 2) {
      b.v[u] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(pages) + row * (DIM / 2) + kg * 16);
      b.sc[u] = e8m0_to_f32(reinterpret_cast<const uint8_t*>(scales)[row * (DIM / 32) + kg]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (KF == 1)
          b.v[u][ks] = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(pages) + row * DIM + ks * 32 + kg * 8);
        else
          b.v[u][ks] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(pages) + row * DIM + ks * 32 + kg * 8);
      }
      if constexpr (KF == 1) b.sc[u] = scales[row];
    }
  }
}

// 8 e2m1 codes (one 32-bit word, channel 2j in the low nibble of byte j) -> 8 bf16 times the block scale
// 2^X (hardware OCP fp4 -> bf16 conversion; exact, since a power-of-two multiple of an e2m1 value has at
// most two significant bits).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8_hw(uint32_t w, float scale) {
  const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8, make_uint4(o0, o1, o2, o3));
}

// 8 e4m3fn codes -> 8 bf16: the gfx950 scaled conversion of a pair of OCP e4m3 codes straight to a bf16 pair, with
// scale 1 (exact: every e4m3 value, subnormals included, is a bf16 value); one instruction per pair instead of a
// conversion to f32 and a byte permute.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8_hw(uint2 v) {
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t x = h ? v.y : v.x;
    w[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
    w[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
  }
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// ReLU of an MFMA result as one v_med3_f32 (the median of x, 0 and +inf). fmaxf(x, 0) costs two instructions here:
// the compiler first quiets a possible signalling NaN in the MFMA result. The infinity passes through an empty asm
// statement so that the optimiser cannot fold the median back into fmaxf. For every non-NaN x the value is
// fmaxf(x, 0)'s, up to the sign of a zero result, which adds nothing to the weighted sums it feeds (they start at +0).
// The prefill score (pages shared by 8 queries, bound by MFMA and VALU issue: 4.67 -> 4.16 ms for 2 x 2048 queries
// at 256K) and the fp8 and MXFP4 decode scores take it (1M-entry decode 2.5 % and 5 % faster); the bf16 decode score
// keeps fmaxf, which measured 2 % faster there (that kernel waits on HBM, not on instruction issue).
__device__ __forceinline__ float opaque_inf() {
  float v = __builtin_inff();
  asm("" : "+v"(v));
  return v;
}
__device__ __forceinline__ float relu_med3(float x, float inf) { return __builtin_amdgcn_fmed3f(x, 0.f, inf); }

// Sum over the four 16-lane rows of a wave, on the VALU: rows (0, 1) and (2, 3) first (16-lane swap), then the two
// pair sums (32-lane swap); every lane ends with (x0 + x1) + (x2 + x3).
__device__ __forceinline__ float rows4_sum_pairs(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int KF, int HT>
__device__ __forceinline__ uint32_t score_page(const PageBuf<KF>& b, const bf16x8 (&qa)[HT][4],
                                               const float (&wv)[HT][4], int kg) {
  uint32_t mine = 0u;
  float mine_f = 0.f;
  const float inf = opaque_inf();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    bf16x8 kb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if constexpr (KF == 2) {
        const uint4 c = b.v[u];
        kb[ks] = fp4x8_to_bf16x8_hw(ks == 0 ? c.x : ks == 1 ? c.y : ks == 2 ? c.z : c.w, b.sc[u]);
      } else if constexpr (KF == 1) {
        kb[ks] = fp8x8_to_bf16x8_hw(b.v[u][ks]);
      } else {
        kb[ks] = __builtin_bit_cast(bf16x8, b.v[u][ks]);
      }
    }
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][ks], kb[ks], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wv[ht][i] * relu_med3(acc[i], inf);
    }
    part = rows4_sum_pairs(part);
    if constexpr (KF == 1) part *= b.sc[u];
    if (kg == u) mine_f = part;
  }
  mine = score_key(mine_f);
  return mine;
}

// The decode step's compress_insert of both caches run inside the index-score launch (csa_compress_index_score):
// one new token per sequence, query q being sequence q's token. The workgroup that scores query q's last page
// (run 0 when the query has none) first runs sequence q's four compress units, one per wave (indexer append and
// entry, main append and entry), then a barrier: the entry the query's own token completes is in that page before
// any wave of the workgroup reads it, and no other workgroup reads that page. OA: main cache output type
// (1 bf16, 2 fp8); the indexer output type follows the page format KF (bf16, fp8, MXFP4).
template <int KF, int OA>
__device__ __forceinline__ void fused_compress(const FusedCompress& fc, int b) {
  constexpr int OB = KF == 0 ? 1 : (KF == 1 ? 2 : 3);
  switch (threadIdx.x >> 6) {  // wave-uniform
    case 0: compress_unit<uint16_t, OB, 128, 4, 8>(fc.idx, b); break;
    case 1: compress_unit<uint16_t, OB, 128, 4, 8>(fc.idx, int64_t(fc.idx.total_new) + b); break;
    case 2: compress_unit<uint16_t, OA, 512, 4, 8>(fc.main, b); break;
    default: compress_unit<uint16_t, OA, 512, 4, 8>(fc.main, int64_t(fc.main.total_new) + b); break;
  }
}

// Decode score for MXFP4 pages: one workgroup per (query, run of pages), blockIdx.x = run. An fp4 row is 64 bytes,
// so the operand-layout loads of a 16-entry tile read whole 128-byte lines and no LDS stage is needed.
template <int KF, int HT, int OA = 0>
__global__ void __launch_bounds__(256, 2) score_mfma_kernel(IndexArgs a, Workspace ws, int run, FusedCompress fc) {
  constexpr int DIM = 128;
  constexpr int E = 64;
  __shared__ uint32_t hist_s[kHistBins];
  __shared__ int32_t pg_phys[kPagesPerBlock];  // physical page of each page of this block, -1 if unmapped
  const int q = blockIdx.y;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  const int64_t n_pages = (n_elig + E - 1) / E;
  const int64_t pg_begin = int64_t(blockIdx.x) * run;
  if constexpr (OA != 0) {
    if (int64_t(blockIdx.x) == (n_pages > 0 ? (n_pages - 1) / run : 0)) {  // uniform per block
      fused_compress<KF, OA>(fc, q);
      __syncthreads();
    }
  }
  if (pg_begin >= n_pages) return;  // uniform per block
  const int64_t pg_end = min(n_pages, pg_begin + run);
  for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) hist_s[b] = 0u;
  if (threadIdx.x < kPagesPerBlock) {
    const int64_t pg = pg_begin + threadIdx.x;
    const int32_t* bt = a.cache.block_table + int64_t(seq) * a.cache.bt_stride;
    const int32_t phys = (pg < pg_end && pg < a.cache.bt_stride) ? bt[pg] : -1;
    pg_phys[threadIdx.x] = (phys >= 0 && phys < a.cache.n_phys) ? phys : -1;
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int H = HT * 16;

  bf16x8 qa[HT][4];
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + int64_t(q) * H * DIM;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                  qp + (ht * 16 + col) * DIM + (KF == 2 ? kg * 32 + ks * 8 : ks * 32 + kg * 8)));
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = a.head_w[int64_t(q) * H + ht * 16 + kg * 4 + i];
  __syncthreads();

  uint32_t* keys_q = ws.keys + int64_t(q) * ws.key_stride;
  // this wave's pages: pg_begin + wave, +4, ... < pg_end
  const int64_t first = __builtin_amdgcn_readfirstlane(int(pg_begin + wave));
  const int n_mine = first < pg_end ? int((pg_end - 1 - first) / 4 + 1) : 0;
  auto page_row = [&](int j, bool* ok) -> int64_t {
    const int slot = wave + 4 * (j < n_mine ? j : n_mine - 1);
    const int32_t phys = pg_phys[slot];
    *ok = phys >= 0;
    return int64_t(*ok ? phys : 0) * E;
  };
  auto finish = [&](int j, uint32_t key, bool ok) {
    const int64_t e = (first + 4 * int64_t(j)) * E + lane;
    if (e < n_elig) {
      const uint32_t k2 = ok ? key : 0u;
      keys_q[e] = k2;
      atomicAdd(&hist_s[k2 >> (32 - kHistBits)], 1u);
    }
  };
  if (n_mine > 0) {
    PageBuf<KF> b0, b1;
    bool ok0, ok1;
    load_page<KF>(b0, a.cache.pages, a.cache.scales, page_row(0, &ok0), col, kg);
    for (int j = 0; j < n_mine; j += 2) {
      load_page<KF>(b1, a.cache.pages, a.cache.scales, page_row(j + 1, &ok1), col, kg);
      finish(j, score_page<KF, HT>(b0, qa, wv, kg), ok0);
      load_page<KF>(b0, a.cache.pages, a.cache.scales, page_row(j + 2, &ok0), col, kg);
      if (j + 1 < n_mine) finish(j + 1, score_page<KF, HT>(b1, qa, wv, kg), ok1);
    }
  }
  flush_hist(hist_s, ws.hist + int64_t(q) * kHistBins);
}

// ------------------------------------------------------------------ MFMA score, pages shared by queries (prefill)
// A prefill chunk has thousands of queries per sequence that all read the same pages, so a workgroup of kShareQ
// waves takes kShareQ consecutive queries (one per wave) and brings every page of its run into LDS once for all of
// them. Pages are copied global -> LDS by global_load_lds (no register staging) into a ring of kShareBufs buffers,
// and scored two per workgroup barrier while the next two are in flight. In LDS, the 16-byte chunk c of page row r sits at chunk
// c ^ (r & (chunks per row - 1)) of its row (the copy picks its source chunks accordingly), so the operand reads of
// 16 rows at one column fall in different banks. Each wave scores the page for its own query with score_page (the
// same arithmetic as the decode kernels, so the scores are identical). Queries of a workgroup that belong to
// different sequences are processed in successive rounds, one sequence per round.
constexpr int kShareQ = 8;
constexpr int kShareThreads = 64 * kShareQ;
constexpr int kShareBufs = 4;  // two pages being scored, two in flight

// Page geometry per key format (KF as for PageBuf): 64 rows of ROW bytes; a page is DMAS copies of 1 KiB, plus for
// fp8 / fp4 one 256-byte copy of its 64 scale words (fp8: the entry's fp32 scale; fp4: its four E8M0 bytes).
template <int KF>
struct SharedPage {
  static constexpr int ROW = KF == 1 ? 128 : (KF == 2 ? 64 : 256);
  static constexpr int BYTES = 64 * ROW;
  static constexpr int CPR = ROW / 16;  // 16-byte chunks per row
  static constexpr int DMAS = BYTES / 1024;
};

// LDS byte offset of bytes [16 c + o, ...) of page row r, 0 <= o < 16.
template <int KF>
__device__ __forceinline__ int swz(int r, int c, int o) {
  using L = SharedPage<KF>;
  return r * L::ROW + ((c ^ (r & (L::CPR - 1))) << 4) + o;
}

// 64 x 4 bytes from global memory into LDS: lane l moves bytes [4 l, 4 l + 4) to lds_byte + 4 l. Like dma_row,
// issued from inline assembly with no output register; the kernel orders it with vmcnt waits and barriers.
__device__ __forceinline__ void dma_words(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_byte), "v"(src) : "m0");
}
__device__ __forceinline__ void dma_chunks(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_byte), "v"(src) : "m0");
}

template <int KF, int HT>
__global__ void __launch_bounds__(kShareThreads, 1) score_shared_kernel(IndexArgs a, Workspace ws) {
  using L = SharedPage<KF>;
  constexpr int DIM = 128;
  constexpr int E = 64;
  // per-query histograms with two 16-bit bins per word (a workgroup counts at most kPagesPerBlock * 64 keys
  // per query)
  __shared__ uint32_t hist_s[kShareQ][kHistBins / 2];
  __shared__ __attribute__((aligned(16))) char page_s[kShareBufs][L::BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t scale_s[kShareBufs][E];
  __shared__ int32_t pg_phys[kPagesPerBlock];
  __shared__ int32_t w_seq[kShareQ];
  __shared__ int32_t w_npages[kShareQ];
  __shared__ int32_t round_seq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int H = HT * 16;
  const int q = blockIdx.x * kShareQ + wave;
  const bool q_ok = q < a.n_q;
  int seq = -1;
  const int64_t n_elig = q_ok ? query_elig(a, q, &seq) : 0;
  const int64_t pg_begin = int64_t(blockIdx.y) * kPagesPerBlock;
  const int64_t n_pages = (n_elig + E - 1) / E;
  for (int b = tid; b < kShareQ * kHistBins / 2; b += kShareThreads) (&hist_s[0][0])[b] = 0u;
  if (lane == 0) {
    w_seq[wave] = (n_pages > pg_begin) ? seq : -1;  // -1: nothing of this run to score
    w_npages[wave] = int32_t(min<int64_t>(n_pages, pg_begin + kPagesPerBlock));
  }
  // this wave's query operands and head weights (registers for the whole kernel)
  bf16x8 qa[HT][4];
  float wv[HT][4];
  {
    const int qq = q_ok ? q : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + int64_t(qq) * H * DIM;
    if constexpr (KF == 2) {  // the fp4 channel order of score_page
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qa[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + (ht * 16 + col) * DIM + kg * 32 + ks * 8));
    } else {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qa[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + (ht * 16 + col) * DIM + ks * 32 + kg * 8));
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[ht][i] = a.head_w[int64_t(qq) * H + ht * 16 + kg * 4 + i];
  }
  uint32_t* keys_q = ws.keys + int64_t(q_ok ? q : 0) * ws.key_stride;
  const char* pages = static_cast<const char*>(a.cache.pages);
  const uint32_t* scales = reinterpret_cast<const uint32_t*>(a.cache.scales);
  __syncthreads();

  bool done = w_seq[wave] < 0;  // per wave; the round bookkeeping below is uniform over the workgroup
  for (int round = 0; round < kShareQ; ++round) {
    if (tid == 0) {
      int rs = -1;
      for (int w = kShareQ - 1; w >= 0; --w)
        if (w_seq[w] >= 0) rs = w_seq[w];  // the first wave's sequence not done yet
      round_seq = rs;
    }
    __syncthreads();
    const int rseq = round_seq;
    if (rseq < 0) break;  // uniform
    const bool active = !done && w_seq[wave] == rseq;
    int64_t run_end = pg_begin;
    for (int w = 0; w < kShareQ; ++w)
      if (w_seq[w] == rseq) run_end = max<int64_t>(run_end, w_npages[w]);
    const int n_pg = int(run_end - pg_begin);
    if (tid < kPagesPerBlock) {
      const int64_t pg = pg_begin + tid;
      const int32_t* bt = a.cache.block_table + int64_t(rseq) * a.cache.bt_stride;
      const int32_t phys = (pg < run_end && pg < a.cache.bt_stride) ? bt[pg] : -1;
      pg_phys[tid] = (phys >= 0 && phys < a.cache.n_phys) ? phys : -1;
    }
    __syncthreads();
    // this wave's share of the copies of page i of the run (i past the run re-copies the last page into a buffer
    // nobody reads)
    auto issue = [&](int i) {
      const int ii = i < n_pg ? i : n_pg - 1;
      const int32_t phys = pg_phys[ii];
      const int64_t page = phys >= 0 ? phys : 0;
      const int buf = i % kShareBufs;
      const char* src = pages + page * L::BYTES;
      const uint32_t dst = uint32_t(reinterpret_cast<uintptr_t>(page_s[buf]));
      // page copy j covers LDS bytes [1024 j, 1024 j + 1024): lane l writes chunk l % CPR of row
      // (1024 j) / ROW + l / CPR, which holds source chunk (l % CPR) ^ (row & (CPR - 1))
      auto page_copy = [&](int j) {
        const int r = (1024 / L::ROW) * j + lane / L::CPR;
        const int c = (lane % L::CPR) ^ (r & (L::CPR - 1));
        dma_chunks(src + r * L::ROW + c * 16, dst + 1024 * j);
      };
      if constexpr (KF == 0) {
        page_copy(2 * wave);
        page_copy(2 * wave + 1);
      } else if constexpr (KF == 1) {
        page_copy(wave);
        if (wave == 0) dma_words(scales + page * E + lane, uint32_t(reinterpret_cast<uintptr_t>(scale_s[buf])));
      } else {
        if (wave < 4) page_copy(wave);
        else if (wave == 4) dma_words(scales + page * E + lane, uint32_t(reinterpret_cast<uintptr_t>(scale_s[buf])));
      }
    };
    // pages are scored two per barrier: pages 2k and 2k + 1 are read while pages 2k + 2 and 2k + 3 are in flight
#pragma unroll
    for (int s = 0; s < 2; ++s) issue(s);
    for (int i0 = 0; i0 < n_pg; i0 += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of pages i0, i0 + 1 have landed
      lds_barrier();  // every wave's copies landed; every wave is done with pages i0 - 2 and i0 - 1
      issue(i0 + 2);  // into the buffers of pages i0 - 2 and i0 - 1
      issue(i0 + 3);
      if (active) {  // both pages in one basic block (a page past the run scores a re-copied page, not stored)
        PageBuf<KF> b[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const char* buf = page_s[(i0 + h) % kShareBufs];
          const uint32_t* sc = scale_s[(i0 + h) % kShareBufs];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = u * 16 + col;
            if constexpr (KF == 2) {
              b[h].v[u] = *reinterpret_cast<const uint4*>(buf + swz<KF>(r, kg, 0));
              b[h].sc[u] = e8m0_to_f32((sc[r] >> (8 * kg)) & 0xFFu);
            } else {
#pragma unroll
              for (int ks = 0; ks < 4; ++ks) {
                if constexpr (KF == 1)
                  b[h].v[u][ks] = *reinterpret_cast<const uint2*>(buf + swz<KF>(r, ks * 2 + (kg >> 1), (kg & 1) * 8));
                else
                  b[h].v[u][ks] = *reinterpret_cast<const uint4*>(buf + swz<KF>(r, ks * 4 + kg, 0));
              }
              if constexpr (KF == 1) b[h].sc[u] = __uint_as_float(sc[r]);
            }
          }
        }
        uint32_t key[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) key[h] = score_page<KF, HT>(b[h], qa, wv, kg);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = i0 + h;
          const int64_t pg = pg_begin + i;
          const int64_t e = pg * E + lane;
          if (i < n_pg && pg < w_npages[wave] && e < n_elig) {
            const uint32_t k2 = pg_phys[i] >= 0 ? key[h] : 0u;
            keys_q[e] = k2;
            const uint32_t bin = k2 >> (32 - kHistBits);
            atomicAdd(&hist_s[wave][bin >> 1], 1u << ((bin & 1u) * 16));
          }
        }
      }
    }
    // the copies are invisible to the compiler's wait tracking: none may be in flight when the next round
    // rewrites the buffers or the workgroup ends
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (active) done = true;
    __syncthreads();
    if (lane == 0 && active) w_seq[wave] = -1;
    __syncthreads();
  }
  if (q_ok) {
    uint32_t* hq = ws.hist + int64_t(q) * kHistBins;
    for (int b = lane; b < kHistBins / 2; b += 64) {
      const uint32_t v = hist_s[wave][b];
      if (v & 0xFFFFu) atomicAdd(hq + 2 * b, v & 0xFFFFu);
      if (v >> 16) atomicAdd(hq + 2 * b + 1, v >> 16);
    }
  }
}

// ------------------------------------------------------------------ MFMA score with contiguous page loads (decode)
// Each wavefront walks its own pages (no workgroup barrier in the loop) with all heads of the query in registers,
// like score_mfma_kernel, but loads a page the way HBM serves it best: every load instruction reads 1 KiB of
// consecutive bytes (full 128-byte lines). The MFMA operand layout wants 16 rows x 64 bytes per instruction instead,
// i.e. half of 16 lines, which costs about 10% of gather bandwidth when MFMA work runs beside it; so the page is
// written to a private LDS stage of the wave and read back in operand layout. kLtAhead pages per wave stay in
// flight in registers. The scores are exactly score_page's.
constexpr int kLtPages = 32;  // pages per workgroup run (8 per wave)
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;  // plain vector: loads and stores
                                                                                // of it stay in registers

template <int KF>
struct LtPage {
  static constexpr int RAW_ROW = KF == 1 ? 128 : (KF == 2 ? 64 : 256);  // bytes per page row in HBM
  static constexpr int ROW = RAW_ROW + 16;                              // LDS bytes per row (rows 4 banks apart)
  static constexpr int LOADS = 64 * RAW_ROW / 1024;                     // 1 KiB load instructions per page: 16, 8, 4
  static constexpr int AHEAD = 2;                                       // pages in flight per wave
};

// Page `phys` (clamped to 0 when unmapped) -> this lane's registers: 16 bytes of each 1 KiB of the page; fp8 / fp4:
// lane l also takes entry l's scale word (fp8 scale bits, fp4 the four E8M0 bytes). bf16 page loads are non-temporal
// (each page is read once per step): 9 % faster on the 128K bf16 decode score than cached loads; on fp8 pages they
// measured no faster, so those stay cached.
template <int KF>
__device__ __forceinline__ void lt_fetch(const IndexArgs& a, int32_t phys, int lane, u32x4 (&c)[LtPage<KF>::LOADS],
                                         uint32_t& sc) {
  using L = LtPage<KF>;
  const int64_t page = phys >= 0 ? phys : 0;
  const char* src = static_cast<const char*>(a.cache.pages) + page * 64 * L::RAW_ROW + lane * 16;
#pragma unroll
  for (int i = 0; i < L::LOADS; ++i) {
    if constexpr (KF == 0) c[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i * 1024));
    else c[i] = *reinterpret_cast<const u32x4*>(src + i * 1024);
  }
  if (KF != 0) sc = reinterpret_cast<const uint32_t*>(a.cache.scales)[page * 64 + lane];
}

// score_page on a page staged in LDS (rows of L::ROW bytes, scale words in sc_s), reading each 16-entry tile's
// operands just before its MFMAs; the arithmetic and its order are score_page's.
template <int KF, int HT>
__device__ __forceinline__ uint32_t lt_score_page(const char* st, const uint32_t* sc_s, const bf16x8 (&qa)[HT][4],
                                                  const float (&wv)[HT][4], int col, int kg) {
  using L = LtPage<KF>;
  float mine_f = 0.f;
  const float inf = opaque_inf();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const char* rowp = st + (u * 16 + col) * L::ROW;
    bf16x8 kb[4];
    float sc = 1.f;
    if constexpr (KF == 2) {
      const uint4 c = *reinterpret_cast<const uint4*>(rowp + kg * 16);
      const float bs = e8m0_to_f32((sc_s[u * 16 + col] >> (8 * kg)) & 0xFFu);
      kb[0] = fp4x8_to_bf16x8_hw(c.x, bs);
      kb[1] = fp4x8_to_bf16x8_hw(c.y, bs);
      kb[2] = fp4x8_to_bf16x8_hw(c.z, bs);
      kb[3] = fp4x8_to_bf16x8_hw(c.w, bs);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (KF == 1) kb[ks] = fp8x8_to_bf16x8_hw(*reinterpret_cast<const uint2*>(rowp + ks * 32 + kg * 8));
        else kb[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rowp + ks * 64 + kg * 16));
      }
      if constexpr (KF == 1) sc = __uint_as_float(sc_s[u * 16 + col]);
    }
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][ks], kb[ks], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wv[ht][i] * (KF == 0 ? fmaxf(acc[i], 0.f) : relu_med3(acc[i], inf));
    }
    part = rows4_sum_pairs(part);
    if constexpr (KF == 1) part *= sc;
    if (kg == u) mine_f = part;
  }
  return score_key(mine_f);
}

template <int KF, int HT, int OA = 0>
__global__ void __launch_bounds__(256, 2) score_lt_kernel(IndexArgs a, Workspace ws, FusedCompress fc) {
  using L = LtPage<KF>;
  constexpr int DIM = 128;
  constexpr int E = 64;
  constexpr int AHEAD = L::AHEAD;
  __shared__ uint32_t hist_s[kHistBins / 2];  // two 16-bit bins per word (at most 2048 keys per workgroup)
  __shared__ __attribute__((aligned(16))) char stage_s[4][E * L::ROW];
  __shared__ uint32_t scale_s[4][E];
  __shared__ int32_t pg_phys[kLtPages];
  const int q = blockIdx.y;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  const int64_t n_pages = (n_elig + E - 1) / E;
  const int64_t pg_begin = int64_t(blockIdx.x) * kLtPages;
  if constexpr (OA != 0) {
    if (int64_t(blockIdx.x) == (n_pages > 0 ? (n_pages - 1) / kLtPages : 0)) {  // uniform per block
      fused_compress<KF, OA>(fc, q);
      __syncthreads();
    }
  }
  if (pg_begin >= n_pages) return;  // uniform per block
  const int64_t pg_end = min(n_pages, pg_begin + kLtPages);
  for (int b = threadIdx.x; b < kHistBins / 2; b += blockDim.x) hist_s[b] = 0u;
  if (threadIdx.x < kLtPages) {
    const int64_t pg = pg_begin + threadIdx.x;
    const int32_t* bt = a.cache.block_table + int64_t(seq) * a.cache.bt_stride;
    const int32_t phys = (pg < pg_end && pg < a.cache.bt_stride) ? bt[pg] : -1;
    pg_phys[threadIdx.x] = (phys >= 0 && phys < a.cache.n_phys) ? phys : -1;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int H = HT * 16;
  bf16x8 qa[HT][4];
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + int64_t(q) * H * DIM;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                  qp + (ht * 16 + col) * DIM + (KF == 2 ? kg * 32 + ks * 8 : ks * 32 + kg * 8)));
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = a.head_w[int64_t(q) * H + ht * 16 + kg * 4 + i];
  lds_barrier();  // pg_phys and the cleared histogram are visible; the loads above stay in flight

  uint32_t* keys_q = ws.keys + int64_t(q) * ws.key_stride;
  char* st = stage_s[wave];
  // this wave's pages: pg_begin + wave, +4, ... < pg_end
  const int64_t first = __builtin_amdgcn_readfirstlane(int(pg_begin + wave));
  const int n_mine = first < pg_end ? int((pg_end - 1 - first) / 4 + 1) : 0;
  if (n_mine > 0) {
    u32x4 land[AHEAD][L::LOADS];
    uint32_t land_sc[AHEAD] = {};
#pragma unroll
    for (int s = 0; s < AHEAD; ++s)
      lt_fetch<KF>(a, pg_phys[wave + 4 * (s < n_mine ? s : n_mine - 1)], lane, land[s], land_sc[s]);
    // The at most kLtPages / 4 steps of this wave are unrolled into straight-line code that a step leaves by a
    // uniform break once the wave's pages are done, and every prefetch is issued (past the last page it re-reads
    // that page). The compiler then knows at every step which loads are older than the other buffer's and waits
    // only for them; in a loop (or with the body or the prefetch under a condition) it waited for both buffers at
    // the top of a step: one page in flight instead of two.
#pragma unroll
    for (int j = 0; j < kLtPages / 4; ++j) {
      if (j >= n_mine) break;  // uniform over the wave
      const int s = j % AHEAD;
      // stage page j: byte offset 16 * (lane + 64 i) of the page is row (lane + 64 i) / (RAW_ROW / 16)
#pragma unroll
      for (int i = 0; i < L::LOADS; ++i) {
        const int chunk = lane + 64 * i;
        const int row = chunk / (L::RAW_ROW / 16), off = (chunk % (L::RAW_ROW / 16)) * 16;
        *reinterpret_cast<u32x4*>(st + row * L::ROW + off) = land[s][i];
      }
      if (KF != 0) scale_s[wave][lane] = land_sc[s];
      const int32_t phys_j = pg_phys[wave + 4 * j];
      const int jn = j + AHEAD < n_mine ? j + AHEAD : n_mine - 1;
      lt_fetch<KF>(a, pg_phys[wave + 4 * jn], lane, land[s], land_sc[s]);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the stage is written before this wave reads it
      __builtin_amdgcn_wave_barrier();
      const uint32_t key = lt_score_page<KF, HT>(st, scale_s[wave], qa, wv, col, kg);
      const int64_t e = (first + 4 * int64_t(j)) * E + lane;
      if (e < n_elig) {
        const uint32_t k2 = phys_j >= 0 ? key : 0u;
        keys_q[e] = k2;
        const uint32_t bin = k2 >> (32 - kHistBits);
        atomicAdd(&hist_s[bin >> 1], 1u << ((bin & 1u) * 16));
      }
    }
  }
  __syncthreads();
  uint32_t* hq = ws.hist + int64_t(q) * kHistBins;
  for (int b = threadIdx.x; b < kHistBins / 2; b += blockDim.x) {
    const uint32_t v = hist_s[b];
    if (v & 0xFFFFu) atomicAdd(hq + 2 * b, v & 0xFFFFu);
    if (v >> 16) atomicAdd(hq + 2 * b + 1, v >> 16);
  }
}

// ------------------------------------------------------------------ VALU score (any head count / dim / dtype)
template <int DT>  // 0 f32, 1 bf16, 2 fp8
__global__ void __launch_bounds__(256) score_valu_kernel(IndexArgs a, Workspace ws) {
  extern __shared__ float smem[];  // [H][D] query, then histogram
  uint32_t* hist_s = reinterpret_cast<uint32_t*>(smem + a.n_heads * a.cache.dim);
  const int q = blockIdx.y;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  const int64_t e_begin = int64_t(blockIdx.x) * 256;
  if (e_begin >= n_elig) return;
  const int H = a.n_heads, D = a.cache.dim;
  for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) hist_s[b] = 0u;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) {
    smem[i] = (a.q_dtype == CSA_F32) ? reinterpret_cast<const float*>(a.q)[int64_t(q) * H * D + i]
                                     : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[int64_t(q) * H * D + i]);
  }
  __syncthreads();
  const int64_t e = e_begin + threadIdx.x;
  if (e < n_elig) {
    const int32_t* bt = a.cache.block_table + int64_t(seq) * a.cache.bt_stride;
    const int64_t row = entry_row(bt, a.cache.bt_stride, a.cache.n_phys, e, kBlock / a.cache.ratio);
    uint32_t key = 0u;
    if (row >= 0) {
      float sc = 1.f;
      if (DT == 2) sc = a.cache.scales[row];
      float total = 0.f;
      for (int h = 0; h < H; ++h) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) {
          float kv;
          if (DT == 0) kv = reinterpret_cast<const float*>(a.cache.pages)[row * D + d];
          else if (DT == 1) kv = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.cache.pages)[row * D + d]);
          else kv = e4m3_to_f32(reinterpret_cast<const uint8_t*>(a.cache.pages)[row * D + d]);
          dot = fmaf(smem[h * D + d], kv, dot);
        }
        if (a.mode == CSA_SCORE_DOT) total += dot;
        else total = fmaf(a.head_w[int64_t(q) * H + h], fmaxf(dot, 0.f), total);
      }
      key = score_key(total * sc);
    }
    ws.keys[int64_t(q) * ws.key_stride + e] = key;
    atomicAdd(&hist_s[key >> (32 - kHistBits)], 1u);
  }
  flush_hist(hist_s, ws.hist + int64_t(q) * kHistBins);
}

// ------------------------------------------------------------------ select
// One 1024-thread workgroup per query: boundary bin from the score histogram (key bits 31..20), one pass
// over the query's keys that marks keys above the bin in a bitmap of chosen entries and lists the keys
// inside it (candidates) with a histogram of their bits 19..8, a last 8-bit digit and, for exact ties,
// the lowest indices first; the bitmap read in word order gives the chosen entries in ascending index.
constexpr int kSelThreads = 1024;
constexpr int kSelLoads = 8;  // 16-byte key loads per thread and chunk of the key pass
constexpr int kCandLds = 6144;  // candidates held in LDS; more spill to the workspace list

__device__ __forceinline__ uint32_t dpp_sum16(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (row shifts within each row of 16, then the row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xF, 0xF, false));  // row_shr:1
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xF, 0xF, false));  // row_shr:2
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xF, 0xF, false));  // row_shr:4
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xF, 0xF, false));  // row_shr:8
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15 into rows 1, 3
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31 into rows 2, 3
  return v;
}

// Block-wide (NT threads) exclusive prefix sum of one value per thread; returns the block total.
template <int NT = kSelThreads>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* excl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = NT / 64;
  const uint32_t incl = wave_incl_scan(v);  // DPP: no LDS round trip per step as with lane shuffles
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  uint32_t base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = tmp[w];
    base += (w < wave) ? t : 0u;
    total += t;
  }
  *excl = base + incl - v;
  __syncthreads();
  return total;
}

// Threshold digit of a descending radix step, found by wave 0: the largest d with
// count(digits >= d) >= need. Writes {d, count(digits > d), count(digit == d)} to out[0..2].
__device__ __forceinline__ void wave0_digit_desc(const uint32_t* dig, int nbins, uint32_t need, uint32_t* out) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int per = (nbins + 63) / 64;
  uint32_t own = 0;
  for (int j = 0; j < per; ++j) {
    const int b = lane * per + j;
    if (b < nbins) own += dig[b];
  }
  const uint32_t incl = wave_incl_scan(own);
  uint32_t run = uint32_t(__builtin_amdgcn_readlane(int(incl), 63)) - incl;  // digits above this lane's range
  for (int j = per - 1; j >= 0; --j) {
    const int b = lane * per + j;
    if (b >= nbins) continue;
    const uint32_t c = dig[b];
    if (run < need && run + c >= need) { out[0] = uint32_t(b); out[1] = run; out[2] = c; }
    run += c;
  }
}

// Ascending counterpart: the smallest d with count(digits <= d) >= want. Writes {d, count(digits < d)}.
__device__ __forceinline__ void wave0_digit_asc(const uint32_t* dig, int nbins, uint32_t want, uint32_t* out) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int per = (nbins + 63) / 64;
  uint32_t own = 0;
  for (int j = 0; j < per; ++j) {
    const int b = lane * per + j;
    if (b < nbins) own += dig[b];
  }
  uint32_t run = wave_incl_scan(own) - own;  // digits below this lane's range
  for (int j = 0; j < per; ++j) {
    const int b = lane * per + j;
    if (b >= nbins) continue;
    const uint32_t c = dig[b];
    if (run < want && run + c >= want) { out[0] = uint32_t(b); out[1] = run; }
    run += c;
  }
}

constexpr int kBitmapLds = 8192;  // LDS bitmap words: queries with up to 262144 eligible entries
constexpr int kSelManyQueries = 256;  // launches of at least this many queries take the half-size select workgroups

// ------------------------------------------------------------------ mark pass (few queries with many entries)
// One workgroup per query cannot scan a long key list quickly, so for few long queries the key pass runs
// first as its own launch, split into chunks of kMarkChunk keys: each workgroup finds the boundary bin from
// the query's histogram, writes the chosen-entry bitmap words of its chunk (a set bit = a key above the
// bin; every word of the chunk is written, so the bitmap needs no clearing), lists the keys inside the bin
// as candidates and counts their bits 19..8 in hist2. The select pass then only resolves the boundary bin.
// 512 threads with 4 loads each: 1M-entry mark + select 22.0 -> 20.2 us against 256 threads with 8 (the same chunk,
// twice the waves to hide the histogram and key round trips; 1024 x 2 measured the same, 256 x 4 and 512 x 8 slower)
constexpr int kMarkThreads = 512;
constexpr int kMarkLoads = 4;  // 16-byte key loads per thread
constexpr int kMarkChunk = kMarkThreads * kMarkLoads * 4;  // 8192 keys = 256 bitmap words
constexpr int kPremarkMaxQueries = 64;
constexpr int64_t kPremarkMinElig = 65536;

__global__ void __launch_bounds__(kMarkThreads) select_mark_kernel(IndexArgs a, Workspace ws) {
  __shared__ uint32_t tmp[kMarkThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t h2_s[kHistBins];
  __shared__ uint2 cand_s[kMarkChunk];  // this chunk's candidates; one global reservation per workgroup
  const int q = blockIdx.y;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  if (n_elig <= a.k) return;  // every entry is chosen: the select pass handles the query alone
  const int64_t c0 = int64_t(blockIdx.x) * kMarkChunk;
  if (c0 >= n_elig) return;  // uniform per block
  const int64_t c1 = min<int64_t>(n_elig, c0 + kMarkChunk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // 4 consecutive keys per 16-byte load (key rows are 256-byte aligned and c0 is a multiple of the chunk)
  const uint4* keys4 = reinterpret_cast<const uint4*>(ws.keys + int64_t(q) * ws.key_stride);
  const uint32_t u0 = uint32_t(c0 / 4), u1 = uint32_t((c1 + 3) / 4);
  uint4 kv[kMarkLoads];
#pragma unroll
  for (int j = 0; j < kMarkLoads; ++j) {
    const uint32_t u = u0 + uint32_t(tid + kMarkThreads * j);
    kv[j] = keys4[u < u1 ? u : u0];  // clamped, unconditional load
  }
  for (int b = tid; b < kHistBins; b += kMarkThreads) h2_s[b] = 0u;
  // boundary bin: the largest b0 with count(bins >= b0) >= k
  constexpr int PER = kHistBins / kMarkThreads;
  const uint32_t* hist = ws.hist + int64_t(q) * kHistBins;
  uint32_t h[PER];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { h[j] = hist[tid * PER + j]; local += h[j]; }
  uint32_t excl;
  const uint32_t total = block_excl_scan<kMarkThreads>(local, tmp, &excl);
  uint32_t run = total - excl - local;
  if (tid == 0) { res[0] = 0xFFFFFFFFu; res[1] = 0u; }
  __syncthreads();
  const uint32_t kk = uint32_t(a.k);
  for (int j = PER - 1; j >= 0; --j) {
    if (run < kk && run + h[j] >= kk) res[0] = uint32_t(tid * PER + j);
    run += h[j];
  }
  __syncthreads();
  const uint32_t b0 = res[0];  // 0xFFFFFFFF only for an inconsistent histogram: nothing is marked then

  uint32_t* bits_q = ws.bits + int64_t(q) * ws.bits_stride;
  uint2* cand_q = ws.cand + int64_t(q) * a.max_elig;
  const int64_t n_words = (n_elig + 31) / 32;
  // Per load j a wave covers 256 consecutive keys; each group of 8 lanes assembles one 32-key bitmap word with
  // lane exchanges (all vector arithmetic). The words are stored after the loop, with every key already read.
  const uint32_t c1u = uint32_t(c1);
  uint32_t wd[kMarkLoads];
  uint32_t cbits = 0;  // candidate flags: bit 4 j + c for key c of load j
#pragma unroll
  for (int j = 0; j < kMarkLoads; ++j) {
    const uint32_t u = u0 + uint32_t(tid + kMarkThreads * j);
    const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
    uint32_t sure = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool in = 4 * u + c < c1u;
      const uint32_t bin = k4[c] >> (32 - kHistBits);
      sure |= uint32_t(in && bin > b0 && b0 != 0xFFFFFFFFu) << c;
      cbits |= uint32_t(in && bin == b0) << (4 * j + c);
    }
    uint32_t w = sure << (4 * (lane & 7));
    w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x141, 0xF, 0xF, false));  // row_half_mirror
    wd[j] = w;
  }
  // candidates go to an LDS list (a returning device-scope atomic per wave would serialise on the query's
  // counter across XCDs): one LDS reservation per wave from a wave prefix sum of the lanes' counts
  const uint32_t nc = uint32_t(__popc(cbits));
  if (__ballot(nc != 0u)) {  // uniform over the wave
    const uint32_t incl = wave_incl_scan(nc);
    const uint32_t total = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
    uint32_t wbase = 0;
    if (lane == 0) wbase = atomicAdd(&res[1], total);
    wbase = uint32_t(__builtin_amdgcn_readfirstlane(int(wbase)));  // every lane is active here
    uint32_t cs = wbase + incl - nc;  // < kMarkChunk: at most one candidate per key of the chunk
#pragma unroll
    for (int j = 0; j < kMarkLoads; ++j) {
      const uint32_t cj = (cbits >> (4 * j)) & 0xFu;
      if (cj) {
        const uint32_t u = u0 + uint32_t(tid + kMarkThreads * j);
        const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if ((cj >> c) & 1u) {
            cand_s[cs++] = make_uint2(k4[c], 4 * u + c);
            atomicAdd(&h2_s[(k4[c] >> 8) & (kHistBins - 1)], 1u);
          }
        }
      }
    }
  }
  // word (u0 + 256 j) / 8 + tid / 8 holds keys 4 (u0 + 256 j + (tid & ~7)) .. +31; every word of the chunk below
  // n_words is stored whole
#pragma unroll
  for (int j = 0; j < kMarkLoads; ++j) {
    const uint32_t word = (u0 + uint32_t(kMarkThreads * j)) / 8 + uint32_t(tid >> 3);
    if ((lane & 7) == 0 && word < uint32_t(n_words)) bits_q[word] = wd[j];
  }
  __syncthreads();
  const uint32_t n_local = res[1];  // <= kMarkChunk
  if (tid == 0) tmp[0] = n_local ? atomicAdd(ws.ncand + q, n_local) : 0u;
  __syncthreads();
  const uint32_t base = tmp[0];
  for (uint32_t j = tid; j < n_local; j += kMarkThreads)
    if (base + j < uint32_t(a.max_elig)) cand_q[base + j] = cand_s[j];
  flush_hist(h2_s, ws.hist2 + int64_t(q) * kHistBins);
}

template <bool PRE, int NT, int BMW, int CLDS, bool BMG>
__global__ void __launch_bounds__(NT, 4) select_kernel(IndexArgs a, Workspace ws) {  // 4 waves per SIMD: 1024 threads per CU
  __shared__ uint32_t tmp[NT / 64];
  __shared__ uint32_t hist2[kHistBins];      // key bits 19..8 of the candidates
  __shared__ uint32_t dig[256];
  __shared__ uint32_t res[4];
  __shared__ uint32_t s_cnt[2];              // sure count, candidate count
  __shared__ uint32_t bitmap_s[BMG ? 1 : BMW];  // chosen entries, one bit each
  __shared__ uint2 cand_s[CLDS];

  const int q = blockIdx.x;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  const int64_t kk = min<int64_t>(a.k, n_elig);  // entries to choose
  const int tid = threadIdx.x;
  uint2* cand_g = ws.cand + int64_t(q) * a.max_elig;  // overflow of the candidate list
  const uint32_t* keys_q = ws.keys + int64_t(q) * ws.key_stride;
  const int64_t n_words = (n_elig + 31) / 32;
  // the mark pass has already scanned this query's keys (bitmap words of keys above the boundary bin,
  // candidate list and hist2 in the workspace)
  const bool pre = PRE && n_elig > a.k;
  uint32_t* bits_g = ws.bits + int64_t(q) * ws.bits_stride;
  // The chosen-entry bitmap is in LDS when every query of the launch has at most BMW words (BMG false), else in the
  // workspace. The choice is made per launch at compile time so that the LDS variant's bitmap accesses are LDS
  // instructions: through a pointer that may point to either they are flat accesses, which count with the key loads,
  // and the key pass then waited for each bitmap store before going on to its next key.
  uint32_t* bitmap = BMG ? bits_g : bitmap_s;
  uint32_t* hist2_g = ws.hist2 + int64_t(q) * kHistBins;
  // after a mark pass every global read of the set-up (score histogram, bitmap words, second histogram) is
  // issued here, before any of them is used, so they cost one round trip together
  constexpr int PER = kHistBins / NT;
  const uint32_t* hist = ws.hist + int64_t(q) * kHistBins;
  uint32_t h[PER];
  if (pre) {
#pragma unroll
    for (int j = 0; j < PER; ++j) h[j] = hist[tid * PER + j];
  }
  if (pre) {
    constexpr int BW = BMW / NT;  // bitmap words per thread when the bitmap fits LDS
    constexpr bool lds_bits = !BMG;
    uint32_t bw[BW], h2[PER];
    if (lds_bits) {
#pragma unroll
      for (int j = 0; j < BW; ++j) {
        const int64_t w = tid + int64_t(NT) * j;
        bw[j] = bits_g[w < n_words ? w : 0];  // clamped, unconditional load
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) h2[j] = hist2_g[tid + NT * j];
    const uint32_t nc = tid == 0 ? ws.ncand[q] : 0u;
    if (lds_bits) {
#pragma unroll
      for (int j = 0; j < BW; ++j) {
        const int64_t w = tid + int64_t(NT) * j;
        if (w < n_words) bitmap[w] = bw[j];
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      hist2[tid + NT * j] = h2[j];
      hist2_g[tid + NT * j] = 0u;  // left zero for the next mark pass
    }
    if (tid == 0) {
      s_cnt[1] = nc;
      ws.ncand[q] = 0u;
    }
  } else {
    // every bitmap word below n_words is stored whole by the key pass, so only hist2 and the counters start at 0
    for (int b = tid; b < kHistBins; b += NT) hist2[b] = 0u;
    if (tid < 2) s_cnt[tid] = 0u;
  }

  // ---- boundary bin of the score histogram: largest b0 with count(bins >= b0) >= kk
  int b0 = -1;
  if (n_elig > a.k) {
    if (!pre) {
#pragma unroll
      for (int j = 0; j < PER; ++j) h[j] = hist[tid * PER + j];
    }
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) local += h[j];
    uint32_t excl;
    const uint32_t total = block_excl_scan<NT>(local, tmp, &excl);
    uint32_t run = total - excl - local;
    if (tid == 0) { res[0] = 0xFFFFFFFFu; res[1] = 0u; }
    __syncthreads();
    for (int j = PER - 1; j >= 0; --j) {
      if (run < uint32_t(kk) && run + h[j] >= uint32_t(kk)) { res[0] = uint32_t(tid * PER + j); res[1] = run; }
      run += h[j];
    }
    __syncthreads();
    b0 = int(res[0]);
    if (pre && tid == 0) s_cnt[0] = res[1];  // keys above the bin, all marked by the mark pass
  }
  __threadfence_block();
  __syncthreads();

  // ---- one pass over the keys: mark keys above the bin, collect keys inside it (and their next 12 bits).
  // A thread reads 4 consecutive keys per 16-byte load, so one load instruction of a wave covers 256 keys; each
  // group of 8 lanes holds one 32-key bitmap word, which it assembles with three lane exchanges and its first
  // lane stores. Every per-key step is vector arithmetic: with a ballot, a mask branch and scalar mask arithmetic
  // per key, 16 waves on one CU were bound by its instruction issue, not by the loads. Candidates (rare) get list
  // slots once per wave and chunk: a wave prefix sum of the lanes' counts and one LDS atomic.
  const int lane = tid & 63;
  const uint32_t n_el32 = uint32_t(n_elig);
  const uint32_t n4 = (n_el32 + 3) / 4;
  const uint4* keys4 = reinterpret_cast<const uint4*>(keys_q);  // key rows are 256-byte aligned
  uint32_t n_sure_l = 0;
  for (uint32_t base4 = 0; base4 < (pre ? 0u : n4); base4 += uint32_t(NT) * kSelLoads) {
    uint4 kv[kSelLoads];
#pragma unroll
    for (int j = 0; j < kSelLoads; ++j) {
      const uint32_t u = base4 + uint32_t(tid + NT * j);
      kv[j] = keys4[u < n4 ? u : 0u];  // clamped, unconditional; a row's last load stays inside its stride
    }
    uint32_t cbits = 0;  // candidate flags: bit 4 j + c for key c of load j
#pragma unroll
    for (int j = 0; j < kSelLoads; ++j) {
      const uint32_t u = base4 + uint32_t(tid + NT * j);
      const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
      uint32_t sure = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool in = 4 * u + c < n_el32;
        const int bin = int(k4[c] >> (32 - kHistBits));
        sure |= uint32_t(in && bin > b0) << c;  // b0 = -1 when every eligible entry is chosen
        cbits |= uint32_t(in && bin == b0) << (4 * j + c);
      }
      n_sure_l += __popc(sure);
      // word (base4 + NT j) / 8 + tid / 8 holds keys 4 (base4 + NT j + (tid & ~7)) .. +31
      uint32_t wd = sure << (4 * (lane & 7));
      wd |= uint32_t(__builtin_amdgcn_mov_dpp(int(wd), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
      wd |= uint32_t(__builtin_amdgcn_mov_dpp(int(wd), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
      wd |= uint32_t(__builtin_amdgcn_mov_dpp(int(wd), 0x141, 0xF, 0xF, false));  // row_half_mirror
      const uint32_t word = (base4 + uint32_t(NT * j)) / 8 + uint32_t(tid >> 3);
      if ((lane & 7) == 0 && word < uint32_t(n_words)) bitmap[word] = wd;
    }
    const uint32_t nc = uint32_t(__popc(cbits));
    if (__ballot(nc != 0u)) {  // uniform over the wave
      const uint32_t incl = wave_incl_scan(nc);
      const uint32_t total = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
      uint32_t wbase = 0;
      if (lane == 0) wbase = atomicAdd(&s_cnt[1], total);
      wbase = uint32_t(__builtin_amdgcn_readfirstlane(int(wbase)));  // every lane is active here
      uint32_t cs = wbase + incl - nc;
#pragma unroll
      for (int j = 0; j < kSelLoads; ++j) {
        const uint32_t cj = (cbits >> (4 * j)) & 0xFu;
        if (cj) {
          const uint32_t u = base4 + uint32_t(tid + NT * j);
          const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if ((cj >> c) & 1u) {
              atomicAdd(&hist2[(k4[c] >> 8) & (kHistBins - 1)], 1u);
              const uint2 item = make_uint2(k4[c], 4 * u + c);
              if (cs < uint32_t(CLDS)) cand_s[cs] = item;
              else if (cs - CLDS < uint32_t(a.max_elig)) cand_g[cs - CLDS] = item;
              ++cs;
            }
          }
        }
      }
    }
  }
  if (!pre) {
    const uint32_t sure_w = uint32_t(__builtin_amdgcn_readlane(int(wave_incl_scan(n_sure_l)), 63));
    if (lane == 0 && sure_w) atomicAdd(&s_cnt[0], sure_w);
  }
  __threadfence_block();
  __syncthreads();

  const uint32_t n_sure = s_cnt[0];
  const uint32_t lds_n = pre ? 0u : uint32_t(CLDS);  // the mark pass lists every candidate in the workspace
  const uint32_t n_cand = min<uint32_t>(s_cnt[1], uint32_t(min<int64_t>(int64_t(lds_n) + a.max_elig, 0xFFFFFFFFll)));
  auto cand_at = [=](uint32_t j) -> uint2 { return j < lds_n ? cand_s[j] : cand_g[j - lds_n]; };
  int64_t need = kk - int64_t(n_sure);
  if (need > 0) {
    // sub-bin of key bits 19..8: largest b1 with count(candidates with bits >= b1) >= need
    constexpr int PER = kHistBins / NT;
    uint32_t h[PER];
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) { h[j] = hist2[tid * PER + j]; local += h[j]; }
    uint32_t excl;
    const uint32_t total = block_excl_scan<NT>(local, tmp, &excl);
    uint32_t run = total - excl - local;
    if (tid == 0) { res[0] = 0u; res[1] = 0u; }
    __syncthreads();
    for (int j = PER - 1; j >= 0; --j) {
      if (run < uint32_t(need) && run + h[j] >= uint32_t(need)) { res[0] = uint32_t(tid * PER + j); res[1] = run; }
      run += h[j];
    }
    __syncthreads();
    uint32_t prefix = (uint32_t(b0) << 20) | (res[0] << 8);
    const uint32_t pmask = 0xFFFFFF00u;
    need -= res[1];
    __syncthreads();
    // last digit: key bits 7..0 among candidates matching the 24-bit prefix
    if (tid < 256) dig[tid] = 0u;
    if (tid < 3) res[tid] = 0u;
    __syncthreads();
    for (uint32_t j = tid; j < n_cand; j += blockDim.x) {
      const uint32_t k2 = cand_at(j).x;
      if ((k2 & pmask) == prefix) atomicAdd(&dig[k2 & 0xFFu], 1u);
    }
    __syncthreads();
    wave0_digit_desc(dig, 256, uint32_t(need), res);
    __syncthreads();
    need -= res[1];
    prefix |= res[0];
    const uint32_t tie_count = res[2];
    __syncthreads();
    // prefix is the exact threshold key; take `need` of its tie_count ties, lowest index first
    uint32_t idx_limit = 0xFFFFFFFFu;
    if (uint32_t(need) < tie_count) {
      uint32_t ipre = 0, imask = 0;
      int64_t want = need;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) dig[tid] = 0u;
        if (tid < 3) res[tid] = 0u;
        __syncthreads();
        for (uint32_t j = tid; j < n_cand; j += blockDim.x) {
          const uint2 c = cand_at(j);
          if (c.x == prefix && (c.y & imask) == ipre) atomicAdd(&dig[(c.y >> shift) & 0xFFu], 1u);
        }
        __syncthreads();
        wave0_digit_asc(dig, 256, uint32_t(want), res);
        __syncthreads();
        want -= res[1];
        ipre |= res[0] << shift;
        imask |= 0xFFu << shift;
        __syncthreads();
      }
      idx_limit = ipre;
    }
    for (uint32_t j = tid; j < n_cand; j += blockDim.x) {
      const uint2 c = cand_at(j);
      if ((c.x > prefix) || (c.x == prefix && c.y <= idx_limit)) atomicOr(&bitmap[c.y >> 5], 1u << (c.y & 31));
    }
  }
  __threadfence_block();
  __syncthreads();

  // ---- compaction of the bitmap in index order (each thread owns a run of consecutive words). The chosen indices
  // go to LDS first (the candidate list is done with), then every output slot is written from there with all of
  // its key loads in flight together: reading each chosen entry's key where its bit is found cost one memory round
  // trip per chosen entry of the thread's run, one after the other.
  static_assert(2 * CLDS >= 2048, "the LDS index list holds the largest k");
  int32_t* chosen_s = reinterpret_cast<int32_t*>(cand_s);
  const int64_t per_t = (n_words + NT - 1) / NT;
  const int64_t w0 = int64_t(tid) * per_t;
  uint32_t mine = 0;
  for (int64_t w = w0; w < w0 + per_t && w < n_words; ++w) mine += __popc(bitmap[w]);
  uint32_t off;
  const uint32_t n_sel_all = block_excl_scan<NT>(mine, tmp, &off);
  const int n_sel = int(min<int64_t>(n_sel_all, kk));
  for (int64_t w = w0; w < w0 + per_t && w < n_words && off < uint32_t(n_sel); ++w) {
    uint32_t bits = bitmap[w];
    while (bits && off < uint32_t(n_sel)) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      chosen_s[off++] = int32_t(w * 32 + b);
    }
  }
  __syncthreads();
  int32_t* outq = a.out_idx + int64_t(q) * a.k;
  constexpr int R = (2048 + NT - 1) / NT;  // output slots per thread at the largest k
  int32_t e[R];
  uint32_t kv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = tid + NT * r;
    e[r] = j < n_sel ? chosen_s[j] : -1;
  }
  if (a.out_scores) {  // uniform
#pragma unroll
    for (int r = 0; r < R; ++r) kv[r] = keys_q[e[r] > 0 ? e[r] : 0];  // unconditional; row 0 exists
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = tid + NT * r;
    if (j < a.k) {
      outq[j] = e[r];
      if (a.out_scores)
        a.out_scores[int64_t(q) * a.k + j] = e[r] >= 0 ? key_score(kv[r]) : __uint_as_float(0x7FC00000u);
    }
  }
  if (tid == 0 && a.out_count) a.out_count[q] = n_sel;
  // leave this query's histogram zeroed for the next score pass on this workspace
  uint32_t* hq = ws.hist + int64_t(q) * kHistBins;
  for (int b = tid; b < kHistBins; b += blockDim.x) hq[b] = 0u;
}

// Queries with no eligible entry never reach the select kernel's last-block path when the grid
// has no block for them; this kernel writes their (empty) outputs.
__global__ void empty_rows_kernel(IndexArgs a) {
  const int q = blockIdx.x;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  if (n_elig > 0) return;
  for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
    a.out_idx[int64_t(q) * a.k + j] = -1;
    if (a.out_scores) a.out_scores[int64_t(q) * a.k + j] = __uint_as_float(0x7FC00000u);
  }
  if (threadIdx.x == 0 && a.out_count) a.out_count[q] = 0;
}

}  // namespace

size_t index_workspace(int n_q, int64_t max_elig, int k) {
  (void)k;
  return clean_bytes(n_q) + align256(size_t(n_q) * size_t(key_stride_of(max_elig)) * 4) +
         align256(size_t(n_q) * size_t(max_elig) * 8) +
         align256(size_t(n_q) * size_t((max_elig + 31) / 32) * 4);
}

size_t index_clean_bytes(int n_q) { return clean_bytes(n_q); }

bool index_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads, csa_score_t mode) {
  if (c.dtype == CSA_F32) return q_dtype == CSA_F32 && n_heads * c.dim <= 8192;
  if (q_dtype != CSA_BF16) return false;
  const bool mfma = mode == CSA_SCORE_WRELU && c.ratio == 4 && c.dim == 128 && n_heads % 16 == 0 && n_heads <= 64;
  if (c.dtype == CSA_FP4_E2M1) return mfma;  // fp4 pages are scored by the MFMA kernel only
  return mfma || n_heads * c.dim <= 8192;
}

hipError_t launch_index_clear(void* ws_base, int n_q, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const int64_t words = int64_t(clean_bytes(n_q) / 4);
  const int64_t nb = (words + 255) / 256;
  const int blocks = int(nb < 4096 ? nb : 4096);
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint32_t*>(ws_base), words);
  return hipGetLastError();
}

template <int HT>
void launch_score_shared(int kf, dim3 grid, const IndexArgs& a, const Workspace& ws, hipStream_t stream) {
  if (kf == 2) hipLaunchKernelGGL((score_shared_kernel<2, HT>), grid, dim3(kShareThreads), 0, stream, a, ws);
  else if (kf == 1) hipLaunchKernelGGL((score_shared_kernel<1, HT>), grid, dim3(kShareThreads), 0, stream, a, ws);
  else hipLaunchKernelGGL((score_shared_kernel<0, HT>), grid, dim3(kShareThreads), 0, stream, a, ws);
}

template <int HT>
void launch_score_fp4(dim3 grid, const IndexArgs& a, const Workspace& ws, int run, hipStream_t stream) {
  hipLaunchKernelGGL((score_mfma_kernel<2, HT>), grid, dim3(256), 0, stream, a, ws, run, FusedCompress{});
}

template <int HT>
void launch_score_lt(int kf, dim3 grid, const IndexArgs& a, const Workspace& ws, hipStream_t stream) {
  if (kf == 2) hipLaunchKernelGGL((score_lt_kernel<2, HT>), grid, dim3(256), 0, stream, a, ws, FusedCompress{});
  else if (kf == 1) hipLaunchKernelGGL((score_lt_kernel<1, HT>), grid, dim3(256), 0, stream, a, ws, FusedCompress{});
  else hipLaunchKernelGGL((score_lt_kernel<0, HT>), grid, dim3(256), 0, stream, a, ws, FusedCompress{});
}

hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream) {
  if (a.n_q == 0 || a.max_elig == 0) return hipSuccess;
  Workspace ws = carve(a.ws, a.n_q, a.max_elig);
  const bool mfma = a.cache.dtype != CSA_F32 && a.mode == CSA_SCORE_WRELU && a.cache.ratio == 4 &&
                    a.cache.dim == 128 && a.n_heads % 16 == 0 && a.n_heads <= 64;
  if (mfma) {
    const int64_t max_pages = (a.max_elig + 63) / 64;
    const int64_t runs = (max_pages + kPagesPerBlock - 1) / kPagesPerBlock;
    const bool fp8s = a.cache.dtype == CSA_FP8_E4M3;
    const bool fp4 = a.cache.dtype == CSA_FP4_E2M1;
    const int kf = fp8s ? 1 : (fp4 ? 2 : 0);
    if (a.n_q >= kQueryFastMin && runs <= 65535) {  // many queries per launch: pages shared through LDS
      const dim3 g2(unsigned((a.n_q + kShareQ - 1) / kShareQ), unsigned(runs));
      switch (a.n_heads / 16) {
        case 1: launch_score_shared<1>(kf, g2, a, ws, stream); break;
        case 2: launch_score_shared<2>(kf, g2, a, ws, stream); break;
        case 3: launch_score_shared<3>(kf, g2, a, ws, stream); break;
        default: launch_score_shared<4>(kf, g2, a, ws, stream); break;
      }
      return hipGetLastError();
    }
    if (fp4) {  // fp4 rows are 64 bytes: the operand-layout loads already read whole lines
      const int run = kPagesPerBlock;
      const dim3 grid(unsigned((max_pages + run - 1) / run), unsigned(a.n_q));
      switch (a.n_heads / 16) {
        case 1: launch_score_fp4<1>(grid, a, ws, run, stream); break;
        case 2: launch_score_fp4<2>(grid, a, ws, run, stream); break;
        case 3: launch_score_fp4<3>(grid, a, ws, run, stream); break;
        default: launch_score_fp4<4>(grid, a, ws, run, stream); break;
      }
    } else {
      const dim3 grid(unsigned((max_pages + kLtPages - 1) / kLtPages), unsigned(a.n_q));
      switch (a.n_heads / 16) {
        case 1: launch_score_lt<1>(kf, grid, a, ws, stream); break;
        case 2: launch_score_lt<2>(kf, grid, a, ws, stream); break;
        case 3: launch_score_lt<3>(kf, grid, a, ws, stream); break;
        default: launch_score_lt<4>(kf, grid, a, ws, stream); break;
      }
    }
  } else {
    const dim3 grid(unsigned((a.max_elig + 255) / 256), unsigned(a.n_q));
    const size_t lds = size_t(a.n_heads) * a.cache.dim * 4 + kHistBins * 4;
    if (a.cache.dtype == CSA_F32) hipLaunchKernelGGL((score_valu_kernel<0>), grid, dim3(256), lds, stream, a, ws);
    else if (a.cache.dtype == CSA_BF16) hipLaunchKernelGGL((score_valu_kernel<1>), grid, dim3(256), lds, stream, a, ws);
    else hipLaunchKernelGGL((score_valu_kernel<2>), grid, dim3(256), lds, stream, a, ws);
  }
  return hipGetLastError();
}

hipError_t launch_compress_index_score(const CompressArgs& main, const CompressArgs& idx, const IndexArgs& a,
                                       hipStream_t stream) {
  // fused: the paired-compress configurations (c4a main D 512 bf16 / fp8 + indexer D 128 bf16 / fp8 / MXFP4, bf16
  // inputs) with the decode score path of 64 indexer heads; anything else runs the two launches one after the other
  const bool main_ok = main.state.dtype == CSA_BF16 && main.cache.ratio == 4 && main.cache.dim == 512 &&
                       (main.cache.dtype == CSA_BF16 || main.cache.dtype == CSA_FP8_E4M3);
  const bool idx_ok = idx.state.dtype == CSA_BF16 && idx.cache.ratio == 4 && idx.cache.dim == 128 &&
                      (idx.cache.dtype == CSA_BF16 || idx.cache.dtype == CSA_FP8_E4M3 || idx.cache.dtype == CSA_FP4_E2M1);
  const bool types_ok = main.cache.dtype == idx.cache.dtype || main.cache.dtype == CSA_FP8_E4M3;
  const bool score_ok = a.n_q > 0 && a.n_q < kQueryFastMin && a.max_elig > 0 && a.mode == CSA_SCORE_WRELU &&
                        a.n_heads == 64 && a.cache.ratio == 4 && a.cache.dim == 128 && a.cache.dtype != CSA_F32;
  if (!(main_ok && idx_ok && types_ok && score_ok)) {
    const hipError_t e = launch_compress_pair(main, idx, stream);
    return e != hipSuccess ? e : launch_index_score(a, stream);
  }
  const FusedCompress fc{main, idx};
  Workspace ws = carve(a.ws, a.n_q, a.max_elig);
  const int64_t max_pages = (a.max_elig + 63) / 64;
  const bool fp8_main = main.cache.dtype == CSA_FP8_E4M3;
  if (a.cache.dtype == CSA_FP4_E2M1) {
    const int run = kPagesPerBlock;
    const dim3 grid(unsigned((max_pages + run - 1) / run), unsigned(a.n_q));
    if (fp8_main) hipLaunchKernelGGL((score_mfma_kernel<2, 4, 2>), grid, dim3(256), 0, stream, a, ws, run, fc);
    else hipLaunchKernelGGL((score_mfma_kernel<2, 4, 1>), grid, dim3(256), 0, stream, a, ws, run, fc);
  } else {
    const dim3 grid(unsigned((max_pages + kLtPages - 1) / kLtPages), unsigned(a.n_q));
    const bool fp8_idx = a.cache.dtype == CSA_FP8_E4M3;
    if (fp8_idx && fp8_main) hipLaunchKernelGGL((score_lt_kernel<1, 4, 2>), grid, dim3(256), 0, stream, a, ws, fc);
    else if (fp8_idx) hipLaunchKernelGGL((score_lt_kernel<1, 4, 1>), grid, dim3(256), 0, stream, a, ws, fc);
    else if (fp8_main) hipLaunchKernelGGL((score_lt_kernel<0, 4, 2>), grid, dim3(256), 0, stream, a, ws, fc);
    else hipLaunchKernelGGL((score_lt_kernel<0, 4, 1>), grid, dim3(256), 0, stream, a, ws, fc);
  }
  return hipGetLastError();
}

template <bool PRE, int NT, int BMW, int CLDS>
void launch_select(const IndexArgs& a, const Workspace& ws, hipStream_t stream) {
  if ((a.max_elig + 31) / 32 <= BMW)
    hipLaunchKernelGGL((select_kernel<PRE, NT, BMW, CLDS, false>), dim3(a.n_q), dim3(NT), 0, stream, a, ws);
  else
    hipLaunchKernelGGL((select_kernel<PRE, NT, BMW, CLDS, true>), dim3(a.n_q), dim3(NT), 0, stream, a, ws);
}

hipError_t launch_index_select(const IndexArgs& a, hipStream_t stream) {
  if (a.n_q == 0) return hipSuccess;
  if (a.max_elig == 0) {
    hipLaunchKernelGGL(empty_rows_kernel, dim3(a.n_q), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  Workspace ws = carve(a.ws, a.n_q, a.max_elig);
  if (a.n_q <= kPremarkMaxQueries && a.max_elig >= kPremarkMinElig) {
    const dim3 grid(unsigned((a.max_elig + kMarkChunk - 1) / kMarkChunk), unsigned(a.n_q));
    hipLaunchKernelGGL(select_mark_kernel, grid, dim3(kMarkThreads), 0, stream, a, ws);
    launch_select<true, kSelThreads, kBitmapLds, kCandLds>(a, ws, stream);
  } else if (a.n_q >= kSelManyQueries) {
    // many queries: half-size workgroups with half-size LDS tables, two per CU, so that one workgroup's
    // scans and barriers overlap the other's key loads
    launch_select<false, kSelThreads / 2, kBitmapLds / 2, kCandLds / 2>(a, ws, stream);
  } else {
    launch_select<false, kSelThreads, kBitmapLds, kCandLds>(a, ws, stream);
  }
  return hipGetLastError();
}

}  // namespace csa
