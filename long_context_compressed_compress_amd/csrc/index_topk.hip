// csa_index_topk kernels: indexer score over the eligible compressed entries of each query,
// then an exact radix top-k select with ties to the lower entry index.
//
// [P1] "DeepSeek V4 Attention Architecture" and [P2] "二、注意力機制為什么這么麻煩": DeepSeek Sparse
// Attention attends only to the top-k compressed entries (k = 512 on c4a layers). [P2] "3.2 內核": the
// indexer pipeline (its own compressor instance, score, top-k) is separate from the main cache.
//
// Two launches on the caller's stream (csa_index_score, then csa_index_select):
//   1. score     -- one workgroup per (query, run of entries). WRELU with 16*HT heads over dim-128
//                   bf16 / fp8 keys runs on MFMA (v_mfma_f32_16x16x32_bf16: heads x 16 entries x 32 dims
//                   per instruction, fp8 codes widened exactly to bf16); other shapes run on a VALU path.
//                   Each score becomes an order-preserving 32-bit key; a 4096-bin LDS histogram of
//                   the top 12 key bits is flushed into the query's global histogram.
//   2. select    -- one workgroup per (query, run of keys): find the histogram bin that holds the
//                   k-th largest key, append keys above it to a "sure" list and keys inside it to a
//                   candidate list. The last workgroup of each query (atomic arrival count) refines the
//                   boundary bin with 8/8/4-bit digit passes over the candidates, breaks exact ties by
//                   ascending index, bitonic-sorts the chosen entries by index and writes the output,
//                   then re-zeroes that query's histogram and counters. The workspace's histogram region
//                   therefore only needs zeroing once (csa_index_workspace_clear) and stays clean.
// The chosen set is unique (score order plus index order is total), so the result does not depend
// on how work is split or on the order of atomics.
#include "csa_internal.h"

namespace csa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kScoreChunk = 1024;   // entries per score workgroup
constexpr int kSelectChunk = 8192;  // keys per select workgroup

struct Workspace {
  uint32_t* keys;   // [n_q][max_elig]
  uint32_t* hist;   // [n_q][kHistBins]
  uint32_t* ctr;    // [n_q][4]: sure count, candidate count, arrivals, unused
  uint2* sure;      // [n_q][k]        (key, index)
  uint2* cand;      // [n_q][max_elig] (key, index)
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline size_t clean_bytes(int n_q) {
  return align256(size_t(n_q) * kHistBins * 4) + align256(size_t(n_q) * 16);
}

// Layout: [hist][ctr] (the region that must be zero between calls), then [keys][sure][cand].
__host__ __device__ inline Workspace carve(void* base, int n_q, int64_t max_elig, int k) {
  char* p = static_cast<char*>(base);
  Workspace w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(n_q) * kHistBins * 4);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(n_q) * 16);
  w.keys = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(n_q) * size_t(max_elig) * 4);
  w.sure = reinterpret_cast<uint2*>(p);
  p += align256(size_t(n_q) * size_t(k) * 8);
  w.cand = reinterpret_cast<uint2*>(p);
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

__global__ void clear_kernel(uint32_t* hist, uint32_t* ctr, int n_q) {
  const int64_t n_h = int64_t(n_q) * kHistBins;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_h + 4 * int64_t(n_q);
       i += int64_t(gridDim.x) * blockDim.x) {
    if (i < n_h) hist[i] = 0u; else ctr[i - n_h] = 0u;
  }
}

__device__ __forceinline__ void flush_hist(uint32_t* hist_s, uint32_t* hist_q) {
  __syncthreads();
  for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) {
    const uint32_t v = hist_s[b];
    if (v) atomicAdd(hist_q + b, v);
  }
}

// fp8 e4m3fn code -> bf16 bits (exact: every e4m3fn value is a bf16 value).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8;
  const uint32_t mag = c & 0x7Fu;
  if (mag >= 8u) return s | ((mag << 4) + (120u << 7));
  // subnormal m * 2^-9 (m = mag < 8)
  return s | (__float_as_uint(float(mag) * 0.001953125f) >> 16);
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint2 v) {
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t x = h ? v.y : v.x;
    w[2 * h] = e4m3_to_bf16_bits(x & 0xFF) | (e4m3_to_bf16_bits((x >> 8) & 0xFF) << 16);
    w[2 * h + 1] = e4m3_to_bf16_bits((x >> 16) & 0xFF) | (e4m3_to_bf16_bits(x >> 24) << 16);
  }
  uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
  return __builtin_bit_cast(bf16x8, u);
}

// ------------------------------------------------------------------ MFMA score (WRELU, dim 128)
// One wavefront handles 16-entry tiles (always inside one 64-entry page, so 4 KiB / 2 KiB contiguous).
// Lane l feeds MFMA row/col l%16 and dims (l/16)*8 .. +8 of each 32-dim k-step; accumulator lane l
// holds heads (l/16)*4 + i of each 16-head tile for entry l%16.
template <bool FP8, int HT>
__global__ void __launch_bounds__(256) score_mfma_kernel(IndexArgs a, Workspace ws) {
  constexpr int DIM = 128;
  constexpr int KS = DIM / 32;
  constexpr int TILES_PER_ITER = 2;
  __shared__ uint32_t hist_s[kHistBins];
  const int q = blockIdx.y;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  const int64_t e_begin = int64_t(blockIdx.x) * kScoreChunk;
  if (e_begin >= n_elig) return;  // uniform per block
  const int64_t e_end = min(n_elig, e_begin + kScoreChunk);
  for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) hist_s[b] = 0u;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int H = HT * 16;

  // query fragments (A operand) and head weights
  bf16x8 qa[HT][KS];
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + int64_t(q) * H * DIM;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + (ht * 16 + col) * DIM + ks * 32 + kg * 8));
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = a.head_w[int64_t(q) * H + ht * 16 + kg * 4 + i];
  __syncthreads();

  const int32_t* bt = a.cache.block_table + int64_t(seq) * a.cache.bt_stride;
  const char* pages = reinterpret_cast<const char*>(a.cache.pages);
  uint32_t* keys_q = ws.keys + int64_t(q) * a.max_elig;

  const int per_block = kBlock / a.cache.ratio;
  const int64_t t_begin = e_begin >> 4;
  const int64_t t_end = (e_end + 15) >> 4;
  for (int64_t t0 = t_begin + wave * TILES_PER_ITER; t0 < t_end; t0 += 4 * TILES_PER_ITER) {
    bf16x8 kb[TILES_PER_ITER][KS];
    float scl[TILES_PER_ITER];
    bool valid[TILES_PER_ITER];
#pragma unroll
    for (int u = 0; u < TILES_PER_ITER; ++u) {
      const int64_t e = (t0 + u) * 16 + col;
      const int64_t row = (e < e_end) ? entry_row(bt, a.cache.bt_stride, a.cache.n_phys, e, per_block) : -1;
      valid[u] = row >= 0;
      scl[u] = 1.f;
      if (FP8) {
        const uint8_t* rp = reinterpret_cast<const uint8_t*>(pages) + (valid[u] ? row : 0) * DIM;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint2 raw = valid[u] ? *reinterpret_cast<const uint2*>(rp + ks * 32 + kg * 8) : make_uint2(0, 0);
          kb[u][ks] = fp8x8_to_bf16x8(raw);
        }
        if (valid[u]) scl[u] = a.cache.scales[row];
      } else {
        const uint16_t* rp = reinterpret_cast<const uint16_t*>(pages) + (valid[u] ? row : 0) * DIM;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 raw = valid[u] ? *reinterpret_cast<const uint4*>(rp + ks * 32 + kg * 8) : make_uint4(0, 0, 0, 0);
          kb[u][ks] = __builtin_bit_cast(bf16x8, raw);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TILES_PER_ITER; ++u) {
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][ks], kb[u][ks], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wv[ht][i] * fmaxf(acc[i], 0.f);
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (FP8) part *= scl[u];
      const int64_t e = (t0 + u) * 16 + col;
      if (kg == 0 && e < e_end) {
        const uint32_t key = valid[u] ? score_key(part) : 0u;
        keys_q[e] = key;
        atomicAdd(&hist_s[key >> (32 - kHistBits)], 1u);
      }
    }
  }
  flush_hist(hist_s, ws.hist + int64_t(q) * kHistBins);
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
    ws.keys[int64_t(q) * a.max_elig + e] = key;
    atomicAdd(&hist_s[key >> (32 - kHistBits)], 1u);
  }
  flush_hist(hist_s, ws.hist + int64_t(q) * kHistBins);
}

// ------------------------------------------------------------------ select
// Wave-aggregated append of the lanes with `take` set; slots at or beyond `cap` are dropped.
__device__ __forceinline__ void wave_append(bool take, uint2 item, uint32_t* counter, uint2* list, uint32_t cap) {
  const uint64_t mask = __ballot(take);
  if (!mask) return;
  const int lane = threadIdx.x & 63;
  uint32_t base = 0;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  if (lane == leader) base = atomicAdd(counter, uint32_t(__popcll(mask)));
  base = __shfl(base, leader);
  if (take) {
    const uint32_t off = __popcll(mask & ((1ull << lane) - 1ull));
    if (base + off < cap) list[base + off] = item;
  }
}

// Bitonic sort of n (power of two, <= 2048) (index, key) pairs in LDS by ascending index.
__device__ void bitonic_by_index(uint32_t* idx, uint32_t* key, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const uint32_t a = idx[lo], b = idx[hi];
        if ((a > b) == up) {
          idx[lo] = b; idx[hi] = a;
          const uint32_t ka = key[lo]; key[lo] = key[hi]; key[hi] = ka;
        }
      }
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(256) select_kernel(IndexArgs a, Workspace ws) {
  __shared__ uint32_t part[256];
  __shared__ uint32_t dig[256];
  __shared__ int s_b0;
  __shared__ int s_last;
  __shared__ uint32_t s_sel_n;
  __shared__ uint32_t sel_idx[kMaxK];
  __shared__ uint32_t sel_key[kMaxK];

  const int q = blockIdx.y;
  int seq;
  const int64_t n_elig = query_elig(a, q, &seq);
  const int64_t kk = min<int64_t>(a.k, n_elig);  // entries to choose
  const uint32_t* hist = ws.hist + int64_t(q) * kHistBins;
  const int tid = threadIdx.x;

  // ---- boundary bin: largest b0 with count(bins >= b0) >= kk
  if (tid == 0) s_b0 = -1;
  if (n_elig > a.k) {
    uint32_t h[16];
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) { h[j] = hist[tid * 16 + j]; local += h[j]; }
    part[tid] = local;
    __syncthreads();
    // inclusive suffix sums over threads (Hillis-Steele from the top)
    for (int off = 1; off < 256; off <<= 1) {
      const uint32_t v = (tid + off < 256) ? part[tid + off] : 0u;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    uint32_t run = part[tid] - local;  // keys in bins above this thread's range
    for (int j = 15; j >= 0; --j) {
      if (run < uint32_t(kk) && run + h[j] >= uint32_t(kk)) s_b0 = tid * 16 + j;
      run += h[j];
    }
  }
  __syncthreads();
  const int b0 = s_b0;

  // ---- partition this block's run of keys
  const uint32_t* keys_q = ws.keys + int64_t(q) * a.max_elig;
  uint32_t* ctr = ws.ctr + 4 * q;
  uint2* sure = ws.sure + int64_t(q) * a.k;
  uint2* cand = ws.cand + int64_t(q) * a.max_elig;
  const int64_t r_begin = int64_t(blockIdx.x) * kSelectChunk;
  const int64_t r_end = min(n_elig, r_begin + kSelectChunk);
  for (int64_t base = r_begin; base < r_end; base += blockDim.x) {
    const int64_t i = base + tid;
    const bool in = i < r_end;
    const uint32_t key = in ? keys_q[i] : 0u;
    const int bin = int(key >> (32 - kHistBits));
    const bool is_sure = in && (b0 < 0 || bin > b0);
    const bool is_cand = in && b0 >= 0 && bin == b0;
    wave_append(is_sure, make_uint2(key, uint32_t(i)), ctr + 0, sure, uint32_t(a.k));
    wave_append(is_cand, make_uint2(key, uint32_t(i)), ctr + 1, cand, uint32_t(a.max_elig));
  }

  // ---- last arriving block of this query finishes the selection
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(ctr + 2, 1u);
    s_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const uint32_t n_sure = min(__hip_atomic_load(ctr + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), uint32_t(a.k));
  const uint32_t n_cand = min(__hip_atomic_load(ctr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), uint32_t(a.max_elig));
  int64_t need = kk - int64_t(n_sure);
  uint32_t prefix = uint32_t(b0 < 0 ? 0 : b0) << (32 - kHistBits);
  uint32_t pmask = (b0 < 0) ? 0u : (0xFFFFFFFFu << (32 - kHistBits));
  uint32_t tie_count = 0;
  uint32_t idx_limit = 0xFFFFFFFFu;
  if (need > 0) {
    // digit passes over key bits 19..12, 11..4, 3..0 among candidates matching the prefix
    const int shifts[3] = {12, 4, 0};
    const uint32_t dmasks[3] = {0xFFu, 0xFFu, 0xFu};
    for (int p = 0; p < 3; ++p) {
      dig[tid] = 0u;
      __syncthreads();
      for (uint32_t j = tid; j < n_cand; j += blockDim.x) {
        const uint32_t key = cand[j].x;
        if ((key & pmask) == prefix) atomicAdd(&dig[(key >> shifts[p]) & dmasks[p]], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t run = 0;
        int d = int(dmasks[p]);
        for (; d > 0; --d) {
          if (run + dig[d] >= uint32_t(need)) break;
          run += dig[d];
        }
        part[0] = uint32_t(d);
        part[1] = run;
        part[2] = dig[d];
      }
      __syncthreads();
      const uint32_t d = part[0];
      need -= part[1];
      prefix |= d << shifts[p];
      pmask |= dmasks[p] << shifts[p];
      tie_count = part[2];
      __syncthreads();
    }
    // prefix is now the exact threshold key; take `need` of its tie_count ties, lowest index first
    if (uint32_t(need) < tie_count) {
      uint32_t ipre = 0, imask = 0;
      int64_t want = need;
      for (int shift = 24; shift >= 0; shift -= 8) {
        dig[tid] = 0u;
        __syncthreads();
        for (uint32_t j = tid; j < n_cand; j += blockDim.x) {
          const uint2 c = cand[j];
          if (c.x == prefix && (c.y & imask) == ipre) atomicAdd(&dig[(c.y >> shift) & 0xFFu], 1u);
        }
        __syncthreads();
        if (tid == 0) {
          uint32_t run = 0;
          int d = 0;
          for (; d < 255; ++d) {
            if (run + dig[d] >= uint32_t(want)) break;
            run += dig[d];
          }
          part[0] = uint32_t(d);
          part[1] = run;
        }
        __syncthreads();
        want -= part[1];
        ipre |= part[0] << shift;
        imask |= 0xFFu << shift;
        __syncthreads();
      }
      idx_limit = ipre;
    }
  }

  // ---- gather the chosen entries into LDS
  if (tid == 0) s_sel_n = 0;
  __syncthreads();
  for (uint32_t j = tid; j < n_sure; j += blockDim.x) {
    const uint2 c = sure[j];
    const uint32_t slot = atomicAdd(&s_sel_n, 1u);
    if (slot < kMaxK) { sel_idx[slot] = c.y; sel_key[slot] = c.x; }
  }
  if (kk - int64_t(n_sure) > 0) {
    for (uint32_t j = tid; j < n_cand; j += blockDim.x) {
      const uint2 c = cand[j];
      const bool take = (c.x > prefix) || (c.x == prefix && c.y <= idx_limit);
      if (take) {
        const uint32_t slot = atomicAdd(&s_sel_n, 1u);
        if (slot < kMaxK) { sel_idx[slot] = c.y; sel_key[slot] = c.x; }
      }
    }
  }
  __syncthreads();
  const int n_sel = int(min<uint32_t>(s_sel_n, uint32_t(kk)));
  int p2 = 1;
  while (p2 < n_sel) p2 <<= 1;
  for (int j = n_sel + tid; j < p2; j += blockDim.x) { sel_idx[j] = 0xFFFFFFFFu; sel_key[j] = 0u; }
  if (p2 > 1) bitonic_by_index(sel_idx, sel_key, p2);
  __syncthreads();
  for (int j = tid; j < a.k; j += blockDim.x) {
    const bool ok = j < n_sel;
    a.out_idx[int64_t(q) * a.k + j] = ok ? int32_t(sel_idx[j]) : -1;
    if (a.out_scores) a.out_scores[int64_t(q) * a.k + j] = ok ? key_score(sel_key[j]) : __uint_as_float(0x7FC00000u);
  }
  if (tid == 0 && a.out_count) a.out_count[q] = n_sel;
  // leave this query's histogram and counters zeroed for the next call on this workspace
  uint32_t* hq = ws.hist + int64_t(q) * kHistBins;
  for (int b = tid; b < kHistBins; b += blockDim.x) hq[b] = 0u;
  if (tid < 4) ctr[tid] = 0u;
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
  return clean_bytes(n_q) + align256(size_t(n_q) * size_t(max_elig) * 4) + align256(size_t(n_q) * size_t(k) * 8) +
         align256(size_t(n_q) * size_t(max_elig) * 8);
}

size_t index_clean_bytes(int n_q) { return clean_bytes(n_q); }

bool index_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads, csa_score_t mode) {
  if (c.dtype == CSA_F32) return q_dtype == CSA_F32 && n_heads * c.dim <= 8192;
  if (q_dtype != CSA_BF16) return false;
  const bool mfma = mode == CSA_SCORE_WRELU && c.dim == 128 && n_heads % 16 == 0 && n_heads <= 64;
  return mfma || n_heads * c.dim <= 8192;
}

hipError_t launch_index_clear(void* ws_base, int n_q, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  Workspace ws = carve(ws_base, n_q, 0, 1);
  const int64_t words = int64_t(n_q) * (kHistBins + 4);
  const int64_t nb = (words + 255) / 256;
  const int blocks = int(nb < 4096 ? nb : 4096);
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, stream, ws.hist, ws.ctr, n_q);
  return hipGetLastError();
}

hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream) {
  if (a.n_q == 0 || a.max_elig == 0) return hipSuccess;
  Workspace ws = carve(a.ws, a.n_q, a.max_elig, a.k);
  const bool mfma = a.cache.dtype != CSA_F32 && a.mode == CSA_SCORE_WRELU && a.cache.dim == 128 &&
                    a.n_heads % 16 == 0 && a.n_heads <= 64;
  if (mfma) {
    const dim3 grid(unsigned((a.max_elig + kScoreChunk - 1) / kScoreChunk), unsigned(a.n_q));
    const bool fp8 = a.cache.dtype == CSA_FP8_E4M3;
    switch (a.n_heads / 16) {
      case 1: if (fp8) hipLaunchKernelGGL((score_mfma_kernel<true, 1>), grid, dim3(256), 0, stream, a, ws);
              else hipLaunchKernelGGL((score_mfma_kernel<false, 1>), grid, dim3(256), 0, stream, a, ws); break;
      case 2: if (fp8) hipLaunchKernelGGL((score_mfma_kernel<true, 2>), grid, dim3(256), 0, stream, a, ws);
              else hipLaunchKernelGGL((score_mfma_kernel<false, 2>), grid, dim3(256), 0, stream, a, ws); break;
      case 3: if (fp8) hipLaunchKernelGGL((score_mfma_kernel<true, 3>), grid, dim3(256), 0, stream, a, ws);
              else hipLaunchKernelGGL((score_mfma_kernel<false, 3>), grid, dim3(256), 0, stream, a, ws); break;
      default: if (fp8) hipLaunchKernelGGL((score_mfma_kernel<true, 4>), grid, dim3(256), 0, stream, a, ws);
               else hipLaunchKernelGGL((score_mfma_kernel<false, 4>), grid, dim3(256), 0, stream, a, ws); break;
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

hipError_t launch_index_select(const IndexArgs& a, hipStream_t stream) {
  if (a.n_q == 0) return hipSuccess;
  if (a.max_elig == 0) {
    hipLaunchKernelGGL(empty_rows_kernel, dim3(a.n_q), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  Workspace ws = carve(a.ws, a.n_q, a.max_elig, a.k);
  const dim3 sgrid(unsigned((a.max_elig + kSelectChunk - 1) / kSelectChunk), unsigned(a.n_q));
  hipLaunchKernelGGL(select_kernel, sgrid, dim3(256), 0, stream, a, ws);
  return hipGetLastError();
}

}  // namespace csa
