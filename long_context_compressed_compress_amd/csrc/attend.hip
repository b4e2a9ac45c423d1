// csa_attend kernels: shared-K=V attention of each query over its selected compressed entries
// (or every eligible entry) plus the raw sliding window, one joint softmax, optional fused
// inverse RoPE at the query position.
//
// [P1] "DeepSeek V4 Attention Architecture": K and V are one shared vector, top-k compressed entries
// (DSA) plus a 128-token sliding window of raw tokens, inverse RoPE on the output.
// [P2] "二、注意力機制為什么這么麻煩": c128a (HCA) layers attend densely; prefill uses bf16 caches and
// decode a token-wise fp8 cache in the same kernel. [P2] "3.2 內核": inverse RoPE fused after attention.
//
// Two kernels:
//   * attend_mfma: bf16 / fp8 caches, D = 512, heads in groups of 16. One workgroup per
//     (query, 16-head group); the groups of one query are placed on the same XCD so their key
//     gathers share that XCD's L2. 64-key tiles are gathered into LDS (fp8 codes widened to bf16
//     exactly, row scale folded into logits and probabilities). S = Q K^T on
//     v_mfma_f32_16x16x32_bf16 (wave w owns keys 16w..16w+15 of the tile); online softmax across
//     tiles; O += P K with P split into bf16 hi + lo parts (fp32-accurate weights), wave w owning
//     dims 128w..128w+127. The PV contraction walks keys in an interleaved order so the four lane
//     groups read LDS rows that fall in disjoint banks.
//   * attend_valu: fp32 caches or other shapes; one workgroup per (query, head), 1024-key chunks.
#include "csa_internal.h"

namespace csa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct KeyRef {
  int64_t row;  // page row, -1 = masked key
  int kind;     // 0 compressed entry, 1 window row
};

__device__ __forceinline__ int64_t attend_elig(const AttendArgs& a, int q) {
  int64_t n = num_eligible(a.q_pos[q], a.cache.ratio, a.cache.window);
  if (n > a.max_elig) n = a.max_elig;
  return n < 0 ? 0 : n;
}

// Key t of query q: t < n_c -> compressed entry (top-k slot t or entry t in dense mode),
// else window position lo + (t - n_c).
__device__ __forceinline__ KeyRef key_ref(const AttendArgs& a, int q, int seq, int64_t t, int64_t n_c, int64_t n_elig,
                                          int64_t lo) {
  KeyRef r{-1, 0};
  if (t < n_c) {
    int64_t e = t;
    if (a.topk) {
      e = a.topk[int64_t(q) * a.k + t];
      if (e < 0 || e >= n_elig) return r;
    }
    if (seq < 0 || seq >= a.cache.batch) return r;
    r.row = entry_row(a.cache.block_table + int64_t(seq) * a.cache.bt_stride, a.cache.bt_stride, a.cache.n_phys, e,
                      kBlock / a.cache.ratio);
    r.kind = 0;
  } else {
    if (seq < 0 || seq >= a.swa.batch) return r;
    r.row = raw_row(a.swa.block_table + int64_t(seq) * a.swa.bt_stride, a.swa.bt_stride, a.swa.n_phys, lo + (t - n_c));
    r.kind = 1;
  }
  return r;
}

// ------------------------------------------------------------------ MFMA path
constexpr int kTile = 64;                      // keys per tile
constexpr int kD = 512;                        // head dim of the MFMA path
constexpr int kRowStride = kD * 2 + 16;        // LDS bytes per key row (bf16 + 16 B pad)
constexpr int kPStride = 64 + 8;               // bf16 elements per P row (16 B pad)
constexpr int kMaxKeys = kMaxK + 1024;         // top-k entries + largest window

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Position, inside a 32-key PV k-step, of key kk in the A/B operand order: lane group g holds
// keys 2g, 2g+1, 2g+8, 2g+9, 2g+16, 2g+17, 2g+24, 2g+25 as its elements 0..7.
__device__ __forceinline__ int perm_pos(int kk) {
  const int g = (kk & 7) >> 1;
  const int j = (kk & 1) + 2 * (kk >> 3);
  return g * 8 + j;
}
__device__ __forceinline__ int perm_key(int g, int j) { return 2 * g + (j & 1) + 8 * (j >> 1); }

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4) of the 64-bit words
// addressed by lanes i/4 + 4j (j = 0..3) of its group, as its elements j.
__device__ __forceinline__ uint2 lds_tr16(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15): quad swaps, half-row and row mirrors.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}
// Value of the lane whose index differs in bit 0 (quad_perm [1,0,3,2]).
__device__ __forceinline__ float pair_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// ---- output epilogue, fp32 or fp8 (the inverse rotation is applied before either).
// A lane holds rr[nt][i] = output of head (kg * 4 + i) of its 16-head group at dim d0 + nt * 16 + col. The fp8
// form stores groups of GN * 16 consecutive channels of one head as e4m3 codes with one fp32 scale: amax over the
// group (GN registers of the lane, then the 16 lanes of its DPP row), code = e4m3_rne(y * (448 / amax)),
// scale = amax / 448, zero codes and scale 1 for an all-zero group.
template <int NT, int GN>
__device__ __forceinline__ void store_fp8_groups(const float (&rr)[NT][4], uint8_t* codes, float* scales, int64_t row0,
                                                 int d0, int col, int group) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint8_t* crow = codes + (row0 + i) * kD;
    float* srow = scales + (row0 + i) * (kD / group);
#pragma unroll
    for (int g = 0; g < NT; g += GN) {
      float amax = 0.f;
#pragma unroll
      for (int n = 0; n < GN; ++n) amax = fmaxf(amax, fabsf(rr[g + n][i]));
      amax = row_max16(amax);
      const float inv = 448.0f / amax;
#pragma unroll
      for (int n = 0; n < GN; ++n)
        crow[d0 + (g + n) * 16 + col] = amax > 0.f ? uint8_t(f32_to_e4m3_rne(rr[g + n][i] * inv)) : uint8_t(0);
      if (col == 0) srow[(d0 + g * 16) / group] = amax > 0.f ? amax / 448.0f : 1.0f;
    }
  }
}

template <int NT>
__device__ __forceinline__ void store_output(const AttendArgs& a, const float (&rr)[NT][4], int q, int h0, int d0,
                                             int col) {
  const int64_t row0 = int64_t(q) * a.n_heads + h0;
  if (a.out) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.out[(row0 + i) * kD + d0 + nt * 16 + col] = rr[nt][i];
    return;
  }
  switch (a.group) {
    case 16: store_fp8_groups<NT, 1>(rr, a.out_codes, a.out_scales, row0, d0, col, 16); break;
    case 32: store_fp8_groups<NT, 2>(rr, a.out_codes, a.out_scales, row0, d0, col, 32); break;
    case 64: store_fp8_groups<NT, 4>(rr, a.out_codes, a.out_scales, row0, d0, col, 64); break;
    default: store_fp8_groups<NT, 8>(rr, a.out_codes, a.out_scales, row0, d0, col, 128); break;
  }
}

template <bool FP8>
struct TileRegs;
template <>
struct TileRegs<false> { uint4 v[16]; };  // 64 rows x 1 KiB / 256 threads
template <>
struct TileRegs<true> { uint4 v[8]; };    // 64 rows x 512 B / 256 threads

template <bool FP8>
__global__ void __launch_bounds__(256) attend_mfma_kernel(AttendArgs a) {
  constexpr int kPassKeys = kMaxKeys;           // keys whose rows are resolved per pass
  constexpr int kPerThread = kPassKeys / 256;
  __shared__ __attribute__((aligned(16))) char k_lds[kTile * kRowStride];
  __shared__ __attribute__((aligned(16))) uint16_t p_hi[16 * kPStride];
  __shared__ __attribute__((aligned(16))) uint16_t p_lo[16 * kPStride];
  __shared__ int32_t key_row[kPassKeys];   // page row of every key of the pass, -1 = masked
  __shared__ uint8_t key_kind[kPassKeys];  // 0 compressed entry, 1 window row
  __shared__ float k_scale[kTile];
  __shared__ float red_max[4][16];
  __shared__ float red_sum[4][16];

  const int HG = a.n_heads / 16;
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int rest = L >> 3;
  const int hg = rest % HG;
  const int q = (rest / HG) * 8 + xcd;
  if (q >= a.n_q) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int seq = a.q_seq[q];
  const int64_t p = a.q_pos[q];
  const int64_t n_elig = attend_elig(a, q);
  const int64_t n_c = a.topk ? a.k : n_elig;
  const int64_t lo = (a.swa_window > 0) ? max<int64_t>(0, p - a.swa_window + 1) : p + 1;
  const int64_t n_swa = (a.swa_window > 0) ? max<int64_t>(0, p - lo + 1) : 0;
  const int64_t n_keys = n_c + n_swa;
  // rows are kept as int32 in LDS; larger pools are rejected at the host (attend_supported)

  bf16x8 qa[16];
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (int64_t(q) * a.n_heads + hg * 16 + col) * kD;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qa[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 32 + kg * 8));

  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  const float scale = a.scale;
  // descriptor fields as locals: selecting between struct fields per lane would turn into vector loads
  // from the kernel-argument block, each followed by a full wait
  // rows of an out-of-range sequence id are never used (seq_c / seq_w mask them); point at row 0 so that the
  // unconditional table loads stay inside the table
  const int32_t* bt_c = a.cache.block_table + int64_t(seq >= 0 && seq < a.cache.batch ? seq : 0) * a.cache.bt_stride;
  const int32_t* bt_w = a.swa.block_table + int64_t(seq >= 0 && seq < a.swa.batch ? seq : 0) * a.swa.bt_stride;
  const int bts_c = a.cache.bt_stride, bts_w = a.swa.bt_stride;
  const int nph_c = a.cache.n_phys, nph_w = a.swa.n_phys;
  const bool seq_c = seq >= 0 && seq < a.cache.batch;
  const bool seq_w = seq >= 0 && seq < a.swa.batch;
  const int per_block = kBlock / a.cache.ratio;
  const int32_t* topk_q = a.topk ? a.topk + int64_t(q) * a.k : nullptr;
  // The window pool is addressed as an integer offset from the cache pool so that choosing a pool per lane
  // is a register select (a per-lane choice between two pointers otherwise becomes an indexed stack load).
  const char* pages_c = static_cast<const char*>(a.cache.pages);
  const int64_t pages_dw = int64_t(reinterpret_cast<uintptr_t>(a.swa.kv_pages)) - int64_t(reinterpret_cast<uintptr_t>(pages_c));
  const float* scales_c = a.cache.scales;
  const int64_t scales_dw = FP8 ? (int64_t(reinterpret_cast<uintptr_t>(a.swa.scales)) - int64_t(reinterpret_cast<uintptr_t>(scales_c))) : 0;

  for (int64_t pass0 = 0; pass0 < n_keys; pass0 += kPassKeys) {
    const int n_pass = int(min<int64_t>(kPassKeys, n_keys - pass0));
    // ---- resolve the page rows of this pass: entry ids first, then block-table lookups. Every load is
    // unconditional (indices clamped into range) so that a thread's loads are all in flight together.
    {
      int32_t ent[kPerThread];  // entry ids and window positions are below 2^31
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int64_t t = pass0 + tid + 256 * j;
        // top-k mode: unconditional load (clamped index); dense mode reads no index list at all
        const int32_t v = topk_q ? topk_q[t < n_c ? t : 0] : 0;
        int64_t e = topk_q ? int64_t(v) : t;
        if (t >= n_c) e = (t < n_keys) ? lo + (t - n_c) : -1;
        ent[j] = int32_t(e);
      }
      int32_t phys[kPerThread];
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int64_t t = pass0 + tid + 256 * j;
        const bool is_c = t < n_c;
        const int64_t blk = ent[j] < 0 ? 0 : ent[j] / (is_c ? per_block : kBlock);
        const int32_t* bt = is_c ? bt_c : bt_w;
        const int bts = is_c ? bts_c : bts_w;
        phys[j] = bt[blk < bts ? blk : bts - 1];
      }
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int local = tid + 256 * j;
        const int64_t t = pass0 + local;
        const bool is_c = t < n_c;
        const int64_t e = ent[j];
        const int per = is_c ? per_block : kBlock;
        const int64_t blk = e < 0 ? 0 : e / per;
        bool ok = e >= 0 && t < n_keys && blk < (is_c ? bts_c : bts_w) && phys[j] >= 0 &&
                  phys[j] < (is_c ? nph_c : nph_w) && (is_c ? (seq_c && e < n_elig) : seq_w);
        const int64_t row = ok ? int64_t(phys[j]) * per + (e - blk * per) : -1;
        if (local < kPassKeys) {
          key_row[local] = int32_t(row);
          key_kind[local] = uint8_t(is_c ? 0 : 1);
        }
      }
    }
    __syncthreads();

    // Global loads of one tile into registers: thread tid covers rows (tid>>6) + 4i, 16-byte chunk (tid & 63)
    // (bf16) or rows (tid>>5) + 8i, chunk (tid & 31) (fp8). Masked rows read row 0 and are zeroed at stash.
    auto issue = [=](int t0, TileRegs<FP8>& R, uint32_t& valid_mask, float& my_scale) {
      valid_mask = 0u;
      constexpr int N = FP8 ? 8 : 16;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int r = FP8 ? (tid >> 5) + 8 * i : (tid >> 6) + 4 * i;
        const int cc = FP8 ? (tid & 31) : (tid & 63);
        const int t = t0 + r;
        const int64_t row = t < n_pass ? key_row[t] : -1;
        const int kind = t < n_pass ? key_kind[t] : 0;
        const bool ok = row >= 0;
        valid_mask |= uint32_t(ok) << i;
        const int64_t off = (kind == 0 ? 0 : pages_dw) + (ok ? row : 0) * (FP8 ? kD : 2 * kD) + cc * 16;
        R.v[i] = *reinterpret_cast<const uint4*>(pages_c + off);
      }
      my_scale = -1.f;  // a negative scale marks a masked key
      if (tid < kTile) {
        const int t = t0 + tid;
        const int64_t row = t < n_pass ? key_row[t] : -1;
        if (row >= 0) {
          my_scale = 1.f;
          if (FP8) my_scale = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(scales_c) +
                                                               (key_kind[t] == 0 ? 0 : scales_dw) + row * 4);
        }
      }
    };
    auto stash = [=](const TileRegs<FP8>& R, uint32_t valid_mask, float my_scale) {
      constexpr int N = FP8 ? 8 : 16;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bool ok = (valid_mask >> i) & 1u;
        if (!FP8) {
          const int r = (tid >> 6) + 4 * i, cc = tid & 63;
          *reinterpret_cast<uint4*>(k_lds + r * kRowStride + cc * 16) = ok ? R.v[i] : make_uint4(0, 0, 0, 0);
        } else {
          const int r = (tid >> 5) + 8 * i, cc = tid & 31;
          const uint4 v = ok ? R.v[i] : make_uint4(0, 0, 0, 0);
          const uint32_t src[4] = {v.x, v.y, v.z, v.w};
          uint32_t w[8];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            // exact pair conversion e4m3 -> bf16 (scale 1)
            w[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[h], 1.0f, false));
            w[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[h], 1.0f, true));
          }
          uint4* dst = reinterpret_cast<uint4*>(k_lds + r * kRowStride + cc * 32);
          dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
          dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
      }
      if (tid < kTile) k_scale[tid] = my_scale;
    };

    TileRegs<FP8> R;
    uint32_t vmask = 0;
    float my_scale = -1.f;
    issue(0, R, vmask, my_scale);
    for (int t0 = 0; t0 < n_pass; t0 += kTile) {
      lds_barrier();  // previous tile's readers of k_lds / p / red are done
      stash(R, vmask, my_scale);
      lds_barrier();
      if (t0 + kTile < n_pass) issue(t0 + kTile, R, vmask, my_scale);  // next tile's loads overlap this tile's math

      // ---- S = Q K^T for this wave's 16 keys (two independent accumulation chains)
      f32x4 s = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
      {
        const char* krow = k_lds + (wave * 16 + col) * kRowStride + kg * 16;
#pragma unroll
        for (int ks = 0; ks < 16; ks += 2) {
          const bf16x8 kb0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 64));
          const bf16x8 kb1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 64 + 64));
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb0, s, 0, 0, 0);
          s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks + 1], kb1, s2, 0, 0, 0);
        }
      }
      const int key_local = wave * 16 + col;
      const float ksc = k_scale[key_local];
      const bool kvalid = ksc >= 0.f;
      float lg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[i] = kvalid ? (s[i] + s2[i]) * (scale * ksc) : -INFINITY;
      // tile max per head (lane holds heads kg*4+i of key col; the 16 keys of a head sit in one DPP row)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mx = row_max16(lg[i]);
        if (col == 0) red_max[wave][kg * 4 + i] = mx;
      }
      lds_barrier();
      float corr[4], pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = kg * 4 + i;
        const float tmax = fmaxf(fmaxf(red_max[0][h], red_max[1][h]), fmaxf(red_max[2][h], red_max[3][h]));
        const float mnew = fmaxf(m_run[i], tmax);
        corr[i] = (m_run[i] == -INFINITY) ? 0.f : __expf(m_run[i] - mnew);
        pv[i] = (lg[i] == -INFINITY) ? 0.f : __expf(lg[i] - mnew);
        m_run[i] = mnew;
        const float sm = row_sum16(pv[i]);
        if (col == 0) red_sum[wave][h] = sm;
      }
      {
        const int ks2 = key_local >> 5;
        const int pos = ks2 * 32 + perm_pos(key_local & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w = kvalid ? pv[i] * ksc : 0.f;  // fp8: the row scale multiplies the value side too
          const uint16_t hi = f32_to_bf16_rne(w);
          const uint16_t lo16 = f32_to_bf16_rne(w - bf16_to_f32(hi));
          p_hi[(kg * 4 + i) * kPStride + pos] = hi;
          p_lo[(kg * 4 + i) * kPStride + pos] = lo16;
        }
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = kg * 4 + i;
        l_run[i] = l_run[i] * corr[i] + (red_sum[0][h] + red_sum[1][h] + red_sum[2][h] + red_sum[3][h]);
      }
      // ---- O = O * corr + P K over this wave's 128 dims (B operand by transposing LDS reads)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= corr[i];
      const int s_lane = lane & 15;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p_hi + col * kPStride + ks2 * 32 + kg * 8));
        const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p_lo + col * kPStride + ks2 * 32 + kg * 8));
        const int r0 = ks2 * 32 + perm_key(kg, s_lane >> 2);
        const int r1 = ks2 * 32 + perm_key(kg, 4 + (s_lane >> 2));
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const int dcol = wave * 128 + nt * 16 + 4 * (s_lane & 3);
          const uint2 e0 = lds_tr16(k_lds + r0 * kRowStride + dcol * 2);
          const uint2 e1 = lds_tr16(k_lds + r1 * kRowStride + dcol * 2);
          const bf16x8 kb = __builtin_bit_cast(bf16x8, make_uint4(e0.x, e0.y, e1.x, e1.y));
          o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, kb, o[nt], 0, 0, 0);
          o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, kb, o[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next pass rewrites the row table
  }

  // ---- epilogue: normalise, optional inverse RoPE, store (fp32 or grouped fp8)
  const int R_ = a.cache.rope_dims;
  const int base = kD - R_;
  const bool rot = a.fuse_inv_rope && R_ > 0 && p >= 0 && p < a.rope_rows;
  const float* cs = rot ? a.rope_cs + p * int64_t(R_) : a.rope_cs;
  float rr[8][4];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int d = wave * 128 + nt * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv_l = (l_run[i] > 0.f) ? 1.f / l_run[i] : 0.f;
      const float v = o[nt][i] * inv_l;
      const float partner = pair_swap(v);
      float r = v;
      if (rot && d >= base) {
        const int j = (d - base) >> 1;
        const float c = cs[2 * j], sn = cs[2 * j + 1];
        r = (d & 1) ? (-partner * sn + v * c) : (v * c + partner * sn);
      }
      rr[nt][i] = r;
    }
  }
  store_output<8>(a, rr, q, hg * 16 + kg * 4, wave * 128, col);
  if (a.out_lse && wave == 0 && col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hg * 16 + kg * 4 + i;
      a.out_lse[int64_t(q) * a.n_heads + h] = (l_run[i] > 0.f) ? m_run[i] + logf(l_run[i]) : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------ split MFMA path (64 heads per block)
// One 512-thread workgroup per (query, 64-head chunk, key split): every key row is gathered once per query
// chunk and feeds all 64 heads. Wave w serves head group hg = w/2 (16 heads) and half sw = w%2: in S it owns
// keys 32sw..32sw+31 of the 64-key tile, in PV dims 256sw..256sw+255. Splits of one query write partial
// (max, sum, unnormalised output) to the workspace and attend_combine merges them; with one split the block
// writes the final output itself.
struct SplitPlan {
  int n_split;      // key splits per query
  int split_keys;   // keys per split (multiple of the tile)
};

__host__ __device__ inline SplitPlan split_plan(int n_q, int n_hchunk, int64_t max_keys) {
  SplitPlan sp;
  const int64_t tiles = (max_keys + kTile - 1) / kTile;
  const int64_t want = (512 + int64_t(n_q) * n_hchunk - 1) / (int64_t(n_q) * n_hchunk);  // about two blocks per CU
  int64_t ns = want < 1 ? 1 : want;
  // at least two tiles per split, unless one tile per split still fits one round of workgroups (one per CU)
  const int64_t max_split = (int64_t(n_q) * n_hchunk * tiles <= 256) ? tiles : (tiles + 1) / 2;
  if (ns > max_split) ns = max_split < 1 ? 1 : max_split;
  const int64_t tiles_per = (tiles + ns - 1) / ns;
  sp.split_keys = int(tiles_per * kTile);
  sp.n_split = int((tiles + tiles_per - 1) / tiles_per);
  if (sp.n_split < 1) sp.n_split = 1;
  return sp;
}

template <bool FP8>
struct TileRegs8;
template <>
struct TileRegs8<false> { uint4 v[8]; };  // 64 rows x 1 KiB / 512 threads
template <>
struct TileRegs8<true> { uint4 v[4]; };   // 64 rows x 512 B / 512 threads

template <bool FP8>
__global__ void __launch_bounds__(512) attend_split_kernel(AttendArgs a, SplitPlan sp, float* part_o, float* part_ml) {
  __shared__ __attribute__((aligned(16))) char k_lds[kTile * kRowStride];
  __shared__ __attribute__((aligned(16))) uint16_t p_hi[4][16 * kPStride];
  __shared__ __attribute__((aligned(16))) uint16_t p_lo[4][16 * kPStride];
  __shared__ int32_t key_row[kMaxKeys];
  __shared__ uint8_t key_kind[kMaxKeys];
  __shared__ float k_scale[kTile];
  __shared__ float red_max[4][2][16];
  __shared__ float red_sum[4][2][16];

  const int n_hchunk = a.n_heads / 64;
  const int split = blockIdx.x % sp.n_split;
  const int hc = (blockIdx.x / sp.n_split) % n_hchunk;
  const int q = blockIdx.x / (sp.n_split * n_hchunk);
  if (q >= a.n_q) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hg = wave >> 1;
  const int sw = wave & 1;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int seq = a.q_seq[q];
  const int64_t p = a.q_pos[q];
  const int64_t n_elig = attend_elig(a, q);
  const int64_t n_c = a.topk ? a.k : n_elig;
  const int64_t lo = (a.swa_window > 0) ? max<int64_t>(0, p - a.swa_window + 1) : p + 1;
  const int64_t n_swa = (a.swa_window > 0) ? max<int64_t>(0, p - lo + 1) : 0;
  const int64_t n_keys = n_c + n_swa;
  const int64_t k_begin = int64_t(split) * sp.split_keys;
  const int64_t k_end = min<int64_t>(n_keys, k_begin + sp.split_keys);

  // rows of an out-of-range sequence id are never used (seq_c / seq_w mask them); point at row 0 so that the
  // unconditional table loads stay inside the table
  const int32_t* bt_c = a.cache.block_table + int64_t(seq >= 0 && seq < a.cache.batch ? seq : 0) * a.cache.bt_stride;
  const int32_t* bt_w = a.swa.block_table + int64_t(seq >= 0 && seq < a.swa.batch ? seq : 0) * a.swa.bt_stride;
  const int bts_c = a.cache.bt_stride, bts_w = a.swa.bt_stride;
  const int nph_c = a.cache.n_phys, nph_w = a.swa.n_phys;
  const bool seq_c = seq >= 0 && seq < a.cache.batch;
  const bool seq_w = seq >= 0 && seq < a.swa.batch;
  const int per_block = kBlock / a.cache.ratio;
  const int32_t* topk_q = a.topk ? a.topk + int64_t(q) * a.k : nullptr;
  const char* pages_c = static_cast<const char*>(a.cache.pages);
  const int64_t pages_dw = int64_t(reinterpret_cast<uintptr_t>(a.swa.kv_pages)) - int64_t(reinterpret_cast<uintptr_t>(pages_c));
  const float* scales_c = a.cache.scales;
  const int64_t scales_dw = FP8 ? (int64_t(reinterpret_cast<uintptr_t>(a.swa.scales)) - int64_t(reinterpret_cast<uintptr_t>(scales_c))) : 0;

  // Keys of a pass: list slots (top-k mode) or entry numbers below n_c, then window positions. Key positions,
  // entries and window positions fit 32 bits (positions are 32-bit at the boundary). Every list load is
  // unconditional (dense mode reads element 0 of the position array and ignores it) and lands in a register of its
  // own; the entries are derived only after every load is out, so the loads overlap. (Overwriting a load's register
  // under a condition before the next load is issued makes each load wait for the one before it.)
  constexpr int PER = (kMaxKeys + 511) / 512;
  const int32_t* lst = topk_q ? topk_q : a.q_pos;
  const int n_c32 = int(n_c), n_keys32 = int(n_keys), lo32 = int(lo);
  auto issue_list = [&](int pass0, int32_t (&raw)[PER]) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int t = pass0 + tid + 512 * j;
      raw[j] = lst[(topk_q != nullptr && t < n_c32) ? t : 0];
    }
  };
  // the first pass's list loads go out before the query fragments: the wait for the list (loads complete in
  // issue order) then does not also wait for the 64 KiB of query
  int32_t raw[PER];
  issue_list(int(k_begin), raw);

  bf16x8 qa[16];
  const int head0 = hc * 64 + hg * 16;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (int64_t(q) * a.n_heads + head0 + col) * kD;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qa[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 32 + kg * 8));

  f32x4 o[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  const float scale = a.scale;

  // page rows of the keys of a pass from its list values (block-table loads unconditional, indices clamped)
  auto resolve = [&](int p0, const int32_t (&raw)[PER]) {
    int32_t ent[PER], phys[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int t = p0 + tid + 512 * j;
      ent[j] = t < n_c32 ? (topk_q ? raw[j] : t) : (t < n_keys32 ? lo32 + (t - n_c32) : -1);
    }
    // entries per block are a power of two (256 / ratio), as is the raw block of 256 positions
    const int lpb = __builtin_ctz(unsigned(per_block));
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool is_c = p0 + tid + 512 * j < n_c32;
      const int e = ent[j] < 0 ? 0 : ent[j];
      const int blk = is_c ? (e >> lpb) : (e >> 8);
      const int bts = is_c ? bts_c : bts_w;
      phys[j] = (is_c ? bt_c : bt_w)[blk < bts ? blk : bts - 1];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int local = tid + 512 * j;
      const int t = p0 + local;
      const bool is_c = t < n_c32;
      const int e = ent[j];
      const int sh = is_c ? lpb : 8;
      const int blk = (e < 0 ? 0 : e) >> sh;
      const bool ok = e >= 0 && t < n_keys32 && blk < (is_c ? bts_c : bts_w) && phys[j] >= 0 &&
                      phys[j] < (is_c ? nph_c : nph_w) && (is_c ? (seq_c && e < n_elig) : seq_w);
      if (local < kMaxKeys) {
        key_row[local] = int32_t(ok ? (int64_t(phys[j]) << sh) + (e - (blk << sh)) : -1);
        key_kind[local] = uint8_t(is_c ? 0 : 1);
      }
    }
  };
  // the first pass is resolved here, in straight-line code after the query loads, so that each wait covers only
  // the loads it needs; later passes (more keys than the row table holds) resolve at the top of their pass
  resolve(int(k_begin), raw);

  for (int64_t pass0 = k_begin; pass0 < k_end; pass0 += kMaxKeys) {
    const int n_pass = int(min<int64_t>(kMaxKeys, k_end - pass0));
    if (pass0 != k_begin) {
      int32_t raw2[PER];
      issue_list(int(pass0), raw2);
      resolve(int(pass0), raw2);
    }
    __syncthreads();

    auto issue = [=](int t0, TileRegs8<FP8>& R, uint32_t& valid_mask, float& my_scale) {
      valid_mask = 0u;
      constexpr int N = FP8 ? 4 : 8;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int r = FP8 ? (tid >> 5) + 16 * i : (tid >> 6) + 8 * i;
        const int cc = FP8 ? (tid & 31) : (tid & 63);
        const int t = t0 + r;
        const int64_t row = t < n_pass ? key_row[t] : -1;
        const int kind = t < n_pass ? key_kind[t] : 0;
        const bool ok = row >= 0;
        valid_mask |= uint32_t(ok) << i;
        const int64_t off = (kind == 0 ? 0 : pages_dw) + (ok ? row : 0) * (FP8 ? kD : 2 * kD) + cc * 16;
        R.v[i] = *reinterpret_cast<const uint4*>(pages_c + off);
      }
      my_scale = -1.f;  // a negative scale marks a masked key
      if (tid < kTile) {
        const int t = t0 + tid;
        const int64_t row = t < n_pass ? key_row[t] : -1;
        if (row >= 0) {
          my_scale = 1.f;
          if (FP8)
            my_scale = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(scales_c) +
                                                        (key_kind[t] == 0 ? 0 : scales_dw) + row * 4);
        }
      }
    };
    auto stash = [=](const TileRegs8<FP8>& R, uint32_t valid_mask, float my_scale) {
      constexpr int N = FP8 ? 4 : 8;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bool ok = (valid_mask >> i) & 1u;
        if (!FP8) {
          const int r = (tid >> 6) + 8 * i, cc = tid & 63;
          *reinterpret_cast<uint4*>(k_lds + r * kRowStride + cc * 16) = ok ? R.v[i] : make_uint4(0, 0, 0, 0);
        } else {
          const int r = (tid >> 5) + 16 * i, cc = tid & 31;
          const uint4 v = ok ? R.v[i] : make_uint4(0, 0, 0, 0);
          const uint32_t src[4] = {v.x, v.y, v.z, v.w};
          uint32_t w[8];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            // exact pair conversion e4m3 -> bf16 (scale 1)
            w[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[h], 1.0f, false));
            w[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[h], 1.0f, true));
          }
          uint4* dst = reinterpret_cast<uint4*>(k_lds + r * kRowStride + cc * 32);
          dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
          dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
      }
      if (tid < kTile) k_scale[tid] = my_scale;
    };

    TileRegs8<FP8> R;
    uint32_t vmask = 0;
    float my_scale = -1.f;
    issue(0, R, vmask, my_scale);
    for (int t0 = 0; t0 < n_pass; t0 += kTile) {
      lds_barrier();
      stash(R, vmask, my_scale);
      lds_barrier();
      if (t0 + kTile < n_pass) issue(t0 + kTile, R, vmask, my_scale);

      // ---- S for this wave's 32 keys (two 16-key column tiles) and its 16 heads
      f32x4 s[2];
#pragma unroll
      for (int n16 = 0; n16 < 2; ++n16) {
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        const char* krow = k_lds + (sw * 32 + n16 * 16 + col) * kRowStride + kg * 16;
#pragma unroll
        for (int ks = 0; ks < 16; ks += 2) {
          const bf16x8 kb0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 64));
          const bf16x8 kb1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 64 + 64));
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb0, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks + 1], kb1, a1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s[n16][i] = a0[i] + a1[i];
      }
      float ksc[2];
      bool kval[2];
      float lg[2][4];
#pragma unroll
      for (int n16 = 0; n16 < 2; ++n16) {
        ksc[n16] = k_scale[sw * 32 + n16 * 16 + col];
        kval[n16] = ksc[n16] >= 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) lg[n16][i] = kval[n16] ? s[n16][i] * (scale * ksc[n16]) : -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mx = row_max16(fmaxf(lg[0][i], lg[1][i]));
        if (col == 0) red_max[hg][sw][kg * 4 + i] = mx;
      }
      lds_barrier();
      float corr[4], pv[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = kg * 4 + i;
        const float tmax = fmaxf(red_max[hg][0][h], red_max[hg][1][h]);
        const float mnew = fmaxf(m_run[i], tmax);
        corr[i] = (m_run[i] == -INFINITY) ? 0.f : __expf(m_run[i] - mnew);
        pv[0][i] = (lg[0][i] == -INFINITY) ? 0.f : __expf(lg[0][i] - mnew);
        pv[1][i] = (lg[1][i] == -INFINITY) ? 0.f : __expf(lg[1][i] - mnew);
        m_run[i] = mnew;
        const float sm = row_sum16(pv[0][i] + pv[1][i]);
        if (col == 0) red_sum[hg][sw][h] = sm;
      }
#pragma unroll
      for (int n16 = 0; n16 < 2; ++n16) {
        const int key_local = sw * 32 + n16 * 16 + col;
        const int pos = (key_local >> 5) * 32 + perm_pos(key_local & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w = kval[n16] ? pv[n16][i] * ksc[n16] : 0.f;
          const uint16_t hi = f32_to_bf16_rne(w);
          const uint16_t lo16 = f32_to_bf16_rne(w - bf16_to_f32(hi));
          p_hi[hg][(kg * 4 + i) * kPStride + pos] = hi;
          p_lo[hg][(kg * 4 + i) * kPStride + pos] = lo16;
        }
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = kg * 4 + i;
        l_run[i] = l_run[i] * corr[i] + red_sum[hg][0][h] + red_sum[hg][1][h];
      }
      // ---- O (16 heads x this wave's 256 dims) = O * corr + P K
#pragma unroll
      for (int nt = 0; nt < 16; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= corr[i];
      const int s_lane = lane & 15;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&p_hi[hg][col * kPStride + ks2 * 32 + kg * 8]));
        const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&p_lo[hg][col * kPStride + ks2 * 32 + kg * 8]));
        const int r0 = ks2 * 32 + perm_key(kg, s_lane >> 2);
        const int r1 = ks2 * 32 + perm_key(kg, 4 + (s_lane >> 2));
#pragma unroll
        for (int nt = 0; nt < 16; ++nt) {
          const int dcol = sw * 256 + nt * 16 + 4 * (s_lane & 3);
          const uint2 e0 = lds_tr16(k_lds + r0 * kRowStride + dcol * 2);
          const uint2 e1 = lds_tr16(k_lds + r1 * kRowStride + dcol * 2);
          const bf16x8 kb = __builtin_bit_cast(bf16x8, make_uint4(e0.x, e0.y, e1.x, e1.y));
          o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, kb, o[nt], 0, 0, 0);
          o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, kb, o[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next pass rewrites the row table
  }

  // ---- epilogue
  if (sp.n_split == 1) {
    const int R_ = a.cache.rope_dims;
    const int base = kD - R_;
    const bool rot = a.fuse_inv_rope && R_ > 0 && p >= 0 && p < a.rope_rows;
    const float* cs = rot ? a.rope_cs + p * int64_t(R_) : a.rope_cs;
    float rr[16][4];
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
      const int d = sw * 256 + nt * 16 + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float inv_l = (l_run[i] > 0.f) ? 1.f / l_run[i] : 0.f;
        const float v = o[nt][i] * inv_l;
        const float partner = pair_swap(v);
        float r = v;
        if (rot && d >= base) {
          const int j = (d - base) >> 1;
          const float c = cs[2 * j], sn = cs[2 * j + 1];
          r = (d & 1) ? (-partner * sn + v * c) : (v * c + partner * sn);
        }
        rr[nt][i] = r;
      }
    }
    store_output<16>(a, rr, q, head0 + kg * 4, sw * 256, col);
    if (a.out_lse && sw == 0 && col == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.out_lse[int64_t(q) * a.n_heads + head0 + kg * 4 + i] = (l_run[i] > 0.f) ? m_run[i] + logf(l_run[i]) : -INFINITY;
  } else {
    // partial: unnormalised output relative to this split's running max, plus (max, sum)
    const int64_t slot = int64_t(q) * sp.n_split + split;
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
      const int d = sw * 256 + nt * 16 + col;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part_o[(slot * a.n_heads + head0 + kg * 4 + i) * kD + d] = o[nt][i];
    }
    if (sw == 0 && col == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t h = slot * a.n_heads + head0 + kg * 4 + i;
        part_ml[2 * h] = m_run[i];
        part_ml[2 * h + 1] = l_run[i];
      }
  }
}

// Merge the key splits of each (query, head): o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, then the
// optional inverse RoPE. One 256-thread workgroup per (query, 4 heads); a thread owns 8 consecutive dims.
template <int NSC>
__global__ void __launch_bounds__(256) attend_combine_kernel(AttendArgs a, SplitPlan sp, const float* part_o,
                                                             const float* part_ml) {
  const int hq = a.n_heads / 4;
  const int q = blockIdx.x / hq;
  const int h = (blockIdx.x % hq) * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  if (q >= a.n_q) return;
  const int64_t p = a.q_pos[q];
  const int ns = sp.n_split;
  const float2* ml = reinterpret_cast<const float2*>(part_ml);
  auto slot_of = [&](int s) { return (int64_t(q) * ns + (s < ns ? s : ns - 1)) * a.n_heads + h; };
  const int R_ = a.cache.rope_dims;
  const int base = kD - R_;
  const bool rot = a.fuse_inv_rope && R_ > 0 && p >= 0 && p < a.rope_rows;
  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float2 csv[4] = {};  // (cos, sin) of the rotation pair of dims d0 + 2 k, k < 4
  // the rotation's table row: loaded once the position is in (a scalar load issued first), beside the split loads
  auto load_cs = [&]() {
    if (!rot) return;  // uniform; the table may be absent without the rotation
    const float2* row = reinterpret_cast<const float2*>(a.rope_cs + p * int64_t(R_));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = d0 + 2 * k;
      csv[k] = row[d >= base ? (d - base) >> 1 : 0];  // clamped into the row
    }
  };
  if constexpr (NSC > 0) {
    // Up to NSC splits: every (max, sum) pair and partial output goes out before any is used, so they cost one
    // memory round trip; surplus slots re-read the last split and get weight 0. The sums are added in split order
    // as in a plain loop.
    float2 v[NSC];
    float4 x0[NSC], x1[NSC];
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      const int64_t slot = slot_of(j);
      v[j] = ml[slot];
      const float4* src = reinterpret_cast<const float4*>(part_o + slot * kD + d0);
      x0[j] = src[0];
      x1[j] = src[1];
    }
    load_cs();
#pragma unroll
    for (int j = 0; j < NSC; ++j)
      if (j < ns) M = fmaxf(M, v[j].x);
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      const float m = v[j].x, l = v[j].y;
      const float w = (j >= ns || m == -INFINITY) ? 0.f : __expf(m - M);
      L += w * l;
      acc[0] += w * x0[j].x; acc[1] += w * x0[j].y; acc[2] += w * x0[j].z; acc[3] += w * x0[j].w;
      acc[4] += w * x1[j].x; acc[5] += w * x1[j].y; acc[6] += w * x1[j].z; acc[7] += w * x1[j].w;
    }
  } else {
    // Any number of splits: a chunk of splits at a time (indices clamped, every load unconditional, surplus splits
    // of a chunk masked afterwards), so a chunk costs one memory round trip: first the (max, sum) pairs of up to
    // kMlChunk splits for the common maximum, then the partial outputs of kOChunk splits at a time.
    constexpr int kMlChunk = 16, kOChunk = 8;
    load_cs();
    for (int s0 = 0; s0 < ns; s0 += kMlChunk) {
      float2 v[kMlChunk];
#pragma unroll
      for (int j = 0; j < kMlChunk; ++j) v[j] = ml[slot_of(s0 + j)];
#pragma unroll
      for (int j = 0; j < kMlChunk; ++j)
        if (s0 + j < ns) M = fmaxf(M, v[j].x);
    }
    for (int s0 = 0; s0 < ns; s0 += kOChunk) {
      float2 v[kOChunk];
      float4 x0[kOChunk], x1[kOChunk];
#pragma unroll
      for (int j = 0; j < kOChunk; ++j) {
        const int64_t slot = slot_of(s0 + j);
        v[j] = ml[slot];
        const float4* src = reinterpret_cast<const float4*>(part_o + slot * kD + d0);
        x0[j] = src[0];
        x1[j] = src[1];
      }
#pragma unroll
      for (int j = 0; j < kOChunk; ++j) {
        // a surplus split of the last chunk gets weight 0 (its clamped loads read a real split, so the products are
        // exact zeros); a branch here would let the compiler move the loads below it, one round trip each
        const float m = v[j].x, l = v[j].y;
        const float w = (s0 + j >= ns || m == -INFINITY) ? 0.f : __expf(m - M);
        L += w * l;
        acc[0] += w * x0[j].x; acc[1] += w * x0[j].y; acc[2] += w * x0[j].z; acc[3] += w * x0[j].w;
        acc[4] += w * x1[j].x; acc[5] += w * x1[j].y; acc[6] += w * x1[j].z; acc[7] += w * x1[j].w;
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] *= inv;
  if (rot) {
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const int d = d0 + k;
      if (d >= base) {
        const float c = csv[k / 2].x, sn = csv[k / 2].y;
        const float u = acc[k], v = acc[k + 1];
        acc[k] = u * c + v * sn;
        acc[k + 1] = -u * sn + v * c;
      }
    }
  }
  if (a.out) {
    float4* dst = reinterpret_cast<float4*>(a.out + (int64_t(q) * a.n_heads + h) * kD + d0);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    // grouped fp8: a group of G channels is G / 8 consecutive lanes of this wave (the R23 rule, as in the
    // single-split epilogue)
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(acc[k]));
    const int lanes = a.group / 8;
    for (int off = 1; off < lanes; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    uint32_t w0 = 0u, w1 = 0u;
    if (amax > 0.f) {
      const float inv = 448.0f / amax;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w0 |= f32_to_e4m3_rne(acc[k] * inv) << (8 * k);
        w1 |= f32_to_e4m3_rne(acc[k + 4] * inv) << (8 * k);
      }
    }
    const int64_t row = int64_t(q) * a.n_heads + h;
    *reinterpret_cast<uint2*>(a.out_codes + row * kD + d0) = make_uint2(w0, w1);
    if ((d0 / 8) % lanes == 0) a.out_scales[row * (kD / a.group) + d0 / a.group] = amax > 0.f ? amax / 448.0f : 1.0f;
  }
  if (a.out_lse && d0 == 0) a.out_lse[int64_t(q) * a.n_heads + h] = (L > 0.f) ? M + logf(L) : -INFINITY;
}

// ------------------------------------------------------------------ VALU path
template <int DT>  // 0 f32, 1 bf16, 2 fp8
__device__ __forceinline__ float load_key(const AttendArgs& a, const KeyRef& r, int d) {
  const void* base = r.kind == 0 ? a.cache.pages : a.swa.kv_pages;
  const int D = a.cache.dim;
  if (DT == 0) return reinterpret_cast<const float*>(base)[r.row * D + d];
  if (DT == 1) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[r.row * D + d]);
  const float sc = r.kind == 0 ? a.cache.scales[r.row] : a.swa.scales[r.row];
  return e4m3_to_f32(reinterpret_cast<const uint8_t*>(base)[r.row * D + d]) * sc;
}

template <int DT>
__global__ void __launch_bounds__(256) attend_valu_kernel(AttendArgs a) {
  constexpr int CHUNK = 1024;
  __shared__ float qv[512];
  __shared__ float pl[CHUNK];
  __shared__ int64_t rows[CHUNK];
  __shared__ int kinds[CHUNK];
  __shared__ float red[256];
  __shared__ float ov[512];
  const int q = blockIdx.x / a.n_heads;
  const int h = blockIdx.x % a.n_heads;
  const int tid = threadIdx.x;
  const int D = a.cache.dim;
  const int seq = a.q_seq[q];
  const int64_t p = a.q_pos[q];
  const int64_t n_elig = attend_elig(a, q);
  const int64_t n_c = a.topk ? a.k : n_elig;
  const int64_t lo = (a.swa_window > 0) ? max<int64_t>(0, p - a.swa_window + 1) : p + 1;
  const int64_t n_keys = n_c + ((a.swa_window > 0) ? p - lo + 1 : 0);
  const int64_t qoff = (int64_t(q) * a.n_heads + h) * D;
  for (int d = tid; d < D; d += 256)
    qv[d] = (a.q_dtype == CSA_F32) ? reinterpret_cast<const float*>(a.q)[qoff + d]
                                   : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qoff + d]);
  float acc[2] = {0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();
  for (int64_t c0 = 0; c0 < n_keys; c0 += CHUNK) {
    const int n = int(min<int64_t>(CHUNK, n_keys - c0));
    float tmax = -INFINITY;
    for (int t = tid; t < n; t += 256) {
      const KeyRef r = key_ref(a, q, seq, c0 + t, n_c, n_elig, lo);
      rows[t] = r.row;
      kinds[t] = r.kind;
      float lgt = -INFINITY;
      if (r.row >= 0) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qv[d], load_key<DT>(a, r, d), dot);
        lgt = dot * a.scale;
      }
      pl[t] = lgt;
      tmax = fmaxf(tmax, lgt);
    }
    red[tid] = tmax;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
      __syncthreads();
    }
    const float mnew = fmaxf(m_run, red[0]);
    __syncthreads();
    const float corr = (m_run == -INFINITY) ? 0.f : expf(m_run - mnew);
    float psum = 0.f;
    for (int t = tid; t < n; t += 256) {
      const float e = (pl[t] == -INFINITY) ? 0.f : expf(pl[t] - mnew);
      pl[t] = e;
      psum += e;
    }
    red[tid] = psum;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] += red[tid + off];
      __syncthreads();
    }
    l_run = l_run * corr + red[0];
    m_run = mnew;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = tid + 256 * j;
      if (d < D) {
        float v = acc[j] * corr;
        for (int t = 0; t < n; ++t) {
          if (rows[t] < 0 || pl[t] == 0.f) continue;
          const KeyRef r{rows[t], kinds[t]};
          v = fmaf(pl[t], load_key<DT>(a, r, d), v);
        }
        acc[j] = v;
      }
    }
    __syncthreads();
  }
  const float inv_l = (l_run > 0.f) ? 1.f / l_run : 0.f;
  for (int j = 0; j < 2; ++j) {
    const int d = tid + 256 * j;
    if (d < D) ov[d] = acc[j] * inv_l;
  }
  __syncthreads();
  const int R = a.cache.rope_dims;
  const int base = D - R;
  const bool rot = a.fuse_inv_rope && R > 0 && p >= 0 && p < a.rope_rows;
  for (int d = tid; d < D; d += 256) {
    float r = ov[d];
    if (rot && d >= base) {
      const int j = (d - base) >> 1;
      const float c = a.rope_cs[p * int64_t(R) + 2 * j], sn = a.rope_cs[p * int64_t(R) + 2 * j + 1];
      r = (d & 1) ? (-ov[d - 1] * sn + ov[d] * c) : (ov[d] * c + ov[d + 1] * sn);
    }
    a.out[qoff + d] = r;
  }
  if (tid == 0 && a.out_lse) a.out_lse[int64_t(q) * a.n_heads + h] = (l_run > 0.f) ? m_run + logf(l_run) : -INFINITY;
}

// ------------------------------------------------------------------ dense path for many queries
// Dense attention (every eligible entry plus the window) when one launch holds many queries, as a prefill
// chunk does: the two queries of a workgroup (consecutive queries of one sequence) share every 64-key tile,
// so each key row fetched feeds 128 (query, head) rows. Scores are computed transposed, S^T = K Q^T, with the
// keys of each 16-row MFMA block permuted so that a lane ends up holding one head's weights for exactly the
// eight keys it supplies as the B operand of O^T = V^T P^T: the weights never pass through LDS and the
// softmax needs no cross-wave reduction. Each of the 8 waves owns 16 heads of one query (Q^T fragments and
// O^T accumulators in registers). Key rows land in LDS straight from global memory, one 1 KiB row per
// global_load_lds_dwordx4, double-buffered: the next tile is in flight while the current one is used.
constexpr int kDenseMinQueries = 512;  // launches with at least this many dense queries take this kernel
constexpr int kDensePairSpan = 64;     // two queries further apart than this walk their keys separately
constexpr float kDenseRescaleMargin = 8.0f;  // natural-log units the running maximum may lag the true one
constexpr int kDenseQueries = 2;      // queries per workgroup (2: eight waves, two per SIMD; 1: four waves)
// Tile rows in LDS: 1056 bytes apart, and 16-byte chunk c of row r stored at c ^ bit 3 of r. Both read patterns of
// the kernel keep this a per-lane constant (the S^T rows a 16-lane group reads share bit 3 with nothing that
// changes along the unrolled loops, and so do the V^T rows), and it spreads the S^T reads of a 16-lane group over
// all banks; rows padded to 1040 bytes without the flip left those reads at about 60 % of the LDS rate.
constexpr int kDenseRowStride = kD * 2 + 32;
__device__ __forceinline__ int dense_chunk_flip(int row) { return (row >> 3) & 1; }

// One 1 KiB key row from global memory into LDS: lane l moves bytes [16 l, 16 l + 16) of the row to
// lds_byte + 16 l. Issued from inline assembly: for the compiler's own form of this copy it orders every later LDS
// read behind the copy's completion (a vmcnt wait per read), which would serialise the next tile's copies with the
// current tile's arithmetic. The kernel orders the copies itself: they only ever target the tile buffer no wave
// reads, and a vmcnt(0) wait plus a barrier (both volatile) come before a buffer is read. No output register.
__device__ __forceinline__ void dma_row(const char* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_byte), "v"(src) : "m0");
}

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48), on the VALU: the 32-lane swap
// pairs rows (0, 2) and (1, 3), the 16-lane swap then pairs rows (0, 1) and (2, 3).
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// fp8 epilogue of the transposed layout: v[db][r] = output at dim db * 16 + kg * 4 + r of one head. A group of
// GN * 16 channels is GN registers of the lane times the four lane groups of its head.
template <int GN>
__device__ __forceinline__ void store_fp8_t(const f32x4 (&v)[32], uint8_t* crow, float* srow, int kg) {
#pragma unroll
  for (int g = 0; g < 32; g += GN) {
    float amax = 0.f;
#pragma unroll
    for (int n = 0; n < GN; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(v[g + n][r]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float inv = 448.0f / amax;
#pragma unroll
    for (int n = 0; n < GN; ++n) {
      uint32_t w = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) w |= (amax > 0.f ? f32_to_e4m3_rne(v[g + n][r] * inv) : 0u) << (8 * r);
      *reinterpret_cast<uint32_t*>(crow + (g + n) * 16 + kg * 4) = w;
    }
    if (kg == 0) srow[g / GN] = amax > 0.f ? amax / 448.0f : 1.0f;
  }
}

template <int QPW>
__global__ void __launch_bounds__(256 * QPW, 1) attend_dense_kernel(AttendArgs a) {
  constexpr int NHB = 1;                  // 16-head blocks per wave
  constexpr int NT = 256 * QPW;           // four waves (64 heads) per query
  constexpr int WPQ = 4;                  // waves per query
  constexpr int RPW = kTile / (4 * QPW);  // tile rows each wave moves
  __shared__ __attribute__((aligned(16))) char kbuf[2][kTile * kDenseRowStride];
  __shared__ int32_t key_row[kMaxKeys];

  // unit = (QPW consecutive queries, 64-head chunk); consecutive units on one XCD (workgroups are dealt to the
  // eight XCDs in turn), so the queries of a sequence read its pages through the same L2
  const int n_hchunk = a.n_heads / 64;
  const int units = ((a.n_q + QPW - 1) / QPW) * n_hchunk;
  const int per_xcd = int(gridDim.x / 8);  // the grid is a multiple of 8
  const int unit = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (unit >= units) return;
  const int hc = unit % n_hchunk;
  const int q0 = QPW * (unit / n_hchunk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform values stay in scalar registers
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int qi = wave / WPQ;  // query of the pair this wave serves
  const bool has1 = QPW == 2 && q0 + 1 < a.n_q;
  const bool wave_has_q = qi == 0 || has1;
  const int q = wave_has_q ? q0 + qi : q0;
  const int head = hc * 64 + (wave % WPQ) * 16 * NHB + col;  // this lane's head in block hb: head + 16 hb

  // positions are 32-bit at the boundary, so every key count and position below fits an int
  const int p_0 = a.q_pos[q0], p_1 = has1 ? a.q_pos[q0 + 1] : p_0;
  const int seq_0 = a.q_seq[q0], seq_1 = has1 ? a.q_seq[q0 + 1] : seq_0;
  const int ne_0 = int(attend_elig(a, q0)), ne_1 = has1 ? int(attend_elig(a, q0 + 1)) : ne_0;
  const int lo_0 = (a.swa_window > 0) ? max(0, p_0 - a.swa_window + 1) : p_0 + 1;
  const int lo_1 = (a.swa_window > 0) ? max(0, p_1 - a.swa_window + 1) : p_1 + 1;
  const int64_t dp = int64_t(p_0) - p_1;
  const bool shared = has1 && seq_0 == seq_1 && dp <= kDensePairSpan && -dp <= kDensePairSpan;
  const int n_ps = (has1 && !shared) ? 2 : 1;
  const int my_ne = qi ? ne_1 : ne_0, my_lo = qi ? lo_1 : lo_0, my_p = qi ? p_1 : p_0;
  // top-k mode (one query per workgroup): the query's list of selected entries
  const int32_t* topk_q = (QPW == 1 && a.topk) ? a.topk + int64_t(q0) * a.k : nullptr;

  bf16x8 qb[NHB][16];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (int64_t(q) * a.n_heads + head) * kD;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qb[hb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + hb * 16 * kD + ks * 32 + kg * 8));
  }

  f32x4 o[32][NHB];
#pragma unroll
  for (int db = 0; db < 32; ++db)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) o[db][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NHB], l_run[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) { m_run[hb] = -INFINITY; l_run[hb] = 0.f; }
  const float scale = a.scale;
  const char* pages_c = static_cast<const char*>(a.cache.pages);
  const char* pages_w = static_cast<const char*>(a.swa.kv_pages);
  const int per_block = kBlock / a.cache.ratio;
  // LDS byte offset of the key this lane reads as MFMA row `col` of 16-key block kb4 in S^T: the permutation
  // that puts the eight keys a lane supplies to PV into its own accumulator registers
  // (blocks kb4 = 1, 2, 3 are the rows of block 0 moved by 16, 32 and 48 keys, which keeps the row's bit 3); the
  // lane's chunk kg of each 64-byte k-step sits at kg ^ that bit
  const int srow = perm_key(col >> 2, col & 3);
  const int soff = srow * kDenseRowStride + (kg ^ dense_chunk_flip(srow)) * 16;
  // LDS byte offsets of the two 4-key rows a lane addresses in the transposing V^T reads of k-step c (a lane's
  // 8 bytes sit in chunk 2 db + bit 1 of col, flipped by the row's bit 3, which the two rows share: they differ by
  // 16 keys)
  const int vchunk = (((col & 3) >> 1) ^ dense_chunk_flip(perm_key(kg, col >> 2))) * 16 + 8 * (col & 1);
  const int voff0 = perm_key(kg, col >> 2) * kDenseRowStride + vchunk;  // + 32 rows for k-step 1
  const int voff1 = perm_key(kg, 4 + (col >> 2)) * kDenseRowStride + vchunk;

  for (int ps = 0; ps < n_ps; ++ps) {
    // queries of the pair in this walk: both when they share their keys, else one walk each
    const bool in0 = shared || ps == 0, in1 = has1 && (shared || ps == 1);
    const bool wave_act = wave_has_q && (qi ? in1 : in0);
    const int seq = in0 ? seq_0 : seq_1;
    int n_cu = 0, lo_u = INT_MAX, hi_u = -1;
    if (in0) {
      n_cu = topk_q ? a.k : ne_0;
      if (p_0 >= lo_0) { lo_u = lo_0; hi_u = p_0; }
    }
    if (in1) {
      n_cu = max(n_cu, ne_1);
      if (p_1 >= lo_1) { lo_u = min(lo_u, lo_1); hi_u = max(hi_u, p_1); }
    }
    if (hi_u < lo_u) { lo_u = 0; hi_u = -1; }  // no window rows (keeps the clamped table loads in range)
    const int n_keys = n_cu + (hi_u - lo_u + 1);
    const bool seq_c = seq >= 0 && seq < a.cache.batch;
    const bool seq_w = seq >= 0 && seq < a.swa.batch;
    const int32_t* bt_c = a.cache.block_table + int64_t(seq_c ? seq : 0) * a.cache.bt_stride;
    const int32_t* bt_w = a.swa.block_table + int64_t(seq_w ? seq : 0) * a.swa.bt_stride;
    const int bts_c = a.cache.bt_stride, bts_w = a.swa.bt_stride;
    const int nph_c = a.cache.n_phys, nph_w = a.swa.n_phys;

    for (int pass0 = 0; pass0 < n_keys; pass0 += kMaxKeys) {
      const int n_pass = min(kMaxKeys, n_keys - pass0);
      // the previous walk or pass is done with the row table and both tile buffers. Not needed before the first
      // pass: skipping it there lets the list and table loads below go out while the query loads are in flight
      // (the barrier waits for every outstanding load)
      if (ps > 0 || pass0 > 0) __syncthreads();
      // ---- page rows of this pass's keys: key t < n_cu is entry t (top-k mode: list slot t, an entry outside
      // [0, eligible) maps to no row), else window position lo_u + t - n_cu
      {
        constexpr int PER = kMaxKeys / NT;
        int32_t ent[PER], phys[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int t = pass0 + tid + NT * j;
          const bool is_c = t < n_cu;
          ent[j] = is_c ? (topk_q ? topk_q[t < a.k ? t : 0] : t) : lo_u + (t - n_cu);  // clamped list load
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int t = pass0 + tid + NT * j;
          const bool is_c = t < n_cu;
          const int e = ent[j] < 0 ? 0 : ent[j];
          const int blk = e / (is_c ? per_block : kBlock);
          const int bts = is_c ? bts_c : bts_w;
          phys[j] = (is_c ? bt_c : bt_w)[blk < bts ? blk : bts - 1];  // clamped, unconditional load
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int local = tid + NT * j;
          const int t = pass0 + local;
          const bool is_c = t < n_cu;
          const int e = ent[j];
          const int per = is_c ? per_block : kBlock;
          const int blk = (e < 0 ? 0 : e) / per;
          const bool ok = local < n_pass && e >= 0 && (!is_c || !topk_q || e < ne_0) && blk < (is_c ? bts_c : bts_w) &&
                          phys[j] >= 0 && phys[j] < (is_c ? nph_c : nph_w) && (is_c ? seq_c : seq_w);
          key_row[local] = ok ? phys[j] * per + (e - blk * per) : -1;
        }
      }
      __syncthreads();

      // this wave moves tile rows RPW w .. RPW w + RPW - 1. Every row is copied unconditionally (a row that maps to
      // no page copies page row 0, so the score loop stays one basic block); such rows are zero-filled once the copy
      // has landed, before the barrier that publishes the tile. bad: bit j = row j of this wave maps to no page.
      auto tile_rows = [&](int tile, int (&rows)[RPW]) -> uint32_t {
        const int t0 = tile * kTile + wave * RPW;
        const int my_row = (t0 + (lane % RPW) < n_pass) ? key_row[t0 + (lane % RPW)] : -1;
        uint32_t bad = 0;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
          rows[j] = __builtin_amdgcn_readlane(my_row, j);
          bad |= uint32_t(rows[j] < 0) << j;
        }
        return bad;
      };
      // lane l lands LDS chunk l of the row, so it copies the row's chunk l ^ (row bit 3)
      auto copy_row = [&](int tile, int buf, const int (&rows)[RPW], int j) {
        const int t = tile * kTile + wave * RPW + j;
        const char* base = (pass0 + t < n_cu) ? pages_c : pages_w;
        dma_row(base + int64_t(rows[j] < 0 ? 0 : rows[j]) * (2 * kD) + (lane ^ dense_chunk_flip(wave * RPW + j)) * 16,
                uint32_t(reinterpret_cast<uintptr_t>(kbuf[buf])) + uint32_t((wave * RPW + j) * kDenseRowStride));
      };
      auto zero_rows = [&](int buf, uint32_t bad) {
        if (bad) {
          char* dst = kbuf[buf] + wave * RPW * kDenseRowStride;
#pragma unroll
          for (int j = 0; j < RPW; ++j)
            if ((bad >> j) & 1u) *reinterpret_cast<uint4*>(dst + j * kDenseRowStride + lane * 16) = make_uint4(0, 0, 0, 0);
        }
      };

      const int n_tiles = (n_pass + kTile - 1) / kTile;
      uint32_t bad_cur;
      {
        int rows0[RPW];
        bad_cur = tile_rows(0, rows0);
#pragma unroll
        for (int j = 0; j < RPW; ++j) copy_row(0, 0, rows0, j);
      }
      for (int tile = 0; tile < n_tiles; ++tile) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows of the tile are in LDS
        zero_rows(tile & 1, bad_cur);
        lds_barrier();                       // every wave's rows are; every wave is done with the other buffer
        // keys of the tile this wave's query sees: lane l tests tile key l; shifted so that the key of
        // accumulator register r of block kb4 is bit (kb4 >> 1) * 32 + (j & 1) + 8 * (j >> 1), j = (kb4 & 1) * 4 + r
        const int tt = tile * kTile + lane;
        const int krow = tt < n_pass ? key_row[tt] : -1;
        // the next tile's copies go out in four groups over the score loop below (each asm statement ends a
        // scheduling region, so they are not spread finer); after the last
        // tile they re-copy rows of this tile into the idle buffer, which nothing reads
        const int ntile = tile + 1 < n_tiles ? tile + 1 : tile;
        const int nbuf = (tile + 1) & 1;
        int nrows[RPW];
        bad_cur = tile_rows(ntile, nrows);
        const char* kb = kbuf[tile & 1];
        uint64_t kmask;
        {
          const int g = pass0 + tt;
          bool ok = krow >= 0;
          if (g < n_cu) ok = ok && (topk_q != nullptr || g < my_ne);
          else {
            const int pos = lo_u + (g - n_cu);
            ok = ok && pos >= my_lo && pos <= my_p;
          }
          kmask = __ballot(ok) >> (2 * kg);
        }

        // ---- S^T (64 keys x 16 NHB heads) = K Q^T
        f32x4 s[4][NHB];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) s[kb4][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // K fragments are loaded two k-steps ahead of their MFMAs (a ring of two k-steps' fragments)
        bf16x8 kf[2][4];
        auto load_k = [&](bf16x8 (&dst)[4], int ks) {
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
            dst[kb4] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + soff + kb4 * 16 * kDenseRowStride + ks * 64));
        };
        load_k(kf[0], 0);
        load_k(kf[1], 1);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          if (ks % 4 == 0)
#pragma unroll
            for (int jj = 0; jj < RPW / 4; ++jj) copy_row(ntile, nbuf, nrows, (ks / 4) * (RPW / 4) + jj);
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb)
              s[kb4][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks & 1][kb4], qb[hb][ks], s[kb4][hb], 0, 0, 0);
          if (ks + 2 < 16) load_k(kf[ks & 1], ks + 2);
        }
        if (!wave_act) continue;

        // ---- online softmax of this lane's heads over its 16 keys of the tile (and the other lane groups'). The
        // weights are taken against the running reference maximum m_run straight away; the tile's maximum only
        // decides whether m_run moves, which it does when the tile exceeds it by more than kDenseRescaleMargin (or
        // on the first keys): then the weights are recomputed and the accumulators rescaled. Weights stay below
        // e^margin. l_part is this lane's share of the running sum; the four lane groups are added at the end.
        bool move_any = false;
        float mx[NHB];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          float m = -INFINITY;
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = (kb4 & 1) * 4 + r;
              const bool v = (kmask >> ((kb4 >> 1) * 32 + (j & 1) + 8 * (j >> 1))) & 1ull;
              const float lg = v ? s[kb4][hb][r] * scale : -INFINITY;
              s[kb4][hb][r] = lg;
              m = fmaxf(m, lg);
            }
          mx[hb] = m;
        }
        float pw[4][NHB][4];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int r = 0; r < 4; ++r) pw[kb4][hb][r] = __expf(s[kb4][hb][r] - m_run[hb]);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          mx[hb] = rows4_max(mx[hb]);
          move_any = move_any || m_run[hb] == -INFINITY || mx[hb] > m_run[hb] + kDenseRescaleMargin;
        }
        if (__ballot(move_any)) {
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            const bool move = m_run[hb] == -INFINITY || mx[hb] > m_run[hb] + kDenseRescaleMargin;
            const float mnew = move ? mx[hb] : m_run[hb];
            const float corr = move ? ((m_run[hb] == -INFINITY) ? 0.f : __expf(m_run[hb] - mnew)) : 1.f;
            m_run[hb] = mnew;
            l_run[hb] *= corr;
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                pw[kb4][hb][r] = (s[kb4][hb][r] == -INFINITY) ? 0.f : __expf(s[kb4][hb][r] - mnew);
#pragma unroll
            for (int db = 0; db < 32; ++db)
#pragma unroll
              for (int r = 0; r < 4; ++r) o[db][hb][r] *= corr;
          }
        }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          float sum = 0.f;
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int r = 0; r < 4; ++r) sum += pw[kb4][hb][r];
          l_run[hb] += sum;
        }

        // ---- O^T (512 dims x 16 NHB heads) += V^T P^T, weights as bf16 hi + lo parts. The 64 (k-step, dim-block)
        // steps read their V^T fragments kPvAhead steps ahead; the hi and lo products of two dim blocks alternate so
        // that no MFMA waits on the one before it.
        bf16x8 ph[2][NHB], pl[2][NHB];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            uint32_t wh[4], wl[4];
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              const float w0 = pw[2 * c + (j >> 2)][hb][j & 3], w1 = pw[2 * c + ((j + 1) >> 2)][hb][(j + 1) & 3];
              const uint16_t h0 = f32_to_bf16_rne(w0), h1 = f32_to_bf16_rne(w1);
              const uint16_t l0 = f32_to_bf16_rne(w0 - bf16_to_f32(h0)), l1 = f32_to_bf16_rne(w1 - bf16_to_f32(h1));
              wh[j >> 1] = uint32_t(h0) | (uint32_t(h1) << 16);
              wl[j >> 1] = uint32_t(l0) | (uint32_t(l1) << 16);
            }
            ph[c][hb] = __builtin_bit_cast(bf16x8, make_uint4(wh[0], wh[1], wh[2], wh[3]));
            pl[c][hb] = __builtin_bit_cast(bf16x8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
          }
        constexpr int kPvAhead = 8;
        bf16x8 vq[kPvAhead];
        auto load_v = [&](int st) -> bf16x8 {
          const int c = st >> 5, db = st & 31;
          const uint2 e0 = lds_tr16(kb + c * 32 * kDenseRowStride + voff0 + db * 32);
          const uint2 e1 = lds_tr16(kb + c * 32 * kDenseRowStride + voff1 + db * 32);
          return __builtin_bit_cast(bf16x8, make_uint4(e0.x, e0.y, e1.x, e1.y));
        };
#pragma unroll
        for (int st = 0; st < kPvAhead; ++st) vq[st] = load_v(st);
#pragma unroll
        for (int st = 0; st < 64; st += 2) {
          const int c = st >> 5, db = st & 31;
          const bf16x8 va = vq[st % kPvAhead], vb = vq[(st + 1) % kPvAhead];
          if (st + kPvAhead < 64) vq[st % kPvAhead] = load_v(st + kPvAhead);
          if (st + 1 + kPvAhead < 64) vq[(st + 1) % kPvAhead] = load_v(st + 1 + kPvAhead);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph[c][hb], o[db][hb], 0, 0, 0);
            o[db + 1][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, ph[c][hb], o[db + 1][hb], 0, 0, 0);
            o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl[c][hb], o[db][hb], 0, 0, 0);
            o[db + 1][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pl[c][hb], o[db + 1][hb], 0, 0, 0);
          }
        }
      }
      // the copies are invisible to the compiler's wait tracking: wait for them here, so that no copy is in flight
      // when the next pass reuses the buffers or the workgroup ends
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  }

  // ---- epilogue: lane holds dims db * 16 + kg * 4 + r of head `head + 16 hb`
  if (!wave_has_q) return;
  const int p = my_p;
  const int R_ = a.cache.rope_dims;
  const int base = kD - R_;
  const bool rot = a.fuse_inv_rope && R_ > 0 && p >= 0 && p < a.rope_rows;
  const float* cs = rot ? a.rope_cs + int64_t(p) * R_ : a.rope_cs;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) l_run[hb] = rows4_sum(l_run[hb]);  // the four lane groups' shares of the sum
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float inv_l = (l_run[hb] > 0.f) ? 1.f / l_run[hb] : 0.f;
    f32x4 v[32];
#pragma unroll
    for (int db = 0; db < 32; ++db) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[db][r] = o[db][hb][r] * inv_l;
      const int d0 = db * 16 + kg * 4;
      if (rot && d0 + 3 >= base) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int d = d0 + 2 * k2;
          if (d >= base) {
            const int j = (d - base) >> 1;
            const float c = cs[2 * j], sn = cs[2 * j + 1];
            const float x = v[db][2 * k2], y = v[db][2 * k2 + 1];
            v[db][2 * k2] = x * c + y * sn;
            v[db][2 * k2 + 1] = -x * sn + y * c;
          }
        }
      }
    }
    const int64_t row = int64_t(q) * a.n_heads + head + 16 * hb;
    if (a.out) {
#pragma unroll
      for (int db = 0; db < 32; ++db) *reinterpret_cast<f32x4*>(a.out + row * kD + db * 16 + kg * 4) = v[db];
    } else {
      uint8_t* crow = a.out_codes + row * kD;
      float* srow_s = a.out_scales + row * (kD / a.group);
      switch (a.group) {
        case 16: store_fp8_t<1>(v, crow, srow_s, kg); break;
        case 32: store_fp8_t<2>(v, crow, srow_s, kg); break;
        case 64: store_fp8_t<4>(v, crow, srow_s, kg); break;
        default: store_fp8_t<8>(v, crow, srow_s, kg); break;
      }
    }
    if (a.out_lse && kg == 0) a.out_lse[row] = (l_run[hb] > 0.f) ? m_run[hb] + logf(l_run[hb]) : -INFINITY;
  }
}
}  // namespace

bool attend_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads) {
  if (int64_t(c.n_phys) * (kBlock / c.ratio) > 0x7FFFFFFF) return false;  // page rows are 32-bit
  if (c.dtype == CSA_F32) return q_dtype == CSA_F32 && c.dim <= 512;
  return q_dtype == CSA_BF16 && c.dim <= 512 && n_heads >= 1;
}

bool attend_quant_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads, int group) {
  const bool g_ok = group == 16 || group == 32 || group == 64 || group == 128;
  return g_ok && attend_supported(c, q_dtype, n_heads) && c.dtype != CSA_F32 && c.dim == kD && n_heads % 16 == 0;
}

static bool use_split_path(const AttendArgs& a) {
  return a.cache.dtype != CSA_F32 && a.cache.dim == kD && a.n_heads % 64 == 0;
}

// Queries per workgroup of the many-query kernel for this launch, 0 when it does not take it: dense launches pair
// consecutive queries (they share their keys), top-k launches take one query per workgroup.
static int dense_queries(const AttendArgs& a) {
  if (a.cache.dtype != CSA_BF16 || a.cache.dim != kD || a.n_heads % 64 != 0 || a.n_q < kDenseMinQueries) return 0;
  return a.topk ? 1 : kDenseQueries;
}

static int64_t max_keys_of(const AttendArgs& a) {
  return (a.topk ? int64_t(a.k) : a.max_elig) + a.swa_window;
}

size_t attend_workspace(int n_q, int n_heads, int dim, int64_t max_keys) {
  if (n_q <= 0 || n_heads % 64 != 0 || dim != kD) return 0;
  const SplitPlan sp = split_plan(n_q, n_heads / 64, max_keys);
  if (sp.n_split <= 1) return 0;
  const size_t slots = size_t(n_q) * sp.n_split * n_heads;
  return slots * kD * 4 + slots * 8 + 256;
}

hipError_t launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (a.n_q == 0) return hipSuccess;
  if (const int qpw = dense_queries(a)) {
    const int64_t units = int64_t((a.n_q + qpw - 1) / qpw) * (a.n_heads / 64);
    const dim3 grid(unsigned((units + 7) / 8 * 8));
    if (qpw == 1) hipLaunchKernelGGL((attend_dense_kernel<1>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((attend_dense_kernel<2>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  if (use_split_path(a)) {
    const int n_hchunk = a.n_heads / 64;
    SplitPlan sp = split_plan(a.n_q, n_hchunk, max_keys_of(a));
    const size_t need = attend_workspace(a.n_q, a.n_heads, kD, max_keys_of(a));
    if (sp.n_split > 1 && (ws == nullptr || ws_bytes < need)) return hipErrorInvalidValue;
    float* part_o = static_cast<float*>(ws);
    float* part_ml = part_o ? part_o + size_t(a.n_q) * sp.n_split * a.n_heads * kD : nullptr;
    const dim3 grid(unsigned(int64_t(a.n_q) * n_hchunk * sp.n_split));
    if (a.cache.dtype == CSA_FP8_E4M3)
      hipLaunchKernelGGL((attend_split_kernel<true>), grid, dim3(512), 0, stream, a, sp, part_o, part_ml);
    else
      hipLaunchKernelGGL((attend_split_kernel<false>), grid, dim3(512), 0, stream, a, sp, part_o, part_ml);
    if (sp.n_split > 1) {
      const dim3 cgrid(unsigned(int64_t(a.n_q) * (a.n_heads / 4)));
      if (sp.n_split <= 4) hipLaunchKernelGGL((attend_combine_kernel<4>), cgrid, dim3(256), 0, stream, a, sp, part_o, part_ml);
      else if (sp.n_split <= 8) hipLaunchKernelGGL((attend_combine_kernel<8>), cgrid, dim3(256), 0, stream, a, sp, part_o, part_ml);
      else if (sp.n_split <= 16) hipLaunchKernelGGL((attend_combine_kernel<16>), cgrid, dim3(256), 0, stream, a, sp, part_o, part_ml);
      else hipLaunchKernelGGL((attend_combine_kernel<0>), cgrid, dim3(256), 0, stream, a, sp, part_o, part_ml);
    }
    return hipGetLastError();
  }
  const bool mfma = a.cache.dtype != CSA_F32 && a.cache.dim == kD && a.n_heads % 16 == 0;
  if (mfma) {
    const int HG = a.n_heads / 16;
    const int64_t blocks = int64_t((a.n_q + 7) / 8) * HG * 8;
    if (a.cache.dtype == CSA_FP8_E4M3)
      hipLaunchKernelGGL((attend_mfma_kernel<true>), dim3(unsigned(blocks)), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((attend_mfma_kernel<false>), dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  } else {
    const dim3 grid(unsigned(int64_t(a.n_q) * a.n_heads));
    if (a.cache.dtype == CSA_F32) hipLaunchKernelGGL((attend_valu_kernel<0>), grid, dim3(256), 0, stream, a);
    else if (a.cache.dtype == CSA_BF16) hipLaunchKernelGGL((attend_valu_kernel<1>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((attend_valu_kernel<2>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace csa
