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

// Position, inside a 32-key PV k-step, of key kk in the A/B operand order: lane group g holds
// keys 2g, 2g+1, 2g+8, 2g+9, 2g+16, 2g+17, 2g+24, 2g+25 as its elements 0..7.
__device__ __forceinline__ int perm_pos(int kk) {
  const int g = (kk & 7) >> 1;
  const int j = (kk & 1) + 2 * (kk >> 3);
  return g * 8 + j;
}
__device__ __forceinline__ int perm_key(int g, int j) { return 2 * g + (j & 1) + 8 * (j >> 1); }

template <bool FP8>
__global__ void __launch_bounds__(256) attend_mfma_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) char k_lds[kTile * kRowStride];
  __shared__ __attribute__((aligned(16))) uint16_t p_hi[16 * kPStride];
  __shared__ __attribute__((aligned(16))) uint16_t p_lo[16 * kPStride];
  __shared__ float k_scale[kTile];
  __shared__ int64_t k_row[kTile];
  __shared__ int k_kind[kTile];
  __shared__ float red[4][16];

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
  const int64_t n_swa = (a.swa_window > 0) ? p - lo + 1 : 0;
  const int64_t n_keys = n_c + n_swa;

  // Q fragments: lane holds Q[head hg*16 + col][ks*32 + kg*8 .. +8], ks = 0..15
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

  for (int64_t t0 = 0; t0 < n_keys; t0 += kTile) {
    // ---- gather the tile into LDS
    if (tid < kTile) {
      const int64_t t = t0 + tid;
      KeyRef r = (t < n_keys) ? key_ref(a, q, seq, t, n_c, n_elig, lo) : KeyRef{-1, 0};
      k_row[tid] = r.row;
      k_kind[tid] = r.kind;
      float sc = 1.f;
      if (FP8 && r.row >= 0) sc = r.kind == 0 ? a.cache.scales[r.row] : a.swa.scales[r.row];
      k_scale[tid] = sc;
    }
    __syncthreads();
    if (!FP8) {
      // 64 rows x 64 chunks of 16 B; each wave copies whole rows
#pragma unroll 4
      for (int c = tid; c < kTile * 64; c += 256) {
        const int r = c >> 6, cc = c & 63;
        const int64_t row = k_row[r];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row >= 0) {
          const uint16_t* base = reinterpret_cast<const uint16_t*>(k_kind[r] == 0 ? a.cache.pages : a.swa.kv_pages);
          v = reinterpret_cast<const uint4*>(base + row * kD)[cc];
        }
        *reinterpret_cast<uint4*>(k_lds + r * kRowStride + cc * 16) = v;
      }
    } else {
      // 64 rows x 32 chunks of 16 codes -> 32 bf16 each
#pragma unroll 2
      for (int c = tid; c < kTile * 32; c += 256) {
        const int r = c >> 5, cc = c & 31;
        const int64_t row = k_row[r];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row >= 0) {
          const uint8_t* base = reinterpret_cast<const uint8_t*>(k_kind[r] == 0 ? a.cache.pages : a.swa.kv_pages);
          v = reinterpret_cast<const uint4*>(base + row * kD)[cc];
        }
        uint32_t w[8];
        const uint32_t src[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t b0 = 0, b1 = 0;
          const float f0 = e4m3_to_f32(src[h] & 0xFF), f1 = e4m3_to_f32((src[h] >> 8) & 0xFF);
          const float f2 = e4m3_to_f32((src[h] >> 16) & 0xFF), f3 = e4m3_to_f32(src[h] >> 24);
          b0 = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
          b1 = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
          w[2 * h] = b0;
          w[2 * h + 1] = b1;
        }
        uint4* dst = reinterpret_cast<uint4*>(k_lds + r * kRowStride + cc * 32);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
    __syncthreads();

    // ---- S = Q K^T for this wave's 16 keys
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    {
      const char* krow = k_lds + (wave * 16 + col) * kRowStride + kg * 16;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 kb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 64));
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, s, 0, 0, 0);
      }
    }
    const int key_local = wave * 16 + col;
    const bool kvalid = k_row[key_local] >= 0;
    const float ksc = k_scale[key_local];
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = kvalid ? s[i] * (scale * ksc) : -INFINITY;
    // tile max per head (lane holds heads kg*4+i for key col)
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = lg[i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
      mx[i] = v;
    }
    if (col == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][kg * 4 + i] = mx[i];
    __syncthreads();
    float corr[4], pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = kg * 4 + i;
      const float tmax = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
      const float mnew = fmaxf(m_run[i], tmax);
      corr[i] = (m_run[i] == -INFINITY) ? 0.f : __expf(m_run[i] - mnew);
      pv[i] = (lg[i] == -INFINITY) ? 0.f : __expf(lg[i] - mnew);
      m_run[i] = mnew;
    }
    __syncthreads();  // everyone has read red[] before it is reused for sums
    float sm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = pv[i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off);
      sm[i] = v;
    }
    if (col == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][kg * 4 + i] = sm[i];
    // probabilities (times the fp8 row scale) to LDS as bf16 hi + lo, in the PV operand order
    {
      const int ks2 = key_local >> 5;
      const int pos = ks2 * 32 + perm_pos(key_local & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = pv[i] * ksc;
        const uint16_t hi = f32_to_bf16_rne(w);
        const uint16_t lo16 = f32_to_bf16_rne(w - bf16_to_f32(hi));
        p_hi[(kg * 4 + i) * kPStride + pos] = hi;
        p_lo[(kg * 4 + i) * kPStride + pos] = lo16;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = kg * 4 + i;
      l_run[i] = l_run[i] * corr[i] + (red[0][h] + red[1][h] + red[2][h] + red[3][h]);
    }
    // ---- O = O * corr + P K over this wave's 128 dims
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= corr[i];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p_hi + col * kPStride + ks2 * 32 + kg * 8));
      const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p_lo + col * kPStride + ks2 * 32 + kg * 8));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int d = wave * 128 + nt * 16 + col;
        uint32_t w[4];
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          const int r0 = ks2 * 32 + perm_key(kg, 2 * j2);
          const int r1 = ks2 * 32 + perm_key(kg, 2 * j2 + 1);
          const uint32_t e0 = *reinterpret_cast<const uint16_t*>(k_lds + r0 * kRowStride + d * 2);
          const uint32_t e1 = *reinterpret_cast<const uint16_t*>(k_lds + r1 * kRowStride + d * 2);
          w[j2] = e0 | (e1 << 16);
        }
        const bf16x8 kb = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, kb, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, kb, o[nt], 0, 0, 0);
      }
    }
    __syncthreads();  // before the next tile overwrites k_lds / p / red
  }

  // ---- epilogue: normalise, optional inverse RoPE, store
  const int R = a.cache.rope_dims;
  const int base = kD - R;
  const bool rot = a.fuse_inv_rope && R > 0 && p >= 0 && p < a.rope_rows;
  const float* cs = rot ? a.rope_cs + p * int64_t(R) : a.rope_cs;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int d = wave * 128 + nt * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv_l = (l_run[i] > 0.f) ? 1.f / l_run[i] : 0.f;
      const float v = o[nt][i] * inv_l;
      const float partner = __shfl_xor(v, 1);
      float r = v;
      if (rot && d >= base) {
        const int j = (d - base) >> 1;
        const float c = cs[2 * j], sn = cs[2 * j + 1];
        r = (d & 1) ? (-partner * sn + v * c) : (v * c + partner * sn);
      }
      const int h = hg * 16 + kg * 4 + i;
      a.out[(int64_t(q) * a.n_heads + h) * kD + d] = r;
    }
  }
  if (a.out_lse && wave == 0 && col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hg * 16 + kg * 4 + i;
      a.out_lse[int64_t(q) * a.n_heads + h] = (l_run[i] > 0.f) ? m_run[i] + logf(l_run[i]) : -INFINITY;
    }
  }
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

}  // namespace

bool attend_supported(const csa_cache_t& c, csa_dtype_t q_dtype, int n_heads) {
  if (c.dtype == CSA_F32) return q_dtype == CSA_F32 && c.dim <= 512;
  return q_dtype == CSA_BF16 && c.dim <= 512 && n_heads >= 1;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream) {
  if (a.n_q == 0) return hipSuccess;
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
