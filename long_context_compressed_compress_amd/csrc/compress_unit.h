// The per-unit work of csa_compress_insert (one wave per unit), shared by the compress kernels and by the decode
// index-score kernels that run the decode step's compress units before scoring (csa_compress_index_score).
//
// [P1] "GPU Compute Saturation" and [P2] "3.2 內核" describe the compressor, RMSNorm, RoPE and the
// cache write as one fused elementwise kernel per cache instance. [P1] "DeepSeek V4 Attention
// Architecture" / [P3] "KV 缓存压缩": c4a entry i = weighted sum of raw tokens 4i .. 4i+7, anchor 4i;
// c128a entry i = weighted sum of 128 raw tokens starting at 128i. [P2] "3.1 顯存": the compressor
// residual is kept as raw sliding-window pages.
//
// Units:
//   * append units: one new raw token; the wave copies its kv row and role logit rows into the state pages.
//   * entry units: one (sequence, new entry). Lanes split into NLC channel lanes (CH consecutive
//     channels each, 16- or 32-byte loads) times G row groups; group g folds window rows
//     t = g, g+G, ... with an online per-channel softmax, then the G partial states merge with
//     butterfly shuffles. Rows of positions before start_pos come from the state pages, rows of new
//     positions straight from the inputs, so append and compress run in the same launch without a
//     dependency between them.
#pragma once
#include "csa_internal.h"

namespace csa {
namespace {

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, int i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t* p, int i) { return bf16_to_f32(p[i]); }
};

// Load N values of type T starting at p (16-byte aligned) into floats.
template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[N]) {
  constexpr int per16 = 16 / sizeof(T);
  static_assert(N % per16 == 0, "vector width");
#pragma unroll
  for (int c = 0; c < N / per16; ++c) {
    const uint4 raw = reinterpret_cast<const uint4*>(p)[c];
    const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int k = 0; k < per16; ++k) v[c * per16 + k] = Elem<T>::get(e, k);
  }
}

template <int N>
__device__ __forceinline__ void zero_vec(float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = 0.f;
}

// The sequence of an appended row: the largest b < batch with cu[b] <= row (cu non-decreasing, cu[0] = 0 <= row),
// with its start position and first row. The whole wave calls it for one row: each lane tests one sequence and
// loads its cu and start position together, so a batch of up to 64 sequences costs one memory round trip (a
// binary search would cost one per step); the found lane's values are broadcast.
__device__ __forceinline__ void find_seq_start(const int32_t* cu, const int32_t* start_pos, int batch, int row,
                                               int& b_out, int& start_out, int& cu_out) {
  const int lane = threadIdx.x & 63;
  int found = 0, f_start = 0, f_cu = 0;
  for (int base = 0; base < batch; base += 64) {
    const int b = base + lane;
    const int bc = b < batch ? b : batch - 1;  // clamped, unconditional loads
    const int c = cu[bc], sp = start_pos[bc];
    asm volatile("" ::"v"(sp));  // keeps the start-position load beside the cu load (it would sink below the ballot)
    const uint64_t le = __ballot(b < batch && c <= row);
    if (le) {
      const int src = 63 - __clzll((unsigned long long)le);
      found = base + src;
      f_start = __shfl(sp, src);
      f_cu = __shfl(c, src);
    }
    if (le != ~0ull) break;  // a lane of this chunk is past the row: later chunks are too
  }
  b_out = found;
  start_out = f_start;
  cu_out = f_cu;
}

// The work of one unit of a compress_insert grid, done by the calling wave: units [0, total_new) append raw token
// `gw`, the following batch x max_entries_bound units build entry (gw - total_new) % bound of sequence
// (gw - total_new) / bound. A unit past the grid returns at once.
template <typename TIn, int OUT, int D, int RATIO, int WINDOW>
__device__ __forceinline__ void compress_unit(const CompressArgs& a, int64_t gw) {
  constexpr int ROLES = WINDOW / RATIO;
  constexpr int VEC = 16 / int(sizeof(TIn));
  constexpr int CH = (D / 64 > VEC) ? D / 64 : VEC;
  constexpr int NLC = D / CH;
  constexpr int G = 64 / NLC;
  constexpr int E = kBlock / RATIO;
  static_assert(D % CH == 0 && NLC <= 64 && (NLC & (NLC - 1)) == 0, "channel split");

  const int lane = threadIdx.x & 63;
  const int64_t n_append = a.total_new;
  const TIn* kv_new = reinterpret_cast<const TIn*>(a.kv_new);
  const TIn* lg_new = reinterpret_cast<const TIn*>(a.logit_new);
  TIn* st_kv = reinterpret_cast<TIn*>(a.state.kv_pages);
  TIn* st_lg = reinterpret_cast<TIn*>(a.state.logit_pages);

  if (gw < n_append) {
    // ---------------- append one raw token to the state pages
    const int row = int(gw);
    int b, start_b, cu_b;
    find_seq_start(a.cu_new, a.start_pos, a.batch, row, b, start_b, cu_b);
    if (b >= a.state.batch) return;
    const int64_t pos = int64_t(start_b) + (row - cu_b);
    const int64_t r = raw_row(a.state.block_table + int64_t(b) * a.state.bt_stride, a.state.bt_stride, a.state.n_phys, pos);
    if (r < 0) return;
    // every chunk of the kv and logit rows is loaded before any is stored: one round trip for the copy
    constexpr int V16_ROW = D * int(sizeof(TIn)) / 16;  // 16-byte chunks per D-row
    constexpr int NKV = (V16_ROW + 63) / 64, NLG = (V16_ROW * ROLES + 63) / 64;
    const uint4* src_kv = reinterpret_cast<const uint4*>(kv_new + int64_t(row) * D);
    uint4* dst_kv = reinterpret_cast<uint4*>(st_kv + r * D);
    const uint4* src_lg = reinterpret_cast<const uint4*>(lg_new + int64_t(row) * ROLES * D);
    uint4* dst_lg = reinterpret_cast<uint4*>(st_lg + r * ROLES * D);
    uint4 vk[NKV], vl[NLG];
#pragma unroll
    for (int j = 0; j < NKV; ++j) {
      const int c = lane + 64 * j;
      vk[j] = src_kv[c < V16_ROW ? c : 0];
    }
#pragma unroll
    for (int j = 0; j < NLG; ++j) {
      const int c = lane + 64 * j;
      vl[j] = src_lg[c < V16_ROW * ROLES ? c : 0];
    }
#pragma unroll
    for (int j = 0; j < NKV; ++j)
      if (lane + 64 * j < V16_ROW) dst_kv[lane + 64 * j] = vk[j];
#pragma unroll
    for (int j = 0; j < NLG; ++j)
      if (lane + 64 * j < V16_ROW * ROLES) dst_lg[lane + 64 * j] = vl[j];
    return;
  }

  // ---------------- build one entry
  const int64_t unit = gw - n_append;
  const int bound = a.max_entries_bound;
  if (unit >= int64_t(a.batch) * bound) return;
  const int b = int(unit / bound);
  const int c_idx = int(unit % bound);
  const int64_t start = a.start_pos[b];
  const int n_new = a.cu_new[b + 1] - a.cu_new[b];
  const int64_t e0 = num_eligible(start - 1, RATIO, WINDOW);          // entries complete before this call
  const int64_t e1 = num_eligible(start + n_new - 1, RATIO, WINDOW);  // after it
  const int64_t count = e1 - e0;
  if (c_idx == 0 && lane == 0) {
    if (a.out_new_entries) a.out_new_entries[b] = int32_t(count);
    if (a.out_slots)
      for (int c = bound; c < a.max_entries_out; ++c) a.out_slots[int64_t(b) * a.max_entries_out + c] = -1;
  }
  if (c_idx >= count) {
    if (a.out_slots && lane == 0 && c_idx < a.max_entries_out) a.out_slots[int64_t(b) * a.max_entries_out + c_idx] = -1;
    return;
  }
  const int64_t i = e0 + c_idx;
  const int64_t first = int64_t(RATIO) * i;
  const int ch_lane = lane % NLC;
  const int grp = lane / NLC;
  const int ch0 = ch_lane * CH;
  const int cu_b = a.cu_new[b];
  const int32_t* st_bt = (b < a.state.batch) ? a.state.block_table + int64_t(b) * a.state.bt_stride : nullptr;
  // everything the epilogue reads that does not depend on the window (the output slot, gamma, the anchor's
  // cos/sin) is loaded now, so its round trip overlaps the window loads
  const int64_t slot = entry_row(a.cache.block_table + int64_t(b) * a.cache.bt_stride, a.cache.bt_stride,
                                 a.cache.n_phys, i, E);
  float gam[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) gam[k] = a.gamma[ch0 + k];
  const int R = a.cache.rope_dims;
  const int base = D - R;
  const bool rot = R > 0 && first < a.rope_rows;
  float rc[CH / 2], rsn[CH / 2];
#pragma unroll
  for (int k = 0; k < CH; k += 2) {
    const int c = ch0 + k;
    rc[k / 2] = 1.f;
    rsn[k / 2] = 0.f;
    if (rot && c >= base) {
      const float* cs = a.rope_cs + first * int64_t(R) + (c - base);  // pair j = (c - base) / 2 at 2j
      rc[k / 2] = cs[0];
      rsn[k / 2] = cs[1];
    }
  }

  float m[CH], s[CH], acc[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) { m[k] = -INFINITY; s[k] = 0.f; acc[k] = 0.f; }

  // The window's state rows lie in at most two 256-position blocks (the window is at most 256 positions long):
  // both table entries are loaded once, unconditionally (clamped), then the rows of a chunk of up to 8 window rows
  // are all loaded before any is used, so a chunk costs one memory round trip. Rows of new positions come from the
  // inputs, older ones from the state pages; a row that maps to no page reads row 0 and counts as zeros.
  static_assert(WINDOW <= kBlock, "a window spans at most two blocks");
  constexpr int ROWS = (WINDOW + G - 1) / G;  // window rows per lane group
  constexpr int CHUNK = ROWS < 8 ? ROWS : 8;  // c4a windows in one chunk; c128a windows in chunks of 8 rows
  const int bts = a.state.bt_stride;
  const int32_t* bt_any = st_bt ? st_bt : a.state.block_table;  // a row that exists, read when b has none
  const int64_t blk0 = first / kBlock;
  const int32_t ph0 = bt_any[blk0 < bts ? blk0 : bts - 1];
  const int32_t ph1 = bt_any[blk0 + 1 < bts ? blk0 + 1 : bts - 1];
#pragma unroll 1
  for (int t0 = 0; t0 < ROWS; t0 += CHUNK) {
    float x[CHUNK][CH], l[CHUNK][CH];
    bool have[CHUNK];
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) {
      const int t = grp + (t0 + k) * G;
      const int64_t pos = first + t;
      const int role = (t < WINDOW ? t : WINDOW - 1) / RATIO;
      const bool from_new = pos >= start;
      const int64_t blk = pos / kBlock;
      const int32_t ph = blk == blk0 ? ph0 : ph1;
      const bool mapped = st_bt != nullptr && blk < bts && ph >= 0 && ph < a.state.n_phys;
      const int64_t r = mapped ? int64_t(ph) * kBlock + (pos - blk * kBlock) : 0;
      have[k] = from_new || mapped;
      const TIn* xs = from_new ? kv_new + (cu_b + (pos - start)) * D : st_kv + r * D;
      const TIn* ls = from_new ? lg_new + ((cu_b + (pos - start)) * ROLES + role) * D : st_lg + (r * ROLES + role) * D;
      load_vec<TIn, CH>(xs + ch0, x[k]);
      load_vec<TIn, CH>(ls + ch0, l[k]);
    }
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) {
      if (grp + (t0 + k) * G >= WINDOW) break;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const float xv = have[k] ? x[k][c] : 0.f, lv = have[k] ? l[k][c] : 0.f;
        const float mn = fmaxf(m[c], lv);
        const float f_old = __expf(m[c] - mn);  // exp(-inf) = 0 on the first row
        const float f_new = __expf(lv - mn);
        s[c] = s[c] * f_old + f_new;
        acc[c] = acc[c] * f_old + f_new * xv;
        m[c] = mn;
      }
    }
  }
  // merge the G row groups (butterfly over the group bits of the lane id)
#pragma unroll
  for (int off = NLC; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const float m2 = __shfl_xor(m[k], off);
      const float s2 = __shfl_xor(s[k], off);
      const float a2 = __shfl_xor(acc[k], off);
      const float mn = fmaxf(m[k], m2);
      const float f1 = (m[k] == -INFINITY) ? 0.f : __expf(m[k] - mn);
      const float f2 = (m2 == -INFINITY) ? 0.f : __expf(m2 - mn);
      s[k] = s[k] * f1 + s2 * f2;
      acc[k] = acc[k] * f1 + a2 * f2;
      m[k] = mn;
    }
  }
  float y[CH];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    y[k] = acc[k] / s[k];
    ss += y[k] * y[k];
  }
#pragma unroll
  for (int off = 1; off < NLC; off <<= 1) ss += __shfl_xor(ss, off);
  const float rms = sqrtf(ss / float(D) + a.eps);
#pragma unroll
  for (int k = 0; k < CH; ++k) y[k] = y[k] / rms * gam[k];

  // RoPE at the anchor on dims [D-R, D), interleaved pairs (each lane owns whole pairs)
  if (rot) {
#pragma unroll
    for (int k = 0; k < CH; k += 2) {
      const int c = ch0 + k;
      if (c >= base) {
        const float co = rc[k / 2], si = rsn[k / 2];
        const float u = y[k], v = y[k + 1];
        y[k] = u * co - v * si;
        y[k + 1] = u * si + v * co;
      }
    }
  }
  const bool in_table = b < a.cache.batch && slot >= 0;
  if (OUT == 3) {
    // MXFP4: the LPB lanes holding one 32-channel block share its amax; X = floor(log2 amax) - 2 comes from
    // the fp32 exponent field (clamped to the E8M0 range), elements are y * 2^-X rounded to nearest-even
    // e2m1 with saturation at 6
    constexpr int LPB = 32 / CH;
    static_assert(32 % CH == 0 && D % 32 == 0, "fp4 block split");
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) amax = fmaxf(amax, fabsf(y[k]));
#pragma unroll
    for (int off = 1; off < LPB; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const int eb = int((__float_as_uint(amax) >> 23) & 0xFFu);  // biased exponent of amax
    const int X = amax > 0.f ? max(eb - 129, -127) : 0;
    const float inv = __uint_as_float(uint32_t(127 - X) << 23);  // 2^-X, normal for X in [-127, 125]
    if (in_table && grp == 0) {
      uint32_t nib[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) nib[k] = f32_to_e2m1_rne(y[k] * inv);
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.cache.pages) + slot * (D / 2) + ch0 / 2;
      if (CH == 8) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < CH; ++k) w |= nib[k] << (4 * k);
        *reinterpret_cast<uint32_t*>(dst) = w;
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < CH; ++k) w |= nib[k] << (4 * k);
        *reinterpret_cast<uint16_t*>(dst) = uint16_t(w);
      }
      if (ch_lane % LPB == 0)
        reinterpret_cast<uint8_t*>(a.cache.scales)[slot * (D / 32) + ch0 / 32] = uint8_t(X + 127);
    }
  } else if (OUT == 2) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) amax = fmaxf(amax, fabsf(y[k]));
#pragma unroll
    for (int off = 1; off < NLC; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (in_table && grp == 0) {
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.cache.pages) + slot * D + ch0;
      uint32_t packed[CH / 4];
      if (amax > 0.f) {
        const float inv = 448.0f / amax;
#pragma unroll
        for (int k = 0; k < CH / 4; ++k) {
          packed[k] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) packed[k] |= f32_to_e4m3_rne(y[4 * k + e] * inv) << (8 * e);
        }
      } else {
#pragma unroll
        for (int k = 0; k < CH / 4; ++k) packed[k] = 0;
      }
#pragma unroll
      for (int k = 0; k < CH / 4; ++k) reinterpret_cast<uint32_t*>(dst)[k] = packed[k];
      if (ch_lane == 0) a.cache.scales[slot] = amax > 0.f ? amax / 448.0f : 1.0f;
    }
  } else if (OUT == 1) {
    if (in_table && grp == 0) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.cache.pages) + slot * D + ch0;
      uint32_t packed[CH / 2];
#pragma unroll
      for (int k = 0; k < CH / 2; ++k)
        packed[k] = uint32_t(f32_to_bf16_rne(y[2 * k])) | (uint32_t(f32_to_bf16_rne(y[2 * k + 1])) << 16);
#pragma unroll
      for (int k = 0; k < CH / 2; ++k) reinterpret_cast<uint32_t*>(dst)[k] = packed[k];
    }
  } else {
    if (in_table && grp == 0) {
      float* dst = reinterpret_cast<float*>(a.cache.pages) + slot * D + ch0;
#pragma unroll
      for (int k = 0; k < CH; ++k) dst[k] = y[k];
    }
  }
  if (a.out_slots && lane == 0 && c_idx < a.max_entries_out)
    a.out_slots[int64_t(b) * a.max_entries_out + c_idx] = in_table ? int32_t(slot) : -1;
}

}  // namespace
}  // namespace csa
