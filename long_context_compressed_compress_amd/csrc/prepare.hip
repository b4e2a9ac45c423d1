// csa_prepare_qk kernel: query RMSNorm + query RoPE and window-key RoPE + window-key insert, fused.
//
// [P1] "GPU Compute Saturation" / [P2] "3.2 內核": the elementwise work on the query heads and on the
// uncompressed sliding-window key in front of the main attention is fused horizontally into one kernel, each
// wave statically assigned to a query head or to the key, with no communication between waves.
#include "csa_internal.h"

namespace csa {
namespace {

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wave per unit: unit u of token t is query head u (u < H) or the token's window key (u == H). Lane l holds
// channels [l*CH, l*CH + CH) with CH >= 2, so every RoPE pair stays in one lane; lanes past D/CH hold nothing.
// KV: 0 fp32, 1 bf16, 2 fp8 e4m3fn with a per-row scale (the window pages' element type).
// A lane's CH channels are contiguous and aligned to their size: each store below is one vector store.
template <int CH>
__device__ __forceinline__ void store_row(float* dst, const float (&y)[CH]) {
  if constexpr (CH == 8) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(y[0], y[1], y[2], y[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(y[4], y[5], y[6], y[7]);
  } else if constexpr (CH == 4) {
    *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
  } else {
    *reinterpret_cast<float2*>(dst) = make_float2(y[0], y[1]);
  }
}
template <int CH>
__device__ __forceinline__ void store_row(uint16_t* dst, const float (&y)[CH]) {
  uint32_t w[CH / 2];
#pragma unroll
  for (int k = 0; k < CH / 2; ++k) w[k] = uint32_t(f32_to_bf16_rne(y[2 * k])) | (uint32_t(f32_to_bf16_rne(y[2 * k + 1])) << 16);
  if constexpr (CH == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  else if constexpr (CH == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  else *reinterpret_cast<uint32_t*>(dst) = w[0];
}
template <int CH>
__device__ __forceinline__ void store_codes(uint8_t* dst, const uint32_t (&c)[CH]) {
  uint32_t w[(CH + 3) / 4] = {};
#pragma unroll
  for (int k = 0; k < CH; ++k) w[k / 4] |= c[k] << (8 * (k % 4));
  if constexpr (CH == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  else if constexpr (CH == 4) *reinterpret_cast<uint32_t*>(dst) = w[0];
  else *reinterpret_cast<uint16_t*>(dst) = uint16_t(w[0]);
}

template <typename TQ, int D, int KV>
__global__ void __launch_bounds__(256) prepare_qk_kernel(PrepareArgs a) {
  constexpr int CH = D / 64 >= 2 ? D / 64 : 2;
  constexpr int NL = D / CH;
  const int lane = threadIdx.x & 63;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int units_per_tok = a.n_heads + 1;
  if (unit >= int64_t(a.n_tok) * units_per_tok) return;  // uniform per wave
  const int64_t t = unit / units_per_tok;
  const int u = int(unit % units_per_tok);
  const bool is_q = u < a.n_heads;
  const bool act = lane < NL;
  const int c0 = act ? lane * CH : 0;  // idle lanes read channel 0 and drop it
  // Round trip 1: position, sequence, the input row and (query heads) gamma, every load unconditional; round trip 2:
  // the cos/sin of the position (clamped into the table) and, for the window key, its block-table entry.
  const int64_t p = a.tok_pos[t];
  const int seq = a.tok_seq[t];
  const TQ* src = is_q ? static_cast<const TQ*>(a.q_in) + (t * a.n_heads + u) * D : static_cast<const TQ*>(a.kv_in) + t * D;
  float y[CH], gm[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    y[k] = load_elem<TQ>(src, c0 + k);
    gm[k] = a.gamma[c0 + k];  // the query gamma has D entries; read but unused for the window key
  }
  const int R = a.rope_dims;
  const int base = D - R;
  const bool rot = R > 0 && p >= 0 && p < a.rope_rows;
  float rc[CH / 2], rs[CH / 2];
#pragma unroll
  for (int k = 0; k < CH; k += 2) {
    const int c = c0 + k;
    const int64_t off = (rot && c >= base) ? p * R + (c - base) : 0;  // clamped: every load is in the table
    rc[k / 2] = R > 0 ? a.rope_cs[off] : 1.f;
    rs[k / 2] = R > 0 ? a.rope_cs[off + 1] : 0.f;
  }
  int64_t row = -1;
  if (!is_q) {
    const bool seq_ok = seq >= 0 && seq < a.swa.batch;
    row = raw_row(a.swa.block_table + int64_t(seq_ok ? seq : 0) * a.swa.bt_stride, a.swa.bt_stride, a.swa.n_phys, p);
    if (!seq_ok) row = -1;
  }
#pragma unroll
  for (int k = 0; k < CH; ++k) y[k] = act ? y[k] : 0.f;
  if (is_q) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) ss += y[k] * y[k];
    ss = wave_sum(ss);
    const float rms = sqrtf(ss / float(D) + a.eps);
#pragma unroll
    for (int k = 0; k < CH; ++k) y[k] = act ? y[k] / rms * gm[k] : 0.f;
  }
  // RoPE at the token's position on dims [D-R, D), interleaved pairs
  if (rot && act) {
#pragma unroll
    for (int k = 0; k < CH; k += 2) {
      const int c = c0 + k;
      if (c >= base) {
        const float co = rc[k / 2], sn = rs[k / 2];
        const float uu = y[k], vv = y[k + 1];
        y[k] = uu * co - vv * sn;
        y[k + 1] = uu * sn + vv * co;
      }
    }
  }
  if (is_q) {
    if (!act) return;
    store_row<CH>(static_cast<TQ*>(a.q_out) + (t * a.n_heads + u) * D + c0, y);
    return;
  }
  // window key: written to `row`, the row of raw position p of sequence tok_seq[t] (-1: not mapped)
  if (KV == 2) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) amax = fmaxf(amax, fabsf(y[k]));
    amax = wave_max(amax);
    if (row < 0) return;
    if (act) {
      const float inv = amax > 0.f ? 448.0f / amax : 0.f;
      uint32_t c[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) c[k] = amax > 0.f ? f32_to_e4m3_rne(y[k] * inv) : 0u;
      store_codes<CH>(static_cast<uint8_t*>(a.swa.kv_pages) + row * D + c0, c);
    }
    if (lane == 0) a.swa.scales[row] = amax > 0.f ? amax / 448.0f : 1.0f;
  } else {
    if (row < 0 || !act) return;
    if constexpr (KV == 0) store_row<CH>(static_cast<float*>(a.swa.kv_pages) + row * D + c0, y);
    else store_row<CH>(static_cast<uint16_t*>(a.swa.kv_pages) + row * D + c0, y);
  }
}

template <typename TQ, int KV>
hipError_t dispatch_dim(const PrepareArgs& a, int dim, dim3 grid, hipStream_t stream) {
  switch (dim) {
    case 32: hipLaunchKernelGGL((prepare_qk_kernel<TQ, 32, KV>), grid, dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((prepare_qk_kernel<TQ, 64, KV>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((prepare_qk_kernel<TQ, 128, KV>), grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((prepare_qk_kernel<TQ, 256, KV>), grid, dim3(256), 0, stream, a); break;
    case 512: hipLaunchKernelGGL((prepare_qk_kernel<TQ, 512, KV>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare_qk(const PrepareArgs& a, csa_dtype_t q_dtype, hipStream_t stream) {
  const int64_t units = int64_t(a.n_tok) * (a.n_heads + 1);
  if (units == 0) return hipSuccess;
  const dim3 grid(unsigned((units + 3) / 4));
  if (q_dtype == CSA_F32) return dispatch_dim<float, 0>(a, a.swa.dim, grid, stream);
  if (a.swa.dtype == CSA_BF16) return dispatch_dim<uint16_t, 1>(a, a.swa.dim, grid, stream);
  return dispatch_dim<uint16_t, 2>(a, a.swa.dim, grid, stream);
}

}  // namespace csa
