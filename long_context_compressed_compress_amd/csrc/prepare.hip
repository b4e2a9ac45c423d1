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
  const int c0 = lane * CH;
  const int64_t p = a.tok_pos[t];
  const TQ* src = is_q ? static_cast<const TQ*>(a.q_in) + (t * a.n_heads + u) * D : static_cast<const TQ*>(a.kv_in) + t * D;
  float y[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) y[k] = act ? load_elem<TQ>(src, c0 + k) : 0.f;
  if (is_q) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) ss += y[k] * y[k];
    ss = wave_sum(ss);
    const float rms = sqrtf(ss / float(D) + a.eps);
#pragma unroll
    for (int k = 0; k < CH; ++k) y[k] = act ? y[k] / rms * a.gamma[c0 + k] : 0.f;
  }
  // RoPE at the token's position on dims [D-R, D), interleaved pairs
  const int R = a.rope_dims;
  const int base = D - R;
  if (R > 0 && p >= 0 && p < a.rope_rows && act) {
#pragma unroll
    for (int k = 0; k < CH; k += 2) {
      const int c = c0 + k;
      if (c >= base) {
        const float co = a.rope_cs[p * R + (c - base)], sn = a.rope_cs[p * R + (c - base) + 1];
        const float uu = y[k], vv = y[k + 1];
        y[k] = uu * co - vv * sn;
        y[k + 1] = uu * sn + vv * co;
      }
    }
  }
  if (is_q) {
    if (!act) return;
    TQ* dst = static_cast<TQ*>(a.q_out) + (t * a.n_heads + u) * D + c0;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if constexpr (sizeof(TQ) == 4) dst[k] = y[k];
      else dst[k] = f32_to_bf16_rne(y[k]);
    }
    return;
  }
  // window key: the row of raw position p of sequence tok_seq[t]
  const int seq = a.tok_seq[t];
  int64_t row = -1;
  if (seq >= 0 && seq < a.swa.batch)
    row = raw_row(a.swa.block_table + int64_t(seq) * a.swa.bt_stride, a.swa.bt_stride, a.swa.n_phys, p);
  if (KV == 2) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) amax = fmaxf(amax, fabsf(y[k]));
    amax = wave_max(amax);
    if (row < 0) return;
    uint8_t* dst = static_cast<uint8_t*>(a.swa.kv_pages) + row * D + c0;
    if (act) {
      const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
      for (int k = 0; k < CH; ++k) dst[k] = amax > 0.f ? uint8_t(f32_to_e4m3_rne(y[k] * inv)) : uint8_t(0);
    }
    if (lane == 0) a.swa.scales[row] = amax > 0.f ? amax / 448.0f : 1.0f;
  } else {
    if (row < 0 || !act) return;
    if (KV == 0) {
      float* dst = static_cast<float*>(a.swa.kv_pages) + row * D + c0;
#pragma unroll
      for (int k = 0; k < CH; ++k) dst[k] = y[k];
    } else {
      uint16_t* dst = static_cast<uint16_t*>(a.swa.kv_pages) + row * D + c0;
#pragma unroll
      for (int k = 0; k < CH; ++k) dst[k] = f32_to_bf16_rne(y[k]);
    }
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
