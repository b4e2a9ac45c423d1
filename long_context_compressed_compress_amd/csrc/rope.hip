// RoPE table construction and the standalone inverse RoPE.
//
// [P1] "DeepSeek V4 Attention Architecture" / [P2] "二、注意力機制為什么這么麻煩": with shared K = V the
// attention output carries absolute rotary phase; an inverse rotation at the query position restores
// relative position. The rotation uses interleaved pairs (D-R+2j, D-R+2j+1) on the last R dims.
#include "csa_internal.h"

namespace csa {
namespace {

// One thread per (position, pair): angle p * theta^(-2j/R) in fp64, cos/sin rounded once to fp32.
__global__ void rope_table_kernel(int rows, int half, int rope_dims, double theta, float* out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(rows) * half) return;
  const int64_t p = i / half;
  const int j = int(i % half);
  const double inv_freq = pow(theta, -2.0 * double(j) / double(rope_dims));
  const double ang = double(p) * inv_freq;
  double s, c;
  sincos(ang, &s, &c);
  out[2 * i] = __double2float_rn(c);
  out[2 * i + 1] = __double2float_rn(s);
}

// One thread per (query, head, pair): (u, v) -> (u c + v s, -u s + v c).
__global__ void inv_rope_kernel(int n_q, int n_heads, int dim, int rope_dims, const int32_t* q_pos,
                                const float* cs, int rope_rows, float* io) {
  const int half = rope_dims / 2;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(n_q) * n_heads * half) return;
  const int j = int(i % half);
  const int64_t qh = i / half;
  const int q = int(qh / n_heads);
  const int64_t p = q_pos[q];
  if (p < 0 || p >= rope_rows) return;
  const float c = cs[p * rope_dims + 2 * j], s = cs[p * rope_dims + 2 * j + 1];
  float* row = io + qh * dim + (dim - rope_dims) + 2 * j;
  const float u = row[0], v = row[1];
  row[0] = u * c + v * s;
  row[1] = -u * s + v * c;
}

// Inverse RoPE fused with fp8 quantisation of the attention output ([P1] "GPU Compute Saturation", [P2] "3.2
// 內核": one pass before the fp8 o_lora matmul instead of two). One thread per 8 consecutive channels of a
// (query, head) row: it rotates its pairs back by the query position, the G/8 threads of a group reduce the
// group's amax with xor-shuffles (a group of G <= 512 channels is G/8 <= 64 aligned lanes of one wave, and never
// straddles a row), then each writes its 8 e4m3fn codes (y * 448/amax, round to nearest even) and the group's
// first thread writes the fp32 scale amax/448 (1 for an all-zero group).
__global__ void __launch_bounds__(256) inv_rope_quant_kernel(int n_q, int n_heads, int dim, int rope_dims,
                                                             const int32_t* q_pos, const float* cs, int rope_rows,
                                                             const float* in, int group, uint8_t* codes,
                                                             float* scales) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = dim / 8;
  const int64_t n_t = int64_t(n_q) * n_heads * per_row;
  const bool live = t < n_t;  // groups are whole: a thread past the end belongs to an all-dead group
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) {
    const float4* src = reinterpret_cast<const float4*>(in + t * 8);
    const float4 a = src[0], b = src[1];
    y[0] = a.x; y[1] = a.y; y[2] = a.z; y[3] = a.w; y[4] = b.x; y[5] = b.y; y[6] = b.z; y[7] = b.w;
    const int q = int(t / (int64_t(per_row) * n_heads));
    const int c0 = int(t % per_row) * 8;
    const int64_t p = q_pos[q];
    const int base = dim - rope_dims;
    if (rope_dims > 0 && p >= 0 && p < rope_rows) {
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        const int c = c0 + k;
        if (c >= base) {
          const float co = cs[p * rope_dims + (c - base)], sn = cs[p * rope_dims + (c - base) + 1];
          const float u = y[k], v = y[k + 1];
          y[k] = u * co + v * sn;
          y[k + 1] = -u * sn + v * co;
        }
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(y[k]));
  const int lanes = group / 8;
  for (int off = 1; off < lanes; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (!live) return;
  uint32_t w0 = 0u, w1 = 0u;
  if (amax > 0.f) {
    const float inv = 448.0f / amax;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w0 |= f32_to_e4m3_rne(y[k] * inv) << (8 * k);
      w1 |= f32_to_e4m3_rne(y[k + 4] * inv) << (8 * k);
    }
  }
  *reinterpret_cast<uint2*>(codes + t * 8) = make_uint2(w0, w1);
  if (t % lanes == 0) scales[t / lanes] = amax > 0.f ? amax / 448.0f : 1.0f;
}

}  // namespace

hipError_t launch_inv_rope_quant(int n_q, int n_heads, int dim, int rope_dims, const int32_t* q_pos,
                                 const float* rope_cs, int rope_rows, const float* in, int group, uint8_t* codes,
                                 float* scales, hipStream_t stream) {
  const int64_t n = int64_t(n_q) * n_heads * (dim / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(inv_rope_quant_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, n_q, n_heads, dim,
                     rope_dims, q_pos, rope_cs, rope_rows, in, group, codes, scales);
  return hipGetLastError();
}

hipError_t launch_rope_table(int rows, int rope_dims, double theta, float* out, hipStream_t stream) {
  const int half = rope_dims / 2;
  const int64_t n = int64_t(rows) * half;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, rows, half, rope_dims,
                     theta, out);
  return hipGetLastError();
}

hipError_t launch_inv_rope(int n_q, int n_heads, int dim, int rope_dims, const int32_t* q_pos, const float* rope_cs,
                           int rope_rows, float* io, hipStream_t stream) {
  const int64_t n = int64_t(n_q) * n_heads * (rope_dims / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(inv_rope_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, n_q, n_heads, dim,
                     rope_dims, q_pos, rope_cs, rope_rows, io);
  return hipGetLastError();
}

}  // namespace csa
