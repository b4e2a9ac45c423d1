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

}  // namespace

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
