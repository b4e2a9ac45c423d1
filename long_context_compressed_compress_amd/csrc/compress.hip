// csa_compress_insert kernels: raw-token append to the compressor state + fused window compression -> RMSNorm ->
// RoPE at anchor -> rounding -> paged cache insert, one wave per unit (compress_unit.h), 4 waves per workgroup.
#include "compress_unit.h"

namespace csa {
namespace {

template <typename TIn, int OUT, int D, int RATIO, int WINDOW>
__global__ void __launch_bounds__(256) compress_insert_kernel(CompressArgs a) {
  compress_unit<TIn, OUT, D, RATIO, WINDOW>(a, int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6));
}

// Two c4a caches' compress_insert in one grid (a decode step's main and indexer caches): blocks [0, blocks_a)
// run cache a's code for head dim DA and output type OA, the rest cache b's for DB and OB. Each cache keeps
// its own code, the step saves one launch.
template <typename TIn, int OA, int OB, int DA, int DB>
__global__ void __launch_bounds__(256) compress_pair_kernel(CompressArgs a, CompressArgs b, int64_t blocks_a) {
  const int w = threadIdx.x >> 6;
  if (int64_t(blockIdx.x) < blocks_a) compress_unit<TIn, OA, DA, 4, 8>(a, int64_t(blockIdx.x) * 4 + w);
  else compress_unit<TIn, OB, DB, 4, 8>(b, (int64_t(blockIdx.x) - blocks_a) * 4 + w);
}

inline int64_t compress_blocks(const CompressArgs& a) {
  return (int64_t(a.total_new) + int64_t(a.batch) * a.max_entries_bound + 3) / 4;
}

template <typename TIn, int OUT, int D>
hipError_t dispatch_ratio(const CompressArgs& a, hipStream_t stream) {
  const int64_t units = int64_t(a.total_new) + int64_t(a.batch) * a.max_entries_bound;
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.cache.ratio == 4)
    hipLaunchKernelGGL((compress_insert_kernel<TIn, OUT, D, 4, 8>), dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((compress_insert_kernel<TIn, OUT, D, 128, 128>), dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename TIn, int OUT>
hipError_t dispatch_dim(const CompressArgs& a, hipStream_t stream) {
  switch (a.cache.dim) {
    case 32: return dispatch_ratio<TIn, OUT, 32>(a, stream);
    case 64: return dispatch_ratio<TIn, OUT, 64>(a, stream);
    case 128: return dispatch_ratio<TIn, OUT, 128>(a, stream);
    case 256: return dispatch_ratio<TIn, OUT, 256>(a, stream);
    case 512: return dispatch_ratio<TIn, OUT, 512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename TIn>
hipError_t dispatch_out(const CompressArgs& a, hipStream_t stream) {
  switch (a.cache.dtype) {
    case CSA_F32: return dispatch_dim<TIn, 0>(a, stream);
    case CSA_BF16: return dispatch_dim<TIn, 1>(a, stream);
    case CSA_FP8_E4M3: return dispatch_dim<TIn, 2>(a, stream);
    case CSA_FP4_E2M1: return dispatch_dim<TIn, 3>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  if (a.state.dtype == CSA_F32) return dispatch_out<float>(a, stream);
  return dispatch_out<uint16_t>(a, stream);
}

hipError_t launch_compress_pair(const CompressArgs& a, const CompressArgs& b, hipStream_t stream) {
  const bool same = a.cache.dtype == b.cache.dtype && (a.cache.dtype == CSA_BF16 || a.cache.dtype == CSA_FP8_E4M3);
  const bool fp8_fp4 = a.cache.dtype == CSA_FP8_E4M3 && b.cache.dtype == CSA_FP4_E2M1;
  const bool fused = a.state.dtype == CSA_BF16 && b.state.dtype == CSA_BF16 && a.cache.ratio == 4 &&
                     b.cache.ratio == 4 && (same || fp8_fp4) && a.cache.dim == 512 && b.cache.dim == 128;
  if (!fused) {  // any other pair: one launch per cache
    const hipError_t e = launch_compress(a, stream);
    return e != hipSuccess ? e : launch_compress(b, stream);
  }
  const int64_t ba = compress_blocks(a), bb = compress_blocks(b);
  if (ba + bb == 0) return hipSuccess;
  if (ba + bb > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(unsigned(ba + bb));
  if (a.cache.dtype == CSA_BF16)
    hipLaunchKernelGGL((compress_pair_kernel<uint16_t, 1, 1, 512, 128>), grid, dim3(256), 0, stream, a, b, ba);
  else if (fp8_fp4)
    hipLaunchKernelGGL((compress_pair_kernel<uint16_t, 2, 3, 512, 128>), grid, dim3(256), 0, stream, a, b, ba);
  else
    hipLaunchKernelGGL((compress_pair_kernel<uint16_t, 2, 2, 512, 128>), grid, dim3(256), 0, stream, a, b, ba);
  return hipGetLastError();
}

}  // namespace csa
