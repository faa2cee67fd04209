// k_diag.hip - a read-only streaming kernel that calibrates the HBM read ceiling the decode
// kernels are measured against (a measurement aid, not part of the method).
#include <hip/hip_runtime.h>

#include "gva_diag.h"
#include "gva_internal.h"

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// Lane l of work-group w reads 16-byte words w * 256 * F + l + 256 * k (k < F) of each stride
// of gridDim.x * 256 * F words: F loads in flight per lane, every word read exactly once. The
// loads are non-temporal (read once, as the decode's cache rows are) and every load
// instruction covers 1 KiB of consecutive words, whole 128-byte lines. Loads past the end
// read the last word again (every load is made and every result used, so none is held back
// behind a branch).
template <int F>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4 *__restrict__ src, int64_t words,
                                                     uint32_t *sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * F;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * F + threadIdx.x; base < words;
       base += stride) {
    u32x4 v[F];
#pragma unroll
    for (int k = 0; k < F; ++k) {
      const int64_t i = base + 256 * k;
      v[k] = __builtin_nontemporal_load(src + (i < words ? i : words - 1));
    }
#pragma unroll
    for (int k = 0; k < F; ++k) acc ^= v[k];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" gva_status gva_diag_stream_read(const void *src, size_t bytes, int32_t work_groups,
                                           int32_t in_flight, uint32_t *sink,
                                           hipStream_t stream) {
  if (!src || !sink || reinterpret_cast<uintptr_t>(src) % 16 != 0 || bytes % 16 != 0)
    return gva::fail(GVA_ERR_INVALID_ARG, "src must be 16-byte aligned, bytes a multiple of 16");
  if (work_groups < 1 || work_groups > 65536)
    return gva::fail(GVA_ERR_INVALID_ARG, "work_groups=%d outside [1, 65536]", work_groups);
  const u32x4 *s = static_cast<const u32x4 *>(src);
  const int64_t words = static_cast<int64_t>(bytes / 16);
  const dim3 grid(static_cast<unsigned>(work_groups));
  switch (in_flight) {
    case 1: hipLaunchKernelGGL(k_stream_read<1>, grid, dim3(256), 0, stream, s, words, sink); break;
    case 2: hipLaunchKernelGGL(k_stream_read<2>, grid, dim3(256), 0, stream, s, words, sink); break;
    case 4: hipLaunchKernelGGL(k_stream_read<4>, grid, dim3(256), 0, stream, s, words, sink); break;
    case 8: hipLaunchKernelGGL(k_stream_read<8>, grid, dim3(256), 0, stream, s, words, sink); break;
    default: return gva::fail(GVA_ERR_INVALID_ARG, "in_flight=%d must be 1, 2, 4 or 8", in_flight);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return gva::fail(GVA_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
  return GVA_OK;
}
