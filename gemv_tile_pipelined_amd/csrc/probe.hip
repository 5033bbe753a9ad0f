// probe.hip -- a read-only stream over a device buffer, for measuring the
// practical HBM read ceiling the GEMV and the skinny GEMM are held against.
//
// A grid-stride loop of 16-byte buffer loads (out-of-range offsets read as
// zero, so no access can leave the buffer) with a chosen cache-policy
// operand; the loaded words are xor-folded and one word per workgroup is
// written only if the fold hits an impossible value, so the loads stay live
// and nothing else touches memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gemvtile.h"

namespace {

typedef unsigned u4 __attribute__((ext_vector_type(4)));

template <int AUX>
__global__ void __launch_bounds__(512) read_stream_kernel(const void *p, uint32_t bytes, unsigned *sink) {
  constexpr int kUnroll = 4;
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
  const uint32_t nthreads = gridDim.x * blockDim.x;
  const uint32_t n16 = bytes / 16;
  unsigned acc = 0;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < n16; base += nthreads * kUnroll) {
    u4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (base + u * nthreads) * 16u, 0, AUX));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int gemvtile_read_stream(const void *p, int64_t bytes, int policy, int blocks, void *sink, void *stream) {
  // bytes <= 1 GiB keeps every offset (base + 3*nthreads)*16 below 2^32.
  if (p == nullptr || sink == nullptr || bytes <= 0 || bytes > (int64_t{1} << 30) || blocks <= 0 || blocks > 4096)
    return GEMVTILE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t b = static_cast<uint32_t>(bytes);
  unsigned *o = static_cast<unsigned *>(sink);
  const dim3 grid(static_cast<unsigned>(blocks)), block(512);
  switch (policy) {
    case 0: hipLaunchKernelGGL(read_stream_kernel<0>, grid, block, 0, s, p, b, o); break;
    case 1: hipLaunchKernelGGL(read_stream_kernel<2>, grid, block, 0, s, p, b, o); break;   // nt
    case 2: hipLaunchKernelGGL(read_stream_kernel<18>, grid, block, 0, s, p, b, o); break;  // sc1 nt
    case 3: hipLaunchKernelGGL(read_stream_kernel<3>, grid, block, 0, s, p, b, o); break;   // sc0 nt
    default: return GEMVTILE_ERR_INVALID_ARG;
  }
  return hipGetLastError() == hipSuccess ? GEMVTILE_OK : GEMVTILE_ERR_LAUNCH;
}
