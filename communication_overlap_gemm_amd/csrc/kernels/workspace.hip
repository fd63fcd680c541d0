// Small kernels around the workspace: initialisation and the flag raised
// after each SDMA copy.
#include "device_common.hpp"

namespace syncov {

// Zero-fills n 32-bit words (workspace initialisation; a kernel rather than a
// memset so the call can sit inside a captured graph).
__global__ __launch_bounds__(256) void fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// Raises flags[c] to the running call's epoch (one lane), after the stream's
// preceding SDMA copy of chunk c has completed.  The call's compute kernel
// cannot finish (and advance the stored epoch) before every such flag is up.
__global__ __launch_bounds__(64) void publish_flag(uint32_t* hdr, uint32_t* flags, int32_t c) {
  if (threadIdx.x == 0) st_release_agent(flags + c, call_epoch(hdr));
}

hipError_t launch_publish_flag(uint32_t* hdr, uint32_t* flags, int32_t c, hipStream_t s) {
  hipLaunchKernelGGL(publish_flag, dim3(1), dim3(64), 0, s, hdr, flags, c);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_u32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace syncov
