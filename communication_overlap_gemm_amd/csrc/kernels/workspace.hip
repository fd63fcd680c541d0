// Small kernels around the workspace: initialisation, and the gate and join
// of the SDMA backend.
#include "device_common.hpp"

namespace syncov {

// Zero-fills n 32-bit words (workspace initialisation; a kernel rather than a
// memset so the call can sit inside a captured graph).
__global__ __launch_bounds__(256) void fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// SDMA backend, first kernel of a call on the caller's stream: fixes the
// call's epoch in the workspace word that the engines copy into the chunk
// flags, writes it past the L2 (the engines read memory, not an XCD's L2),
// then opens the gate signal that every SDMA copy of the call waits for.
__global__ __launch_bounds__(64) void sdma_gate(uint32_t* hdr, int64_t* gate) {
  if (threadIdx.x == 0) {
    __hip_atomic_store(hdr + WS_SDMA_EPOCH, call_epoch(hdr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(gate, int64_t(0), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// SDMA backend, copy-only: ends the call once every copied chunk's flag is up
// (bounded waits; a timeout is recorded like any other), then stores the
// call's epoch as the compute kernel's last workgroup would.
__global__ __launch_bounds__(64) void sdma_join(uint32_t* hdr, const uint32_t* flags, const int32_t* arrival,
                                                const int32_t* resident, int32_t num_chunks, uint64_t timeout_ticks) {
  if (threadIdx.x == 0) {
    const uint32_t e = call_epoch(hdr);
    for (int32_t p = 0; p < num_chunks; ++p) {
      const int32_t c = arrival[p];
      if (!resident[c] && !wait_flag(flags, c, e, hdr, timeout_ticks)) break;
    }
    st_release_agent(hdr + WS_EPOCH, e);
  }
}

hipError_t launch_sdma_gate(uint32_t* hdr, int64_t* gate, hipStream_t s) {
  hipLaunchKernelGGL(sdma_gate, dim3(1), dim3(64), 0, s, hdr, gate);
  return hipGetLastError();
}

hipError_t launch_sdma_join(uint32_t* hdr, const uint32_t* flags, const int32_t* arrival, const int32_t* resident,
                            int32_t num_chunks, uint64_t timeout_ticks, hipStream_t s) {
  hipLaunchKernelGGL(sdma_join, dim3(1), dim3(64), 0, s, hdr, flags, arrival, resident, num_chunks, timeout_ticks);
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
