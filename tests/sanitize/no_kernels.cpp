// Stand-ins for the kernel launchers, for the host-only sanitizer build: the
// host checks never get a device, so no launch is reached; these return an
// error if one were.  The variant table mirrors the kernels' instances.
#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace syncov {
struct GemmArgs;
struct AttnArgs;

hipError_t launch_gemm(const GemmArgs&, int, int, int, int, bool, int, hipStream_t, int*) { return hipErrorNoDevice; }
int gemm_wg_per_cu(int tm, int tn) { return (tm == 128 && tn == 128) ? 2 : 1; }
bool gemm_variant_exists(int tm, int tn) {
  return (tm == 256 && tn == 256) || (tm == 256 && tn == 128) || (tm == 128 && tn == 128);
}
hipError_t launch_fill_u32(uint32_t*, int64_t, uint32_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_sdma_gate(uint32_t*, int64_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_sdma_join(uint32_t*, const uint32_t*, const int32_t*, const int32_t*, int32_t, uint64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_ring_attn(const AttnArgs&, int, hipStream_t) { return hipErrorNoDevice; }
int attn_wg_per_cu() { return 1; }
int attn_query_block(int hg) { return 32 * (8 / hg); }

}  // namespace syncov
