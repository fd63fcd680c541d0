// Copy agent on dedicated CUs, and the per-call begin kernel.
//
// The Syncopate summary page ("Core method", paper sec. 5.2, Fig. 7) lowers a
// chunk plan to load/store on dedicated SMs among other backends, signalling
// through global-memory flags; the review page's Fig. 5 caption shows that
// communication as an independent kernel on specialised SMs.  The Entwine
// abstract pairs a tile-reordered GEMM with SM-based fine-grained
// communication and sizes the SM share against compute slowdown.
//
// Here one kernel runs on a CU-masked stream (the GEMM gets the other CUs):
//   copy-in  (AG, attention): for each chunk in arrival order, every
//            workgroup copies its slice of the chunk's rows from the peer
//            region to the local buffer; the last workgroup to finish raises
//            ready[c] = epoch.
//   copy-out (RS): for each chunk in send order, every workgroup waits for
//            done[c] (raised by the GEMM), copies its slice of the chunk's
//            rows of C into the staging slot, and the last one raises
//            sent[c] = epoch.
// All workgroups walk the same order, so chunks complete one after another
// at the agent's full bandwidth.
#include "device_common.hpp"
#include "launch_args.hpp"

namespace syncov {


typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Copies bytes [lo, hi) of src to dst (16-byte granules; both 16-byte aligned),
// kUnroll loads in flight per thread.  STREAM selects non-temporal accesses.
template <bool STREAM>
__device__ __forceinline__ void copy_range(const char* __restrict__ src, char* __restrict__ dst, int64_t lo,
                                           int64_t hi) {
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src);
  u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
  int64_t g = lo / 16 + threadIdx.x;
  const int64_t gend = hi / 16;
  const int64_t step = kCopyThreads;
  auto ld = [](const u32x4_t* p) { return STREAM ? __builtin_nontemporal_load(p) : *p; };
  auto st = [](u32x4_t v, u32x4_t* p) {
    if constexpr (STREAM)
      __builtin_nontemporal_store(v, p);
    else
      *p = v;
  };
  for (; g + (kUnroll - 1) * step < gend; g += kUnroll * step) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld(s + g + u * step);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) st(v[u], d + g + u * step);
  }
  for (; g < gend; g += step) st(ld(s + g), d + g);
}

// Publication.  A chunk is complete when every workgroup's stores of it are
// visible device-wide.  Each workgroup first drains its stores into its XCD's
// L2 (workgroup-scope release = wait for the stores), then counts itself in a
// per-(chunk, XCD) counter; the last workgroup of each XCD writes that L2 back
// with one agent-scope release (which covers the other workgroups' lines in
// the same L2) and adds the XCD's workgroups to the chunk's total; whoever
// completes the total raises the flag.  One L2 writeback per XCD per chunk
// instead of one per workgroup.  A census at kernel start tells each
// workgroup how many of the grid's workgroups share its XCD.
__global__ __launch_bounds__(kCopyThreads) void copy_agent(CopyArgs a) {
  __shared__ int32_t s_ok;
  __shared__ uint32_t s_mine;
  const uint32_t epoch = a.hdr[WS_EPOCH];
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int xcc = xcc_id();
  if (threadIdx.x == 0) {
    add_acq_rel_agent(a.hdr + WS_CENSUS + xcc, 1u);
    add_acq_rel_agent(a.hdr + WS_CENSUS_TOTAL, 1u);
    // every workgroup of this grid is resident at once (the grid is sized to
    // the dedicated CUs), so the census completes; the wait is still bounded
    const uint64_t t0 = wall_clock64();
    bool ok = true;
    while (ld_relaxed_agent(a.hdr + WS_CENSUS_TOTAL) < static_cast<uint32_t>(G)) {
      __builtin_amdgcn_s_sleep(1);
      if (wall_clock64() - t0 > a.timeout_ticks) {
        record_timeout(a.hdr, -1);
        ok = false;
        break;
      }
    }
    s_mine = ok ? ld_relaxed_agent(a.hdr + WS_CENSUS + xcc) : 0u;
  }
  __syncthreads();
  const uint32_t mine = s_mine;
  if (mine == 0) return;
  for (int32_t p = 0; p < a.num_chunks; ++p) {
    const int32_t c = a.arrival[p];
    if (!a.copy_out && a.resident[c]) continue;
    if (a.copy_out) {
      if (threadIdx.x == 0) {
        const bool ok = wait_flag(a.wait_flags, c, epoch, a.hdr, a.timeout_ticks);
        if (ok) acquire_agent();
        s_ok = ok;
      }
      __syncthreads();
      const int ok = s_ok;
      __syncthreads();
      if (!ok) continue;  // chunk never completed: nothing to send
    }
    const int64_t r0 = a.chunk_begin[c], r1 = a.chunk_begin[c + 1];
    const int64_t drow = a.copy_out ? a.slot_row[p] : r0;
    for (int x = 0; x < a.ntensors; ++x) {
      const int64_t bytes = (r1 - r0) * a.row_bytes[x];
      const int64_t granules = bytes / 16;
      const int64_t lo = granules * b / G * 16, hi = granules * (b + 1) / G * 16;
      if (a.streaming)
        copy_range<true>(a.src[x] + r0 * a.row_bytes[x], a.dst[x] + drow * a.row_bytes[x], lo, hi);
      else
        copy_range<false>(a.src[x] + r0 * a.row_bytes[x], a.dst[x] + drow * a.row_bytes[x], lo, hi);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // this thread's stores have reached the L2
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = add_acq_rel_agent(a.xparts + c * kMaxXcd + xcc, 1u);
      if (old + 1u == mine) {
        release_agent();  // write this XCD's L2 back: every workgroup of this XCD has stored
        const uint32_t done = add_acq_rel_agent(a.parts + c, mine);
        if (done + mine == static_cast<uint32_t>(G)) st_release_agent(a.out_flags + c, epoch);
      }
    }
  }
}

// Opens a call: bumps the epoch, clears the error word and the per-chunk
// counters, and raises the flags of chunks that need no copy (resident ones,
// or all of them for compute-only runs).  One workgroup.
__global__ __launch_bounds__(256) void begin_call(uint32_t* hdr, uint32_t* flags, uint32_t* counters,
                                                  uint32_t* parts, uint32_t* xparts, int32_t num_chunks,
                                                  const int32_t* resident, int32_t preset_all) {
  __shared__ uint32_t s_epoch;
  if (threadIdx.x == 0) {
    uint32_t e = hdr[WS_EPOCH] + 1u;
    if (e == 0u) e = 1u;
    hdr[WS_EPOCH] = e;
    hdr[WS_ERR_CODE] = 0u;
    hdr[WS_ERR_CHUNK] = 0u;
    hdr[WS_TICKET] = 0u;
    hdr[WS_CENSUS_TOTAL] = 0u;
    s_epoch = e;
  }
  if (threadIdx.x < kMaxXcd) hdr[WS_CENSUS + threadIdx.x] = 0u;
  for (int32_t i = threadIdx.x; i < num_chunks * kMaxXcd; i += blockDim.x) xparts[i] = 0u;
  __syncthreads();
  const uint32_t e = s_epoch;
  for (int32_t c = threadIdx.x; c < num_chunks; c += blockDim.x) {
    counters[c] = 0u;
    parts[c] = 0u;
    if (preset_all || (resident && resident[c])) flags[c] = e;
  }
}

// Zero-fills n 32-bit words (workspace initialisation; a kernel rather than a
// memset so the call can sit inside a captured graph).
__global__ __launch_bounds__(256) void fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// Raises flags[c] to the current epoch (one lane), after the stream's
// preceding SDMA copy of chunk c has completed.
__global__ __launch_bounds__(64) void publish_flag(uint32_t* hdr, uint32_t* flags, int32_t c) {
  if (threadIdx.x == 0) st_release_agent(flags + c, hdr[WS_EPOCH]);
}

hipError_t launch_publish_flag(uint32_t* hdr, uint32_t* flags, int32_t c, hipStream_t s) {
  hipLaunchKernelGGL(publish_flag, dim3(1), dim3(64), 0, s, hdr, flags, c);
  return hipGetLastError();
}

// Copy-agent workgroups that fit on one CU at once (the census needs the whole
// grid resident).
int copy_agent_max_wg_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, copy_agent, kCopyThreads, 0) != hipSuccess) return 1;
  return n < 1 ? 1 : n;
}

hipError_t launch_copy_agent(const CopyArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(copy_agent, dim3(grid), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_begin_call(uint32_t* hdr, uint32_t* flags, uint32_t* counters, uint32_t* parts, uint32_t* xparts,
                             int32_t num_chunks, const int32_t* resident, int32_t preset_all, hipStream_t s) {
  hipLaunchKernelGGL(begin_call, dim3(1), dim3(256), 0, s, hdr, flags, counters, parts, xparts, num_chunks, resident,
                     preset_all);
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
