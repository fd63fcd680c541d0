// Device helpers shared by the gfx950 kernels: bf16 vector types, the
// cross-XCD flag protocol (bounded relaxed polling, one acquire; release then
// publish), and the workspace layout.
//
// Flag protocol.  The pages' asynchronous backends signal chunk completion
// through global-memory flags (Syncopate summary page, "Core method", paper
// sec. 5.2, Fig. 7).  On MI355X the producer (copy agent, SDMA engine or GEMM
// epilogue) and the consumer may sit on different XCDs, each with its own L2,
// so the producer publishes with an agent-scope release (its stores are
// written back past its L2) and the consumer, after seeing the flag with
// relaxed agent-scope polls, performs one agent-scope acquire (stale lines in
// its own caches are dropped) before it reads the chunk.  Flags hold the
// epoch of the call that raised them, so they are never cleared between
// calls; every wait is bounded by a wall-clock limit and reports the chunk it
// gave up on in the workspace error word.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch_args.hpp"

namespace syncov {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Workspace header words (uint32 index).  The flag and counter arrays follow
// at offsets the host computes from the plan's chunk count.
enum : int {
  WS_EPOCH = 0,       // epoch of the last completed call
  WS_ERR_CODE = 1,    // 0 = fine, else ERR_* below (sticky until re-initialisation)
  WS_ERR_CHUNK = 2,   // chunk whose wait expired first
  WS_EXIT = 3,        // finished groups of workgroups of the running call (tree level 2)
  WS_SDMA_EPOCH = 8,  // SDMA backend: the running call's epoch, copied into each chunk flag by the engine
  WS_EXIT_GROUP = 16, // finished workgroups per group of kTreeFan (tree level 1, 16 slots)
  WS_HEADER_WORDS = 64
};
constexpr int kMaxXcd = 16;

// XCD (XCC) this wave runs on.
__device__ __forceinline__ int xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kMaxXcd - 1); }
enum : uint32_t { ERR_TIMEOUT = 1u };

__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

__device__ __forceinline__ uint32_t ld_relaxed_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_relaxed_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_release_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t add_relaxed_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool epoch_reached(uint32_t flag, uint32_t epoch) {
  return static_cast<int32_t>(flag - epoch) >= 0;
}

// Records a timeout for `chunk` if no error is recorded yet.
__device__ __forceinline__ void record_timeout(uint32_t* hdr, int32_t chunk) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(hdr + WS_ERR_CODE, &expected, ERR_TIMEOUT, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    __hip_atomic_store(hdr + WS_ERR_CHUNK, static_cast<uint32_t>(chunk), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  release_agent();  // ordered before this workgroup's exit count, which the call's last workgroup acquires
}

// Single-lane bounded wait for flags[c] to reach `epoch`.  Returns false when
// the wall-clock limit passes or another wait has already recorded an error
// (so that every waiter on a withheld chunk gives up promptly).  No acquire
// here: the caller performs one after all its waits succeed.
// Polls back off exponentially (64 to 1024 cycles between loads): many
// waiters on one flag would otherwise flood its memory channel and slow the
// producers' stores and counters on it.
__device__ __forceinline__ void backoff_sleep(int& n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_sleep(1); break;
    case 1: __builtin_amdgcn_s_sleep(2); break;
    case 2: __builtin_amdgcn_s_sleep(4); break;
    case 3: __builtin_amdgcn_s_sleep(8); break;
    default: __builtin_amdgcn_s_sleep(16); break;
  }
  if (n < 4) ++n;
}

__device__ __forceinline__ bool wait_flag(const uint32_t* flags, int32_t c, uint32_t epoch, uint32_t* hdr,
                                          uint64_t timeout_ticks) {
  if (epoch_reached(ld_relaxed_agent(flags + c), epoch)) return true;
  const uint64_t t0 = wall_clock64();
  int b = 0;
  for (;;) {
    backoff_sleep(b);
    if (epoch_reached(ld_relaxed_agent(flags + c), epoch)) return true;
    if (ld_relaxed_agent(hdr + WS_ERR_CODE) != 0) return false;
    if (wall_clock64() - t0 > timeout_ticks) {
      record_timeout(hdr, c);
      return false;
    }
  }
}


// Round-to-nearest-even float -> bf16 bits (inputs are finite in this library;
// NaN is kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Counting tree.  Many workgroups incrementing one word serialise on it; a
// two-level tree keyed by the caller's rank (groups of `fan` workgroups, sizes
// known from the count alone) keeps at most `fan` atomics on any word (16 for
// up to 256 workgroups).  One lane per workgroup calls it; it returns true for
// exactly one caller, the one that completes the count, after clearing the
// words for the next use.  level1 holds up to 16 words.
// Ordering: whatever a caller ordered before its call with an agent-scope
// release fence happens-before everything the completing caller does after
// the call.  The counts themselves are relaxed: an agent-scope acquire or
// release on gfx950 is an L2 invalidate or write-back, so only the completer
// of a group (acquire-release fence: it takes the group's releases over and
// passes them on through its level-2 count) and the completer of the tree
// (acquire fence) pay for one; every other caller pays only for its own
// release.  (Each relaxed count returns its old value, which the caller
// compares before it goes on, so its count is performed before anything the
// caller issues after it.)
__device__ __forceinline__ bool tree_count(uint32_t* level1, uint32_t* level2, int32_t rank, int32_t count) {
  const int32_t fan = count > 256 ? (count + 15) / 16 : 16;
  const int32_t g = rank / fan, groups = (count + fan - 1) / fan;
  const uint32_t in_group = static_cast<uint32_t>(count - g * fan < fan ? count - g * fan : fan);
  if (add_relaxed_agent(level1 + g, 1u) + 1u != in_group) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
  st_relaxed_agent(level1 + g, 0u);
  if (add_relaxed_agent(level2, 1u) + 1u != static_cast<uint32_t>(groups)) return false;
  acquire_agent();
  st_relaxed_agent(level2, 0u);
  return true;
}

// ---- one launch per call --------------------------------------------------
// Every call is one kernel launch on the caller's stream.  Its epoch is one
// past the epoch of the last completed call on this workspace; the last
// workgroup of the grid to finish stores it, after every workgroup has read
// the old value (each reads it before it counts itself out).  Flags are
// compared against the epoch, so they are never cleared; per-chunk counters
// are cleared by the workgroup that completes them.  A recorded error is
// sticky: waits give up at once until the workspace is initialised again, and
// the last workgroup clears the counters that a failed call left behind.
__device__ __forceinline__ uint32_t call_epoch(const uint32_t* hdr) {
  const uint32_t e = __hip_atomic_load(hdr + WS_EPOCH, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  return e == 0u ? 1u : e;
}

// Last action of every workgroup (all threads).  The exit count carries no
// release of its own: the stores of the call are made visible by the end of
// the kernel, and a recorded error by the release in record_timeout.  Each
// workgroup's read of the old epoch was issued at its start, before the
// barrier below, and the last workgroup stores the new epoch only after every
// workgroup has counted out.
__device__ __forceinline__ void end_call(uint32_t* hdr, uint32_t epoch, const CounterArrays& ca) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (tree_count(hdr + WS_EXIT_GROUP, hdr + WS_EXIT, blockIdx.x, gridDim.x)) {
      if (ld_relaxed_agent(hdr + WS_ERR_CODE) != 0u) {
        for (int32_t c = 0; c < ca.num_chunks; ++c) {
          st_relaxed_agent(ca.counters + c, 0u);
          st_relaxed_agent(ca.parts + c, 0u);
          for (int x = 0; x < kMaxXcd; ++x) st_relaxed_agent(ca.xparts + c * kMaxXcd + x, 0u);
          for (int h = 0; h < kMaxSlices; ++h) {
            st_relaxed_agent(ca.sparts + c * kMaxSlices + h, 0u);
            for (int x = 0; x < kMaxXcd; ++x) st_relaxed_agent(ca.sxparts + (c * kMaxSlices + h) * kMaxXcd + x, 0u);
          }
        }
      }
      st_release_agent(hdr + WS_EPOCH, epoch);
    }
  }
}

// Persistent-kernel slot of workgroup `b` out of `g`: workgroups are handed to
// XCDs round-robin, so consecutive slots are made to live on one XCD, and the
// tiles one XCD works on at a time are neighbours in the traversal order
// (they share A rows or B columns in that XCD's L2).
__device__ __forceinline__ int32_t xcd_slot(int32_t b, int32_t g, int32_t nxcd) {
  if (nxcd <= 1 || g % nxcd) return b;
  return (b % nxcd) * (g / nxcd) + b / nxcd;
}

}  // namespace syncov
