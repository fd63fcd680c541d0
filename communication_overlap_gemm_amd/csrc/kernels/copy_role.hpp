// Copy role: the workgroups of a call's launch that move chunks instead of
// computing.
//
// The Syncopate summary page ("Core method", paper sec. 5.2, Fig. 7) lowers a
// chunk plan to load/store on dedicated SMs among other backends, signalling
// through global-memory flags; the review page's Fig. 5 caption shows that
// communication on specialised SMs beside the compute.  The Entwine abstract
// pairs a tile-reordered GEMM with SM-based fine-grained communication and
// sizes the SM share against compute slowdown.
//
// Here the copy agent is not a kernel of its own: the first `count`
// workgroups of the compute kernel's grid take this role, so a call is one
// launch on one stream.  The dispatcher places workgroup b on XCD b % 8 and
// issues workgroups in order, so with a multiple of 8 of them they are
// spread evenly over the XCDs and resident before any compute workgroup.
//   copy-in  (AG, attention): for each chunk in arrival order, every
//            workgroup copies its slice of the chunk's rows from the peer
//            region to the local buffer; the chunk's flag is raised once all
//            slices are visible device-wide.
//   copy-out (RS): for each chunk in send order, every workgroup waits for
//            done[c] (raised by the GEMM role), copies its slice of the
//            chunk's rows of C into the staging slot, and sent[c] is raised
//            the same way.
//   K-sliced copy-in: the chunks move as column slices of their rows, slice 0
//            of every chunk first, each slice with a ready flag of its own, so
//            a tile can start on the first K-slice of its rows before the rest
//            of them has landed.
// All workgroups walk the same order, so chunks complete one after another at
// the role's full bandwidth.
#pragma once

#include "device_common.hpp"
#include "launch_args.hpp"

namespace syncov {

typedef uint32_t copy_u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCopyUnroll = 16;  // 16-byte loads in flight per thread

// The copy stores (unless STREAM) carry the device-scope cache policy (SC1):
// the copied rows reach memory as they are written, so the agent-scope
// release that publishes them finds little left to write back.  They go
// through a buffer resource over the destination of one chunk, so every
// offset must stay below 2 GiB; the runtime refuses larger chunks for the
// backends that copy on CUs.
constexpr int kCopyStorePolicy = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t copy_dst_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), 0x7fffffff, 0x00020000);
}

// Copies bytes [lo, hi) of src to dst (16-byte granules; both 16-byte
// aligned), kCopyUnroll loads in flight per thread.  STREAM selects
// non-temporal accesses; otherwise the stores carry kCopyStorePolicy and hi
// stays below 2 GiB.
template <int THREADS, bool STREAM>
__device__ __forceinline__ void copy_range(const char* __restrict__ src, char* __restrict__ dst, int64_t lo,
                                           int64_t hi) {
  const copy_u32x4_t* s = reinterpret_cast<const copy_u32x4_t*>(src);
  copy_u32x4_t* d = reinterpret_cast<copy_u32x4_t*>(dst);
  const __amdgpu_buffer_rsrc_t drs = copy_dst_rsrc(dst);
  int64_t g = lo / 16 + threadIdx.x;
  const int64_t gend = hi / 16;
  constexpr int64_t step = THREADS;
  auto ld = [](const copy_u32x4_t* p) { return STREAM ? __builtin_nontemporal_load(p) : *p; };
  auto st = [&](copy_u32x4_t v, int64_t gi) {  // granule gi of dst
    if constexpr (STREAM)
      __builtin_nontemporal_store(v, d + gi);
    else
      __builtin_amdgcn_raw_buffer_store_b128(v, drs, static_cast<uint32_t>(gi * 16), 0, kCopyStorePolicy);
  };
  for (; g + (kCopyUnroll - 1) * step < gend; g += kCopyUnroll * step) {
    copy_u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = ld(s + g + u * step);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) st(v[u], g + u * step);
  }
  if (g < gend) {  // the remainder, still with every load in flight before the stores
    copy_u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (g + u * step < gend) v[u] = ld(s + g + u * step);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (g + u * step < gend) st(v[u], g + u * step);
  }
}

// Copies granules [lo, hi) of a column block: the block is `rows` rows of
// `seg` bytes (a multiple of 16) at byte column col of rows `pitch` bytes
// apart in src and dst, its granules numbered row by row.  Same loads in
// flight per thread as copy_range; each thread steps its (row, column) by the
// block stride instead of dividing.
template <int THREADS, bool STREAM>
__device__ __forceinline__ void copy_block(const char* __restrict__ src, char* __restrict__ dst, int64_t pitch,
                                           int64_t col, int64_t seg, int64_t lo, int64_t hi) {
  const int64_t gpr = seg / 16;  // granules per row
  int64_t g = lo + threadIdx.x;
  if (g >= hi) return;
  int64_t row = g / gpr, cg = g - row * gpr;
  const int64_t drow = THREADS / gpr, dcg = THREADS - drow * gpr;  // one step of THREADS granules
  auto ld = [](const char* p) {
    const copy_u32x4_t* q = reinterpret_cast<const copy_u32x4_t*>(p);
    return STREAM ? __builtin_nontemporal_load(q) : *q;
  };
  const __amdgpu_buffer_rsrc_t drs = copy_dst_rsrc(dst);
  auto st = [&](copy_u32x4_t v, int64_t off) {  // byte offset in dst
    if constexpr (STREAM)
      __builtin_nontemporal_store(v, reinterpret_cast<copy_u32x4_t*>(dst + off));
    else
      __builtin_amdgcn_raw_buffer_store_b128(v, drs, static_cast<uint32_t>(off), 0, kCopyStorePolicy);
  };
  while (g < hi) {
    copy_u32x4_t v[kCopyUnroll];
    int64_t off[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      off[u] = row * pitch + col + cg * 16;
      if (g + u * THREADS < hi) v[u] = ld(src + off[u]);
      row += drow;
      cg += dcg;
      if (cg >= gpr) {
        cg -= gpr;
        ++row;
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (g + u * THREADS < hi) st(v[u], off[u]);
    g += kCopyUnroll * THREADS;
  }
}

// Thread 0 of a workgroup that has copied (and released) its share of slice h
// of chunk c, rank-th of `count`: the completer of the slice's count raises
// the slice flag, and the completer of the chunk's last slice raises the chunk
// flag (counted with acquire-release, so it sees the others' publications)
// and clears the count.
__device__ __forceinline__ void slice_done(const CopyArgs& a, int32_t c, int32_t h, int32_t S, int32_t rank,
                                           int32_t count, uint32_t epoch) {
  const int32_t sl = c * kMaxSlices + h;
  if (!tree_count(a.sxparts + sl * kMaxXcd, a.sparts + sl, rank, count)) return;
  st_release_agent(a.slice_flags + sl, epoch);
  const uint32_t done = __hip_atomic_fetch_add(a.parts + c, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  if (done == static_cast<uint32_t>(S)) {
    st_relaxed_agent(a.parts + c, 0u);
    if (a.trace_chunks) a.trace_chunks[2 * c] = wall_clock64();
    st_release_agent(a.out_flags + c, epoch);
  }
}

// Publication.  A chunk is complete when every copy workgroup's stores of it
// are visible device-wide.  Each workgroup drains its stores into its XCD's L2
// (workgroup-scope release = wait for the stores), writes that L2 back with an
// agent-scope release, and counts itself in the chunk's counting tree; the
// workgroup that completes the count raises the flag.  No workgroup waits for
// another.  `rank` in [0, count) is this workgroup's index among the copy
// workgroups.
// BATCH: copy this workgroup's slice of every chunk, then publish them all
// with one completion round (co-located copy: nothing computes until its own
// share is copied, so per-chunk publication would only add latency).
template <int THREADS, bool BATCH = false>
__device__ __forceinline__ void copy_role(const CopyArgs& a, int32_t rank, int32_t count, uint32_t epoch) {
  __shared__ int32_t s_ok;
  const int64_t G = count, b = rank;
  auto skipped = [&](int32_t c) { return !a.copy_out && (a.resident[c] || a.skip_chunk == c || a.skip_chunk == -1); };
  if constexpr (BATCH) {
    // Published all at once, so the copied rows are split evenly in row
    // order, not chunk by chunk: each workgroup copies one contiguous share
    // of the concatenated copied granules (one or two large ranges).
    int32_t first = -1;  // the batch counts in the slots of its first copied chunk
    int64_t total = 0;
    for (int x = 0; x < a.ntensors; ++x)
      for (int32_t c = 0; c < a.num_chunks; ++c)
        if (!skipped(c)) total += (a.chunk_begin[c + 1] - a.chunk_begin[c]) * a.row_bytes[x] / 16;
    const int64_t lo = total * b / G, hi = total * (b + 1) / G;
    int64_t pos = 0;
    for (int x = 0; x < a.ntensors; ++x)
      for (int32_t c = 0; c < a.num_chunks; ++c) {
        if (skipped(c)) continue;
        if (first < 0) first = c;  // the lowest copied chunk id: the same for every workgroup
        const int64_t r0 = a.chunk_begin[c], n = (a.chunk_begin[c + 1] - r0) * a.row_bytes[x] / 16;
        const int64_t a0 = lo > pos ? lo : pos, a1 = hi < pos + n ? hi : pos + n;
        if (a0 < a1)
          copy_range<THREADS, false>(a.src[x] + r0 * a.row_bytes[x], a.dst[x] + r0 * a.row_bytes[x], (a0 - pos) * 16,
                                     (a1 - pos) * 16);
        pos += n;
      }
    if (first < 0) return;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
      release_agent();
      if (tree_count(a.xparts + first * kMaxXcd, a.parts + first, rank, count)) {
        const uint64_t now = wall_clock64();
        release_agent();  // one release for every flag below (a waiter polls relaxed, then acquires)
        for (int32_t p = 0; p < a.num_chunks; ++p) {
          const int32_t c = a.arrival[p];
          if (skipped(c)) continue;
          if (a.trace_chunks) a.trace_chunks[2 * c] = now;
          for (int32_t h = 0; a.kslices > 1 && h < a.kslices; ++h) st_relaxed_agent(a.slice_flags + c * kMaxSlices + h, epoch);
          st_relaxed_agent(a.out_flags + c, epoch);
        }
      }
    }
    return;
  }
  // Teams: the workgroups split into `teams` teams by rank; team t copies
  // every teams-th copied item (in arrival / send order) from the t-th on, so
  // up to `teams` items are in flight at once and one team's drain, waits and
  // publication overlap the others' copying.  An item is a chunk, or with a
  // K-sliced copy-in one column slice of a chunk, slice-major: slice 0 of
  // every chunk in arrival order, then slice 1, ...
  const int32_t teams = (a.teams > 1 && a.teams <= count) ? a.teams : 1;
  const int32_t team = rank % teams, trank = rank / teams;
  const int32_t tcount = count / teams + (team < count % teams ? 1 : 0);
  const int32_t S = (!a.copy_out && a.kslices > 1) ? a.kslices : 1;
  int32_t seq = -1;  // index of the item among the copied ones
  uint64_t link_free = 0;  // thread 0, paced copies: when this team's link is next free
  for (int32_t h = 0; h < S; ++h)
    for (int32_t p = 0; p < a.num_chunks; ++p) {
      const int32_t c = a.arrival[p];
      if (skipped(c)) continue;
      if (h < a.lead_slices && a.lead_count && a.lead_count[c] > 0) continue;  // the compute workgroups copy it
      if (++seq % teams != team) continue;
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
      if (a.pace_q16 && threadIdx.x == 0) {  // the item holds the link from when both are ready
        int64_t bytes = 0;
        for (int x = 0; x < a.ntensors; ++x) {
          const int64_t lines = a.row_bytes[x] / 128;
          bytes += (r1 - r0) * (S == 1 ? a.row_bytes[x] : ((h + 1) * lines / S - h * lines / S) * 128);
        }
        const uint64_t now = wall_clock64();
        link_free = (link_free > now ? link_free : now) + ((static_cast<uint64_t>(bytes) * a.pace_q16) >> 36);
      }
      for (int x = 0; x < a.ntensors; ++x) {
        const int64_t rb = a.row_bytes[x];
        if (S == 1) {
          const int64_t granules = (r1 - r0) * rb / 16;
          const int64_t lo = granules * trank / tcount * 16, hi = granules * (trank + 1) / tcount * 16;
          if (a.streaming)
            copy_range<THREADS, true>(a.src[x] + r0 * rb, a.dst[x] + drow * rb, lo, hi);
          else
            copy_range<THREADS, false>(a.src[x] + r0 * rb, a.dst[x] + drow * rb, lo, hi);
        } else {
          const int64_t lines = rb / 128;  // 128-byte columns per row
          const int64_t col = h * lines / S * 128, seg = (h + 1) * lines / S * 128 - col;
          const int64_t granules = (r1 - r0) * (seg / 16);
          const int64_t lo = granules * trank / tcount, hi = granules * (trank + 1) / tcount;
          if (a.streaming)
            copy_block<THREADS, true>(a.src[x] + r0 * rb, a.dst[x] + r0 * rb, rb, col, seg, lo, hi);
          else
            copy_block<THREADS, false>(a.src[x] + r0 * rb, a.dst[x] + r0 * rb, rb, col, seg, lo, hi);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // this thread's stores have reached the L2
      __syncthreads();
      if (threadIdx.x == 0) {
        if (a.pace_q16) {  // paced: the item is delivered when its link time has passed
          int n = 0;
          while (wall_clock64() < link_free) backoff_sleep(n);
        }
        release_agent();  // write this XCD's L2 back
        if (S == 1) {
          if (tree_count(a.xparts + c * kMaxXcd, a.parts + c, trank, tcount)) {
            if (a.trace_chunks) a.trace_chunks[2 * c + (a.copy_out ? 1 : 0)] = wall_clock64();
            st_release_agent(a.out_flags + c, epoch);
          }
        } else {
          slice_done(a, c, h, S, trank, tcount, epoch);
        }
      }
    }
}

// Lead slices of a K-sliced copy-in, run by compute workgroup g before its
// first tile: for each (chunk c, share rank) of its lead items, copy share
// rank of lead_count[c] of the first lead_slices slices of chunk c's rows (the
// first floor(L lines / S) 128-byte columns of each row, L = lead_slices),
// then publish each of those slices with the other workgroups of the share
// group.  The shares of one chunk are held by the workgroups whose first tile
// reads it, which all start together.
template <int THREADS>
__device__ __forceinline__ void lead_slice(const CopyArgs& a, const int32_t* lead_ptr, const int32_t* lead_item,
                                           int32_t g, uint32_t epoch) {
  const int32_t S = a.kslices, L = a.lead_slices;
  for (int32_t e = lead_ptr[g]; e < lead_ptr[g + 1]; ++e) {
    const int32_t c = lead_item[2 * e], rank = lead_item[2 * e + 1], count = a.lead_count[c];
    const int64_t r0 = a.chunk_begin[c], r1 = a.chunk_begin[c + 1], rb = a.row_bytes[0];
    const int64_t seg = L * (rb / 128) / S * 128;  // slices [0, L): the columns before slice L's first
    const int64_t granules = (r1 - r0) * (seg / 16);
    const int64_t lo = granules * rank / count, hi = granules * (rank + 1) / count;
    if (a.streaming)
      copy_block<THREADS, true>(a.src[0] + r0 * rb, a.dst[0] + r0 * rb, rb, 0, seg, lo, hi);
    else
      copy_block<THREADS, false>(a.src[0] + r0 * rb, a.dst[0] + r0 * rb, rb, 0, seg, lo, hi);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
      release_agent();  // write this XCD's L2 back
      for (int32_t h = 0; h < L; ++h) slice_done(a, c, h, S, rank, count, epoch);
    }
  }
}

}  // namespace syncov
