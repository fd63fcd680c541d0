// Kernel argument blocks shared by the host runtime and the kernels.
#pragma once

#include <stdint.h>

namespace syncov {

constexpr int kMaxSlices = 8;  // K-slices per chunk (copy_kslices) the workspace holds
constexpr int kMaxCopyTensors = 3;  // tensors staged per chunk (head-parallel attention: Q, K and V)

// Per-chunk counter arrays of the workspace (cleared by the workgroup that
// completes them; after a failed call, by the call's last workgroup).
struct CounterArrays {
  uint32_t* counters;  // GEMM-RS: tiles stored per chunk
  uint32_t* parts;     // copy role: XCDs finished per chunk (K-sliced copy: slices finished)
  uint32_t* xparts;    // copy role: workgroups finished per (chunk, XCD), C x 16
  uint32_t* sparts;    // K-sliced copy: XCDs finished per (chunk, slice), C x kMaxSlices
  uint32_t* sxparts;   // K-sliced copy: workgroups finished per (chunk, slice, XCD), C x kMaxSlices x 16
  int32_t num_chunks;
};

// Copy role (copy_role.hpp): chunk copy-in or copy-out.
struct CopyArgs {
  const char* src[kMaxCopyTensors];  // tensors per chunk (ring attention: K and V; head-parallel: Q, K, V)
  char* dst[kMaxCopyTensors];
  int64_t row_bytes[kMaxCopyTensors];
  int32_t ntensors;
  int32_t num_chunks;
  const int64_t* chunk_begin;  // C+1 row bounds
  const int32_t* arrival;      // chunk id per position
  const int32_t* resident;     // copy-in: chunks already in place (skipped)
  const int64_t* slot_row;     // copy-out: first staging row of each position (C+1)
  uint32_t* out_flags;         // raised per chunk when its copy is complete
  const uint32_t* wait_flags;  // copy-out: done flags to wait for
  uint32_t* parts;             // per-chunk count of finished XCD groups
  uint32_t* xparts;            // per (chunk, XCD) count of finished workgroups, C x 16
  uint32_t* hdr;
  uint64_t timeout_ticks;
  int32_t copy_out;
  int32_t streaming;   // non-temporal loads and stores
  int32_t skip_chunk;  // copy-in: chunk left out (failure-path tests); -1 = all, -2 = none
  int32_t teams;       // copy-in: chunks in flight at once (1 = one after another)
  uint64_t* trace_chunks;  // SYNC_RUN_TRACE: per chunk {ready, sent} wall-clock stamps, or null
  // copy-in K-slices: with kslices > 1 every chunk moves as kslices column
  // blocks of its rows, slice by slice across all chunks (slice 0 of every
  // chunk first); slice h of chunk c raises slice_flags[c * kMaxSlices + h]
  // and the last of a chunk's slices raises out_flags[c].  Slice h holds the
  // 128-byte row columns [h * R / kslices, (h + 1) * R / kslices) of each
  // tensor, R = row_bytes / 128.
  int32_t kslices;
  // Link pacing (0 = none): each team stands for one link; an item occupies
  // its team's link for bytes * pace_q16 / 2^36 wall-clock ticks (pace_q16 =
  // ticks per MiB in 16.16 fixed point), starting when both the link is free
  // and the item may start, and is published only when that time has passed.
  uint64_t pace_q16;
  uint32_t* slice_flags;
  uint32_t* sparts;
  uint32_t* sxparts;
  // K-sliced copy-in with lead slices: chunks with lead_count[c] > 0 have
  // their first lead_slices slices copied by compute workgroups (GemmArgs
  // lead tables); the copy role leaves those items out.  Null: the copy role
  // moves every item.
  const int32_t* lead_count;
  int32_t lead_slices;
};

// Persistent GEMM (gemm_persistent.hip).  Workgroups [0, copy_blocks) of the
// grid run the copy role with `copy`; the others compute tiles.
struct GemmArgs {
  const uint16_t* A;  // bf16 [M][K]
  const uint16_t* B;  // bf16 [K][N] (KN) or [N][K] (NK)
  void* C;            // [M][N] fp32 or bf16
  int64_t M, N, K;
  const int32_t* order;  // tile traversal, num_tiles entries
  int32_t num_tiles, tiles_n;
  const int64_t* dep_ptr;  // tile -> chunks CSR
  const int32_t* dep_idx;
  const int32_t* tiles_in;  // RS: tiles per chunk
  const int32_t* resident;  // AG: chunks in place before the call (never waited for)
  uint32_t* flags;          // AG: ready flags; RS: done flags
  uint32_t* hdr;            // workspace header
  CounterArrays cnt;
  uint64_t timeout_ticks;   // wall-clock ticks allowed per wait
  int32_t nxcd;             // XCDs (for the workgroup -> slot remap)
  int32_t wait_chunks;      // AG: 0 = every chunk is in place (compute-only)
  int32_t copy_blocks;
  int32_t colocated;        // AG: every compute workgroup first copies its share of each chunk
  int32_t tile_grid;        // > 0: only compute workgroups [0, tile_grid) take tiles (the others only copy)
  uint64_t* trace_tiles;    // SYNC_RUN_TRACE: per tile {wait begin, wait end, end, xcc<<32 | slot}, or null
  uint64_t* trace_chunks;   // SYNC_RUN_TRACE: per chunk {ready/done, sent}, or null
  // AG with a K-sliced copy (kslices > 1): a tile waits for slice 0 of its
  // chunks before its first loads and for slice h before the loads of the
  // first K-step of slice h (slice_flags as in CopyArgs)
  int32_t kslices;
  const uint32_t* slice_flags;
  // GEMM-RS with the epilogue backend (push_rows non-null): the epilogue also
  // stores tile t's rows into `staging` from row push_rows[t] on (its send
  // slot; every tile lies in one chunk), and the tile that completes chunk c
  // raises sent[c] with done[c]
  const int32_t* push_rows;
  void* staging;
  uint32_t* sent;
  // reduce-scatter step (non-null with push_rows; fp32 C): [M][N] fp32, the
  // partial sums arriving from the ring predecessor; a send slot receives
  // the tile plus these rows
  const void* partials;
  // GEMM-AR share (ar_count > 0; RS instances): the copy workgroups gather the
  // all-reduced rows into ar_out instead of copying out.  Item i is
  // ar_items[5 i .. 5 i + 4] = {source (0: staging, 1: ar_peer), source row,
  // destination row, rows, gate chunk}; it waits until the gate chunk is done.
  const int64_t* ar_items;
  int32_t ar_count;
  const char* ar_src[2];
  char* ar_out;
  int64_t ar_row_bytes;
  // AG with a K-sliced copy and lead slices (lead_ptr non-null): compute
  // workgroup g first copies share lead_item[2 e + 1] of copy.lead_count[c] of
  // the lead slices of chunk c = lead_item[2 e], for e in [lead_ptr[g],
  // lead_ptr[g + 1]), and publishes them with the others of that share group
  const int32_t* lead_ptr;
  const int32_t* lead_item;
  CopyArgs copy;
};

// Ring-attention step (ring_attn.hip).  Same role split as GemmArgs.
struct AttnArgs {
  const uint16_t* q;  // bf16 [sq][heads_q][128]
  const uint16_t* k;  // bf16 [world*n][heads_kv][128] (local copy, filled by the copy role)
  const uint16_t* v;
  float* o;           // [sq][heads_q][128]
  float* m_state;     // [heads_q][sq] (null: not kept; only with init and finalize)
  float* l_state;
  float* lse;         // [heads_q][sq] or null
  int64_t sq;
  int32_t heads_q, heads_kv, heads_per_item;
  float scale;
  int32_t init, finalize;
  const int64_t* chunk_begin;  // key-row bounds of the KV chunks
  const int32_t* arrival;
  const int32_t* resident;
  int32_t num_chunks;
  // Head-parallel attention: the queries arrive with the keys.  items[it] is
  // the plan tile (i * heads_q + h, h the first head of the item's group,
  // tile_m = the item's query rows) taken it-th; the item waits for the chunks
  // dep_idx[dep_ptr[t] ..) holding its query rows before it reads them.  Null
  // items: ring attention (queries resident, items head-group-major).
  const int32_t* items;
  int32_t num_items;
  const int64_t* dep_ptr;
  const int32_t* dep_idx;
  const uint32_t* flags;
  uint32_t* hdr;
  CounterArrays cnt;
  uint64_t timeout_ticks;
  int32_t nxcd;
  int32_t wait_chunks;
  int32_t copy_blocks;
  int32_t colocated;
  CopyArgs copy;
};

}  // namespace syncov
