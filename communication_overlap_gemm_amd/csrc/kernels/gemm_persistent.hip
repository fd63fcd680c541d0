// Persistent bf16 MFMA GEMM for gfx950 whose tile traversal follows a chunk
// plan: in AG mode every tile first waits for the ready flags of the chunks of
// A it reads; in RS mode every stored tile counts toward the chunks of C it
// wrote and the last one raises the chunk's done flag.
//
// Method: Syncopate summary page, "Core method" (paper sec. 5, 5.2, Fig. 6):
// one fused kernel; the chunk-tile dependency graph tells each tile which
// chunks it consumes or produces; waits are inserted before consumption; the
// tile scheduler visits chunks in communication order.  Entwine abstract:
// tiles are ordered so output is produced for communication at a steady pace.
//
// gfx950 design (not the pages' Hopper/Triton design):
//  * A grid of wave64s per workgroup (2x2, or 2x4 for 256x256 tiles: two
//    waves per SIMD); each wave owns a block of C built from
//    v_mfma_f32_32x32x16_bf16 (fp32 accumulate).
//  * K advances 64 at a time through a ring of LDS stages filled by
//    direct-to-LDS buffer loads (no staging registers), one barrier per stage.
//  * Operands are read from a per-tile buffer base (32-bit offsets; reads
//    past the end return zero, so ragged M/N need no branches).
//  * A (and B stored [n][k]) sit k-contiguous in LDS, one ds_read_b128 per
//    fragment; B stored [k][n] sits as it is in memory and is turned into
//    k-contiguous fragments by gfx950's transposing LDS reads.  16-byte XOR
//    swizzles keep both kinds of read free of bank conflicts.
//  * The epilogue stages row strips of the accumulators through LDS and
//    writes C with 16-byte buffer stores, rows past M dropped by the hardware.
//  * One workgroup per CU (two for 128x128) walks the plan's tile order with
//    a static stride; slots are remapped so that each XCD takes consecutive
//    tiles of the order.
#include <type_traits>
#include <utility>

#include "copy_role.hpp"
#include "device_common.hpp"
#include "launch_args.hpp"

namespace syncov {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));


// Raw buffer resource over [base, base + bytes); word 3 selects 32-bit data
// format as gfx9 raw buffer accesses expect.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Cache policy of the output stores (C and the send slots): SC1, device
// scope.  No tile of the launch reads them back, and stored with device scope
// they reach memory during the launch instead of sitting dirty in the XCD's
// L2 until the launch ends and its caches are written back (measured: C
// stores with the default policy left 3-10 us of write-back at the end of
// the call, most for GEMM-RS, whose C is 134 MB).
constexpr int kOutputStorePolicy = 16;


// Epilogue.  Accumulator element e of a 32x32 block sits at row
// 8*(e/4) + 4*(lane/32) + e%4, column lane%32.  Each wave writes one 32-row
// strip at a time into its own LDS region (row-major, padded pitch), then
// reads it back 16 bytes per lane and stores whole rows with buffer stores
// (rows past M fall outside num_records and are dropped).
// WGM x WGN waves, each owning a (TM/WGM) x (TN/WGN) block; RPP staged rows
// per pass (32, or 16 when the LDS ring cannot hold every wave's 32-row strip).
// 16 bytes of fp32 C plus 16 bytes of incoming fp32 partials, element-wise.
__device__ __forceinline__ u32x4_t add_partials(u32x4_t c, u32x4_t p) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(__uint_as_float(c[i]) + __uint_as_float(p[i]));
  return r;
}

// PUSH (GEMM-RS instances): with push_row0 >= 0 the tile's rows also go to
// staging from row push_row0 on (its send slot; the tile lies in one chunk).
template <int TM, int TN, int CT, int WGM, int WGN, int RPP, bool PUSH = false>
__device__ __forceinline__ void store_tile_w(const GemmArgs& a,
                                             const f32x16_t (&acc)[TM / WGM / 32][TN / WGN / 32], char* lds,
                                             int64_t m0, int64_t n0, int rows_valid, int cols_valid, int wave,
                                             int lane, int64_t push_row0 = -1) {
  constexpr int WM = TM / WGM, WN = TN / WGN, MI = WM / 32, NI = WN / 32;
  constexpr int ES = CT == 0 ? 4 : 2;
  constexpr int SP = WN + 32 / ES;   // staged strip pitch (elements), +32 B
  constexpr int LPR = WN * ES / 16;  // lanes per staged row
  constexpr int RPI = 64 / LPR;      // rows per store instruction
  static_assert(RPP == 32 || RPP == 16, "rows per pass");
  const int wm = wave / WGN, wn = wave % WGN;
  char* const stage = lds + wave * RPP * SP * ES;
  const int rr = lane / LPR, rc = (lane % LPR) * (16 / ES);
  const bool col_ok = wn * WN + rc < cols_valid;
  const int64_t N = a.N;
  const int row_bytes = static_cast<int>(N) * ES;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int h = 0; h < 32 / RPP; ++h) {
      const int strip = wm * WM + i * 32 + h * RPP;  // first tile row of this pass
      const int rows_left = rows_valid - strip;
      const bool push = PUSH && push_row0 >= 0;
      // reduce-scatter step (fp32 C): this pass's incoming partials are loaded
      // first, so that their latency overlaps the staging through LDS (rows
      // past M lie outside the resource and read as zero)
      const bool reduce = CT == 0 && push && a.partials;
      [[maybe_unused]] const __amdgpu_buffer_rsrc_t ps =
          make_rsrc(static_cast<const char*>(reduce ? a.partials : a.C) + ((m0 + strip) * N + n0 + wn * WN) * ES,
                    reduce && rows_left > 0 ? static_cast<int64_t>(rows_left) * row_bytes : 0);
      [[maybe_unused]] u32x4_t pv[PUSH && CT == 0 ? RPP / RPI : 1];
      if constexpr (PUSH && CT == 0) {
        if (reduce && col_ok) {
#pragma unroll
          for (int it = 0; it < RPP / RPI; ++it)
            pv[it] = buf_load_b128(ps, static_cast<uint32_t>((it * RPI + rr) * row_bytes + rc * ES));
        }
      }
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3) - h * RPP, c = j * 32 + (lane & 31);
          if (RPP == 32 || (e >> 3) == h) {  // accumulator rows 0-15 hold e < 8, rows 16-31 e >= 8
            if constexpr (CT == 0)
              *reinterpret_cast<float*>(stage + (r * SP + c) * ES) = acc[i][j][e];
            else
              *reinterpret_cast<uint16_t*>(stage + (r * SP + c) * ES) = f32_to_bf16_rne(acc[i][j][e]);
          }
        }
      __syncthreads();
      // RS with a send slot may leave C unwritten (C null): its stores then
      // fall outside a zero-record resource and are dropped
      const bool c_out = !PUSH || a.C != nullptr;
      const __amdgpu_buffer_rsrc_t cs =
          make_rsrc(static_cast<char*>(c_out ? a.C : a.staging) + ((m0 + strip) * N + n0 + wn * WN) * ES,
                    c_out && rows_left > 0 ? static_cast<int64_t>(rows_left) * row_bytes : 0);
      [[maybe_unused]] const __amdgpu_buffer_rsrc_t ss =
          make_rsrc(static_cast<char*>(push ? a.staging : a.C) + ((push_row0 + strip) * N + n0 + wn * WN) * ES,
                    push && rows_left > 0 ? static_cast<int64_t>(rows_left) * row_bytes : 0);
#pragma unroll
      for (int it = 0; it < RPP / RPI; ++it) {
        const int r = it * RPI + rr;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + (r * SP + rc) * ES);
        if (col_ok) {
          __builtin_amdgcn_raw_buffer_store_b128(v, cs, static_cast<uint32_t>(r * row_bytes + rc * ES), 0,
                                                 kOutputStorePolicy);
          if constexpr (PUSH) {
            if (push) {
              const uint32_t off = static_cast<uint32_t>(r * row_bytes + rc * ES);
              u32x4_t w = v;
              if constexpr (CT == 0) {
                if (reduce) w = add_partials(v, pv[it]);
              }
              __builtin_amdgcn_raw_buffer_store_b128(w, ss, off, 0, kOutputStorePolicy);
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

// GEMM-RS completion of tile t: every wave's C stores have reached the L2;
// then one agent-scope release (a write-back of this XCD's L2, covering all
// the waves) before the tile is counted toward each chunk it wrote, with
// relaxed counts; the last tile of a chunk acquires the other tiles' releases
// and raises the chunk's done flag.
__device__ __forceinline__ void publish_rs_tile(const GemmArgs& a, int32_t t, uint32_t epoch, int tid) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0) {
    release_agent();
    for (int64_t e = a.dep_ptr[t]; e < a.dep_ptr[t + 1]; ++e) {
      const int32_t c = a.dep_idx[e];
      const uint32_t old = add_relaxed_agent(a.cnt.counters + c, 1u);
      if (old + 1u == static_cast<uint32_t>(a.tiles_in[c])) {
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");  // the chunk's other tiles, released onward with it
        st_relaxed_agent(a.cnt.counters + c, 0u);  // every tile of c has counted: ready for the next call
        if (a.trace_chunks) a.trace_chunks[2 * c] = wall_clock64();
        st_relaxed_agent(a.flags + c, epoch);
        if (a.push_rows) {  // the tiles also wrote the chunk into its send slot
          if (a.trace_chunks) a.trace_chunks[2 * c + 1] = wall_clock64();
          st_relaxed_agent(a.sent + c, epoch);
        }
      }
    }
  }
}

// GEMM-AR share, all-gather half: workgroups walk the items in ring
// all-gather order (dedicated copy workgroups from the start, compute
// workgroups once their tiles are stored); for each, thread 0 waits until the
// item's gate chunk is done (the rank's own chunk with the same sub-chunk
// index: in a ring all-reduce the all-gather of a sub-chunk follows the end
// of its reduce-scatter on every rank), then the workgroup copies share
// `rank` of `count` of the item's rows.  Nothing is published per item: the
// call's end covers them.
template <int THREADS>
__device__ void ar_gather(const GemmArgs& a, int32_t rank, int32_t count, uint32_t epoch) {
  __shared__ int32_t s_ok;
  for (int32_t i = 0; i < a.ar_count; ++i) {
    const int64_t* it = a.ar_items + 5 * i;
    if (threadIdx.x == 0) {
      const bool ok = wait_flag(a.flags, static_cast<int32_t>(it[4]), epoch, a.hdr, a.timeout_ticks);
      if (ok) acquire_agent();
      s_ok = ok;
    }
    __syncthreads();
    const int ok = s_ok;
    __syncthreads();
    if (!ok) return;  // the call failed: the error is recorded
    const int64_t granules = it[3] * a.ar_row_bytes / 16;
    const int64_t lo = granules * rank / count * 16, hi = granules * (rank + 1) / count * 16;
    const char* const src = it[0] ? a.ar_src[1] : a.ar_src[0];
    copy_range<THREADS, true>(src + it[1] * a.ar_row_bytes, a.ar_out + it[2] * a.ar_row_bytes, lo, hi);
  }
}

// AG: lane 0 waits for every chunk tile t reads that was not in place before
// the call, then one acquire.  Returns false (uniformly) when a wait gave up,
// so the tile is skipped.
// Thread 0 waits for flags[c * stride + slice] of every chunk c tile t reads
// (resident chunks excepted), then makes their data visible to this CU.
// False if one never arrived (timeout or an error of the call).
__device__ __forceinline__ bool wait_tile_deps(const GemmArgs& a, int32_t t, uint32_t epoch, const uint32_t* flags,
                                               int32_t stride, int32_t slice) {
  bool ok = true, waited = false;
  for (int64_t e = a.dep_ptr[t]; ok && e < a.dep_ptr[t + 1]; ++e) {
    const int32_t c = a.dep_idx[e];
    if (a.resident[c]) continue;
    // reads flags[c * stride + slice]; a timeout names chunk c
    ok = wait_flag(flags + c * (stride - 1) + slice, c, epoch, a.hdr, a.timeout_ticks);
    waited = true;
  }
  if (ok && waited) acquire_agent();
  return ok;
}

// Tile start: every chunk of tile t (with a K-sliced copy, their slice 0).
__device__ __forceinline__ bool wait_tile_chunks(const GemmArgs& a, int32_t t, uint32_t epoch, int tid,
                                                 int32_t* s_skip) {
  if (!a.wait_chunks) return true;
  if (tid == 0) {
    const bool ok = a.kslices > 1 ? wait_tile_deps(a, t, epoch, a.slice_flags, kMaxSlices, 0)
                                  : wait_tile_deps(a, t, epoch, a.flags, 1, 0);
    *s_skip = ok ? 0 : 1;
  }
  __syncthreads();
  const int skip = *s_skip;
  __syncthreads();
  return !skip;
}

// Workgroups per CU a tile shape is launched with: 128x128 runs two per CU
// (its LDS ring and registers fit twice), larger tiles one.  The kernels
// declare it in their launch bounds, so the compiler holds each instance to
// that register budget; the runtime checks the resulting occupancy before a
// launch whose workgroups must all be resident at once.
template <int TM, int TN> constexpr int kWgPerCu = (TM == 128 && TN == 128) ? 2 : 1;

// ---------------------------------------------------------------------------
// The GEMM kernel (gemm_dma), for B stored [n][k] or [k][n].
//  * K advances TK at a time through an NS-stage LDS ring.  Loads go straight
//    from HBM to LDS (buffer_load ... lds, 16 bytes per lane): no staging
//    registers, no ds_write pass.  A wave's load fills 1 KB of LDS, lane l at
//    byte 16*l; the 16-byte-slot swizzle is applied by choosing which global
//    slot each lane fetches.
//  * The prologue fills every slot; right after the barrier that publishes
//    stage kt+1 (which also proves every wave is done with stage kt), the load
//    of stage kt+NS goes into stage kt's slot, so a load has NS-1 stages of
//    MFMA work to land in.
//  * Two register sets of fragments (one k16 step each) alternate: the MFMAs
//    of one step are interleaved with the LDS reads of the next step (for the
//    last step of a stage, the first step of the next stage, read after that
//    stage's barrier), so LDS latency hides behind the MFMA pipe.
//  * Fragment reads are inline asm: the compiler's wait insertion cannot tell
//    them apart from the in-flight LDS-DMA writes and would put vmcnt(0) in
//    front of each; the kernel waits explicitly instead (lgkmcnt before use,
//    vmcnt + raw barrier per stage).
// ---------------------------------------------------------------------------

// s_waitcnt with vmcnt = n and the other counters unconstrained (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// s_waitcnt with lgkmcnt = n and the other counters unconstrained.
template <int n>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(n >= 0 && n < 16, "lgkmcnt");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (n << 8) | (3 << 14));
}

// (The LDS-address-space casts and the asm are device-only: a host pass that
// sees them drops the kernel's host stub, so they sit behind the device guard.)
__device__ __forceinline__ bf16x8_t lds_read_b128(uint32_t addr) {
  bf16x8_t r{};
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
#endif
  return r;
}
// The same with a constant byte offset in the instruction's 16-bit field.
template <int OFF>
__device__ __forceinline__ bf16x8_t lds_read_b128_at(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  bf16x8_t r{};
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF));
#endif
  return r;
}

// gfx950's transposing LDS read of 16-bit elements, with a constant byte
// offset.  Each lane names 8 bytes (four elements); within every group of 16
// lanes, lane i receives element i % 4 of the lanes i / 4, i / 4 + 4,
// i / 4 + 8 and i / 4 + 12 of its group, in that order.  When source lane r
// points at row (r / 4) and columns 4 (r % 4) .. 4 (r % 4) + 3 of a row-major
// 4 x 16 block, destination lane i therefore holds column i, rows 0..3.
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr16_at(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2_t r{};
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF));
#endif
  return r;
}

// Calls f(std::integral_constant<int, X>{}) for X = 0 .. N-1 in order, so X
// can name a template argument or an instruction's immediate.
template <typename F, int... X>
__device__ __forceinline__ void unroll_each(F&& f, std::integer_sequence<int, X...>) {
  (f(std::integral_constant<int, X>{}), ...);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
#else
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
#endif
}

// 16 bytes per lane from buffer offset voff straight into LDS at lds + 16*lane
// (lds wave-uniform).
__device__ __forceinline__ void dma_load_16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16, voff, 0, 0, 0);
#endif
}

// Slot swizzle for rows of SLOTS 16-byte slots.  A fragment read has lanes
// 0..15 (and 16..31) on 16 consecutive rows at one logical slot; the XOR term
// spreads them over distinct 16-byte bank groups whether the LDS serves 8 or
// 16 lanes of a 128-bit read per cycle.  It uses row bits 0..3 only, so a
// fragment's 32-aligned base row does not change it.
template <int SLOTS>
__device__ __forceinline__ int rswz(int row, int slot) {
  if constexpr (SLOTS == 4)
    return slot ^ (((row >> 1) & 3) ^ ((row >> 3) & 1));
  else
    return slot ^ ((row & 7) ^ ((row >> 3) & 1));
}

// B stored [k][n] (BKN): a stage holds TK rows of TN columns, and 16-byte slot
// s of row k sits at slot s ^ 4 kn_swz(k).  The swizzle term uses row bits 0,
// 1 and (with 32 slots per row) 3: the rows that one transposing read touches
// (four consecutive rows per 32 lanes, two such sets 8 rows apart) then fall
// on distinct 64-byte bank groups, and within a k16 step the term depends only
// on the lane, so every read of a fragment is one base plus an immediate.
template <int TN>
__device__ __forceinline__ int kn_swz(int k) {
  if constexpr (TN >= 256)
    return (k & 3) | (((k >> 3) & 1) << 2);
  else
    return k & 3;
}

// FEED: how a stage reaches the LDS.  0: direct-to-LDS loads, all issued
// right after the barrier that frees the slot; F > 0: direct-to-LDS loads
// spread over the first F k16 steps after that barrier, between the MFMAs;
// kFeedReg: through registers (global loads one stage ahead, written to the
// free slot with ds_write between the MFMAs).
constexpr int kFeedReg = -1;

template <int TM, int TN, int CT, bool RS, int TK, int NS, int WGM, int WGN, int FEED, bool BKN>
__global__ __launch_bounds__(64 * WGM * WGN, (kWgPerCu<TM, TN>)) void gemm_dma(GemmArgs a) {
  constexpr int NW = WGM * WGN, THREADS = 64 * NW;  // waves, as a WGM x WGN grid over the tile
  constexpr int WM = TM / WGM, WN = TN / WGN;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int ROWB = TK * 2;                      // bytes per LDS row
  constexpr int SLOTS = ROWB / 16;
  constexpr int RPL = 1024 / ROWB;                  // rows per 1 KB wave load
  constexpr int KS = TK / 16;                       // k16 steps per stage
  constexpr int A_BYTES = TM * ROWB, B_BYTES = TN * ROWB;
  constexpr int ROWB_B = BKN ? TN * 2 : ROWB;       // bytes per LDS row of B
  constexpr int RPLB = 1024 / ROWB_B;               // rows of B per 1 KB wave load
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_LD = A_BYTES / 1024 / NW;         // 1 KB wave loads per wave per stage
  constexpr int B_LD = B_BYTES / 1024 / NW;
  constexpr int LPW = A_LD + B_LD;                  // loads per wave per stage
  constexpr int NFRAG = MI + NI;                    // fragments per k16 step: A frags, then B frags
  constexpr int NB = BKN ? 2 * NI : NI;             // B reads per k16 step (two transposing halves per fragment)
  constexpr int NRD = MI + NB;                      // LDS reads per k16 step
  static_assert(WM % 32 == 0 && WN % 32 == 0 && A_LD >= 1 && B_LD >= 1 && A_LD * NW * 1024 == A_BYTES &&
                B_LD * NW * 1024 == B_BYTES, "tile");
  static_assert((SLOTS == 4 || SLOTS == 8) && KS % 2 == 0, "stage depth");
  static_assert(NS >= 2 && (NS - 2) * LPW < 64, "ring");
  static_assert(NFRAG <= MI * NI && (!BKN || (WN == 64 && (TN == 128 || TN == 256))), "reads per MFMA slot");
  constexpr bool REG = FEED == kFeedReg, SPREAD = FEED > 0;
  constexpr int PPW = LPW / KS;  // REG: staged loads written (and refetched) per k16 step
  static_assert(!REG || (!BKN && NS == 2 && LPW % KS == 0 && NFRAG + PPW <= MI * NI && SLOTS == 8 && A_LD == B_LD &&
                         A_LD % 2 == 0),
                "register staging");
  constexpr int LPG = SPREAD ? LPW / FEED : 1;          // SPREAD: loads per k16 step
  constexpr int GAP = SPREAD ? MI * NI / LPG : 1;       // SPREAD: MFMAs between loads
  static_assert(FEED >= kFeedReg && (!SPREAD || (NS == 2 && FEED <= KS && LPW % FEED == 0 && LPG <= MI * NI &&
                                                 MI * NI % LPG == 0)),
                "spread feed");
  constexpr int ES = CT == 0 ? 4 : 2;
  constexpr int RPP = NW * 32 * (WN + 32 / ES) * ES <= NS * STAGE ? 32 : 16;  // epilogue rows per pass
  static_assert(NW * RPP * (WN + 32 / ES) * ES <= NS * STAGE, "epilogue staging must fit the LDS ring");

  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];
  __shared__ int32_t s_skip;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const uint32_t epoch = call_epoch(a.hdr);
  const int64_t M = a.M, N = a.N, K = a.K;
  const int nk = static_cast<int>(K / TK);

  // per-lane global offsets (bytes, relative to the tile's first row at k0)
  uint32_t a_off[A_LD], b_off[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int row = (wave * A_LD + i) * RPL + lane / SLOTS;
    a_off[i] = static_cast<uint32_t>((row * K + rswz<SLOTS>(row, lane % SLOTS) * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    if constexpr (BKN) {  // row k of the stage, physical slot lane % (TN / 8)
      const int k = (wave * B_LD + i) * RPLB + lane / (TN / 8);
      b_off[i] = static_cast<uint32_t>((k * N + ((lane % (TN / 8)) ^ (4 * kn_swz<TN>(k))) * 8) * 2);
    } else {
      const int row = (wave * B_LD + i) * RPL + lane / SLOTS;
      b_off[i] = static_cast<uint32_t>((row * K + rswz<SLOTS>(row, lane % SLOTS) * 8) * 2);
    }
  }
  // REG: A and B rows are indexed alike, and with 8 slots per row the swizzle
  // depends only on bit 3 of the row, i.e. on the parity of the load index:
  // load i's lane offset is reg_off[i % 2] from a buffer that starts
  // (i - i % 2) * RPL rows further (in the base, not the scalar offset, which
  // the range check of a raw buffer leaves out)
  uint32_t reg_off[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = (wave * A_LD + p) * RPL + lane / SLOTS;  // swizzled as the direct-to-LDS loads
    reg_off[p] = static_cast<uint32_t>(((p * RPL + lane / SLOTS) * K + rswz<SLOTS>(row, lane % SLOTS) * 8) * 2);
  }
  // per-lane LDS offset of a fragment read for k16 step kk (rows are 32-aligned,
  // so the swizzle depends only on the lane's row within the block)
  // plus the wave's first A row; its B rows sit a wave-uniform distance
  // further (b_delta), and the fragment's row block is the read's immediate
  const int frow = lane & 31;
  uint32_t frag_off[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    frag_off[kk] = (wm * WM + frow) * ROWB + rswz<SLOTS>(frow, kk * 2 + (lane >> 5)) * 16;
  const uint32_t b_delta = static_cast<uint32_t>(A_BYTES + (wn * WN - wm * WM) * ROWB);
  // BKN: per-lane offset in a stage of fragment j's first transposing read at
  // k16 step 0.  Lane group g = lane / 16 reads rows 8 (g / 2) + r / 4 (r =
  // lane % 16) and columns 16 (g % 2) + 4 (r % 4) .. + 3 of the fragment's 32,
  // so lane l receives column l % 32 at rows 8 (l / 32) .. + 3, the B-operand
  // layout of the 32x32x16 MFMA; the second half is 4 rows further, the k16
  // step 16 rows further (immediates).
  uint32_t kn_off[BKN ? NI : 1];
  if constexpr (BKN) {
    const int g = lane >> 4, r = lane & 15, k = 8 * (g >> 1) + (r >> 2);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = wn * WN + 32 * j + 16 * (g & 1) + 4 * (r & 3);
      kn_off[j] = static_cast<uint32_t>(A_BYTES + k * ROWB_B + (((n >> 3) ^ (4 * kn_swz<TN>(k))) << 4) + 8 * (r & 1));
    }
  }

  if (static_cast<int32_t>(blockIdx.x) < a.copy_blocks) {
    if constexpr (RS && CT == 0) {  // GEMM-AR is fp32 only
      if (a.ar_count) {  // every workgroup of the launch takes a share of each item
        ar_gather<THREADS>(a, blockIdx.x, gridDim.x, epoch);
        end_call(a.hdr, epoch, a.cnt);
        return;
      }
    }
    copy_role<THREADS>(a.copy, blockIdx.x, a.copy_blocks, epoch);
    end_call(a.hdr, epoch, a.cnt);
    return;
  }
  const int32_t gb = blockIdx.x - a.copy_blocks, gn = gridDim.x - a.copy_blocks;
  if (!RS && a.colocated) {  // co-located: pull this workgroup's share first
    if (a.copy.teams > 1)
      copy_role<THREADS>(a.copy, gb, gn, epoch);  // teams: each chunk published as soon as its team is done
    else
      copy_role<THREADS, true>(a.copy, gb, gn, epoch);  // one publication for all chunks
  }
  if constexpr (!RS) {
    if (a.lead_ptr) lead_slice<THREADS>(a.copy, a.lead_ptr, a.lead_item, gb, epoch);  // slice 0 of the first tile's chunk
  }
  const int32_t tg = (a.tile_grid > 0 && a.tile_grid < gn) ? a.tile_grid : gn;  // workgroups that take tiles
  const int32_t slot0 = gb < tg ? xcd_slot(gb, tg, a.nxcd) : a.num_tiles;
  for (int32_t p = slot0; p < a.num_tiles; p += tg) {
    const int32_t t = a.order[p];
    const int32_t ti = t / a.tiles_n, tj = t - ti * a.tiles_n;
    const int64_t m0 = static_cast<int64_t>(ti) * TM, n0 = static_cast<int64_t>(tj) * TN;
    const int rows_valid = static_cast<int>((M - m0) < TM ? (M - m0) : TM);
    const int cols_valid = static_cast<int>((N - n0) < TN ? (N - n0) : TN);
    if (a.trace_tiles && tid == 0) {
      a.trace_tiles[4 * t] = wall_clock64();
      a.trace_tiles[4 * t + 3] = (static_cast<uint64_t>(xcc_id()) << 32) | static_cast<uint32_t>(p);
    }
    if constexpr (!RS) {
      if (!wait_tile_chunks(a, t, epoch, tid, &s_skip)) continue;  // a chunk never arrived: tile left untouched
    }
    if (a.trace_tiles && tid == 0) a.trace_tiles[4 * t + 1] = wall_clock64();
    const uint16_t* const a_tile = a.A + m0 * K;
    const uint16_t* const b_tile = BKN ? a.B + n0 : a.B + n0 * K;
    // B's buffer for the stage at k0: its rows (B [n][k]: the tile's columns
    // from k0; B [k][n]: rows k0.. of B from column n0, to the end of B)
    auto b_rsrc = [&](int64_t k0, bool live) {
      if constexpr (BKN)
        return make_rsrc(b_tile + k0 * N, live ? (K - k0) * N * 2 - n0 * 2 : 0);
      else
        return make_rsrc(b_tile + k0, live ? static_cast<int64_t>(cols_valid) * K * 2 - k0 * 2 : 0);
    };

    auto issue = [&](int kt) {  // loads of k-step kt into slot kt % NS
      char* st = smem + (kt % NS) * STAGE;
      const int64_t k0 = static_cast<int64_t>(kt) * TK;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_tile + k0, static_cast<int64_t>(rows_valid) * K * 2 - k0 * 2);
      const __amdgpu_buffer_rsrc_t rb = b_rsrc(k0, true);
#pragma unroll
      for (int i = 0; i < A_LD; ++i) dma_load_16(ra, st + (wave * A_LD + i) * 1024, a_off[i]);
#pragma unroll
      for (int i = 0; i < B_LD; ++i) dma_load_16(rb, st + A_BYTES + (wave * B_LD + i) * 1024, b_off[i]);
    };
    // stage kt is in LDS for every wave; the loads of later stages (at most
    // NS - 2 of them) may still be in flight
    auto landed = [&](int kt) {
      const int later = nk - 1 - kt < NS - 2 ? nk - 1 - kt : NS - 2;
      if constexpr (NS >= 4) {
        if (later >= 2) {
          wait_vmcnt<2 * LPW>();
        } else if (later == 1) {
          wait_vmcnt<LPW>();
        } else {
          wait_vmcnt<0>();
        }
      } else if constexpr (NS == 3) {
        if (later >= 1)
          wait_vmcnt<LPW>();
        else
          wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    // REG: load `i` of stage kt (A loads first, then B) goes through a
    // register; a stage past the last is a zero-length buffer (no access, the
    // register reads zero), so the loads need no branch
    u32x4_t rv[REG ? LPW : 1];
    auto fetch = [&](int kt, int i) {
      const bool live = kt < nk;
      const int64_t k0 = static_cast<int64_t>(live ? kt : 0) * TK;
      const int li = i < A_LD ? i : i - A_LD;
      const int64_t r0 = static_cast<int64_t>(wave * A_LD + li - li % 2) * RPL;  // the buffer's first row
      const __amdgpu_buffer_rsrc_t r =
          i < A_LD ? make_rsrc(a_tile + r0 * K + k0, live ? (rows_valid - r0) * K * 2 - k0 * 2 : 0)
                   : make_rsrc(b_tile + r0 * K + k0, live ? (cols_valid - r0) * K * 2 - k0 * 2 : 0);
      rv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, reg_off[li % 2], 0, 0));
    };
    // REG: register `i` into stage kt's slot, at the place its direct-to-LDS
    // load would have written (lane l's 16 bytes at 16 l of the wave's 1 KB)
    auto put = [&](int kt, int i) {
      char* const st = smem + (kt % NS) * STAGE;
      char* const dst = i < A_LD ? st + (wave * A_LD + i) * 1024 : st + A_BYTES + (wave * B_LD + i - A_LD) * 1024;
      *reinterpret_cast<u32x4_t*>(dst + lane * 16) = rv[i];
    };
    // SPREAD: direct-to-LDS load `i` of stage kt; past the last stage a
    // zero-length buffer (nothing is read; zeros land in the free slot)
    auto dma_one = [&](int kt, int i) {
      char* const st = smem + (kt % NS) * STAGE;
      const bool live = kt < nk;
      const int64_t k0 = static_cast<int64_t>(live ? kt : 0) * TK;
      if (i < A_LD)
        dma_load_16(make_rsrc(a_tile + k0, live ? static_cast<int64_t>(rows_valid) * K * 2 - k0 * 2 : 0),
                    st + (wave * A_LD + i) * 1024, a_off[i]);
      else
        dma_load_16(b_rsrc(k0, live), st + A_BYTES + (wave * B_LD + i - A_LD) * 1024, b_off[i - A_LD]);
    };

    f32x16_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = f32x16_t{};

    __syncthreads();  // the previous tile's epilogue is done with the LDS
    if constexpr (REG) {
      // stage 0 into its slot, stage 1 into the registers, then the first part
      // of stage 1 into its slot with stage 2's loads behind it (the rest of
      // stage 1 is written during stage 0's first k16 steps)
#pragma unroll
      for (int i = 0; i < LPW; ++i) fetch(0, i);
#pragma unroll
      for (int i = 0; i < LPW; ++i) put(0, i);
#pragma unroll
      for (int i = 0; i < LPW; ++i) fetch(1, i);
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        put(1, i);
        fetch(2, i);
      }
    } else if constexpr (SPREAD) {
      // stage 0, then the first part of stage 1 (its other parts go out
      // during stage 0's first k16 steps)
      if (0 < nk) issue(0);
#pragma unroll
      for (int i = 0; i < LPG; ++i) dma_one(1, i);
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (s < nk) issue(s);
    }

    const uint32_t ring = lds_addr(smem);
    // One k16 step's fragments: A blocks, then B (BKN: two transposing halves
    // per block, rows 0..3 and 4..7 of each lane's eight)
    using BFrag = std::conditional_t<BKN, u32x2_t, bf16x8_t>;
    struct Frags {
      bf16x8_t a[MI];
      BFrag b[NB];
    };
    struct Bases {
      uint32_t a, b, kn[BKN ? NI : 1];
    };
    auto bases = [&](uint32_t nst, int nkk) {
      Bases q;
      q.a = nst + frag_off[nkk];
      q.b = q.a + b_delta;
      if constexpr (BKN) {
#pragma unroll
        for (int j = 0; j < NI; ++j) q.kn[j] = nst + nkk * (16 * ROWB_B) + kn_off[j];
      }
      return q;
    };
    // read R of one k16 step (A first, then B) into f
    auto read_one = [&](Frags& f, const Bases& q, auto rc) {
      constexpr int R = decltype(rc)::value;
      if constexpr (R < MI)
        f.a[R] = lds_read_b128_at<R * 32 * ROWB>(q.a);
      else if constexpr (BKN)
        f.b[R - MI] = lds_read_tr16_at<((R - MI) % 2) * 4 * ROWB_B>(q.kn[(R - MI) / 2]);
      else
        f.b[R - MI] = lds_read_b128_at<(R - MI) * 32 * ROWB>(q.b);
    };
    // B operand of fragment j
    auto b_op = [&](const Frags& f, auto jc) -> bf16x8_t {
      constexpr int j = decltype(jc)::value;
      if constexpr (BKN)
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(f.b[2 * j], f.b[2 * j + 1], 0, 1, 2, 3));
      else
        return f.b[j];
    };
    // MFMA slot after which read R is issued: one read per slot while they
    // fit, else spread evenly
    constexpr auto read_slot = [](int r) { return NRD <= MI * NI ? r : r * (MI * NI) / NRD; };
    // MFMAs on one fragment set, interleaved with the reads of the next set.
    // The reads are unconditional: a read whose result the compiler might
    // discard would let it emit select/copy code on registers that an
    // in-flight asm read is still going to write.
    // REG: after the reads, part `part` of the staged registers is written
    // into stage pst's slot and refetched with stage pst + 1; the wait then
    // leaves those PPW writes in flight (LDS operations complete in order, so
    // the reads before them have landed).  SPREAD: part `part` (< FEED) of
    // stage pst's direct-to-LDS loads, one every GAP MFMAs.
    auto mma = [&](Frags& cur, Frags& nxt, uint32_t nst, int nkk, int pst, int part) {
      const Bases q = bases(nst, nkk);
      unroll_each(
          [&](auto xc) {
            constexpr int x = decltype(xc)::value, i = x / NI, j = x % NI;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[i], b_op(cur, std::integral_constant<int, j>{}),
                                                                acc[i][j], 0, 0, 0);
            unroll_each(
                [&](auto rc) {
                  if constexpr (read_slot(decltype(rc)::value) == x) read_one(nxt, q, rc);
                },
                std::make_integer_sequence<int, NRD>{});
            if constexpr (REG && x >= NFRAG && x < NFRAG + PPW) {
              put(pst, part * PPW + x - NFRAG);
              fetch(pst + 1, part * PPW + x - NFRAG);
            }
            if constexpr (SPREAD && x % GAP == 0) {
              if (part < FEED) dma_one(pst, part * LPG + x / GAP);
            }
            __builtin_amdgcn_sched_barrier(0);
          },
          std::make_integer_sequence<int, MI * NI>{});
      if constexpr (REG)
        wait_lgkmcnt<PPW>();
      else
        wait_lgkmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
    };

    // K-sliced copy: the first loads of stage s go out right after the
    // barrier that ends stage s - LEAD, so thread 0 waits for slice h of the
    // tile's chunks just before the barrier that precedes the first loads of
    // slice h (its first stage is h * nk / kslices; slice 0 was waited for at
    // the tile start, and every slice spans more stages than the prologue
    // loads).  A slice that never arrives leaves the tile unstored (s_skip),
    // as at the start.
    constexpr int LEAD = REG ? 3 : (SPREAD ? 2 : NS);
    const bool sliced = !RS && a.wait_chunks && a.kslices > 1;
    int next_h = 1, next_stage = sliced ? nk / a.kslices : nk + LEAD;
    auto wait_slice = [&](int kt) {
      if (kt + LEAD == next_stage) {
        if (tid == 0 && !wait_tile_deps(a, t, epoch, a.slice_flags, kMaxSlices, next_h)) s_skip = 1;
        ++next_h;
        next_stage = next_h < a.kslices ? next_h * nk / a.kslices : nk + LEAD;
      }
    };

    Frags fp, fq;
    if constexpr (REG) {
      wait_lgkmcnt<0>();
      __builtin_amdgcn_s_barrier();  // stage 0 is in its slot for every wave
      __builtin_amdgcn_sched_barrier(0);
    } else {
      landed(0);
    }
    {
      const Bases q = bases(ring, 0);
      unroll_each([&](auto rc) { read_one(fp, q, rc); }, std::make_integer_sequence<int, NRD>{});
    }
    wait_lgkmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < nk; ++kt) {
      const uint32_t st = ring + (kt % NS) * STAGE;
      // REG: these steps write parts 1.. of stage kt + 1 into its slot
#pragma unroll
      for (int kk = 0; kk < KS - 1; kk += 2) {
        mma(fp, fq, st, kk + 1, kt + 1, kk + 1);
        if (kk + 2 < KS) mma(fq, fp, st, kk + 2, kt + 1, kk + 2);
      }
      // last k16 step of the stage: its MFMAs read fq; the next stage's first
      // step is read into fp once that stage has landed (after the last
      // stage, a read of an idle slot whose result goes unused)
      wait_slice(kt);
      if constexpr (REG) {
        // every wave has written stage kt + 1 and read its last fragments of
        // stage kt: the one slot becomes readable, the other writable (part 0
        // of stage kt + 2 goes in during the last step)
        wait_lgkmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (SPREAD) {
        // the same after the last stage too: the zero-length loads that follow
        // write into a slot other waves may still be reading until then
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      } else if (kt + 1 < nk) {
        landed(kt + 1);
        if (kt + NS < nk) issue(kt + NS);  // into stage kt's slot, free now
      }
      mma(fq, fp, ring + ((kt + 1) % NS) * STAGE, 0, kt + 2, 0);
    }
    if constexpr (SPREAD) wait_vmcnt<0>();  // the zero-length loads after the last stage have landed
    __syncthreads();  // every wave is done reading the ring before the epilogue reuses it
    if (sliced && s_skip) continue;  // a slice never arrived: tile left untouched
    store_tile_w<TM, TN, CT, WGM, WGN, RPP, RS>(a, acc, smem, m0, n0, rows_valid, cols_valid, wave, lane,
                                                RS && a.push_rows ? a.push_rows[t] : -1);
    if constexpr (RS) publish_rs_tile(a, t, epoch, tid);
    if (a.trace_tiles && tid == 0) a.trace_tiles[4 * t + 2] = wall_clock64();
  }
  // co-located GEMM-RS: every workgroup joins the copy-out once its tiles are
  // stored, chunk by chunk in send order (the first chunks are done first)
  if (RS && a.colocated) copy_role<THREADS>(a.copy, gb, gn, epoch);
  // GEMM-AR: every compute workgroup joins the all-gather once its tiles are stored
  if constexpr (RS && CT == 0) {
    if (a.ar_count) ar_gather<THREADS>(a, blockIdx.x, gridDim.x, epoch);
  }
  end_call(a.hdr, epoch, a.cnt);
}

// Host-side launcher: picks the template instance; hipErrorInvalidValue for a
// variant that does not exist.
// K per stage, ring depth and wave grid of the direct-to-LDS GEMM, per tile:
// 64-deep stages read whole 128-byte lines per row; the ring takes what the
// LDS holds at the tile's workgroups per CU (128x128 runs two per CU); the
// 256x256 tile runs eight waves, two per SIMD, so that one wave's waits are
// covered by the other's MFMAs (measured 124 us against 137 us with four
// waves on 8192x1792x4096).  Its stage loads go out spread over the first two
// k16 steps after the barrier rather than in one burst, which keeps the
// vector-memory queue from holding up the MFMA issue (8192x1792x4096 with 32
// copy CUs: 170 us against 179 us).
template <int TM, int TN> struct DmaShape { static constexpr int TK = 64, NS = 2, WGM = 2, WGN = 2, FEED = 0; };
template <> struct DmaShape<256, 128> { static constexpr int TK = 64, NS = 3, WGM = 2, WGN = 2, FEED = 0; };
template <> struct DmaShape<256, 256> { static constexpr int TK = 64, NS = 2, WGM = 2, WGN = 4, FEED = 2; };

// With max_per_cu non-null nothing is launched: *max_per_cu receives how many
// workgroups of the chosen instance can be resident on one CU.
hipError_t launch_gemm(const GemmArgs& a, int tm, int tn, int b_layout, int c_dtype, bool rs, int grid,
                       hipStream_t stream, int* max_per_cu) {
  auto go = [&](auto kernel, int threads) -> hipError_t {
    if (max_per_cu)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(max_per_cu, reinterpret_cast<const void*>(kernel), threads,
                                                          0);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, a);
    return hipGetLastError();
  };
#define SYNC_GEMM_DMA_CASE(TM_, TN_, BL_, CT_)                                                               \
  if (tm == TM_ && tn == TN_ && b_layout == BL_ && c_dtype == CT_) {                                         \
    using S_ = DmaShape<TM_, TN_>;                                                                           \
    constexpr int threads_ = 64 * S_::WGM * S_::WGN;                                                         \
    return rs ? go(gemm_dma<TM_, TN_, CT_, true, S_::TK, S_::NS, S_::WGM, S_::WGN, S_::FEED, BL_ == 0>,      \
                   threads_)                                                                                 \
              : go(gemm_dma<TM_, TN_, CT_, false, S_::TK, S_::NS, S_::WGM, S_::WGN, S_::FEED, BL_ == 0>,     \
                   threads_);                                                                                \
  }
#define SYNC_GEMM_DMA_TILES(BL_, CT_) \
  SYNC_GEMM_DMA_CASE(256, 256, BL_, CT_) SYNC_GEMM_DMA_CASE(256, 128, BL_, CT_) SYNC_GEMM_DMA_CASE(128, 128, BL_, CT_)
  SYNC_GEMM_DMA_TILES(1, 0)
  SYNC_GEMM_DMA_TILES(1, 1)
  SYNC_GEMM_DMA_TILES(0, 0)
  SYNC_GEMM_DMA_TILES(0, 1)
#undef SYNC_GEMM_DMA_TILES
#undef SYNC_GEMM_DMA_CASE
  return hipErrorInvalidValue;
}

int gemm_wg_per_cu(int tm, int tn) {
  if (tm == 128 && tn == 128) return kWgPerCu<128, 128>;
  return 1;
}

bool gemm_variant_exists(int tm, int tn) {
  return (tm == 256 && tn == 256) || (tm == 256 && tn == 128) || (tm == 128 && tn == 128);
}

}  // namespace syncov
