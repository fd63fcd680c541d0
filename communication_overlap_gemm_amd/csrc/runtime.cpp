// Host runtime behind the C ABI in sync_overlap.h: plans with lazily uploaded
// device tables, the workspace layout, the library's streams (plain and
// CU-masked) and events, and the launch sequences of the copy backends.
//
// Call shape (Syncopate summary page, "Core method", paper sec. 5.2 and
// Fig. 7; review page, Fig. 5 caption): the communication of a plan runs
// beside one fused compute kernel and signals chunk completion through
// global-memory flags.  On one MI355X the "peers" are a second HBM region;
// the copy agent is either the SDMA engine or a copy kernel on CUs that the
// GEMM does not use.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <tuple>
#include <memory>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

#include "kernels/device_common.hpp"
#include "kernels/launch_args.hpp"
#include "planner.hpp"
#include "sdma_engine.hpp"
#include "sync_overlap.h"

namespace syncov {

hipError_t launch_gemm(const GemmArgs& a, int tm, int tn, int b_layout, int c_dtype, bool rs, int grid, hipStream_t s,
                       int* max_per_cu = nullptr);
int gemm_wg_per_cu(int tm, int tn);
bool gemm_variant_exists(int tm, int tn);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
hipError_t launch_sdma_gate(uint32_t* hdr, int64_t* gate, hipStream_t s);
hipError_t launch_sdma_join(uint32_t* hdr, const uint32_t* flags, const int32_t* arrival, const int32_t* resident,
                            int32_t num_chunks, uint64_t timeout_ticks, hipStream_t s);
hipError_t launch_ring_attn(const AttnArgs& a, int grid, hipStream_t s);
int attn_wg_per_cu();
int attn_query_block(int hg);
constexpr int64_t kAttnHeadDim = 128;

}  // namespace syncov

using namespace syncov;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

}  // namespace

namespace syncov {
// Sets the thread's last-error message (other translation units of the library).
int set_error(int code, const std::string& msg) { return fail(code, msg); }
}  // namespace syncov

namespace {

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return SYNC_EHIP;
}

#define HIP_TRY(expr)                             \
  do {                                            \
    hipError_t _e = (expr);                       \
    if (_e != hipSuccess) return hip_fail(_e, #expr); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// ---- per-device state ----------------------------------------------------
// Workspace of sync_ag_gemm_noalloc: a file-scope device array, so that the
// call allocates nothing.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, once per device
// (DeviceState::scratch), and only that address is passed to kernels.
constexpr int64_t kScratchBytes = int64_t(1) << 20;
__device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

// Per-device facts and the ring of timing events.  Every call runs on the
// caller's stream: the library creates no streams.
struct DeviceState {
  bool ready = false;
  int device = 0;
  void* scratch = nullptr;        // device address of `scratch` on this device
  hipError_t scratch_err = hipSuccess;
  int num_cus = 0, num_xcds = 1, clock_khz = 0;
  int64_t wall_khz = 100000;
  std::string arch;
  // SYNC_RUN_TIMED: ring of event quadruples (kernel start/end, copy start/end)
  struct Timed {
    hipEvent_t k0 = nullptr, k1 = nullptr, c0 = nullptr, c1 = nullptr;
    bool has_kernel = false, has_copy = false;
  };
  std::vector<Timed> ring;
  int64_t ring_head = 0, ring_count = 0;
  std::vector<hipEvent_t> split_events;  // sync_gemm_split: one per chunk hand-over, plus the join
  std::mutex mu;  // serialises launch sequences (the events and streams are shared)
};

std::mutex g_devices_mu;
std::map<int, std::unique_ptr<DeviceState>> g_devices;

int current_device_state(DeviceState** out) {
  int dev = 0;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge == hipErrorNoDevice || ge == hipErrorInsufficientDriver)
    return fail(SYNC_ENODEV, std::string("no HIP device: ") + hipGetErrorString(ge));
  if (ge != hipSuccess) return hip_fail(ge, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_devices_mu);
  auto& slot = g_devices[dev];
  if (!slot) slot = std::make_unique<DeviceState>();
  DeviceState& d = *slot;
  if (!d.ready) {
    d.device = dev;
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, dev));
    d.arch = prop.gcnArchName;
    if (d.arch.rfind("gfx950", 0) != 0) return fail(SYNC_ENODEV, "device " + std::to_string(dev) + " is " + d.arch + ", not gfx950");
    d.num_cus = prop.multiProcessorCount;
    d.clock_khz = prop.clockRate;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0) d.num_xcds = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) == hipSuccess && v > 0) d.wall_khz = v;
    // this device is current: its own copy of the scratch array
    d.scratch_err = hipGetSymbolAddress(&d.scratch, HIP_SYMBOL(scratch));
    if (d.scratch_err != hipSuccess) d.scratch = nullptr;
    d.ready = true;
  }
  *out = &d;
  return SYNC_OK;
}

constexpr int kTimingRing = 1024;

// Next timing slot (creates its events on first use); nullptr when not timed.
int timing_slot(DeviceState& d, bool timed, DeviceState::Timed** out) {
  *out = nullptr;
  if (!timed) return SYNC_OK;
  if (d.ring.empty()) d.ring.resize(kTimingRing);
  DeviceState::Timed& t = d.ring[d.ring_head % kTimingRing];
  if (!t.k0) {
    HIP_TRY(hipEventCreate(&t.k0));
    HIP_TRY(hipEventCreate(&t.k1));
    HIP_TRY(hipEventCreate(&t.c0));
    HIP_TRY(hipEventCreate(&t.c1));
  }
  t.has_kernel = t.has_copy = false;
  ++d.ring_head;
  if (d.ring_count < kTimingRing) ++d.ring_count;
  *out = &t;
  return SYNC_OK;
}

}  // namespace

// ---- plans -------------------------------------------------------------------
struct DeviceTables {
  int32_t* tile_order = nullptr;
  int64_t* dep_ptr = nullptr;
  int32_t* dep_idx = nullptr;
  int32_t* tiles_in = nullptr;
  int64_t* chunk_begin = nullptr;
  int32_t* arrival = nullptr;
  int32_t* resident = nullptr;
  int64_t* slot_row = nullptr;
  int32_t* push_rows = nullptr;  // GEMM-RS: staging row of each tile's first row (tiles in one chunk)
  int64_t* ar_items = nullptr;   // GEMM-RS plans: the all-gather items of a GEMM-AR share
  int32_t* ident = nullptr;      // 0 .. T-1: the traversal of one chunk's GEMM in sync_gemm_split
  int32_t* head_items = nullptr; // HEAD_ATTN plans: the tiles that start a kernel work item, in order
  void* block = nullptr;  // one allocation holding all of the above
};

// Lead-slice tables of an AG plan for one launch shape (see GemmArgs):
// lead_ptr[gn + 1], lead_item[2 x items], lead_count[C], one device block.
struct LeadTables {
  int32_t* lead_ptr = nullptr;
  int32_t* lead_item = nullptr;
  int32_t* lead_count = nullptr;
  void* block = nullptr;
};

struct sync_plan_s {
  Plan plan;
  std::vector<int64_t> slot_row;   // staging row of each send position (C+1)
  std::vector<int32_t> push_rows;  // GEMM-RS, every tile in one chunk: staging row of each tile's first row (T)
  std::vector<int64_t> ar_items;   // GEMM-RS: GEMM-AR all-gather items, 5 per item (see GemmArgs)
  std::vector<int32_t> head_items; // HEAD_ATTN: tiles whose head starts a kernel work item, in traversal order
  std::mutex mu;
  std::map<int, DeviceTables> dev;
  // (device, compute workgroups, XCDs, withheld chunk) -> lead-slice tables
  std::map<std::tuple<int, int, int, int>, LeadTables> lead;
};

namespace {

template <typename T>
void put(char*& cur, std::vector<char>& host, const std::vector<T>& v, T** dst, char* base) {
  const size_t off = cur - host.data();
  std::memcpy(cur, v.data(), v.size() * sizeof(T));
  *dst = reinterpret_cast<T*>(base + off);
  cur += align_up(static_cast<int64_t>(v.size() * sizeof(T)), 256);
}

int device_tables(sync_plan_s* p, int dev, DeviceTables** out) {
  std::lock_guard<std::mutex> lk(p->mu);
  auto it = p->dev.find(dev);
  if (it != p->dev.end()) {
    *out = &it->second;
    return SYNC_OK;
  }
  const Plan& pl = p->plan;
  auto sz = [](size_t n, size_t e) { return align_up(static_cast<int64_t>(n * e), 256); };
  const int64_t total = sz(pl.tile_order.size(), 4) + sz(pl.dep_ptr.size(), 8) + sz(pl.dep_idx.size(), 4) +
                        sz(pl.tiles_in.size(), 4) + sz(pl.chunk_begin.size(), 8) + sz(pl.arrival.size(), 4) +
                        sz(pl.resident.size(), 4) + sz(p->slot_row.size(), 8) + sz(p->push_rows.size(), 4) +
                        sz(p->ar_items.size(), 8) + sz(pl.tile_order.size(), 4) + sz(p->head_items.size(), 4) +
                        256;
  std::vector<char> host(static_cast<size_t>(total), 0);
  void* block = nullptr;
  HIP_TRY(hipMalloc(&block, static_cast<size_t>(total)));
  DeviceTables t;
  t.block = block;
  char* cur = host.data();
  char* base = static_cast<char*>(block);
  put(cur, host, pl.tile_order, &t.tile_order, base);
  put(cur, host, pl.dep_ptr, &t.dep_ptr, base);
  put(cur, host, pl.dep_idx, &t.dep_idx, base);
  put(cur, host, pl.tiles_in, &t.tiles_in, base);
  put(cur, host, pl.chunk_begin, &t.chunk_begin, base);
  put(cur, host, pl.arrival, &t.arrival, base);
  put(cur, host, pl.resident, &t.resident, base);
  put(cur, host, p->slot_row, &t.slot_row, base);
  if (!p->push_rows.empty()) put(cur, host, p->push_rows, &t.push_rows, base);
  if (!p->ar_items.empty()) put(cur, host, p->ar_items, &t.ar_items, base);
  std::vector<int32_t> ident(pl.tile_order.size());
  std::iota(ident.begin(), ident.end(), 0);
  put(cur, host, ident, &t.ident, base);
  if (!p->head_items.empty()) put(cur, host, p->head_items, &t.head_items, base);
  hipError_t e = hipMemcpy(block, host.data(), static_cast<size_t>(total), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(block);
    return hip_fail(e, "hipMemcpy(plan tables)");
  }
  *out = &p->dev.emplace(dev, t).first->second;
  return SYNC_OK;
}

// The plan's tables on `dev` if an earlier call put them there; EINVAL
// otherwise (for callers that may not allocate).
int resident_tables(sync_plan_s* p, int dev, DeviceTables** out) {
  std::lock_guard<std::mutex> lk(p->mu);
  auto it = p->dev.find(dev);
  if (it == p->dev.end())
    return fail(SYNC_EINVAL, "the plan's tables are not on this device yet: call sync_workspace_init or a launch "
                             "call with this plan on the device first");
  *out = &it->second;
  return SYNC_OK;
}

// Host twin of the kernels' xcd_slot: the traversal position compute
// workgroup b of g takes first.
int32_t first_slot(int32_t b, int32_t g, int32_t nxcd) {
  if (nxcd <= 1 || g % nxcd) return b;
  return (b % nxcd) * (g / nxcd) + b / nxcd;
}

// Lead-slice tables for a launch with gn compute workgroups: workgroup g's
// first tile is order[first_slot(g)]; for every non-resident, non-withheld
// chunk it reads, g takes the next share of that chunk's slice 0.  Built once
// per (plan, device, gn, XCDs, withheld chunk) and kept with the plan.
int lead_tables(sync_plan_s* p, int dev, int32_t gn, int32_t nxcd, int32_t withheld, LeadTables** out) {
  std::lock_guard<std::mutex> lk(p->mu);
  const auto key = std::make_tuple(dev, gn, nxcd, withheld);
  auto it = p->lead.find(key);
  if (it != p->lead.end()) {
    *out = &it->second;
    return SYNC_OK;
  }
  const Plan& pl = p->plan;
  std::vector<int32_t> ptr(static_cast<size_t>(gn) + 1, 0), item, count(static_cast<size_t>(pl.num_chunks), 0);
  for (int32_t g = 0; g < gn; ++g) {
    const int32_t pos = first_slot(g, gn, nxcd);
    if (pos < pl.num_tiles) {
      const int32_t t = pl.tile_order[pos];
      for (int64_t e = pl.dep_ptr[t]; e < pl.dep_ptr[t + 1]; ++e) {
        const int32_t c = pl.dep_idx[e];
        if (pl.resident[c] || c == withheld || withheld == -1) continue;
        item.push_back(c);
        item.push_back(count[c]++);
      }
    }
    ptr[g + 1] = static_cast<int32_t>(item.size() / 2);
  }
  const int64_t n0 = align_up(static_cast<int64_t>(ptr.size()) * 4, 256);
  const int64_t n1 = align_up(static_cast<int64_t>(std::max<size_t>(item.size(), 1)) * 4, 256);
  const int64_t n2 = align_up(static_cast<int64_t>(count.size()) * 4, 256);
  std::vector<char> host(static_cast<size_t>(n0 + n1 + n2), 0);
  std::memcpy(host.data(), ptr.data(), ptr.size() * 4);
  if (!item.empty()) std::memcpy(host.data() + n0, item.data(), item.size() * 4);
  std::memcpy(host.data() + n0 + n1, count.data(), count.size() * 4);
  LeadTables t;
  HIP_TRY(hipMalloc(&t.block, host.size()));
  hipError_t e = hipMemcpy(t.block, host.data(), host.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(t.block);
    return hip_fail(e, "hipMemcpy(lead tables)");
  }
  char* b = static_cast<char*>(t.block);
  t.lead_ptr = reinterpret_cast<int32_t*>(b);
  t.lead_item = reinterpret_cast<int32_t*>(b + n0);
  t.lead_count = reinterpret_cast<int32_t*>(b + n0 + n1);
  *out = &p->lead.emplace(key, t).first->second;
  return SYNC_OK;
}

// Workspace layout: 256-byte header, then four uint32[C] arrays, each padded
// to 256 bytes: flags (ready / done), counters (GEMM tiles stored per chunk),
// parts (copy XCD groups finished per chunk), sent (copy-out done); then
// xparts, uint32[C][16] (copy workgroups finished per chunk and XCD); then the
// K-sliced copy's sflags and sparts, uint32[C][8] each (ready flag and XCD
// groups finished per chunk slice), and sxparts, uint32[C][8][16]; then the
// trace: uint64[T][4] per tile and uint64[C][2] per chunk (SYNC_RUN_TRACE).
struct WsView {
  uint32_t *hdr, *flags, *counters, *parts, *sent, *xparts, *sflags, *sparts, *sxparts;
  uint64_t *trace_tiles, *trace_chunks;
};

int64_t ws_array_bytes(int32_t C) { return align_up(static_cast<int64_t>(C) * 4, 256); }
int64_t ws_xparts_bytes(int32_t C) { return align_up(static_cast<int64_t>(C) * 4 * kMaxXcd, 256); }
int64_t ws_slice_bytes(int32_t C) { return align_up(static_cast<int64_t>(C) * 4 * kMaxSlices, 256); }

int64_t ws_trace_offset(int32_t C) {
  return 256 + 4 * ws_array_bytes(C) + ws_xparts_bytes(C) + 2 * ws_slice_bytes(C) +
         align_up(static_cast<int64_t>(C) * 4 * kMaxSlices * kMaxXcd, 256);
}

int64_t ws_total_bytes(int32_t C, int32_t T) {
  return ws_trace_offset(C) + align_up(static_cast<int64_t>(T) * 32, 256) + align_up(static_cast<int64_t>(C) * 16, 256);
}

WsView ws_view(void* ws, int32_t C, int32_t T) {
  char* b = static_cast<char*>(ws);
  const int64_t a = ws_array_bytes(C);
  WsView v;
  v.hdr = reinterpret_cast<uint32_t*>(b);
  v.flags = reinterpret_cast<uint32_t*>(b + 256);
  v.counters = reinterpret_cast<uint32_t*>(b + 256 + a);
  v.parts = reinterpret_cast<uint32_t*>(b + 256 + 2 * a);
  v.sent = reinterpret_cast<uint32_t*>(b + 256 + 3 * a);
  v.xparts = reinterpret_cast<uint32_t*>(b + 256 + 4 * a);
  const int64_t s0 = 256 + 4 * a + ws_xparts_bytes(C);
  v.sflags = reinterpret_cast<uint32_t*>(b + s0);
  v.sparts = reinterpret_cast<uint32_t*>(b + s0 + ws_slice_bytes(C));
  v.sxparts = reinterpret_cast<uint32_t*>(b + s0 + 2 * ws_slice_bytes(C));
  const int64_t t0 = ws_trace_offset(C);
  v.trace_tiles = reinterpret_cast<uint64_t*>(b + t0);
  v.trace_chunks = reinterpret_cast<uint64_t*>(b + t0 + align_up(static_cast<int64_t>(T) * 32, 256));
  return v;
}

struct CallCtx {
  DeviceState* dev = nullptr;
  DeviceTables* tab = nullptr;
  WsView ws{};
  sync_copy_cfg cfg{};
  uint64_t timeout_ticks = 0;
};

// ws == nullptr with `noalloc`: the call runs on the device's static scratch
// and must not allocate (the plan's tables must already be on the device).
int prepare(sync_plan_t plan, const sync_copy_cfg* cfg_in, void* ws, int op, CallCtx& cx, bool noalloc = false) {
  if (!plan) return fail(SYNC_EINVAL, "plan is NULL");
  if (plan->plan.desc.op != op) return fail(SYNC_EINVAL, "plan was built for a different op");
  if (!noalloc && (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u)))
    return fail(SYNC_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  sync_copy_cfg cfg{};
  cfg.backend = SYNC_COPY_SDMA;
  if (cfg_in) cfg = *cfg_in;
  if (cfg.backend == SYNC_COPY_SDMA ? (cfg.copy_teams < 0 || cfg.copy_teams > std::max(plan->plan.num_chunks, kMaxSdmaEngines))
                                     : (cfg.copy_teams < 0 || cfg.copy_teams > plan->plan.num_chunks))
    return fail(SYNC_EINVAL, "copy_teams must be in [0, number of chunks] (SDMA: [0, max(number of chunks, 16)])");
  if (cfg.copy_teams == 0) cfg.copy_teams = 1;
  if (cfg.copy_kslices < 0 || cfg.copy_kslices > kMaxSlices) return fail(SYNC_EINVAL, "copy_kslices must be in [0, 8]");
  if (cfg.copy_kslices == 0) cfg.copy_kslices = 1;
  if (cfg.copy_kslices > 1) {
    const sync_plan_desc& d = plan->plan.desc;
    if (op != SYNC_OP_AG_GEMM) return fail(SYNC_EINVAL, "copy_kslices > 1 is for AG-GEMM");
    if (cfg.backend == SYNC_COPY_SDMA)
      return fail(SYNC_EINVAL, "copy_kslices > 1 needs the CU, COLOCATED or PRESET backend");
    if (d.k / 64 < 4 * static_cast<int64_t>(cfg.copy_kslices))
      return fail(SYNC_EINVAL, "copy_kslices > 1 needs K/64 >= 4 x copy_kslices");
  }
  if (cfg.copy_streaming != 0 && cfg.copy_streaming != 1) return fail(SYNC_EINVAL, "copy_streaming must be 0 or 1");
  if (cfg.copy_lead_slice < 0 || (cfg.copy_lead_slice > 0 && (cfg.copy_kslices < 2 || cfg.copy_lead_slice > cfg.copy_kslices)))
    return fail(SYNC_EINVAL, "copy_lead_slice must be 0, or in [1, copy_kslices] with copy_kslices > 1");
  if (cfg.copy_lead_slice && (op != SYNC_OP_AG_GEMM || cfg.backend != SYNC_COPY_CU || cfg.copy_link_gbps != 0.f))
    return fail(SYNC_EINVAL, "copy_lead_slice is for AG-GEMM with the CU backend, copy_kslices > 1 and no pacing");
  if (cfg.copy_link_gbps != 0.f) {
    if (!(cfg.copy_link_gbps >= 1.f && cfg.copy_link_gbps <= 10000.f))
      return fail(SYNC_EINVAL, "copy_link_gbps must be 0 or in [1, 10000]");
    if (cfg.backend != SYNC_COPY_CU) return fail(SYNC_EINVAL, "copy_link_gbps paces the CU backend's copy teams");
  }
  if (cfg.backend < SYNC_COPY_PRESET || cfg.backend > SYNC_COPY_EPILOGUE) return fail(SYNC_EINVAL, "bad backend");
  if (cfg.backend == SYNC_COPY_EPILOGUE && op != SYNC_OP_GEMM_RS)
    return fail(SYNC_EUNSUPPORTED, "the EPILOGUE backend sends GEMM-RS output; AG and attention copy in");
  if (cfg.backend == SYNC_COPY_HOST_GATED)
    return fail(SYNC_EUNSUPPORTED, "the HOST_GATED backend was withdrawn (stream-ordered runtime copies cannot start "
                                   "while the persistent kernel runs); SYNC_RUN_WITHHOLD covers failure-path tests");
  if (cfg.flags & ~(SYNC_RUN_COPY_ONLY | SYNC_RUN_COMPUTE_ONLY | SYNC_RUN_TIMED | SYNC_RUN_WITHHOLD | SYNC_RUN_TRACE))
    return fail(SYNC_EINVAL, "unknown cfg.flags bits");
  if ((cfg.flags & SYNC_RUN_TRACE) && (op == SYNC_OP_RING_ATTN || op == SYNC_OP_HEAD_ATTN))
    return fail(SYNC_EINVAL, "TRACE is for GEMM calls");
  if ((cfg.flags & SYNC_RUN_WITHHOLD) && (cfg.withhold_chunk < -1 || cfg.withhold_chunk >= plan->plan.num_chunks))
    return fail(SYNC_EINVAL, "withhold_chunk must be -1 or a chunk id");
  if ((cfg.flags & SYNC_RUN_WITHHOLD) &&
      (cfg.backend != SYNC_COPY_CU || op == SYNC_OP_GEMM_RS || (cfg.flags & (SYNC_RUN_COPY_ONLY | SYNC_RUN_COMPUTE_ONLY))))
    return fail(SYNC_EINVAL, "WITHHOLD needs the CU backend, an AG or attention plan, and no other run mode");
  if ((cfg.flags & SYNC_RUN_COPY_ONLY) && (cfg.flags & SYNC_RUN_COMPUTE_ONLY))
    return fail(SYNC_EINVAL, "COPY_ONLY and COMPUTE_ONLY are exclusive");
  if ((cfg.flags & SYNC_RUN_COPY_ONLY) && cfg.backend == SYNC_COPY_PRESET)
    return fail(SYNC_EINVAL, "COPY_ONLY needs a copy backend");
  int rc = current_device_state(&cx.dev);
  if (rc) return rc;
  if (cfg.backend == SYNC_COPY_CU) {
    if (cfg.copy_cus < cx.dev->num_xcds || cfg.copy_cus % cx.dev->num_xcds || cfg.copy_cus > cx.dev->num_cus / 2)
      return fail(SYNC_EINVAL, "copy_cus must be a multiple of the XCD count and at most half the CUs");
  }
  if (noalloc) {
    if (!cx.dev->scratch)
      return fail(SYNC_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(cx.dev->scratch_err));
    ws = cx.dev->scratch;
    if ((rc = resident_tables(plan, cx.dev->device, &cx.tab))) return rc;
  } else if ((rc = device_tables(plan, cx.dev->device, &cx.tab))) {
    return rc;
  }
  cx.ws = ws_view(ws, plan->plan.num_chunks, plan->plan.num_tiles);
  cx.cfg = cfg;
  const uint64_t ns = cfg.timeout_ns ? cfg.timeout_ns : 2000000000ull;
  cx.timeout_ticks = ns / 1000000ull * static_cast<uint64_t>(cx.dev->wall_khz) +
                     (ns % 1000000ull) * static_cast<uint64_t>(cx.dev->wall_khz) / 1000000ull;
  return SYNC_OK;
}

int check_gemm_shape(const Plan& pl) {
  const auto& d = pl.desc;
  if (d.k % 64) return fail(SYNC_EUNSUPPORTED, "k must be a multiple of 64");
  if (d.n % 8) return fail(SYNC_EUNSUPPORTED, "n must be a multiple of 8");
  if (!gemm_variant_exists(d.tile_m, d.tile_n))
    return fail(SYNC_EUNSUPPORTED, "no kernel for tile " + std::to_string(d.tile_m) + "x" + std::to_string(d.tile_n));
  if (d.m * d.k * 2 >= (int64_t(1) << 40) || d.k * d.n * 2 >= (int64_t(1) << 31) ||
      static_cast<int64_t>(d.tile_m) * d.k * 2 >= (int64_t(1) << 31) ||
      static_cast<int64_t>(d.tile_m) * d.n * 4 >= (int64_t(1) << 31))
    return fail(SYNC_EUNSUPPORTED, "operand too large for 32-bit buffer offsets");
  return SYNC_OK;
}

// Compute workgroups per CU (the kernel's occupancy; copy workgroups of the
// same launch take CUs at the same rate).
int gemm_wg_per_cu(const Plan& pl) { return syncov::gemm_wg_per_cu(pl.desc.tile_m, pl.desc.tile_n); }

// A launch of num_cus x wpc workgroups assumes every one of them is resident
// at once: the co-located copy publishes every chunk once all workgroups have
// copied, and co-located copy-out and the GEMM-AR all-gather wait for chunks
// that other workgroups of the grid produce.  The instance's occupancy (from
// its registers and LDS) is read once per device and variant; an instance
// that fits fewer workgroups per CU is refused rather than left to time out.
std::mutex g_occ_mu;
std::map<std::tuple<int, int, int, int, int, int>, int> g_occ;

int check_residency(const Plan& pl, int device, int c_dtype, bool rs) {
  const auto key = std::make_tuple(device, pl.desc.tile_m, pl.desc.tile_n, pl.desc.b_layout, c_dtype, rs ? 1 : 0);
  int occ = -1;
  {
    std::lock_guard<std::mutex> lk(g_occ_mu);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) occ = it->second;
  }
  if (occ < 0) {
    GemmArgs none{};
    HIP_TRY(launch_gemm(none, pl.desc.tile_m, pl.desc.tile_n, pl.desc.b_layout, c_dtype, rs, 0, nullptr, &occ));
    std::lock_guard<std::mutex> lk(g_occ_mu);
    g_occ[key] = occ;
  }
  const int need = gemm_wg_per_cu(pl);
  if (occ < need)
    return fail(SYNC_EUNSUPPORTED, "the " + std::to_string(pl.desc.tile_m) + "x" + std::to_string(pl.desc.tile_n) +
                                       " kernel fits " + std::to_string(occ) + " workgroup(s) per CU; its launch "
                                       "needs " + std::to_string(need));
  return SYNC_OK;
}

CounterArrays counter_arrays(const CallCtx& cx, int32_t C) {
  return CounterArrays{cx.ws.counters, cx.ws.parts, cx.ws.xparts, cx.ws.sparts, cx.ws.sxparts, C};
}

GemmArgs make_gemm_args(const Plan& pl, const CallCtx& cx, const void* A, const void* B, void* C) {
  GemmArgs g{};
  g.A = static_cast<const uint16_t*>(A);
  g.B = static_cast<const uint16_t*>(B);
  g.C = C;
  g.M = pl.desc.m;
  g.N = pl.desc.n;
  g.K = pl.desc.k;
  g.order = cx.tab->tile_order;
  g.num_tiles = pl.num_tiles;
  g.tiles_n = pl.tiles_n;
  g.dep_ptr = cx.tab->dep_ptr;
  g.dep_idx = cx.tab->dep_idx;
  g.tiles_in = cx.tab->tiles_in;
  g.resident = cx.tab->resident;
  g.flags = cx.ws.flags;
  g.hdr = cx.ws.hdr;
  g.cnt = counter_arrays(cx, pl.num_chunks);
  g.timeout_ticks = cx.timeout_ticks;
  g.nxcd = cx.dev->num_xcds;
  g.wait_chunks = 1;
  g.copy_blocks = 0;
  g.trace_tiles = (cx.cfg.flags & SYNC_RUN_TRACE) ? cx.ws.trace_tiles : nullptr;
  g.trace_chunks = (cx.cfg.flags & SYNC_RUN_TRACE) ? cx.ws.trace_chunks : nullptr;
  g.kslices = cx.cfg.copy_kslices;
  g.slice_flags = cx.ws.sflags;
  return g;
}

// Copy role arguments: copy-in stages chunks from src[x] to dst[x] at the same
// rows (ntensors tensors of rb[x]-byte rows) and raises the ready flags.
CopyArgs make_copy_in(const Plan& pl, const CallCtx& cx, const char* const src[kMaxCopyTensors],
                      char* const dst[kMaxCopyTensors], const int64_t rb[kMaxCopyTensors], int ntensors) {
  CopyArgs ca{};
  for (int x = 0; x < ntensors; ++x) {
    ca.src[x] = src[x];
    ca.dst[x] = dst[x];
    ca.row_bytes[x] = rb[x];
  }
  ca.ntensors = ntensors;
  ca.num_chunks = pl.num_chunks;
  ca.chunk_begin = cx.tab->chunk_begin;
  ca.arrival = cx.tab->arrival;
  ca.resident = cx.tab->resident;
  ca.slot_row = cx.tab->slot_row;
  ca.out_flags = cx.ws.flags;
  ca.parts = cx.ws.parts;
  ca.xparts = cx.ws.xparts;
  ca.hdr = cx.ws.hdr;
  ca.timeout_ticks = cx.timeout_ticks;
  ca.streaming = cx.cfg.copy_streaming;
  ca.skip_chunk = (cx.cfg.flags & SYNC_RUN_WITHHOLD) ? cx.cfg.withhold_chunk : -2;
  ca.teams = cx.cfg.copy_teams;
  ca.trace_chunks = (cx.cfg.flags & SYNC_RUN_TRACE) ? cx.ws.trace_chunks : nullptr;
  ca.kslices = cx.cfg.copy_kslices;  // > 1 only for AG-GEMM (checked by prepare)
  ca.slice_flags = cx.ws.sflags;
  ca.sparts = cx.ws.sparts;
  ca.sxparts = cx.ws.sxparts;
  if (cx.cfg.copy_link_gbps > 0.f) {  // wall-clock ticks per MiB at the link rate, 16.16 fixed point
    const double ticks_per_mib = static_cast<double>(cx.dev->wall_khz) * 1e3 * 1048576.0 /
                                 (static_cast<double>(cx.cfg.copy_link_gbps) * 1e9);
    ca.pace_q16 = static_cast<uint64_t>(ticks_per_mib * 65536.0 + 0.5);
    if (!ca.pace_q16) ca.pace_q16 = 1;
  }
  return ca;
}

// How one call's launch is split between roles.
struct Roles {
  int grid = 0;         // workgroups of the launch (0: no compute launch)
  int copy_blocks = 0;  // leading workgroups that run the copy role
  int wait = 1;         // compute waits for non-resident chunks
  int colocated = 0;    // every compute workgroup copies its share first
  bool no_compute = false;  // co-located copy-only: the copy phase alone
  bool engines = false; // SDMA: copies queued on the SDMA engines through HSA, gated by the call
  bool push = false;    // EPILOGUE: the RS epilogue stores every tile into its send slot too
};

// CU backend: one launch, copy_cus * wpc copy workgroups first, then one
// compute workgroup per remaining CU slot.  PRESET: compute alone, nothing to
// wait for.  SDMA: compute on every CU, copies on the SDMA engines.
Roles roles_for(const CallCtx& cx, const DeviceState& d, int wpc) {
  Roles r;
  const bool copy_only = cx.cfg.flags & SYNC_RUN_COPY_ONLY;
  const bool compute_only = cx.cfg.flags & SYNC_RUN_COMPUTE_ONLY;
  switch (cx.cfg.backend) {
    case SYNC_COPY_PRESET:
      r.grid = d.num_cus * wpc;
      r.wait = 0;
      break;
    case SYNC_COPY_CU:
      if (copy_only) {
        r.grid = r.copy_blocks = cx.cfg.copy_cus * wpc;
      } else if (compute_only) {
        r.grid = (d.num_cus - cx.cfg.copy_cus) * wpc;
        r.wait = 0;
      } else {
        r.grid = d.num_cus * wpc;
        r.copy_blocks = cx.cfg.copy_cus * wpc;
      }
      break;
    case SYNC_COPY_COLOCATED:
      r.grid = d.num_cus * wpc;
      if (copy_only) {
        r.colocated = 1;  // the copy phase of every workgroup, no tiles after it
        r.no_compute = true;
      } else if (compute_only)
        r.wait = 0;
      else
        r.colocated = 1;
      break;
    case SYNC_COPY_EPILOGUE:
      r.grid = d.num_cus * wpc;
      r.wait = 0;
      r.push = !compute_only;
      break;
    case SYNC_COPY_SDMA:
      r.grid = copy_only ? 0 : d.num_cus * wpc;
      if (compute_only)
        r.wait = 0;
      else
        r.engines = true;
      break;
    default:  // rejected by prepare()
      break;
  }
  return r;
}

// A GEMM launch whose workgroups only compute takes no more of them than the
// plan has tiles, rounded up to a multiple of the XCD count, so the slot remap
// gives every XCD an equal run of consecutive tiles.  (224 tiles on 256
// workgroups would leave one XCD idle and give the other seven 32 tiles each,
// spanning more distinct A rows per L2.)
// A co-located launch keeps its whole grid for the copy and hands the tiles
// to that many of its workgroups (GemmArgs::tile_grid).
int32_t tile_workgroups(int32_t tiles, int32_t workgroups, int nxcd) {
  const int32_t want = nxcd < 1 ? tiles : (tiles + nxcd - 1) / nxcd * nxcd;
  return want > 0 && want < workgroups ? want : workgroups;
}
void fit_grid_to_tiles(Roles& r, int32_t tiles, int nxcd) {
  if (r.grid <= 0 || r.copy_blocks || r.colocated || r.no_compute) return;
  r.grid = tile_workgroups(tiles, r.grid, nxcd);
}

// SDMA backend: reserve the call's signals; on the caller's stream the gate
// kernel; every copied chunk queued on the SDMA engines (each copy waits for
// the gate, so launch and queueing may happen in either order); then the
// compute kernel (copy-only: the join kernel).  If queueing fails, the join
// kernel ends the call instead, the missing chunks' waits timing out.
template <typename Launch>
int run_engines(const Plan& pl, CallCtx& cx, DeviceState& d, DeviceState::Timed* tm, hipStream_t cs, const Roles& r,
                const char* const src[kMaxCopyTensors], char* const dst[kMaxCopyTensors],
                const int64_t rb[kMaxCopyTensors], int ntensors, Launch launch) {
  int32_t copied = 0;
  for (int32_t c = 0; c < pl.num_chunks; ++c) copied += pl.resident[c] ? 0 : 1;
  SdmaCall call;
  int rc = sdma_begin(d.device, copied, ntensors, cx.cfg.copy_teams, &call);
  if (rc) return rc;
  SdmaJob job{};
  for (int x = 0; x < ntensors; ++x) {
    job.src[x] = src[x];
    job.dst[x] = dst[x];
    job.row_bytes[x] = rb[x];
  }
  job.ntensors = ntensors;
  job.num_chunks = pl.num_chunks;
  job.chunk_begin = pl.chunk_begin.data();
  job.arrival = pl.arrival.data();
  job.resident = pl.resident.data();
  job.flags = cx.ws.flags;
  job.epoch_word = cx.ws.hdr + WS_SDMA_EPOCH;
  if (tm) {
    HIP_TRY(hipEventRecord(tm->k0, cs));
    HIP_TRY(hipEventRecord(tm->c0, cs));
  }
  HIP_TRY(launch_sdma_gate(cx.ws.hdr, call.gate_value, cs));
  const int queued = sdma_submit(d.device, call, job);
  if (r.grid > 0 && queued == SYNC_OK) {
    if ((rc = launch(cs, r))) return rc;
  } else {
    HIP_TRY(launch_sdma_join(cx.ws.hdr, cx.ws.flags, cx.tab->arrival, cx.tab->resident, pl.num_chunks,
                             cx.timeout_ticks, cs));
  }
  if (tm) {
    HIP_TRY(hipEventRecord(tm->k1, cs));
    HIP_TRY(hipEventRecord(tm->c1, cs));
    tm->has_kernel = tm->has_copy = true;
  }
  return queued;
}

// Enqueues one call on the caller's stream `cs`: `launch(stream, roles)` puts
// the compute kernel (with its copy workgroups, if any) there; the SDMA
// backend adds its gate kernel and queues the copies on the engines.
template <typename Launch>
int run_call(const Plan& pl, CallCtx& cx, DeviceState& d, DeviceState::Timed* tm, hipStream_t cs,
             const Roles& r, const char* const src[kMaxCopyTensors], char* const dst[kMaxCopyTensors],
             const int64_t rb[kMaxCopyTensors], int ntensors, Launch launch) {
  if (r.copy_blocks || r.colocated) {  // the copy role stores with 32-bit offsets within one chunk
    int64_t rows = 0;
    for (int32_t c = 0; c < pl.num_chunks; ++c) rows = std::max(rows, pl.chunk_begin[c + 1] - pl.chunk_begin[c]);
    for (int x = 0; x < ntensors; ++x)
      if (rows * rb[x] >= (int64_t(1) << 31))
        return fail(SYNC_EUNSUPPORTED, "the CU and COLOCATED backends copy chunks of under 2 GiB per tensor");
  }
  auto timed = [&](hipStream_t st) -> int {
    if (tm) HIP_TRY(hipEventRecord(tm->k0, st));
    int rc = launch(st, r);
    if (rc) return rc;
    if (tm) {
      HIP_TRY(hipEventRecord(tm->k1, st));
      tm->has_kernel = true;
    }
    return SYNC_OK;
  };
  if (cx.cfg.flags & SYNC_RUN_TRACE) {  // stamps start at zero: "nothing recorded"
    const int64_t words = (ws_total_bytes(pl.num_chunks, pl.num_tiles) - ws_trace_offset(pl.num_chunks)) / 4;
    HIP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(cx.ws.trace_tiles), words, 0u, cs));
  }
  if (r.engines) return run_engines(pl, cx, d, tm, cs, r, src, dst, rb, ntensors, launch);
  return timed(cs);
}

}  // namespace

// ---- C ABI ---------------------------------------------------------------------
extern "C" {

int sync_plan(const sync_plan_desc* desc, sync_plan_t* out) {
  if (!desc || !out) return fail(SYNC_EINVAL, "desc and out must be non-NULL");
  *out = nullptr;
  auto p = std::make_unique<sync_plan_s>();
  std::string err;
  if (!build_plan(*desc, p->plan, err)) return fail(SYNC_EINVAL, err);
  const Plan& pl = p->plan;
  p->slot_row.assign(pl.num_chunks + 1, 0);
  for (int32_t s = 0; s < pl.num_chunks; ++s) {
    const int32_t c = pl.arrival[s];
    p->slot_row[s + 1] = p->slot_row[s] + (pl.chunk_begin[c + 1] - pl.chunk_begin[c]);
  }
  if (pl.desc.op == SYNC_OP_GEMM_RS) {
    // GEMM-AR all-gather order: ring step k brings shard (r - d k) mod W (k = 0:
    // this rank's own, fully reduced in its staging slots), sub-chunks in
    // order; sub-chunk q of every shard waits for this rank's own sub-chunk q
    const auto& d = pl.desc;
    const int32_t W = d.world, S = pl.num_chunks / W;
    for (int32_t kstep = 0; kstep < W; ++kstep) {
      const int32_t w = static_cast<int32_t>((((d.rank - d.ring_dir * kstep) % W) + W) % W);
      for (int32_t q = 0; q < S; ++q) {
        const int32_t c = w * S + q, own = d.rank * S + q;
        const int64_t r0 = pl.chunk_begin[c], rows = pl.chunk_begin[c + 1] - r0;
        const int64_t item[5] = {kstep == 0 ? 0 : 1, kstep == 0 ? p->slot_row[pl.chunk_pos[c]] : r0, r0, rows, own};
        p->ar_items.insert(p->ar_items.end(), item, item + 5);
      }
    }
  }
  if (pl.desc.op == SYNC_OP_HEAD_ATTN) {
    // the attention kernel's work item is a group of hg query heads sharing
    // one KV head: the plan tiles of each group's first head stand for it
    const int32_t group = pl.desc.heads_q / pl.desc.heads_kv, hg = std::min(group, 4);
    for (int32_t t : pl.tile_order)
      if ((t % pl.tiles_n) % hg == 0) p->head_items.push_back(t);
  }
  bool one_chunk = pl.desc.op == SYNC_OP_GEMM_RS && pl.rows < (int64_t(1) << 31);
  for (int32_t t = 0; one_chunk && t < pl.num_tiles; ++t) one_chunk = pl.dep_ptr[t + 1] - pl.dep_ptr[t] == 1;
  if (one_chunk) {
    p->push_rows.resize(static_cast<size_t>(pl.num_tiles));
    for (int32_t t = 0; t < pl.num_tiles; ++t) {
      const int32_t c = pl.dep_idx[pl.dep_ptr[t]];
      const int64_t m0 = static_cast<int64_t>(t / pl.tiles_n) * pl.desc.tile_m;
      p->push_rows[t] = static_cast<int32_t>(p->slot_row[pl.chunk_pos[c]] + (m0 - pl.chunk_begin[c]));
    }
  }
  *out = p.release();
  return SYNC_OK;
}

void sync_plan_destroy(sync_plan_t plan) {
  if (!plan) return;
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : plan->dev) {
    if (have) (void)hipSetDevice(kv.first);
    (void)hipFree(kv.second.block);
  }
  for (auto& kv : plan->lead) {
    if (have) (void)hipSetDevice(std::get<0>(kv.first));
    (void)hipFree(kv.second.block);
  }
  if (have) (void)hipSetDevice(cur);
  delete plan;
}

int sync_plan_get_info(sync_plan_t plan, sync_plan_info* out) {
  if (!plan || !out) return fail(SYNC_EINVAL, "plan and out must be non-NULL");
  const Plan& p = plan->plan;
  out->num_chunks = p.num_chunks;
  out->num_tiles = p.num_tiles;
  out->tiles_m = p.tiles_m;
  out->tiles_n = p.tiles_n;
  out->num_deps = static_cast<int64_t>(p.dep_idx.size());
  return SYNC_OK;
}

int sync_plan_export(sync_plan_t plan, sync_plan_tables* out) {
  if (!plan || !out) return fail(SYNC_EINVAL, "plan and out must be non-NULL");
  const Plan& p = plan->plan;
  auto cp = [](auto* dst, const auto& v) {
    if (dst) std::memcpy(dst, v.data(), v.size() * sizeof(v[0]));
  };
  cp(out->chunk_begin, p.chunk_begin);
  cp(out->chunk_pos, p.chunk_pos);
  cp(out->arrival, p.arrival);
  cp(out->resident, p.resident);
  cp(out->tiles_in, p.tiles_in);
  cp(out->tile_order, p.tile_order);
  cp(out->tile_key, p.tile_key);
  cp(out->dep_ptr, p.dep_ptr);
  cp(out->dep_idx, p.dep_idx);
  cp(out->inv_ptr, p.inv_ptr);
  cp(out->inv_idx, p.inv_idx);
  return SYNC_OK;
}

size_t sync_workspace_size(sync_plan_t plan) {
  if (!plan) return 0;
  return static_cast<size_t>(ws_total_bytes(plan->plan.num_chunks, plan->plan.num_tiles));
}

int sync_workspace_init(sync_plan_t plan, void* ws, void* stream) {
  if (!plan || !ws || (reinterpret_cast<uintptr_t>(ws) & 255u)) return fail(SYNC_EINVAL, "bad plan or workspace");
  DeviceState* d = nullptr;
  int rc = current_device_state(&d);
  if (rc) return rc;
  // SDMA flag copies of earlier calls must not land after the fill
  if ((rc = sdma_quiesce_all(d->device))) return rc;
  DeviceTables* tab = nullptr;  // set-up: the plan's tables go to the device now, not on the first launch
  if ((rc = device_tables(plan, d->device, &tab))) return rc;
  HIP_TRY(launch_fill_u32(static_cast<uint32_t*>(ws), static_cast<int64_t>(sync_workspace_size(plan) / 4), 0u,
                          static_cast<hipStream_t>(stream)));
  return SYNC_OK;
}

int sync_trace_export(sync_plan_t plan, const void* ws, void* stream, sync_trace* out) {
  if (!plan || !ws || !out) return fail(SYNC_EINVAL, "plan, ws and out must be non-NULL");
  DeviceState* d = nullptr;
  int rc = current_device_state(&d);
  if (rc) return rc;
  const int32_t C = plan->plan.num_chunks, T = plan->plan.num_tiles;
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  const int64_t off = ws_trace_offset(C);
  const int64_t chunk_off = align_up(static_cast<int64_t>(T) * 32, 256);
  std::vector<uint64_t> tiles(static_cast<size_t>(T) * 4), chunks(static_cast<size_t>(C) * 2);
  const char* b = static_cast<const char*>(ws);
  if (T) HIP_TRY(hipMemcpy(tiles.data(), b + off, tiles.size() * 8, hipMemcpyDeviceToHost));
  if (C) HIP_TRY(hipMemcpy(chunks.data(), b + off + chunk_off, chunks.size() * 8, hipMemcpyDeviceToHost));
  uint64_t t0 = ~0ull;
  for (int32_t t = 0; t < T; ++t)
    for (int i = 0; i < 3; ++i)
      if (tiles[4 * t + i]) t0 = std::min(t0, tiles[4 * t + i]);
  for (uint64_t v : chunks)
    if (v) t0 = std::min(t0, v);
  const double ns_per_tick = 1e6 / static_cast<double>(d->wall_khz);
  auto ns = [&](uint64_t v) -> int64_t {
    return v ? static_cast<int64_t>(std::llround(static_cast<double>(v - t0) * ns_per_tick)) : -1;
  };
  for (int32_t t = 0; t < T; ++t) {
    const uint64_t* r = &tiles[4 * static_cast<size_t>(t)];
    if (out->tile_wait_begin) out->tile_wait_begin[t] = ns(r[0]);
    if (out->tile_wait_end) out->tile_wait_end[t] = ns(r[1]);
    if (out->tile_end) out->tile_end[t] = ns(r[2]);
    if (out->tile_xcc) out->tile_xcc[t] = r[0] ? static_cast<int32_t>(r[3] >> 32) : -1;
    if (out->tile_slot) out->tile_slot[t] = r[0] ? static_cast<int32_t>(r[3] & 0xffffffffu) : -1;
  }
  for (int32_t c = 0; c < C; ++c) {
    if (out->chunk_ready) out->chunk_ready[c] = ns(chunks[2 * c]);
    if (out->chunk_sent) out->chunk_sent[c] = ns(chunks[2 * c + 1]);
  }
  return SYNC_OK;
}

int sync_workspace_status(const void* ws, void* stream, int32_t* err_chunk) {
  if (!ws) {  // the static scratch of sync_ag_gemm_noalloc on the current device
    DeviceState* d = nullptr;
    int rc = current_device_state(&d);
    if (rc) return rc;
    if (!d->scratch)
      return fail(SYNC_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(d->scratch_err));
    ws = d->scratch;
  }
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  uint32_t h[3] = {0, 0, 0};
  HIP_TRY(hipMemcpy(h, ws, sizeof h, hipMemcpyDeviceToHost));
  if (err_chunk) *err_chunk = h[WS_ERR_CODE] ? static_cast<int32_t>(h[WS_ERR_CHUNK]) : -1;
  if (h[WS_ERR_CODE] == ERR_TIMEOUT)
    return fail(SYNC_ETIMEOUT, "a device-side wait timed out on chunk " + std::to_string(h[WS_ERR_CHUNK]));
  if (h[WS_ERR_CODE]) return fail(SYNC_EHIP, "unknown workspace error word");
  return SYNC_OK;
}

static int ag_gemm_impl(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a_peer, void* a_local, const void* b,
                        void* c, int32_t c_dtype, void* ws, void* compute, bool noalloc) {
  CallCtx cx;
  if (noalloc) {  // nothing that allocates: no SDMA signals, no timing events, no trace, no lead tables
    const int32_t backend = cfg ? cfg->backend : SYNC_COPY_SDMA;
    if (backend != SYNC_COPY_PRESET && backend != SYNC_COPY_CU && backend != SYNC_COPY_COLOCATED)
      return fail(SYNC_EUNSUPPORTED, "sync_ag_gemm_noalloc runs the PRESET, CU and COLOCATED backends");
    if (cfg->flags & (SYNC_RUN_TIMED | SYNC_RUN_TRACE))
      return fail(SYNC_EUNSUPPORTED, "sync_ag_gemm_noalloc takes no TIMED or TRACE mode");
    if (cfg->copy_lead_slice) return fail(SYNC_EUNSUPPORTED, "sync_ag_gemm_noalloc takes no copy_lead_slice");
  }
  int rc = prepare(plan, cfg, ws, SYNC_OP_AG_GEMM, cx, noalloc);
  if (rc) return rc;
  const Plan& pl = plan->plan;
  if ((rc = check_gemm_shape(pl))) return rc;
  if (noalloc) {
    const int64_t need = ws_trace_offset(pl.num_chunks);
    if (need > kScratchBytes)
      return fail(SYNC_EINVAL, "the plan needs " + std::to_string(need) + " bytes of workspace; the static scratch "
                               "holds " + std::to_string(kScratchBytes));
  }
  if (c_dtype != SYNC_DTYPE_F32 && c_dtype != SYNC_DTYPE_BF16) return fail(SYNC_EINVAL, "bad c_dtype");
  const bool need_peer = cx.cfg.backend != SYNC_COPY_PRESET && !(cx.cfg.flags & SYNC_RUN_COMPUTE_ONLY);
  if (!a_local || !b || !c || (need_peer && !a_peer)) return fail(SYNC_EINVAL, "NULL operand");
  if (!aligned16(a_local) || !aligned16(b) || !aligned16(c) || (a_peer && !aligned16(a_peer)))
    return fail(SYNC_EINVAL, "operands must be 16-byte aligned");
  DeviceState& d = *cx.dev;
  if ((rc = check_residency(pl, d.device, c_dtype, false))) return rc;
  std::lock_guard<std::mutex> lk(d.mu);
  DeviceState::Timed* tm = nullptr;
  if ((rc = timing_slot(d, cx.cfg.flags & SYNC_RUN_TIMED, &tm))) return rc;
  if (noalloc)  // the scratch keeps the last call's contents: epoch, flags and counters start from zero
    HIP_TRY(launch_fill_u32(cx.ws.hdr, ws_trace_offset(pl.num_chunks) / 4, 0u, static_cast<hipStream_t>(compute)));
  const char* src[kMaxCopyTensors] = {static_cast<const char*>(a_peer)};
  char* dst[kMaxCopyTensors] = {static_cast<char*>(a_local)};
  const int64_t rb[kMaxCopyTensors] = {pl.desc.k * 2};
  GemmArgs g = make_gemm_args(pl, cx, a_local, b, c);
  g.copy = make_copy_in(pl, cx, src, dst, rb, 1);
  Roles r = roles_for(cx, d, gemm_wg_per_cu(pl));
  fit_grid_to_tiles(r, pl.num_tiles, d.num_xcds);
  if (r.colocated && !r.no_compute) g.tile_grid = tile_workgroups(pl.num_tiles, r.grid, d.num_xcds);
  if (cx.cfg.copy_lead_slice && r.wait && r.grid > r.copy_blocks) {
    const int32_t withheld = (cx.cfg.flags & SYNC_RUN_WITHHOLD) ? cx.cfg.withhold_chunk : -2;
    LeadTables* lt = nullptr;
    if ((rc = lead_tables(plan, d.device, r.grid - r.copy_blocks, d.num_xcds, withheld, &lt))) return rc;
    g.lead_ptr = lt->lead_ptr;
    g.lead_item = lt->lead_item;
    g.copy.lead_count = lt->lead_count;
    g.copy.lead_slices = cx.cfg.copy_lead_slice;
  }
  return run_call(pl, cx, d, tm, static_cast<hipStream_t>(compute), r, src, dst, rb, 1,
                  [&](hipStream_t st, const Roles& rr) -> int {
                    g.copy_blocks = rr.copy_blocks;
                    g.wait_chunks = rr.wait;
                    g.colocated = rr.colocated;
                    if (rr.no_compute) g.num_tiles = 0;
                    HIP_TRY(launch_gemm(g, pl.desc.tile_m, pl.desc.tile_n, pl.desc.b_layout, c_dtype, false, rr.grid,
                                        st));
                    return SYNC_OK;
                  });
}

int sync_ag_gemm(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a_peer, void* a_local, const void* b, void* c,
                 int32_t c_dtype, void* ws, void* compute, void* copy) {
  (void)copy;
  return ag_gemm_impl(plan, cfg, a_peer, a_local, b, c, c_dtype, ws, compute, false);
}

int sync_ag_gemm_noalloc(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a_peer, void* a_local,
                         const void* b, void* c, int32_t c_dtype, void* compute) {
  if (!cfg) return fail(SYNC_EINVAL, "sync_ag_gemm_noalloc needs a copy configuration");
  return ag_gemm_impl(plan, cfg, a_peer, a_local, b, c, c_dtype, nullptr, compute, true);
}

// GEMM-RS share; `partials` (fp32 [m][n], or null) makes the send the
// reduce-scatter step: slot data = tile + the incoming partial sums.
static int gemm_rs_impl(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a, const void* b, void* c,
                        int32_t c_dtype, const void* partials, void* staging, void* ws, void* compute, void* copy,
                        const void* ar_peer = nullptr, void* ar_out = nullptr) {
  CallCtx cx;
  int rc = prepare(plan, cfg, ws, SYNC_OP_GEMM_RS, cx);
  if (rc) return rc;
  const bool ar = ar_out != nullptr;
  if (ar) {
    if (cx.cfg.flags & (SYNC_RUN_COMPUTE_ONLY | SYNC_RUN_TRACE))
      return fail(SYNC_EUNSUPPORTED, "GEMM-AR calls take no COMPUTE_ONLY or TRACE mode");
    if (cx.cfg.copy_cus < 0 || cx.cfg.copy_cus % cx.dev->num_xcds || cx.cfg.copy_cus > cx.dev->num_cus / 2)
      return fail(SYNC_EINVAL, "GEMM-AR: copy_cus (CUs set aside for the all-gather) must be 0 or a multiple of "
                               "the XCD count, at most half the CUs");
    if (!ar_peer || !aligned16(ar_peer) || !aligned16(ar_out))
      return fail(SYNC_EINVAL, "GEMM-AR: reduced_peer and out must be non-NULL and 16-byte aligned");
  }
  if (partials) {
    if (cx.cfg.backend != SYNC_COPY_EPILOGUE || (cx.cfg.flags & SYNC_RUN_COMPUTE_ONLY))
      return fail(SYNC_EUNSUPPORTED, "the reduce-scatter step runs in the EPILOGUE backend's stores");
    if (c_dtype != SYNC_DTYPE_F32) return fail(SYNC_EUNSUPPORTED, "the reduce-scatter step needs fp32 C");
    if (!aligned16(partials)) return fail(SYNC_EINVAL, "partials must be 16-byte aligned");
  }
  const Plan& pl = plan->plan;
  if ((rc = check_gemm_shape(pl))) return rc;
  if (c_dtype != SYNC_DTYPE_F32 && c_dtype != SYNC_DTYPE_BF16) return fail(SYNC_EINVAL, "bad c_dtype");
  if (cx.cfg.backend == SYNC_COPY_SDMA)
    return fail(SYNC_EUNSUPPORTED, "GEMM-RS copy-out runs on CUs (CU or COLOCATED backend) or not at all (PRESET)");
  const bool compute_only = cx.cfg.backend == SYNC_COPY_PRESET || (cx.cfg.flags & SYNC_RUN_COMPUTE_ONLY);
  if (cx.cfg.flags & SYNC_RUN_COPY_ONLY) return fail(SYNC_EINVAL, "COPY_ONLY is not defined for GEMM-RS");
  // the EPILOGUE backend's tiles go straight to their send slots, so C is optional there
  const bool c_optional = cx.cfg.backend == SYNC_COPY_EPILOGUE && !compute_only;
  if (!a || !b || (!c && !c_optional) || (!compute_only && !staging)) return fail(SYNC_EINVAL, "NULL operand");
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || (staging && !aligned16(staging)))
    return fail(SYNC_EINVAL, "operands must be 16-byte aligned");
  DeviceState& d = *cx.dev;
  if ((rc = check_residency(pl, d.device, c_dtype, true))) return rc;
  std::lock_guard<std::mutex> lk(d.mu);
  DeviceState::Timed* tm = nullptr;
  if ((rc = timing_slot(d, cx.cfg.flags & SYNC_RUN_TIMED, &tm))) return rc;
  GemmArgs g = make_gemm_args(pl, cx, a, b, c);
  {
    // copy-out: rows of C, in send order, into the packed staging slots
    const int64_t es = c_dtype == SYNC_DTYPE_F32 ? 4 : 2;
    const char* src[kMaxCopyTensors] = {static_cast<const char*>(c)};
    char* dst[kMaxCopyTensors] = {static_cast<char*>(staging)};
    const int64_t rb[kMaxCopyTensors] = {pl.desc.n * es};
    g.copy = make_copy_in(pl, cx, src, dst, rb, 1);
    g.copy.copy_out = 1;
    g.copy.out_flags = cx.ws.sent;
    g.copy.wait_flags = cx.ws.flags;
  }
  Roles r = roles_for(cx, d, gemm_wg_per_cu(pl));
  if (!ar) fit_grid_to_tiles(r, pl.num_tiles, d.num_xcds);
  if (r.push) {
    const int64_t es = c_dtype == SYNC_DTYPE_F32 ? 4 : 2;
    if (pl.desc.m * pl.desc.n * es >= (int64_t(1) << 31))
      return fail(SYNC_EUNSUPPORTED, "the EPILOGUE backend needs m x n x element size below 2 GiB");
    if (!cx.tab->push_rows)
      return fail(SYNC_EUNSUPPORTED, "the EPILOGUE backend needs every tile inside one chunk (chunk rows a "
                                     "multiple of tile_m)");
    g.push_rows = cx.tab->push_rows;
    g.staging = staging;
    g.sent = cx.ws.sent;
    g.partials = partials;
  }
  Roles rar = r;
  if (ar) {  // the all-gather runs on copy_cus dedicated CUs of the same launch
    rar.copy_blocks = cx.cfg.copy_cus * gemm_wg_per_cu(pl);
    g.ar_items = cx.tab->ar_items;
    g.ar_count = pl.num_chunks;
    g.ar_src[0] = static_cast<const char*>(staging);
    g.ar_src[1] = static_cast<const char*>(ar_peer);
    g.ar_out = static_cast<char*>(ar_out);
    g.ar_row_bytes = pl.desc.n * 4;
  }
  return run_call(pl, cx, d, tm, static_cast<hipStream_t>(compute), rar, nullptr, nullptr, nullptr, 0,
                  [&](hipStream_t st, const Roles& rr) -> int {
                    g.copy_blocks = rr.copy_blocks;
                    g.colocated = rr.colocated;
                    HIP_TRY(launch_gemm(g, pl.desc.tile_m, pl.desc.tile_n, pl.desc.b_layout, c_dtype, true, rr.grid,
                                        st));
                    return SYNC_OK;
                  });
}

int sync_gemm_rs(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a, const void* b, void* c, int32_t c_dtype,
                 void* staging, void* ws, void* compute, void* copy) {
  return gemm_rs_impl(plan, cfg, a, b, c, c_dtype, nullptr, staging, ws, compute, copy);
}

int sync_gemm_rs_reduce(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a, const void* b, void* c,
                        const float* partials, void* staging, void* ws, void* compute, void* copy) {
  if (!partials) return fail(SYNC_EINVAL, "partials is NULL");
  return gemm_rs_impl(plan, cfg, a, b, c, SYNC_DTYPE_F32, partials, staging, ws, compute, copy);
}

int sync_gemm_ar(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a, const void* b, void* c,
                 const float* partials, const float* reduced_peer, float* out, void* staging, void* ws, void* compute,
                 void* copy) {
  if (!partials || !out) return fail(SYNC_EINVAL, "partials and out must be non-NULL");
  return gemm_rs_impl(plan, cfg, a, b, c, SYNC_DTYPE_F32, partials, staging, ws, compute, copy, reduced_peer, out);
}

// Kernel-level overlap baseline (Syncopate summary page, "Key observations",
// observation 1, Fig. 2(a)-(b): the operator split into per-chunk kernels,
// overlapped by streams).  Same GEMM kernel and K order as the fused calls;
// the hand-over of every chunk is a runtime copy plus a pair of events.
int sync_gemm_split(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a_peer, void* a, const void* b, void* c,
                    int32_t c_dtype, void* staging, void* ws, void* compute, void* copy) {
  if (!plan) return fail(SYNC_EINVAL, "plan is NULL");
  const Plan& pl = plan->plan;
  const int32_t op = pl.desc.op;
  if (op != SYNC_OP_AG_GEMM && op != SYNC_OP_GEMM_RS) return fail(SYNC_EINVAL, "sync_gemm_split takes a GEMM plan");
  const int32_t backend = cfg ? cfg->backend : SYNC_COPY_CU;
  if (backend != SYNC_COPY_CU && backend != SYNC_COPY_SDMA)
    return fail(SYNC_EINVAL, "sync_gemm_split copies with the runtime: backend CU (blit kernels) or SDMA (engines)");
  if (cfg && cfg->flags) return fail(SYNC_EINVAL, "sync_gemm_split takes no run-mode flags");
  if (!copy) return fail(SYNC_EINVAL, "sync_gemm_split needs a copy stream");
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u)) return fail(SYNC_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  int rc = check_gemm_shape(pl);
  if (rc) return rc;
  if (c_dtype != SYNC_DTYPE_F32 && c_dtype != SYNC_DTYPE_BF16) return fail(SYNC_EINVAL, "bad c_dtype");
  const bool ag = op == SYNC_OP_AG_GEMM;
  if (!a || !b || !c || (ag && !a_peer) || (!ag && !staging)) return fail(SYNC_EINVAL, "NULL operand");
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || (a_peer && !aligned16(a_peer)) ||
      (staging && !aligned16(staging)))
    return fail(SYNC_EINVAL, "operands must be 16-byte aligned");
  DeviceState* dp = nullptr;
  if ((rc = current_device_state(&dp))) return rc;
  DeviceState& d = *dp;
  if ((rc = check_residency(pl, d.device, c_dtype, false))) return rc;
  DeviceTables* tab = nullptr;
  if ((rc = device_tables(plan, d.device, &tab))) return rc;
  std::lock_guard<std::mutex> lk(d.mu);
  const int32_t C = pl.num_chunks;
  while (static_cast<int32_t>(d.split_events.size()) < C + 1) {
    hipEvent_t e = nullptr;
    HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    d.split_events.push_back(e);
  }
  hipStream_t cs = static_cast<hipStream_t>(compute), xs = static_cast<hipStream_t>(copy);
  const hipMemcpyKind kind = backend == SYNC_COPY_SDMA ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
  const int64_t K = pl.desc.k, N = pl.desc.n, es = c_dtype == SYNC_DTYPE_F32 ? 4 : 2;
  const int32_t TM = pl.desc.tile_m, Tn = pl.tiles_n, full = d.num_cus * gemm_wg_per_cu(pl);
  CallCtx cx;
  cx.dev = &d;
  cx.tab = tab;
  cx.ws = ws_view(ws, C, pl.num_tiles);
  cx.timeout_ticks = 2000ull * static_cast<uint64_t>(d.wall_khz);
  // the GEMM over the rows of one chunk: every tile in place, the identity traversal
  auto gemm_rows = [&](int64_t r0, int64_t r1) -> int {
    GemmArgs g = make_gemm_args(pl, cx, static_cast<const uint16_t*>(a) + r0 * K, b,
                                static_cast<char*>(c) + r0 * N * es);
    g.M = r1 - r0;
    g.order = tab->ident;
    g.num_tiles = static_cast<int32_t>((r1 - r0 + TM - 1) / TM) * Tn;
    g.wait_chunks = 0;
    const int grid = std::min(full, g.num_tiles);
    HIP_TRY(launch_gemm(g, pl.desc.tile_m, pl.desc.tile_n, pl.desc.b_layout, c_dtype, false, grid, cs));
    return SYNC_OK;
  };
  for (int32_t p = 0; p < C; ++p) {
    const int32_t ch = pl.arrival[p];
    const int64_t r0 = pl.chunk_begin[ch], r1 = pl.chunk_begin[ch + 1];
    if (ag) {  // copy in the chunk, then its GEMM once the copy has landed
      if (!pl.resident[ch]) {
        HIP_TRY(hipMemcpyAsync(static_cast<char*>(a) + r0 * K * 2, static_cast<const char*>(a_peer) + r0 * K * 2,
                               static_cast<size_t>((r1 - r0) * K * 2), kind, xs));
        HIP_TRY(hipEventRecord(d.split_events[p], xs));
        HIP_TRY(hipStreamWaitEvent(cs, d.split_events[p], 0));
      }
      if ((rc = gemm_rows(r0, r1))) return rc;
    } else {  // the chunk's GEMM, then its copy-out to send slot p
      if ((rc = gemm_rows(r0, r1))) return rc;
      HIP_TRY(hipEventRecord(d.split_events[p], cs));
      HIP_TRY(hipStreamWaitEvent(xs, d.split_events[p], 0));
      HIP_TRY(hipMemcpyAsync(static_cast<char*>(staging) + plan->slot_row[p] * N * es,
                             static_cast<const char*>(c) + r0 * N * es, static_cast<size_t>((r1 - r0) * N * es), kind,
                             xs));
    }
  }
  HIP_TRY(hipEventRecord(d.split_events[C], xs));  // the call ends on `compute` once every copy has
  HIP_TRY(hipStreamWaitEvent(cs, d.split_events[C], 0));
  return SYNC_OK;
}

int sync_ring_attn_step(sync_plan_t plan, const sync_copy_cfg* cfg, const void* q, const void* k_peer,
                        const void* v_peer, void* k_local, void* v_local, float* o, float* m_state, float* l_state,
                        float* lse, float scale, int32_t flags, void* ws, void* compute, void* copy) {
  CallCtx cx;
  int rc = prepare(plan, cfg, ws, SYNC_OP_RING_ATTN, cx);
  if (rc) return rc;
  const Plan& pl = plan->plan;
  const auto& dsc = pl.desc;
  if (dsc.k != kAttnHeadDim) return fail(SYNC_EUNSUPPORTED, "head dim (k) must be 128");
  const int group = dsc.heads_q / dsc.heads_kv;
  if (!(group == 1 || group == 2 || group % 4 == 0))
    return fail(SYNC_EUNSUPPORTED, "heads_q / heads_kv must be 1, 2 or a multiple of 4");
  if (flags & ~(SYNC_ATTN_INIT | SYNC_ATTN_FINALIZE)) return fail(SYNC_EINVAL, "unknown attention flags");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SYNC_EINVAL, "scale must be positive and finite");
  const bool need_peer = cx.cfg.backend != SYNC_COPY_PRESET && !(cx.cfg.flags & SYNC_RUN_COMPUTE_ONLY);
  if (!q || !k_local || !v_local || !o || !m_state || !l_state || (need_peer && (!k_peer || !v_peer)))
    return fail(SYNC_EINVAL, "NULL operand");
  if (!aligned16(q) || !aligned16(k_local) || !aligned16(v_local) || !aligned16(o) ||
      (k_peer && !aligned16(k_peer)) || (v_peer && !aligned16(v_peer)))
    return fail(SYNC_EINVAL, "operands must be 16-byte aligned");
  if (dsc.m * dsc.heads_q * dsc.k * 2 >= (int64_t(1) << 31))
    return fail(SYNC_EUNSUPPORTED, "query tensor too large for 32-bit buffer offsets");
  DeviceState& d = *cx.dev;
  std::lock_guard<std::mutex> lk(d.mu);
  DeviceState::Timed* tm = nullptr;
  if ((rc = timing_slot(d, cx.cfg.flags & SYNC_RUN_TIMED, &tm))) return rc;
  const int64_t row = static_cast<int64_t>(dsc.heads_kv) * dsc.k * 2;  // bytes per token of K or V
  const char* src[kMaxCopyTensors] = {static_cast<const char*>(k_peer), static_cast<const char*>(v_peer)};
  char* dst[kMaxCopyTensors] = {static_cast<char*>(k_local), static_cast<char*>(v_local)};
  const int64_t rb[kMaxCopyTensors] = {row, row};
  AttnArgs at{};
  at.q = static_cast<const uint16_t*>(q);
  at.k = static_cast<const uint16_t*>(k_local);
  at.v = static_cast<const uint16_t*>(v_local);
  at.o = o;
  at.m_state = m_state;
  at.l_state = l_state;
  at.lse = lse;
  at.sq = dsc.m;
  at.heads_q = dsc.heads_q;
  at.heads_kv = dsc.heads_kv;
  at.heads_per_item = std::min(group, 4);
  at.scale = scale;
  at.init = (flags & SYNC_ATTN_INIT) ? 1 : 0;
  at.finalize = (flags & SYNC_ATTN_FINALIZE) ? 1 : 0;
  at.chunk_begin = cx.tab->chunk_begin;
  at.arrival = cx.tab->arrival;
  at.resident = cx.tab->resident;
  at.num_chunks = pl.num_chunks;
  at.flags = cx.ws.flags;
  at.hdr = cx.ws.hdr;
  at.cnt = counter_arrays(cx, pl.num_chunks);
  at.timeout_ticks = cx.timeout_ticks;
  at.nxcd = d.num_xcds;
  at.copy = make_copy_in(pl, cx, src, dst, rb, 2);
  const Roles r = roles_for(cx, d, attn_wg_per_cu());
  return run_call(pl, cx, d, tm, static_cast<hipStream_t>(compute), r, src, dst, rb, 2,
                  [&](hipStream_t st, const Roles& rr) -> int {
                    at.copy_blocks = rr.copy_blocks;
                    at.wait_chunks = rr.wait;
                    at.colocated = rr.colocated;
                    if (rr.no_compute) at.sq = 0;
                    HIP_TRY(launch_ring_attn(at, rr.grid, st));
                    return SYNC_OK;
                  });
}

int sync_head_attn(sync_plan_t plan, const sync_copy_cfg* cfg, const void* q_peer, const void* k_peer,
                   const void* v_peer, void* q, void* k, void* v, float* o, float* lse, float scale, void* ws,
                   void* compute, void* copy) {
  CallCtx cx;
  int rc = prepare(plan, cfg, ws, SYNC_OP_HEAD_ATTN, cx);
  if (rc) return rc;
  const Plan& pl = plan->plan;
  const auto& dsc = pl.desc;
  if (dsc.k != kAttnHeadDim) return fail(SYNC_EUNSUPPORTED, "head dim (k) must be 128");
  const int group = dsc.heads_q / dsc.heads_kv;
  if (!(group == 1 || group == 2 || group % 4 == 0))
    return fail(SYNC_EUNSUPPORTED, "heads_q / heads_kv must be 1, 2 or a multiple of 4");
  const int hg = std::min(group, 4), qb = attn_query_block(hg);
  if (dsc.tile_m != qb)
    return fail(SYNC_EUNSUPPORTED, "tile_m must be the kernel's query block: " + std::to_string(qb) +
                                       " rows for heads_q / heads_kv = " + std::to_string(group));
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SYNC_EINVAL, "scale must be positive and finite");
  const bool need_peer = cx.cfg.backend != SYNC_COPY_PRESET && !(cx.cfg.flags & SYNC_RUN_COMPUTE_ONLY);
  if (!q || !k || !v || !o || (need_peer && (!q_peer || !k_peer || !v_peer))) return fail(SYNC_EINVAL, "NULL operand");
  for (const void* x : {q_peer, k_peer, v_peer, static_cast<const void*>(q), static_cast<const void*>(k),
                        static_cast<const void*>(v), static_cast<const void*>(o)})
    if (x && !aligned16(x)) return fail(SYNC_EINVAL, "operands must be 16-byte aligned");
  if (dsc.m * dsc.heads_q * dsc.k * 2 >= (int64_t(1) << 31))
    return fail(SYNC_EUNSUPPORTED, "query tensor too large for 32-bit buffer offsets");
  DeviceState& d = *cx.dev;
  std::lock_guard<std::mutex> lk(d.mu);
  DeviceState::Timed* tm = nullptr;
  if ((rc = timing_slot(d, cx.cfg.flags & SYNC_RUN_TIMED, &tm))) return rc;
  const int64_t qrow = static_cast<int64_t>(dsc.heads_q) * dsc.k * 2;   // bytes per token of Q
  const int64_t kvrow = static_cast<int64_t>(dsc.heads_kv) * dsc.k * 2;  // of K or V
  const char* src[kMaxCopyTensors] = {static_cast<const char*>(q_peer), static_cast<const char*>(k_peer),
                                      static_cast<const char*>(v_peer)};
  char* dst[kMaxCopyTensors] = {static_cast<char*>(q), static_cast<char*>(k), static_cast<char*>(v)};
  const int64_t rb[kMaxCopyTensors] = {qrow, kvrow, kvrow};
  AttnArgs at{};
  at.q = static_cast<const uint16_t*>(q);
  at.k = static_cast<const uint16_t*>(k);
  at.v = static_cast<const uint16_t*>(v);
  at.o = o;
  at.lse = lse;
  at.sq = dsc.m;
  at.heads_q = dsc.heads_q;
  at.heads_kv = dsc.heads_kv;
  at.heads_per_item = hg;
  at.scale = scale;
  at.init = 1;
  at.finalize = 1;
  at.chunk_begin = cx.tab->chunk_begin;
  at.arrival = cx.tab->arrival;
  at.resident = cx.tab->resident;
  at.num_chunks = pl.num_chunks;
  at.items = cx.tab->head_items;
  at.num_items = static_cast<int32_t>(plan->head_items.size());
  at.dep_ptr = cx.tab->dep_ptr;
  at.dep_idx = cx.tab->dep_idx;
  at.flags = cx.ws.flags;
  at.hdr = cx.ws.hdr;
  at.cnt = counter_arrays(cx, pl.num_chunks);
  at.timeout_ticks = cx.timeout_ticks;
  at.nxcd = d.num_xcds;
  at.copy = make_copy_in(pl, cx, src, dst, rb, 3);
  const Roles r = roles_for(cx, d, attn_wg_per_cu());
  return run_call(pl, cx, d, tm, static_cast<hipStream_t>(compute), r, src, dst, rb, 3,
                  [&](hipStream_t st, const Roles& rr) -> int {
                    at.copy_blocks = rr.copy_blocks;
                    at.wait_chunks = rr.wait;
                    at.colocated = rr.colocated;
                    if (rr.no_compute) at.num_items = 0;
                    HIP_TRY(launch_ring_attn(at, rr.grid, st));
                    return SYNC_OK;
                  });
}

int32_t sync_attn_query_block(int32_t heads_q, int32_t heads_kv) {
  if (heads_q < 1 || heads_kv < 1 || heads_q % heads_kv) return 0;
  const int32_t group = heads_q / heads_kv;
  if (!(group == 1 || group == 2 || group % 4 == 0)) return 0;
  return attn_query_block(std::min(group, 4));
}

int sync_get_device_info(sync_device_info* out) {
  if (!out) return fail(SYNC_EINVAL, "out is NULL");
  DeviceState* d = nullptr;
  int rc = current_device_state(&d);
  if (rc) return rc;
  std::memset(out, 0, sizeof *out);
  out->device = d->device;
  out->num_cus = d->num_cus;
  out->num_xcds = d->num_xcds;
  out->clock_khz = d->clock_khz;
  out->wall_clock_khz = d->wall_khz;
  std::snprintf(out->arch, sizeof out->arch, "%s", d->arch.c_str());
  return SYNC_OK;
}

int sync_read_timings(int32_t max, sync_timing* out, int32_t* count) {
  if (!count || (max > 0 && !out)) return fail(SYNC_EINVAL, "bad arguments");
  *count = 0;
  DeviceState* d = nullptr;
  int rc = current_device_state(&d);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(d->mu);
  const int64_t n = d->ring_count;
  for (int64_t i = 0; i < n; ++i) {
    DeviceState::Timed& t = d->ring[(d->ring_head - n + i) % kTimingRing];
    sync_timing r{0.f, 0.f};
    if (t.has_kernel) {
      HIP_TRY(hipEventSynchronize(t.k1));
      HIP_TRY(hipEventElapsedTime(&r.kernel_ms, t.k0, t.k1));
    }
    if (t.has_copy) {
      HIP_TRY(hipEventSynchronize(t.c1));
      HIP_TRY(hipEventElapsedTime(&r.copy_ms, t.c0, t.c1));
    }
    if (*count < max) out[(*count)++] = r;
  }
  d->ring_count = 0;
  return SYNC_OK;
}

const char* sync_last_error(void) { return g_err.c_str(); }

void sync_shutdown(void) {
  sdma_release_all();
  std::lock_guard<std::mutex> lk(g_devices_mu);
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_devices) {
    DeviceState& d = *kv.second;
    if (!d.ready) continue;
    (void)hipSetDevice(kv.first);
    for (auto& t : d.ring)
      for (hipEvent_t e : {t.k0, t.k1, t.c0, t.c1})
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : d.split_events) (void)hipEventDestroy(e);
  }
  g_devices.clear();
  if (have) (void)hipSetDevice(cur);
}

}  // extern "C"
