// SDMA copy agent driven through HSA.
//
// The Syncopate summary page ("Core method", paper sec. 5.2, Fig. 7) lists a
// copy-engine backend beside load/store on dedicated SMs; both signal chunk
// completion through global-memory flags.  On MI355X the copy engines are the
// SDMA engines.  This file queues a call's chunk copies on them directly with
// hsa_amd_memory_async_copy_on_engine, with no HIP stream in between:
//
//   caller stream:  gate kernel -> compute kernel (or, copy-only, a join kernel)
//   SDMA engine e:  [wait gate] copy chunk c (each tensor; with more engines
//                   than copied chunks, one row piece of it per engine) ->
//                   4-byte copy of the call's epoch into flag[c] (after every
//                   piece of the chunk completed)
//
// The gate kernel runs when the caller's stream reaches the call: it fixes the
// call's epoch in the workspace (the word the flag copies read) and opens the
// gate signal, which every copy of the call waits for.  So the copies start
// after the work queued before the call, and the compute kernel, which runs on
// every CU, waits on the flags in-kernel as with the CU backend.  Nothing on a
// second HIP stream orders anything, so no kernel on the GPU delays a copy.
//
// Signals are kept per device in a ring of call records; a record is reused
// once every flag copy of its previous call has completed (host wait).
#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <algorithm>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "sdma_engine.hpp"
#include "sync_overlap.h"

namespace syncov {

int set_error(int code, const std::string& msg);

namespace {

constexpr int kRecords = 16;                      // calls in flight per device
constexpr uint64_t kReuseWaitNs = 10000000000ull;  // bound on waiting for a record's previous call

struct Record {
  hsa_signal_t gate{};                 // opened (0) by the gate kernel
  volatile hsa_signal_value_t* gate_value = nullptr;
  hsa_signal_t done{};                 // counts down the call's flag copies
  std::vector<hsa_signal_t> chunk;     // per copied chunk: counts down its data copies
  bool used = false;
};

struct Engines {
  bool ready = false;
  hsa_agent_t gpu{};
  std::vector<hsa_amd_sdma_engine_id_t> ids;  // available engines, in id order
  Record rec[kRecords];
  int next = 0;
  std::mutex mu;
};

std::mutex g_mu;
std::map<int, std::unique_ptr<Engines>> g_engines;

struct FindAgent {
  uint32_t bdf, domain;
  hsa_agent_t agent, cpu;
  bool found, found_cpu;
};

hsa_status_t find_agent(hsa_agent_t a, void* data) {
  auto* f = static_cast<FindAgent*>(data);
  hsa_device_type_t type;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS) return HSA_STATUS_SUCCESS;
  if (type == HSA_DEVICE_TYPE_CPU && !f->found_cpu) {
    f->cpu = a;
    f->found_cpu = true;
  }
  if (type != HSA_DEVICE_TYPE_GPU || f->found) return HSA_STATUS_SUCCESS;
  uint32_t bdf = 0, domain = 0;
  if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) != HSA_STATUS_SUCCESS)
    return HSA_STATUS_SUCCESS;
  (void)hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN), &domain);
  if (bdf == f->bdf && domain == f->domain) {
    f->agent = a;
    f->found = true;
  }
  return HSA_STATUS_SUCCESS;
}

int hsa_fail(hsa_status_t s, const char* what) {
  const char* msg = nullptr;
  (void)hsa_status_string(s, &msg);
  return set_error(SYNC_EHIP, std::string(what) + ": " + (msg ? msg : "HSA error"));
}

#define HSA_TRY(expr)                                   \
  do {                                                  \
    const hsa_status_t s_ = (expr);                     \
    if (s_ != HSA_STATUS_SUCCESS) return hsa_fail(s_, #expr); \
  } while (0)

int make_signal(hsa_signal_value_t v, hsa_signal_t* out, uint64_t attributes = 0) {
  HSA_TRY(hsa_amd_signal_create(v, 0, nullptr, attributes, out));
  return SYNC_OK;
}

// Engine state of HIP device `dev` (agent matched by PCI location).
int engines_for(int dev, Engines** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto& slot = g_engines[dev];
  if (!slot) slot = std::make_unique<Engines>();
  Engines& e = *slot;
  if (!e.ready) {
    HSA_TRY(hsa_init());  // reference-counted; the HIP runtime holds its own
    int bus = 0, devno = 0, domain = 0;
    if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev) != hipSuccess ||
        hipDeviceGetAttribute(&devno, hipDeviceAttributePciDeviceId, dev) != hipSuccess ||
        hipDeviceGetAttribute(&domain, hipDeviceAttributePciDomainID, dev) != hipSuccess)
      return set_error(SYNC_EHIP, "cannot read the device's PCI location");
    FindAgent f{static_cast<uint32_t>((bus << 8) | (devno << 3)), static_cast<uint32_t>(domain), {}, {}, false, false};
    HSA_TRY(hsa_iterate_agents(find_agent, &f));
    if (!f.found) return set_error(SYNC_EHIP, "no HSA agent at the device's PCI location");
    e.gpu = f.agent;
    // The engine status is reported per direction between two agents; a copy
    // within one device may use the engines of either host direction.
    uint32_t mask = 0, m2 = 0;
    if (hsa_amd_memory_copy_engine_status(e.gpu, e.gpu, &mask) != HSA_STATUS_SUCCESS) mask = 0;
    if (!mask && f.found_cpu) {
      if (hsa_amd_memory_copy_engine_status(e.gpu, f.cpu, &m2) == HSA_STATUS_SUCCESS) mask |= m2;
      if (hsa_amd_memory_copy_engine_status(f.cpu, e.gpu, &m2) == HSA_STATUS_SUCCESS) mask |= m2;
    }
    for (int b = 0; b < 32; ++b)
      if (mask & (1u << b)) e.ids.push_back(static_cast<hsa_amd_sdma_engine_id_t>(1u << b));
    if (e.ids.empty()) return set_error(SYNC_EUNSUPPORTED, "no SDMA engine is available on this device");
    e.ready = true;
  }
  *out = &e;
  return SYNC_OK;
}

// Waits until every flag copy of the record's last call has completed.
int quiesce(Record& r) {
  if (!r.used) return SYNC_OK;
  const hsa_signal_value_t v =
      hsa_signal_wait_scacquire(r.done, HSA_SIGNAL_CONDITION_LT, 1, kReuseWaitNs, HSA_WAIT_STATE_BLOCKED);
  if (v > 0) return set_error(SYNC_ETIMEOUT, "an earlier call's SDMA copies did not complete");
  if (v < 0) return set_error(SYNC_EHIP, "an SDMA copy reported an error");
  return SYNC_OK;
}

}  // namespace

int sdma_engine_count(int dev, int* out) {
  Engines* e = nullptr;
  int rc = engines_for(dev, &e);
  if (rc) return rc;
  *out = static_cast<int>(e->ids.size());
  return SYNC_OK;
}

int sdma_begin(int dev, int32_t copied_chunks, int32_t ntensors, int32_t engines, SdmaCall* out) {
  Engines* e = nullptr;
  int rc = engines_for(dev, &e);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(e->mu);
  Record& r = e->rec[e->next];
  if ((rc = quiesce(r))) return rc;
  if (!r.gate.handle) {
    // The gate is consumed by the SDMA engines only, and the gate kernel
    // writes its value word itself: a GPU-only signal, whose value pointer
    // HSA hands out for that purpose.
    if ((rc = make_signal(1, &r.gate, HSA_AMD_SIGNAL_AMD_GPU_ONLY)) || (rc = make_signal(0, &r.done))) return rc;
    HSA_TRY(hsa_amd_signal_value_pointer(r.gate, &r.gate_value));
  }
  while (static_cast<int32_t>(r.chunk.size()) < copied_chunks) {
    hsa_signal_t s{};
    if ((rc = make_signal(0, &s))) return rc;
    r.chunk.push_back(s);
  }
  const int32_t used = std::max(1, std::min<int32_t>(engines, static_cast<int32_t>(e->ids.size())));
  const int32_t pieces = std::max(1, copied_chunks > 0 ? used / copied_chunks : 1);
  hsa_signal_store_screlease(r.gate, 1);
  hsa_signal_store_screlease(r.done, copied_chunks);
  for (int32_t i = 0; i < copied_chunks; ++i) hsa_signal_store_screlease(r.chunk[i], ntensors * pieces);
  r.used = true;
  out->engines = used;
  out->pieces = pieces;
  out->record = e->next;
  out->gate_value = const_cast<int64_t*>(reinterpret_cast<volatile int64_t*>(r.gate_value));
  e->next = (e->next + 1) % kRecords;
  return SYNC_OK;
}

int sdma_submit(int dev, const SdmaCall& call, const SdmaJob& job) {
  Engines* e = nullptr;
  int rc = engines_for(dev, &e);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(e->mu);
  Record& r = e->rec[call.record];
  const int32_t used = call.engines, P = call.pieces;
  int32_t copied = 0;
  for (int32_t p = 0; p < job.num_chunks; ++p) copied += job.resident[job.arrival[p]] ? 0 : 1;
  int32_t i = 0;
  hsa_status_t s = HSA_STATUS_SUCCESS;
  const char* what = nullptr;
  for (int32_t p = 0; p < job.num_chunks && s == HSA_STATUS_SUCCESS; ++p) {
    const int32_t c = job.arrival[p];
    if (job.resident[c]) continue;
    const int64_t r0 = job.chunk_begin[c], r1 = job.chunk_begin[c + 1];
    int32_t queued = 0;  // data copies of this chunk queued (the chunk signal starts at ntensors x P)
    for (int32_t q = 0; q < P && s == HSA_STATUS_SUCCESS; ++q) {
      const hsa_amd_sdma_engine_id_t eng = e->ids[(i * P + q) % used];
      const int64_t p0 = r0 + (r1 - r0) * q / P, p1 = r0 + (r1 - r0) * (q + 1) / P;
      for (int x = 0; x < job.ntensors && s == HSA_STATUS_SUCCESS; ++x) {
        if (p1 == p0) {  // an empty piece (fewer rows than pieces): nothing to copy
          hsa_signal_subtract_screlease(r.chunk[i], 1);
          ++queued;
          continue;
        }
        const int64_t off = p0 * job.row_bytes[x], bytes = (p1 - p0) * job.row_bytes[x];
        s = hsa_amd_memory_async_copy_on_engine(job.dst[x] + off, e->gpu, job.src[x] + off, e->gpu,
                                                static_cast<size_t>(bytes), 1, &r.gate, r.chunk[i], eng, true);
        what = "SDMA chunk copy";
        if (s == HSA_STATUS_SUCCESS) ++queued;
      }
    }
    if (s != HSA_STATUS_SUCCESS) {
      // the copies not queued will never count the chunk signal down
      hsa_signal_subtract_screlease(r.chunk[i], job.ntensors * P - queued);
      break;
    }
    s = hsa_amd_memory_async_copy_on_engine(job.flags + c, e->gpu, job.epoch_word, e->gpu, sizeof(uint32_t), 1,
                                            &r.chunk[i], r.done, e->ids[(i * P) % used], true);
    what = "SDMA flag copy";
    if (s == HSA_STATUS_SUCCESS) ++i;
  }
  if (s != HSA_STATUS_SUCCESS) {
    // flag copies that were not queued will never count the record down; the
    // queued ones still run once the gate opens
    hsa_signal_subtract_screlease(r.done, copied - i);
    return hsa_fail(s, what);
  }
  return SYNC_OK;
}

void sdma_release_all() {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& kv : g_engines) {
    Engines& e = *kv.second;
    if (!e.ready) continue;
    std::lock_guard<std::mutex> lk2(e.mu);
    for (Record& r : e.rec) {
      (void)quiesce(r);  // bounded; a record still busy after the bound is released anyway
      if (r.gate.handle) (void)hsa_signal_destroy(r.gate);
      if (r.done.handle) (void)hsa_signal_destroy(r.done);
      for (hsa_signal_t s : r.chunk) (void)hsa_signal_destroy(s);
      r = Record{};
    }
    (void)hsa_shut_down();  // the reference taken when the engines were first used
  }
  g_engines.clear();
}

int sdma_quiesce_all(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_engines.find(dev);
  if (it == g_engines.end() || !it->second->ready) return SYNC_OK;
  Engines& e = *it->second;
  std::lock_guard<std::mutex> lk2(e.mu);
  for (Record& r : e.rec) {
    const int rc = quiesce(r);
    if (rc) return rc;
  }
  return SYNC_OK;
}

}  // namespace syncov
