// Autotuner over the overlapped GEMM's configuration space (split factor,
// tile shape, tile order, copy-CU count), built on the public C ABI: each
// candidate is planned, run and timed with device events on the caller's
// stream, and the fastest is kept.  Results are cached in-process and,
// optionally, in a text file (SYNC_TUNE_CACHE).
//
// The pages tune chunk size, split factor and communication backend per
// workload and leave the tuning cost out of their measurements (Syncopate
// summary page, "Core method" and "Limits"); the tile order and tile shape
// are the knobs of the reordered GEMM (Entwine abstract).
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "sync_overlap.h"

namespace syncov {
int set_error(int code, const std::string& msg);
}

namespace {

using syncov::set_error;

std::mutex g_cache_mu;
std::map<std::string, sync_tune_result> g_cache;
std::string g_file_loaded;  // cache file already read into g_cache ("" = none)

const char* cache_path() {
  const char* p = std::getenv("SYNC_TUNE_CACHE");
  return (p && *p) ? p : nullptr;
}

// Cache file: one line per result,
// "key<TAB>split tile_m tile_n order copy_cus best_ms backend agent search_wall_ms".
void load_file_locked() {
  const char* path = cache_path();
  if (!path || g_file_loaded == path) return;
  g_file_loaded = path;
  std::ifstream f(path);
  std::string line;
  while (std::getline(f, line)) {
    const size_t tab = line.find('\t');
    if (tab == std::string::npos) continue;
    sync_tune_result r{};
    std::istringstream in(line.substr(tab + 1));
    if (in >> r.split >> r.tile_m >> r.tile_n >> r.tile_order >> r.copy_cus >> r.best_ms >> r.backend >> r.agent) {
      if (!(in >> r.search_wall_ms)) r.search_wall_ms = 0.f;  // lines written before the field existed
      g_cache[line.substr(0, tab)] = r;
    }
  }
}

void append_file_locked(const std::string& key, const sync_tune_result& r) {
  const char* path = cache_path();
  if (!path) return;
  std::ofstream f(path, std::ios::app);
  f << key << '\t' << r.split << ' ' << r.tile_m << ' ' << r.tile_n << ' ' << r.tile_order << ' ' << r.copy_cus << ' '
    << r.best_ms << ' ' << r.backend << ' ' << r.agent << ' ' << r.search_wall_ms << '\n';
}

std::string list_str(const int32_t* v, int32_t n) {
  std::string s;
  for (int32_t i = 0; i < n; ++i) s += (i ? "," : "") + std::to_string(v[i]);
  return s;
}

std::string cache_key(const sync_plan_desc& b, const sync_tune_space& sp, int32_t c_dtype) {
  sync_device_info di{};
  (void)sync_get_device_info(&di);
  int hip_version = 0;
  (void)hipRuntimeGetVersion(&hip_version);
  std::ostringstream k;
  k << di.arch << '/' << di.num_cus << " hip" << hip_version << " op" << b.op << " m" << b.m << " n" << b.n << " k" << b.k << " W" << b.world
    << " r" << b.rank << " d" << b.ring_dir << " pat" << b.pattern << " res" << b.local_resident << " B"
    << b.b_layout << " g" << b.group_m << " h" << b.hier_group << " C" << c_dtype << " S[" << list_str(sp.splits, sp.n_splits) << "] T["
    << list_str(sp.tiles, 2 * sp.n_tiles) << "] O[" << list_str(sp.orders, sp.n_orders) << "] U["
    << list_str(sp.copy_cus, sp.n_copy_cus) << "]";
  if (sp.n_agents > 0) {
    k << " A[";
    for (int32_t i = 0; i < sp.n_agents; ++i) {
      const sync_copy_cfg& c = sp.agents[i];
      k << (i ? ";" : "") << c.backend << ',' << c.copy_cus << ',' << c.copy_teams << ',' << c.copy_kslices << ','
        << c.copy_streaming << ',' << c.copy_link_gbps << ',' << c.copy_lead_slice;
    }
    k << "]";
  }
  if (b.pattern == SYNC_PAT_EXPLICIT && b.explicit_order) k << " E[" << list_str(b.explicit_order, b.world) << "]";
  return k.str();
}

int check_space(const sync_plan_desc* base, const sync_tune_space* sp) {
  if (!base || !sp) return set_error(SYNC_EINVAL, "base and space must be non-NULL");
  if (base->op != SYNC_OP_AG_GEMM && base->op != SYNC_OP_GEMM_RS)
    return set_error(SYNC_EINVAL, "the autotuner covers the GEMM ops (AG, RS)");
  if (sp->reserved) return set_error(SYNC_EINVAL, "sync_tune_space.reserved must be zero");
  if (!sp->splits || sp->n_splits < 1 || !sp->tiles || sp->n_tiles < 1 || !sp->orders || sp->n_orders < 1)
    return set_error(SYNC_EINVAL, "every list of the space needs at least one entry");
  if (sp->n_agents < 0 || (sp->n_agents > 0 && !sp->agents))
    return set_error(SYNC_EINVAL, "agents must hold n_agents copy configurations");
  if (sp->n_agents == 0 && (!sp->copy_cus || sp->n_copy_cus < 1))
    return set_error(SYNC_EINVAL, "the space needs copy-CU counts or a list of copy agents");
  for (int32_t i = 0; i < sp->n_agents; ++i) {
    const sync_copy_cfg& c = sp->agents[i];
    if (c.flags || c.host_gates)
      return set_error(SYNC_EINVAL, "tuned copy agents take no run-mode flags and no host gates");
    if (c.backend != SYNC_COPY_SDMA && c.backend != SYNC_COPY_CU && c.backend != SYNC_COPY_COLOCATED &&
        c.backend != SYNC_COPY_EPILOGUE)
      return set_error(SYNC_EINVAL, "tuned copy agents are SDMA, CU, COLOCATED or EPILOGUE");
  }
  if (sp->warmup < 0 || sp->iters < 0) return set_error(SYNC_EINVAL, "warmup and iters must be >= 0");
  return SYNC_OK;
}

template <typename F>
void for_each_candidate(const sync_plan_desc& base, const sync_tune_space& sp, F f) {
  for (int32_t a = 0; a < sp.n_splits; ++a)
    for (int32_t t = 0; t < sp.n_tiles; ++t)
      for (int32_t o = 0; o < sp.n_orders; ++o) {
        sync_plan_desc d = base;
        d.split = sp.splits[a];
        d.tile_m = sp.tiles[2 * t];
        d.tile_n = sp.tiles[2 * t + 1];
        d.tile_order = sp.orders[o];
        f(d);
      }
}

}  // namespace

extern "C" {

size_t sync_tune_workspace_size(const sync_plan_desc* base, const sync_tune_space* space) {
  if (check_space(base, space)) return 0;
  size_t need = 0;
  for_each_candidate(*base, *space, [&](const sync_plan_desc& d) {
    sync_plan_t p = nullptr;
    if (sync_plan(&d, &p) == SYNC_OK) {
      const size_t s = sync_workspace_size(p);
      if (s > need) need = s;
      sync_plan_destroy(p);
    }
  });
  return need;
}

int sync_autotune(const sync_plan_desc* base, const sync_tune_space* space, const sync_tune_buffers* bufs,
                  sync_tune_result* out) {
  int rc = check_space(base, space);
  if (rc) return rc;
  if (!bufs || !out) return set_error(SYNC_EINVAL, "bufs and out must be non-NULL");
  if (!bufs->ws || (reinterpret_cast<uintptr_t>(bufs->ws) & 255u))
    return set_error(SYNC_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  const sync_tune_space& sp = *space;
  const auto t_start = std::chrono::steady_clock::now();
  auto wall_ms = [&]() {
    return std::chrono::duration<float, std::milli>(std::chrono::steady_clock::now() - t_start).count();
  };
  const std::string key = cache_key(*base, sp, bufs->c_dtype);
  if (!sp.force) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    load_file_locked();
    auto it = g_cache.find(key);
    if (it != g_cache.end()) {
      *out = it->second;
      out->candidates_run = 0;
      out->candidates_skipped = 0;
      out->from_cache = 1;
      out->call_wall_ms = wall_ms();
      return SYNC_OK;
    }
  }
  const int warmup = sp.warmup ? sp.warmup : 3, iters = sp.iters ? sp.iters : 10;
  hipStream_t st = static_cast<hipStream_t>(bufs->stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
    return set_error(SYNC_EHIP, "hipEventCreate failed");
  sync_tune_result best{};
  best.best_ms = -1.f;
  int run = 0, skipped = 0;
  int hard = SYNC_OK;
  for_each_candidate(*base, sp, [&](const sync_plan_desc& d) {
    if (hard) return;
    sync_plan_t p = nullptr;
    const int32_t n_cfg = sp.n_agents > 0 ? sp.n_agents : sp.n_copy_cus;
    if (sync_plan(&d, &p) != SYNC_OK) {
      skipped += n_cfg;
      return;
    }
    for (int32_t u = 0; u < n_cfg && !hard; ++u) {
      sync_copy_cfg cfg{};
      if (sp.n_agents > 0) {
        cfg = sp.agents[u];
      } else {
        cfg.backend = SYNC_COPY_CU;
        cfg.copy_cus = sp.copy_cus[u];
      }
      cfg.timeout_ns = sp.timeout_ns ? sp.timeout_ns : 100000000ull;
      auto call = [&]() -> int {
        if (d.op == SYNC_OP_AG_GEMM)
          return sync_ag_gemm(p, &cfg, bufs->a_peer, bufs->a, bufs->b, bufs->c, bufs->c_dtype, bufs->ws, bufs->stream,
                              nullptr);
        return sync_gemm_rs(p, &cfg, bufs->a, bufs->b, bufs->c, bufs->c_dtype, bufs->staging, bufs->ws, bufs->stream,
                            nullptr);
      };
      int crc = sync_workspace_init(p, bufs->ws, bufs->stream);
      for (int i = 0; i < warmup && crc == SYNC_OK; ++i) crc = call();
      if (crc == SYNC_EINVAL || crc == SYNC_EUNSUPPORTED) {  // not a valid candidate for these kernels
        ++skipped;
        continue;
      }
      if (crc != SYNC_OK) {
        hard = crc;
        break;
      }
      int32_t ch = -1;
      if (sync_workspace_status(bufs->ws, bufs->stream, &ch) != SYNC_OK) {  // timed out: drop it
        ++skipped;
        (void)sync_workspace_init(p, bufs->ws, bufs->stream);
        continue;
      }
      if (hipEventRecord(e0, st) != hipSuccess) {
        hard = set_error(SYNC_EHIP, "hipEventRecord failed");
        break;
      }
      for (int i = 0; i < iters && crc == SYNC_OK; ++i) crc = call();
      if (crc != SYNC_OK) {
        hard = crc;
        break;
      }
      float ms = 0.f;
      if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
          hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
        hard = set_error(SYNC_EHIP, "event timing failed");
        break;
      }
      if (sync_workspace_status(bufs->ws, bufs->stream, &ch) != SYNC_OK) {
        ++skipped;
        (void)sync_workspace_init(p, bufs->ws, bufs->stream);
        continue;
      }
      ++run;
      ms /= static_cast<float>(iters);
      if (best.best_ms < 0.f || ms < best.best_ms) {
        best.split = d.split;
        best.tile_m = d.tile_m;
        best.tile_n = d.tile_n;
        best.tile_order = d.tile_order;
        best.copy_cus = cfg.copy_cus;
        best.backend = cfg.backend;
        best.agent = sp.n_agents > 0 ? u : -1;
        best.best_ms = ms;
      }
    }
    sync_plan_destroy(p);
  });
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (hard) return hard;
  if (run == 0) return set_error(SYNC_EUNSUPPORTED, "no candidate of the space could run");
  best.candidates_run = run;
  best.candidates_skipped = skipped;
  best.from_cache = 0;
  best.search_wall_ms = wall_ms();
  best.call_wall_ms = best.search_wall_ms;
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    load_file_locked();
    g_cache[key] = best;
    append_file_locked(key, best);
  }
  *out = best;
  return SYNC_OK;
}

void sync_tune_forget(void) {
  std::lock_guard<std::mutex> lk(g_cache_mu);
  g_cache.clear();
  g_file_loaded.clear();
}

}  // extern "C"
