// Host-side checks of the C ABI, built with AddressSanitizer and UBSan and
// run without a GPU: plans over a wide enumeration of descriptors (valid and
// invalid, every op and pattern, uneven shards), the invariants of their
// exported tables, and every entry point's argument checks.  Calls that get
// past the checks end with SYNC_ENODEV (no device), so only host code runs.
// Exit status 0 when every check holds; a sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sync_overlap.h"

namespace {

int g_fail = 0, g_plans = 0, g_rejected = 0, g_calls = 0;

#define CHECK(c)                                                                \
  do {                                                                          \
    if (!(c)) {                                                                 \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);       \
      ++g_fail;                                                                 \
    }                                                                           \
  } while (0)

// Invariants of a plan's exported tables (the oracle tests pin the values;
// here only that every index stays inside its array).
void check_tables(sync_plan_t p, const sync_plan_desc& d) {
  sync_plan_info in{};
  CHECK(sync_plan_get_info(p, &in) == SYNC_OK);
  const int32_t C = in.num_chunks, T = in.num_tiles;
  CHECK(C == d.world * d.split && T == in.tiles_m * in.tiles_n && in.num_deps >= T);
  std::vector<int64_t> cb(C + 1), dptr(T + 1), iptr(C + 1);
  std::vector<int32_t> pos(C), arr(C), res(C), tin(C), ord(T), key(T), didx(in.num_deps), iidx(in.num_deps);
  sync_plan_tables t{cb.data(), pos.data(), arr.data(), res.data(), tin.data(), ord.data(),
                     key.data(), dptr.data(), didx.data(), iptr.data(), iidx.data()};
  CHECK(sync_plan_export(p, &t) == SYNC_OK);
  std::vector<int> seen_c(C, 0), seen_t(T, 0);
  for (int32_t c = 0; c < C; ++c) {
    CHECK(cb[c] < cb[c + 1]);
    CHECK(arr[c] >= 0 && arr[c] < C);
    if (arr[c] >= 0 && arr[c] < C) {
      ++seen_c[arr[c]];
      CHECK(pos[arr[c]] == c);
    }
    CHECK(res[c] == 0 || res[c] == 1);
  }
  for (int32_t c = 0; c < C; ++c) CHECK(seen_c[c] == 1);
  for (int32_t i = 0; i < T; ++i) {
    CHECK(ord[i] >= 0 && ord[i] < T);
    if (ord[i] >= 0 && ord[i] < T) ++seen_t[ord[i]];
    CHECK(dptr[i] <= dptr[i + 1]);
  }
  for (int32_t i = 0; i < T; ++i) CHECK(seen_t[i] == 1);
  CHECK(dptr[0] == 0 && dptr[T] == in.num_deps && iptr[0] == 0 && iptr[C] == in.num_deps);
  for (int64_t e = 0; e < in.num_deps; ++e) CHECK(didx[e] >= 0 && didx[e] < C && iidx[e] >= 0 && iidx[e] < T);
  for (int32_t c = 0; c < C; ++c) CHECK(tin[c] == iptr[c + 1] - iptr[c]);
  CHECK(sync_workspace_size(p) > 0);
  // a partial export (NULL members skipped) must not write through them
  sync_plan_tables part{};
  part.arrival = arr.data();
  CHECK(sync_plan_export(p, &part) == SYNC_OK);
}

void try_plan(sync_plan_desc d) {
  sync_plan_t p = nullptr;
  const int rc = sync_plan(&d, &p);
  if (rc == SYNC_OK) {
    ++g_plans;
    CHECK(p != nullptr);
    check_tables(p, d);
    sync_plan_destroy(p);
  } else {
    ++g_rejected;
    CHECK(rc == SYNC_EINVAL && p == nullptr && std::strlen(sync_last_error()) > 0);
  }
}

sync_plan_desc base_desc(int32_t op, int64_t m, int64_t n, int64_t k, int32_t world) {
  sync_plan_desc d{};
  d.op = op;
  d.m = m;
  d.n = n;
  d.k = k;
  d.world = world;
  d.ring_dir = 1;
  d.split = 1;
  d.tile_m = 4;
  d.tile_n = 2;
  d.tile_order = SYNC_ORDER_CHUNK_MAJOR;
  d.local_resident = 1;
  d.b_layout = SYNC_B_KN;
  return d;
}

void enumerate_plans() {
  const int32_t ops[] = {SYNC_OP_AG_GEMM, SYNC_OP_GEMM_RS, SYNC_OP_RING_ATTN, SYNC_OP_HEAD_ATTN, 0, 7};
  const int32_t orders_all[] = {SYNC_ORDER_ROW_MAJOR, SYNC_ORDER_CHUNK_MAJOR, SYNC_ORDER_SWIZZLED};
  for (int32_t op : ops)
    for (int32_t W : {1, 2, 3, 4, 6, 8})
      for (int32_t r : {0, W / 2, W - 1, W})  // W: out of range
        for (int32_t dir : {1, -1, 0})
          for (int32_t pat : {int32_t{SYNC_PAT_RING}, int32_t{SYNC_PAT_EXPLICIT}, int32_t{SYNC_PAT_HIER_SWIZZLE},
                              int32_t{SYNC_PAT_MESH}, int32_t{9}})
            for (int32_t s : {1, 2, 3, 7})
              for (int32_t tm : {1, 3, 4, 64})
                for (int32_t order : orders_all) {
                  const bool attn = op == SYNC_OP_RING_ATTN || op == SYNC_OP_HEAD_ATTN;
                  const int64_t n = attn ? 5 : 6, m = op == SYNC_OP_HEAD_ATTN ? W * n : (attn ? 9 : W * 5);
                  sync_plan_desc d = base_desc(op, m, n, attn ? 128 : 64, W);
                  d.rank = r;
                  d.ring_dir = dir;
                  d.pattern = pat;
                  d.split = s;
                  d.tile_m = tm;
                  d.tile_order = order;
                  d.group_m = 2;
                  if (attn) {
                    d.heads_q = 4;
                    d.heads_kv = 2;
                  }
                  std::vector<int32_t> perm(W);
                  for (int32_t i = 0; i < W; ++i) perm[i] = (i * 3 + 1) % W;  // a permutation only for some W
                  if (pat == SYNC_PAT_EXPLICIT) d.explicit_order = perm.data();
                  if (pat == SYNC_PAT_HIER_SWIZZLE) {
                    for (int32_t g : {1, 2, 3, W}) {
                      d.hier_group = g;
                      try_plan(d);
                    }
                    continue;
                  }
                  try_plan(d);
                }
  // uneven shards (an all-to-all's receive side), valid and invalid
  const int64_t rows_sets[][4] = {{3, 1, 4, 1}, {1, 1, 1, 1}, {5, 0, 2, 2}, {7, 9, 2, 6}, {-1, 4, 4, 4}};
  for (const auto& rows : rows_sets)
    for (int32_t op : {int32_t{SYNC_OP_AG_GEMM}, int32_t{SYNC_OP_GEMM_RS}, int32_t{SYNC_OP_RING_ATTN}})
      for (int32_t s : {1, 2})
        for (int64_t m : {9, 10, 24}) {
          sync_plan_desc d = base_desc(op, m, 6, 64, 4);
          d.shard_rows = rows;
          d.split = s;
          d.heads_q = d.heads_kv = 1;
          try_plan(d);
        }
  // degenerate and hostile sizes
  for (int64_t m : {0, -4, 1, 3}) {
    sync_plan_desc d = base_desc(SYNC_OP_AG_GEMM, m, 4, 64, 1);
    try_plan(d);
  }
  {
    sync_plan_desc d = base_desc(SYNC_OP_AG_GEMM, 8, 4, 64, 4);
    d.reserved[0] = 1;
    try_plan(d);
    d = base_desc(SYNC_OP_AG_GEMM, 8, 4, 64, 4);
    d.pattern = SYNC_PAT_EXPLICIT;  // no order given
    try_plan(d);
    d.tile_m = 0;
    try_plan(d);
  }
  CHECK(sync_plan(nullptr, nullptr) == SYNC_EINVAL);
  sync_plan_t p = nullptr;
  CHECK(sync_plan(nullptr, &p) == SYNC_EINVAL && p == nullptr);
  sync_plan_destroy(nullptr);
}

// Every entry point with a plan of each op and argument sets that the host
// checks accept or reject; none may reach device work.
void entry_points() {
  struct P {
    int32_t op;
    sync_plan_t p;
  } plans[4] = {{SYNC_OP_AG_GEMM, nullptr}, {SYNC_OP_GEMM_RS, nullptr}, {SYNC_OP_RING_ATTN, nullptr},
                {SYNC_OP_HEAD_ATTN, nullptr}};
  for (auto& x : plans) {
    const bool attn = x.op == SYNC_OP_RING_ATTN || x.op == SYNC_OP_HEAD_ATTN;
    sync_plan_desc d = base_desc(x.op, x.op == SYNC_OP_HEAD_ATTN ? 256 : 1024, attn ? 64 : 512, attn ? 128 : 256, 4);
    d.tile_m = attn ? 64 : 128;
    d.tile_n = 128;
    if (attn) {
      d.heads_q = 4;
      d.heads_kv = 1;
    }
    CHECK(sync_plan(&d, &x.p) == SYNC_OK);
  }
  alignas(256) static char buf[1 << 16];
  void* ws = buf;  // host memory: only passed through the checks, never read by the device
  const void* in = buf;
  float* f = reinterpret_cast<float*>(buf);
  sync_copy_cfg good{};
  good.backend = SYNC_COPY_CU;
  good.copy_cus = 32;
  std::vector<sync_copy_cfg> cfgs;
  cfgs.push_back(good);
  for (int i = 0; i < 12; ++i) {
    sync_copy_cfg c = good;
    switch (i) {
      case 0: c.backend = 99; break;
      case 1: c.copy_teams = -1; break;
      case 2: c.copy_kslices = 9; break;
      case 3: c.copy_kslices = 2; break;
      case 4: c.copy_streaming = 2; break;
      case 5: c.copy_lead_slice = 1; break;
      case 6: c.copy_link_gbps = -3.f; break;
      case 7: c.flags = 1 << 20; break;
      case 8: c.flags = SYNC_RUN_COPY_ONLY | SYNC_RUN_COMPUTE_ONLY; break;
      case 9: c.flags = SYNC_RUN_WITHHOLD; c.withhold_chunk = 99; break;
      case 10: c.backend = SYNC_COPY_HOST_GATED; break;
      case 11: c.backend = SYNC_COPY_EPILOGUE; break;
    }
    cfgs.push_back(c);
  }
  for (auto& x : plans) {
    for (sync_plan_t p : {x.p, static_cast<sync_plan_t>(nullptr)})
      for (size_t ci = 0; ci <= cfgs.size(); ++ci) {
        const sync_copy_cfg* c = ci == 0 ? nullptr : &cfgs[ci - 1];
        for (void* w : {ws, static_cast<void*>(buf + 1), static_cast<void*>(nullptr)}) {
          int rc[8];
          rc[0] = sync_ag_gemm(p, c, in, buf, in, buf, SYNC_DTYPE_F32, w, nullptr, nullptr);
          rc[1] = sync_ag_gemm_noalloc(p, c, in, buf, in, buf, SYNC_DTYPE_BF16, nullptr);
          rc[2] = sync_gemm_rs(p, c, in, in, buf, SYNC_DTYPE_F32, buf, w, nullptr, nullptr);
          rc[3] = sync_gemm_rs_reduce(p, c, in, in, buf, f, buf, w, nullptr, nullptr);
          rc[4] = sync_gemm_ar(p, c, in, in, buf, f, f, f, buf, w, nullptr, nullptr);
          rc[5] = sync_gemm_split(p, c, in, buf, in, buf, SYNC_DTYPE_F32, buf, w, nullptr, buf);
          rc[6] = sync_ring_attn_step(p, c, in, in, in, buf, buf, f, f, f, f, 0.1f, SYNC_ATTN_INIT, w, nullptr,
                                      nullptr);
          rc[7] = sync_head_attn(p, c, in, in, in, buf, buf, buf, f, f, 0.1f, w, nullptr, nullptr);
          for (int i = 0; i < 8; ++i) {
            ++g_calls;
            CHECK(rc[i] == SYNC_EINVAL || rc[i] == SYNC_EUNSUPPORTED || rc[i] == SYNC_ENODEV);
            CHECK(std::strlen(sync_last_error()) > 0);
          }
        }
      }
    CHECK(sync_workspace_init(x.p, ws, nullptr) != SYNC_OK);
    CHECK(sync_workspace_init(x.p, nullptr, nullptr) == SYNC_EINVAL);
    sync_trace tr{};
    CHECK(sync_trace_export(x.p, ws, nullptr, &tr) != SYNC_OK);
    CHECK(sync_trace_export(x.p, ws, nullptr, nullptr) != SYNC_OK);
    sync_plan_destroy(x.p);
  }
  int32_t ch = 0;
  CHECK(sync_workspace_status(nullptr, nullptr, &ch) != SYNC_OK);
  CHECK(sync_workspace_status(ws, nullptr, nullptr) != SYNC_OK);
  sync_timing tm[4];
  int32_t count = -1;
  CHECK(sync_read_timings(4, tm, &count) != SYNC_OK || count == 0);
  CHECK(sync_read_timings(4, nullptr, &count) == SYNC_EINVAL);
  CHECK(sync_read_timings(0, nullptr, nullptr) == SYNC_EINVAL);
  sync_device_info di{};
  CHECK(sync_get_device_info(&di) == SYNC_ENODEV);
  CHECK(sync_get_device_info(nullptr) == SYNC_EINVAL);
}

void autotune_checks() {
  const int32_t splits[] = {1, 2, 4}, tiles[] = {256, 256, 128, 128}, orders[] = {SYNC_ORDER_CHUNK_MAJOR},
                cus[] = {16, 32};
  sync_copy_cfg agents[3]{};
  agents[0].backend = SYNC_COPY_SDMA;
  agents[1].backend = SYNC_COPY_CU;
  agents[1].copy_cus = 32;
  agents[2].backend = SYNC_COPY_CU;
  agents[2].flags = SYNC_RUN_TIMED;  // rejected: tuned agents take no run flags
  for (int32_t op : {int32_t{SYNC_OP_AG_GEMM}, int32_t{SYNC_OP_GEMM_RS}, int32_t{SYNC_OP_RING_ATTN}})
    for (int variant = 0; variant < 6; ++variant) {
      sync_plan_desc b = base_desc(op, 8192, 1792, 4096, 8);
      b.heads_q = b.heads_kv = 1;
      sync_tune_space sp{};
      sp.splits = splits;
      sp.n_splits = 3;
      sp.tiles = tiles;
      sp.n_tiles = 2;
      sp.orders = orders;
      sp.n_orders = 1;
      sp.copy_cus = cus;
      sp.n_copy_cus = 2;
      if (variant == 1) sp.n_splits = 0;
      if (variant == 2) sp.reserved = 1;
      if (variant == 3) {
        sp.agents = agents;
        sp.n_agents = 2;
      }
      if (variant == 4) {
        sp.agents = agents;
        sp.n_agents = 3;
      }
      if (variant == 5) sp.warmup = -1;
      const size_t need = sync_tune_workspace_size(&b, &sp);
      CHECK((need > 0) == (op != SYNC_OP_RING_ATTN && (variant == 0 || variant == 3)));
      sync_tune_buffers bufs{};
      alignas(256) static char wsb[256];
      bufs.ws = wsb;
      sync_tune_result r{};
      const int rc = sync_autotune(&b, &sp, &bufs, &r);
      ++g_calls;
      CHECK(rc != SYNC_OK);
    }
  CHECK(sync_tune_workspace_size(nullptr, nullptr) == 0);
  sync_tune_forget();
}

}  // namespace

int main() {
  enumerate_plans();
  entry_points();
  autotune_checks();
  sync_shutdown();
  std::printf("host checks: %d plans built, %d rejected, %d calls checked, %d failures\n", g_plans, g_rejected, g_calls,
              g_fail);
  return g_fail ? 1 : 0;
}
