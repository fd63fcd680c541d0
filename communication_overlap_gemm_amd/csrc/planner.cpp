// Chunk planner (see planner.hpp for what it encodes and where from).
#include "planner.hpp"

#include <algorithm>
#include <numeric>
#include <tuple>

namespace syncov {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t wrap(int64_t x, int32_t w) {
  int64_t r = x % w;
  return static_cast<int32_t>(r < 0 ? r + w : r);
}

}  // namespace

bool build_plan(const sync_plan_desc& d, Plan& p, std::string& err) {
  p = Plan{};
  p.desc = d;
  p.desc.explicit_order = nullptr;
  const bool head = d.op == SYNC_OP_HEAD_ATTN;
  const bool attn = d.op == SYNC_OP_RING_ATTN || head;
  const bool rs = d.op == SYNC_OP_GEMM_RS;
  if (d.op != SYNC_OP_AG_GEMM && !rs && !attn) {
    err = "op must be AG_GEMM, GEMM_RS, RING_ATTN or HEAD_ATTN";
    return false;
  }
  if (d.world < 1) { err = "world must be >= 1"; return false; }
  if (d.rank < 0 || d.rank >= d.world) { err = "rank out of range"; return false; }
  if (d.ring_dir != 1 && d.ring_dir != -1) { err = "ring_dir must be +1 or -1"; return false; }
  if (d.m < 1 || d.n < 1 || d.k < 1) { err = "m, n, k must be positive"; return false; }
  if (d.tile_m < 1) { err = "tile_m must be positive"; return false; }
  if (d.tile_order < SYNC_ORDER_ROW_MAJOR || d.tile_order > SYNC_ORDER_SWIZZLED) { err = "bad tile_order"; return false; }
  if (d.group_m < 0) { err = "group_m must be >= 0"; return false; }
  if (d.reserved[0]) { err = "reserved fields must be zero"; return false; }
  p.desc.shard_rows = nullptr;
  const int32_t W = d.world, s = d.split;
  const int64_t G = d.group_m > 0 ? d.group_m : 4;

  std::vector<int64_t> rows_of(W), base(W + 1, 0);  // rows of each shard and their prefix sums
  if (attn) {
    if (d.heads_q < 1 || d.heads_kv < 1 || d.heads_q % d.heads_kv) { err = "heads_q must be a positive multiple of heads_kv"; return false; }
    if (d.shard_rows) { err = "shard_rows is for the GEMM ops"; return false; }
    if (head && d.m != static_cast<int64_t>(W) * d.n) {
      err = "head-parallel attention: the queries are every token (m = world * n)";
      return false;
    }
    p.shard_rows = d.n;
    p.rows = static_cast<int64_t>(W) * d.n;
    std::fill(rows_of.begin(), rows_of.end(), p.shard_rows);
  } else {
    if (d.tile_n < 1) { err = "tile_n must be positive"; return false; }
    if (d.b_layout != SYNC_B_KN && d.b_layout != SYNC_B_NK) { err = "bad b_layout"; return false; }
    if (d.shard_rows) {
      int64_t total = 0;
      for (int32_t w = 0; w < W; ++w) {
        if (d.shard_rows[w] < 1) { err = "shard_rows must be positive"; return false; }
        rows_of[w] = d.shard_rows[w];
        total += rows_of[w];
      }
      if (total != d.m) { err = "shard_rows must sum to m"; return false; }
      p.shard_rows = *std::min_element(rows_of.begin(), rows_of.end());
    } else {
      if (d.m % W) { err = "m must be divisible by world"; return false; }
      p.shard_rows = d.m / W;
      std::fill(rows_of.begin(), rows_of.end(), p.shard_rows);
    }
    p.rows = d.m;
  }
  for (int32_t w = 0; w < W; ++w) base[w + 1] = base[w] + rows_of[w];
  if (s < 1 || s > p.shard_rows) { err = "split must be in [1, rows per shard]"; return false; }

  // shard consumed (AG, attention) or sent (RS) at each ring step
  std::vector<int32_t> step_shard(W);
  if ((d.pattern == SYNC_PAT_HIER_SWIZZLE) != (d.hier_group != 0)) {
    err = "hier_group is set exactly for the hierarchical swizzle pattern";
    return false;
  }
  if (d.pattern == SYNC_PAT_RING || d.pattern == SYNC_PAT_MESH) {
    for (int32_t st = 0; st < W; ++st)
      step_shard[st] = wrap(static_cast<int64_t>(d.rank) - static_cast<int64_t>(d.ring_dir) * (rs ? st + 1 : st), W);
  } else if (d.pattern == SYNC_PAT_EXPLICIT) {
    if (!d.explicit_order) { err = "EXPLICIT pattern needs explicit_order"; return false; }
    std::vector<char> seen(W, 0);
    for (int32_t st = 0; st < W; ++st) {
      int32_t w = d.explicit_order[st];
      if (w < 0 || w >= W || seen[w]) { err = "explicit_order is not a permutation of shards"; return false; }
      seen[w] = 1;
      step_shard[st] = w;
    }
    p.explicit_order = step_shard;
  } else if (d.pattern == SYNC_PAT_HIER_SWIZZLE) {
    // groups of g consecutive ranks: own group first, then each group in
    // turn; inside a group, start at this rank's local index (at every step
    // the ranks of a group pull from distinct peers).  RS: reversed.
    const int32_t g = d.hier_group;
    if (g < 1 || W % g) { err = "hier_group must divide world"; return false; }
    const int32_t groups = W / g, my_group = d.rank / g, my_local = d.rank % g;
    for (int32_t a = 0; a < groups; ++a)
      for (int32_t b = 0; b < g; ++b) {
        const int32_t st = a * g + b, w = ((my_group + a) % groups) * g + (my_local + b) % g;
        step_shard[rs ? W - 1 - st : st] = w;
      }
  } else {
    err = "bad pattern";
    return false;
  }
  std::vector<int32_t> step_of(W);
  for (int32_t st = 0; st < W; ++st) step_of[step_shard[st]] = st;

  const int32_t C = W * s;
  p.num_chunks = C;
  p.chunk_begin.resize(C + 1);
  p.chunk_pos.resize(C);
  p.arrival.resize(C);
  p.resident.resize(C);
  for (int32_t w = 0; w < W; ++w)
    for (int32_t q = 0; q < s; ++q) {
      const int32_t c = w * s + q;
      p.chunk_begin[c] = base[w] + (static_cast<int64_t>(q) * rows_of[w]) / s;
      // mesh: every peer's link runs at once, so sub-chunk q of every shard
      // arrives before sub-chunk q + 1 of any (ties in ring step order)
      p.chunk_pos[c] = d.pattern == SYNC_PAT_MESH ? q * W + step_of[w] : step_of[w] * s + q;
      p.resident[c] = (!rs && d.local_resident && w == d.rank) ? 1 : 0;
    }
  p.chunk_begin[C] = p.rows;
  for (int32_t c = 0; c < C; ++c) p.arrival[p.chunk_pos[c]] = c;

  // tile grid
  const int64_t tm = ceil_div(d.m, d.tile_m);
  const int64_t tn = attn ? d.heads_q : ceil_div(d.n, d.tile_n);
  if (tm * tn > INT32_MAX / 2) { err = "too many tiles"; return false; }
  p.tiles_m = static_cast<int32_t>(tm);
  p.tiles_n = static_cast<int32_t>(tn);
  const int32_t T = p.tiles_m * p.tiles_n;
  p.num_tiles = T;

  // chunks met by each tile row: a contiguous id range [lo, hi)
  std::vector<int32_t> row_lo(tm), row_hi(tm);
  for (int64_t i = 0; i < tm; ++i) {
    if (attn && !head) { row_lo[i] = 0; row_hi[i] = C; continue; }  // ring: every KV block
    const int64_t r0 = i * d.tile_m, r1 = std::min<int64_t>(r0 + d.tile_m, d.m);
    // first chunk whose end is past r0; last chunk whose begin is before r1
    auto first = std::upper_bound(p.chunk_begin.begin() + 1, p.chunk_begin.end(), r0) - (p.chunk_begin.begin() + 1);
    auto last = std::lower_bound(p.chunk_begin.begin(), p.chunk_begin.end() - 1, r1) - p.chunk_begin.begin();
    row_lo[i] = static_cast<int32_t>(first);
    row_hi[i] = static_cast<int32_t>(last);
  }
  p.dep_ptr.resize(T + 1);
  p.tile_key.resize(T);
  p.dep_ptr[0] = 0;
  for (int32_t t = 0; t < T; ++t) {
    const int32_t i = t / p.tiles_n;
    int32_t key = rs ? INT32_MAX : -1;
    for (int32_t c = row_lo[i]; c < row_hi[i]; ++c) {
      p.dep_idx.push_back(c);
      key = rs ? std::min(key, p.chunk_pos[c]) : std::max(key, p.chunk_pos[c]);
    }
    p.dep_ptr[t + 1] = static_cast<int64_t>(p.dep_idx.size());
    p.tile_key[t] = key;
  }
  // transpose: tiles per chunk, ascending tile id
  p.tiles_in.assign(C, 0);
  for (int32_t c : p.dep_idx) ++p.tiles_in[c];
  p.inv_ptr.assign(C + 1, 0);
  for (int32_t c = 0; c < C; ++c) p.inv_ptr[c + 1] = p.inv_ptr[c] + p.tiles_in[c];
  p.inv_idx.resize(p.dep_idx.size());
  {
    std::vector<int64_t> fill(p.inv_ptr.begin(), p.inv_ptr.end() - 1);
    for (int32_t t = 0; t < T; ++t)
      for (int64_t e = p.dep_ptr[t]; e < p.dep_ptr[t + 1]; ++e) p.inv_idx[fill[p.dep_idx[e]]++] = t;
  }

  // traversal order
  p.tile_order.resize(T);
  std::iota(p.tile_order.begin(), p.tile_order.end(), 0);
  const int32_t Tn = p.tiles_n;
  if (d.tile_order == SYNC_ORDER_CHUNK_MAJOR) {
    std::sort(p.tile_order.begin(), p.tile_order.end(), [&](int32_t a, int32_t b) {
      return std::make_tuple(p.tile_key[a], a / Tn, a % Tn) < std::make_tuple(p.tile_key[b], b / Tn, b % Tn);
    });
  } else if (d.tile_order == SYNC_ORDER_SWIZZLED) {
    std::sort(p.tile_order.begin(), p.tile_order.end(), [&](int32_t a, int32_t b) {
      return std::make_tuple(p.tile_key[a], (a / Tn) / G, a % Tn, a / Tn) <
             std::make_tuple(p.tile_key[b], (b / Tn) / G, b % Tn, b / Tn);
    });
  }
  return true;
}

}  // namespace syncov
