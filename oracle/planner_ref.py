"""ORACLE -- reference chunk planner.  Test infrastructure only: nothing on the
product path imports it; only the tests, the smoke check and the bench's CPU
baseline leg do.

What the pages fix (Syncopate summary page, "Core method", paper sec. 5.1-5.2
and Fig. 6; Syncopate review page, captions of Fig. 4-6; Entwine abstract):
  * communication is a plan of P2P/collective operations on *chunks*, each a
    block of a logical tensor that holds one or more compute tiles; a ring is
    one of the patterns a plan expresses;
  * the compiler builds the chunk-tile dependency graph (which chunks each tile
    consumes or produces) and makes a tile wait until its chunks are done;
  * the tile scheduler is rewritten: chunks are first put in communication
    order, then the traversal inside a chunk is kept or adjusted for locality;
  * (Entwine) tiles are reordered so that output for communication is produced
    at a steady pace, in the order it is sent.

The pages give no formula for any of this, so the encoding below is a reading;
parity of this planner with the pages is *unpinned* beyond the invariants,
brute-force enumerations and hand-worked fixtures the tests check.

Reading, in the order the planner applies it:
  R = M / W rows per shard (attention: M := W * n tokens, R = n); s = split.
  chunk c = w*s + q  (shard w, sub-chunk q):
      begin(c) = w*R + floor(q*R/s),  end(c) = w*R + floor((q+1)*R/s)
  Uneven shards (an all-to-all's receive side, GEMM ops only): shard w has
  R_w rows (given, summing to M) and starts at B_w = R_0 + ... + R_(w-1);
      begin(c) = B_w + floor(q*R_w/s),  with s <= min R_w
  ring step -> shard:
      AG, attention:  shard_at(k) = (r - d*k) mod W        (k = 0 is local)
      RS:             shard_at(k) = (r - d*(k+1)) mod W    (own chunk last)
      explicit:       shard_at(k) = user order (a permutation)
      hierarchical swizzle (the summary page names the pattern, sec. 5.1, and
      defines none; this is the reading): ranks form W/g groups of g
      consecutive ranks; rank r = G_r*g + l_r takes at step k = a*g + b
          AG, attention:  shard_at(k) = ((G_r + a) mod (W/g))*g + (l_r + b) mod g
          RS:             shard_at(k) = the AG order reversed (own shard last)
      so its own group comes first, every group in turn, and at each step the
      ranks of a group pull from distinct peers (each (a, b) is a bijection of
      ranks);
      mesh: the ring's step order, but every peer's link runs at once, so
      sub-chunk q of every shard arrives before sub-chunk q + 1 of any.
  pos(w*s+q) = kpos(w)*s + q with kpos = inverse of shard_at (mesh: q*W + kpos(w));
  arrival[p] = the chunk whose pos is p;
  resident(c) = local_resident and w == r and op != RS.
  tiles: Tm = ceil(M/TM), Tn = ceil(N/TN), t = i*Tn + j, rows(i) = [i*TM, min((i+1)*TM, M))
         attention: Tm = ceil(Sq/TM), Tn = Hq (work item t = i*Hq + h), deps = all chunks
         head-parallel attention (the all-to-all receive side of sequence
         parallelism: every rank holds all Sq = W*n tokens of its heads, token
         block w from peer w; Q, K and V arrive together): Tm = ceil(Sq/TM),
         Tn = Hq, deps = the chunks holding the item's query rows (its K and V
         blocks are folded in as they land)
  deps(t) = {c : [begin(c), end(c)) meets rows(i)} ascending; inv = its transpose
  key(t)  = max pos over deps (AG, attention) / min pos over deps (RS)
  orders: ROW_MAJOR  t ascending
          CHUNK_MAJOR sort by (key, i, j)
          SWIZZLED   sort by (key, i // G, j, i)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

OP_AG_GEMM, OP_GEMM_RS, OP_RING_ATTN, OP_HEAD_ATTN = 1, 2, 3, 4
PAT_RING, PAT_EXPLICIT, PAT_HIER_SWIZZLE, PAT_MESH = 0, 1, 2, 3
ORDER_ROW_MAJOR, ORDER_CHUNK_MAJOR, ORDER_SWIZZLED = 0, 1, 2
DEFAULT_GROUP_M = 4


class PlanError(ValueError):
    pass


@dataclass
class PlanDesc:
    op: int
    m: int
    n: int
    k: int
    world: int
    rank: int = 0
    ring_dir: int = 1
    pattern: int = PAT_RING
    explicit_order: Optional[List[int]] = None
    split: int = 1
    tile_m: int = 128
    tile_n: int = 128
    tile_order: int = ORDER_CHUNK_MAJOR
    group_m: int = 0
    local_resident: int = 1
    heads_q: int = 0
    heads_kv: int = 0
    shard_rows: Optional[List[int]] = None
    hier_group: int = 0


@dataclass
class PlanTables:
    num_chunks: int
    num_tiles: int
    tiles_m: int
    tiles_n: int
    chunk_begin: List[int] = field(default_factory=list)   # C+1
    chunk_pos: List[int] = field(default_factory=list)     # C
    arrival: List[int] = field(default_factory=list)       # C
    resident: List[int] = field(default_factory=list)      # C
    tile_order: List[int] = field(default_factory=list)    # T
    tile_key: List[int] = field(default_factory=list)      # T (indexed by tile id)
    dep_ptr: List[int] = field(default_factory=list)       # T+1
    dep_idx: List[int] = field(default_factory=list)
    inv_ptr: List[int] = field(default_factory=list)       # C+1
    inv_idx: List[int] = field(default_factory=list)
    tiles_in: List[int] = field(default_factory=list)      # C


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def plan_ref(desc: PlanDesc) -> PlanTables:
    """Build the chunk and tile tables for one descriptor (reading above)."""
    d = desc
    if d.op not in (OP_AG_GEMM, OP_GEMM_RS, OP_RING_ATTN, OP_HEAD_ATTN):
        raise PlanError("op")
    attn = d.op in (OP_RING_ATTN, OP_HEAD_ATTN)
    if d.world < 1 or not (0 <= d.rank < d.world) or d.ring_dir not in (1, -1):
        raise PlanError("world/rank/ring_dir")
    if d.m < 1 or d.n < 1 or d.k < 1 or d.tile_m < 1:
        raise PlanError("sizes")
    if d.tile_order not in (ORDER_ROW_MAJOR, ORDER_CHUNK_MAJOR, ORDER_SWIZZLED):
        raise PlanError("tile_order")
    G = d.group_m if d.group_m > 0 else DEFAULT_GROUP_M
    W, r, s = d.world, d.rank, d.split

    if attn:
        if d.heads_q < 1 or d.heads_kv < 1 or d.heads_q % d.heads_kv:
            raise PlanError("heads")
        if d.shard_rows is not None:
            raise PlanError("shard_rows")
        if d.op == OP_HEAD_ATTN and d.m != W * d.n:
            raise PlanError("head-parallel attention: the queries are every token (m = world * n)")
        R = d.n                       # tokens per KV block
        M_rows = W * d.n              # rows of the chunked (KV) tensor
        rows_of = [R] * W
    else:
        if d.tile_n < 1:
            raise PlanError("tile_n")
        if d.shard_rows is not None:
            rows_of = list(d.shard_rows)
            if len(rows_of) != W or min(rows_of) < 1 or sum(rows_of) != d.m:
                raise PlanError("shard_rows")
        else:
            if d.m % W:
                raise PlanError("m % world")
            rows_of = [d.m // W] * W
        R = min(rows_of)
        M_rows = d.m
    if not (1 <= s <= R):
        raise PlanError("split")
    shard_base = [sum(rows_of[:w]) for w in range(W)]

    # ring step -> shard
    if (d.pattern == PAT_HIER_SWIZZLE) != (d.hier_group != 0):
        raise PlanError("hier_group is set exactly for the hierarchical swizzle")
    if d.pattern in (PAT_RING, PAT_MESH):
        if d.op == OP_GEMM_RS:
            shard_at = [(r - d.ring_dir * (k + 1)) % W for k in range(W)]
        else:
            shard_at = [(r - d.ring_dir * k) % W for k in range(W)]
    elif d.pattern == PAT_EXPLICIT:
        order = list(d.explicit_order or [])
        if sorted(order) != list(range(W)):
            raise PlanError("explicit order is not a permutation")
        shard_at = order
    elif d.pattern == PAT_HIER_SWIZZLE:
        g = d.hier_group
        if g < 1 or W % g:
            raise PlanError("hier_group must divide world")
        groups, my_group, my_local = W // g, r // g, r % g
        shard_at = [((my_group + a) % groups) * g + (my_local + b) % g for a in range(groups) for b in range(g)]
        if d.op == OP_GEMM_RS:
            shard_at = shard_at[::-1]
    else:
        raise PlanError("pattern")
    kpos = [0] * W
    for k, w in enumerate(shard_at):
        kpos[w] = k

    C = W * s
    chunk_begin = []
    for w in range(W):
        for q in range(s):
            chunk_begin.append(shard_base[w] + (q * rows_of[w]) // s)
    chunk_begin.append(M_rows)
    if d.pattern == PAT_MESH:
        chunk_pos = [(c % s) * W + kpos[c // s] for c in range(C)]
    else:
        chunk_pos = [kpos[c // s] * s + (c % s) for c in range(C)]
    arrival = [0] * C
    for c, p in enumerate(chunk_pos):
        arrival[p] = c
    resident = [1 if (d.local_resident and (c // s) == r and d.op != OP_GEMM_RS) else 0
                for c in range(C)]

    # tile grid and dependencies
    if d.op == OP_RING_ATTN:
        Tm, Tn = _ceil_div(d.m, d.tile_m), d.heads_q
        deps_of_row = [list(range(C)) for _ in range(Tm)]
    else:
        Tm = _ceil_div(d.m, d.tile_m)
        Tn = d.heads_q if d.op == OP_HEAD_ATTN else _ceil_div(d.n, d.tile_n)
        deps_of_row = []
        for i in range(Tm):
            lo, hi = i * d.tile_m, min((i + 1) * d.tile_m, d.m)
            deps_of_row.append([c for c in range(C)
                                if chunk_begin[c] < hi and lo < chunk_begin[c + 1]])
    T = Tm * Tn
    dep_ptr, dep_idx = [0], []
    tile_key = []
    for t in range(T):
        deps = deps_of_row[t // Tn]
        dep_idx.extend(deps)
        dep_ptr.append(len(dep_idx))
        ps = [chunk_pos[c] for c in deps]
        tile_key.append(min(ps) if d.op == OP_GEMM_RS else max(ps))
    inv_lists = [[] for _ in range(C)]
    for t in range(T):
        for c in dep_idx[dep_ptr[t]:dep_ptr[t + 1]]:
            inv_lists[c].append(t)
    inv_ptr, inv_idx = [0], []
    for c in range(C):
        inv_idx.extend(inv_lists[c])
        inv_ptr.append(len(inv_idx))
    tiles_in = [len(x) for x in inv_lists]

    def sort_key(t):
        i, j = divmod(t, Tn)
        if d.tile_order == ORDER_CHUNK_MAJOR:
            return (tile_key[t], i, j)
        if d.tile_order == ORDER_SWIZZLED:
            return (tile_key[t], i // G, j, i)
        return (t,)

    tile_order = sorted(range(T), key=sort_key)
    return PlanTables(C, T, Tm, Tn, chunk_begin, chunk_pos, arrival, resident, tile_order,
                      tile_key, dep_ptr, dep_idx, inv_ptr, inv_idx, tiles_in)
