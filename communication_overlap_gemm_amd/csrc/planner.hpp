// Chunk planner: chunk row bounds, ring positions, tile dependency tables and
// the reordered tile traversal.  Host-only C++ (no HIP), so plans can be built
// and checked without a GPU.
//
// The plan encodes the ideas of the Syncopate summary page ("Core method",
// paper sec. 5.1-5.2, Fig. 6): chunks are blocks of a tensor holding one or
// more tiles; every tile waits on the chunks it reads; chunks are visited in
// communication order and tiles inside a chunk keep (CHUNK_MAJOR) or adjust
// (SWIZZLED) their traversal.  For reduce-scatter the key is the earliest send
// slot a tile feeds, so output leaves in send order at a steady pace (Entwine
// abstract).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "sync_overlap.h"

namespace syncov {

struct Plan {
  sync_plan_desc desc{};
  std::vector<int32_t> explicit_order;
  int64_t rows = 0;        // rows of the chunked tensor (m, or world*n for attention)
  int64_t shard_rows = 0;  // R (uneven shards: the smallest shard's rows)
  int32_t num_chunks = 0, num_tiles = 0, tiles_m = 0, tiles_n = 0;
  std::vector<int64_t> chunk_begin;  // C+1
  std::vector<int32_t> chunk_pos, arrival, resident, tiles_in;  // C
  std::vector<int32_t> tile_order, tile_key;                    // T
  std::vector<int64_t> dep_ptr;                                  // T+1
  std::vector<int32_t> dep_idx;
  std::vector<int64_t> inv_ptr;                                  // C+1
  std::vector<int32_t> inv_idx;
};

// Fills `out` from `d`; on failure returns false and sets `err`.
bool build_plan(const sync_plan_desc& d, Plan& out, std::string& err);

}  // namespace syncov
