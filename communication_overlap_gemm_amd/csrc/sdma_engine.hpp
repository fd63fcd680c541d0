// SDMA copy agent driven through HSA (sdma_engine.cpp).
#pragma once

#include <stdint.h>

#include "kernels/launch_args.hpp"

namespace syncov {

// Bound on copy_teams for the SDMA backend (the engines' ids form a 16-bit mask).
constexpr int32_t kMaxSdmaEngines = 16;

// One call's copies: every non-resident chunk, in arrival order, each tensor
// row block [chunk_begin[c], chunk_begin[c+1]) from src to dst, then flags[c]
// set to the 32-bit word at epoch_word.  With E engines used (of those
// available) and C copied chunks, each chunk is cut into P = max(1, E / C)
// row pieces; piece q of copied chunk i goes to engine (i P + q) mod E, and
// the flag is written once every piece of every tensor has landed.
struct SdmaJob {
  const char* src[kMaxCopyTensors];
  char* dst[kMaxCopyTensors];
  int64_t row_bytes[kMaxCopyTensors];
  int32_t ntensors;
  int32_t num_chunks;
  const int64_t* chunk_begin;  // host tables
  const int32_t* arrival;
  const int32_t* resident;
  uint32_t* flags;             // device
  const uint32_t* epoch_word;  // device word the gate kernel fills with the call's epoch
};

struct SdmaCall {
  int record = 0;
  int64_t* gate_value = nullptr;  // the gate kernel stores 0 here to start the copies
  int32_t engines = 1;            // engines used
  int32_t pieces = 1;             // row pieces per copied chunk
};

// Reserves a call record on HIP device dev (waiting, bounded, for its previous
// call's copies to complete), fixes the engines used (at most `engines`) and
// the pieces per chunk, and arms its signals.
int sdma_begin(int dev, int32_t copied_chunks, int32_t ntensors, int32_t engines, SdmaCall* out);
// Queues the copies and flag writes of a call reserved with sdma_begin.
int sdma_submit(int dev, const SdmaCall& call, const SdmaJob& job);
// Waits for every queued SDMA copy of device dev to complete.
int sdma_quiesce_all(int dev);
// Waits (bounded) for every queued SDMA copy, then destroys the signals and
// drops the HSA reference of every device's engine state.
void sdma_release_all();
// Number of SDMA engines available for device-to-device copies on dev.
int sdma_engine_count(int dev, int* out);

}  // namespace syncov
