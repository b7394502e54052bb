// The fused decode / verify layer launch (layer.hip).
#pragma once

#include "common.h"

namespace moe {

// Cross-workgroup bookkeeping of the fused layer, in 32-bit words at the
// start of the workspace (a region no other call touches).  It must be zero
// before the first call on a workspace.  Word 0 counts calls; every other
// word is a flag that holds the number of the call that last set it, so
// nothing has to be cleared between calls.
constexpr int kSyncCalls = 0;
constexpr int kSyncArrive = 1024;       // one word per workgroup (<= 1024)
constexpr int kSyncTasks = 2048;        // one word per gate/up task
constexpr size_t layer_sync_bytes(int max_active, int I) {
  return size_t(kSyncTasks) * 4 + size_t(max_active) * (I / 4) * 4;
}

struct LayerArgs {
  const uint16_t* x;
  int T, E, k, H, I, S, fmt;
  int rfmt;
  const void* W;
  const float* bias;
  const int32_t* slot_of;
  MatView g, u, d, sg, su, sd;
  int has_sh;
  // outputs
  float* y;
  int32_t* idx;
  float* gate;
  int32_t* slot_idx;       // may be null
  moe_miss* miss;
  int32_t* miss_off;
  // workspace
  float* logits;           // [T][E]
  float* h;                // [T*k][I]
  float* h_sh;             // [T][I]
  uint32_t* sync;          // kSyncWords
};

bool layer_fused_ok(int fmt, int T, int k, int E, int H, int I);
size_t layer_fused_lds(int fmt, int T, int E, int H, int I);
hipError_t launch_layer_fused(const LayerArgs& a, hipStream_t st, int* grid);

}  // namespace moe
