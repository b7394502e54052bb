// The fused decode / verify layer launch (layer.hip).
#pragma once

#include "common.h"

namespace moe {

// Hand-off region of the fused layer, at the start of the workspace, sized
// from the layer shape only (never from T) so that every call on one
// workspace finds it at the same place.  It must be zero before the first
// call.  Word 0 counts calls.  Every other entry is a 64-bit word {value,
// call number}: a workgroup publishes a value together with the number of
// the call that made it in one store, and a reader knows the value is
// current when the number matches -- no separate flag, no reset.
//   [0, 256)           call counter (uint32)
//   arrive [1024]      one tagged word per workgroup
//   logits [16][E]     tagged router logits
//   h      [hrows][I]  tagged SwiGLU activations: pairs first, then the
//                      shared expert's rows (one per token)
constexpr int kLayerMaxGrid = 1024;
constexpr int kLayerMaxPairs = 256;
__host__ __device__ inline int layer_h_rows(int k) {
  const int p = MOE_LAYER_MAX_T * k;
  return (p < kLayerMaxPairs ? p : kLayerMaxPairs) + MOE_LAYER_MAX_T;
}
inline size_t layer_region_bytes(int E, int k, int I) {
  return 256 + size_t(kLayerMaxGrid) * 8 + size_t(MOE_LAYER_MAX_T) * E * 8 +
         size_t(layer_h_rows(k)) * I * 8;
}

// Data planes of one expert matrix pool (sizes are common to all six).
struct Planes {
  const uint8_t* codes;    // Q formats: codes; F32: fp32 data as bytes
  const uint16_t* scale;
  const uint16_t* mn;
};

// Kernel arguments, kept small: every field lives in scalar registers for
// the whole launch.
struct LayerArgs {
  const uint16_t* x;
  int T, E, k, H, I, S;
  int rfmt;
  int has_sh;
  const void* W;
  const float* bias;
  const int32_t* slot_of;
  Planes g, u, d, sg, su, sd;
  int64_t mat_bytes;       // bytes of one matrix's data plane
  int64_t mat_blocks;      // 32-weight blocks of one matrix
  // outputs
  float* y;
  int32_t* idx;
  float* gate;
  int32_t* slot_idx;       // may be null
  moe_miss* miss;
  int32_t* miss_off;
  uint32_t* usage;         // [E] choice counts (may be null)
  uint8_t* region;         // hand-off region (layout above)
};

bool layer_fused_ok(int fmt, int T, int k, int E, int H, int I);
size_t layer_fused_lds(int fmt, int T, int E, int H, int I);
hipError_t launch_layer_fused(const LayerArgs& a, int fmt, hipStream_t st, int* grid);

}  // namespace moe
