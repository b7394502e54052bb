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
//   [0, 256)           header: call counter (uint32, byte 0), error word
//                      (uint32, byte 4: nonzero once a call gave up a
//                      bounded wait), a word nothing writes (byte 128: the
//                      test hook's wait)
//   arrive [1024]      one tagged word per workgroup
//   logits [16][E]     tagged router logits
//   h      [hrows][I]  tagged SwiGLU activations: pairs first, then the
//                      shared expert's rows (one per token)
//   part   [hrows][H]  tagged down-projection rows, the same row order
//                      (pair rows already times their gate; the fixed-order
//                      sum of y reads them)
constexpr int kLayerMaxGrid = 1024;
constexpr int kLayerMaxPairs = 256;
__host__ __device__ inline int layer_h_rows(int k) {
  const int p = MOE_LAYER_MAX_T * k;
  return (p < kLayerMaxPairs ? p : kLayerMaxPairs) + MOE_LAYER_MAX_T;
}
inline size_t layer_region_bytes(int E, int k, int H, int I) {
  return 256 + size_t(kLayerMaxGrid) * 8 + size_t(MOE_LAYER_MAX_T) * E * 8 +
         size_t(layer_h_rows(k)) * (size_t(I) + H) * 8;
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
  uint64_t wait_ticks;     // budget of every wait, in ticks of the 100 MHz real-time counter
  int debug_hold;          // test hook: workgroup 0 first waits on a word nothing writes
  uint64_t* trace;         // phase stamps [grid][kTraceSlots] (null: off)
  int det;                 // 1: y summed in a fixed order (no float atomics)
};

// Phase stamps of the fused launch (real-time counter ticks, 100 MHz), one
// row per workgroup, written by its thread 0 when LayerArgs.trace is set.
enum TraceSlot {
  kTrStart = 0,        // workgroup start
  kTrXcd = 1,          // the XCD it runs on (hardware register, not a time)
  kTrStaged = 2,       // tokens staged (first barrier)
  kTrTasksA = 3,       // wave 0's router / shared-expert tasks done
  kTrLogits = 4,       // every logit seen
  kTrRouted = 5,       // routing and resolution done
  kTrGateUp0 = 6,      // wave 0's gate/up tasks done
  kTrGateUpAll = 7,    // the workgroup's last wave's gate/up tasks done
  kTrStagedH = 8,      // the first down unit's h staged
  kTrDown = 9,         // the workgroup's down units done
  kTrEnd = 10,         // end (workgroup 0: after the arrival check)
  kTrLogitsAll = 11,   // every wave has seen every logit (the barrier after the polls)
  kTrDStart = 12,      // down phase entered (the workgroup's gate/up tasks issued and done)
  kTrHPolled = 13,     // the first down unit's h all present (thread 0's poll)
  kTrHPolls = 14,      // thread 0's poll rounds for that h (a count, not a time)
  kTrLgPolls = 15,     // thread 0's poll rounds for the logits (a count)
  // routing, step by step (17 is stamped for one token only)
  kTrRtCand = 16,      // candidates listed (one token: before the second barrier;
                       // several: the threshold selection done)
  kTrRtBar2 = 17,      // after the second barrier
  kTrRtRank = 18,      // ranks taken (several tokens: the per-wave fallback done)
  kTrRtGate = 19,      // gates made
  kTrRtResolved = 20,  // slots and miss list resolved
  kTrTasksAAll = 21,   // the workgroup's last wave's router / shared-expert tasks done
  kTrTkSeg = 22,       // several tokens: segment maxima published (first top-k barrier)
  kTrTkTau = 23,       // several tokens: thresholds found (second barrier)
  // first down unit
  kTrDBar1 = 24,       // after the barrier that ends the LDS use of gate/up
  kTrDBar2 = 25,       // after the barrier that publishes the h sources
  kTrHConv = 26,       // h converted and stored in LDS (thread 0)
  kTrHBar = 27,        // after the staging barrier
  kTrTkCand = 28,      // several tokens: candidates listed (third barrier)
  kTraceSlots = 32
};

// Byte offsets in the region header.
constexpr int kRegionErr = 4;
constexpr int kRegionHold = 128;

bool layer_fused_ok(int fmt, int T, int k, int E, int H, int I);
size_t layer_fused_lds(int fmt, int T, int E, int H, int I);
hipError_t launch_layer_fused(const LayerArgs& a, int fmt, hipStream_t st, int* grid);

// The fused launch on the library's static hand-off region of the current
// device (moe_layer_noalloc): a.region is set here.
hipError_t launch_layer_noalloc(LayerArgs a, int fmt, hipStream_t st);
// Device address of that region (set up on first use: *ptr = null if it
// never was), and a clear of it on stream st.
hipError_t layer_scratch_address(uint8_t** ptr);
hipError_t layer_scratch_clear(hipStream_t st);

}  // namespace moe
