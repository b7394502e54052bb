// Host-side launchers of the gfx950 kernels (one translation unit each).
#pragma once

#include "common.h"

namespace moe {

// verify-pass acceptance: partial argmax blocks per row, then one block
int verify_parts(int T, int V);
hipError_t launch_verify_accept(const float* logits, int T, int V, const int32_t* draft,
                                int32_t* out, int32_t* n_out, void* ws, hipStream_t st);

// router
constexpr int kRouterNT = 8;              // tokens per router block
constexpr int kRouterLdsBytes = 64 * 1024;
hipError_t launch_router(const uint16_t* x, int T, int H, int E, int rfmt, const void* W,
                         const float* bias, float* logits, hipStream_t st);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                       hipStream_t st);
// bf16 MFMA router GEMM for large T (BF16 router weights).
hipError_t launch_router_mfma(const uint16_t* x, int T, int H, int E, const uint16_t* W,
                              const float* bias, float* logits, hipStream_t st);

// Active bucket list: slots with a non-empty bucket in ascending order,
// where their bucket starts, and how many there are.
struct ActiveList {
  int32_t* slot;    // [cap]
  int32_t* start;   // [cap + 1]; start[n] = total pairs
  int32_t* count;   // [1]
};

// resolve
constexpr int kResolveSmallMax = 256;     // pairs handled by one block
constexpr int kResolveChunk = 1024;       // pairs per block in the large path
hipError_t launch_resolve_small(int T, int k, int E, int S, const int32_t* idx,
                                const float* gate, const int32_t* slot_of, int32_t* slot_idx,
                                int32_t* bucket_off, int32_t* bucket_pair, moe_miss* miss,
                                int32_t* miss_off, ActiveList act, hipStream_t st);
size_t resolve_large_ws(int T, int k, int S);
hipError_t launch_resolve_large(int T, int k, int E, int S, const int32_t* idx,
                                const float* gate, const int32_t* slot_of, int32_t* slot_idx,
                                int32_t* bucket_off, int32_t* bucket_pair, moe_miss* miss,
                                int32_t* miss_off, ActiveList act, void* ws, hipStream_t st);
hipError_t launch_active_from_offsets(int S, const int32_t* bucket_off, ActiveList act,
                                      hipStream_t st);

// usage counts and the adaptive slot table
hipError_t launch_count_usage(int P, int E, const int32_t* idx, uint32_t* usage, hipStream_t st);
struct RefreshMat {          // one of gate / up / down
  uint8_t* pool_codes;       // [S] matrices (codes, or fp32 data)
  uint16_t* pool_scale;      // [S] planes (nullptr for fp32)
  uint16_t* pool_min;
  const uint8_t* store_codes;   // [N] matrices
  const uint16_t* store_scale;
  const uint16_t* store_min;
  int64_t mat_bytes, mat_blocks;
};
struct RefreshArgs {
  int N, S, max_swaps;
  uint32_t* usage;           // [N]
  int32_t* slot_of;          // [N]
  int32_t* expert_of;        // [S]
  int32_t* swaps;            // [max_swaps][3]
  int32_t* n_swaps;          // [1]
  RefreshMat mats[3];
};
hipError_t launch_slot_refresh(const RefreshArgs& a, hipStream_t st);

// expert FFN (decode GEMV)
struct FfnArgs {
  const uint16_t* x;     // bf16 [T][H]
  int T, k, H, I, fmt;
  MatView g, u, d;       // routed pools (by slot)
  MatView sg, su, sd;    // shared expert (codes == nullptr: none)
  ActiveList act;        // buckets to run
  const int32_t* bucket_pair;
  int active_cap;        // upper bound of act.count
  float* h;              // fp32 [T*k][I] by pair id
  float* h_sh;           // fp32 [T][I]
  float* pair_out;       // fp32 [T*k][H]
  float* shared_out;     // fp32 [T][H]
  // accumulate mode (y_acc set): y_acc[t] += gate[t*k+j] * o for every hit
  // pair and += the shared expert's output, with device-scope float atomic
  // adds; pair_out and shared_out are then unused
  float* y_acc;          // fp32 [T][H]
  const float* gate;     // fp32 [T*k]
};
hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t st);

// expert FFN (prefill grouped GEMM, fp16 MFMA)
size_t ffn_gemm_ws(int T, int k, int H, int I, int S);
bool ffn_gemm_ok(int fmt, int H, int I);
bool ffn_gemm_fits(int T, int k, int H, int I);
hipError_t launch_ffn_gemm(const FfnArgs& a, int S, const int32_t* bucket_off, void* ws,
                           hipStream_t st);

// combine
hipError_t launch_combine(int T, int k, int H, const int32_t* slot_idx, const float* gate,
                          const float* pair_out, const float* shared_out, float* y,
                          hipStream_t st);

}  // namespace moe
