// Dequant-fused expert FFN for decode and verify batches (few tokens per
// expert): gate/up GEMV + SwiGLU, then the down GEMV.
//
// [MD] = ModelDock, "Strata はなぜ少ない VRAM でも速いのか": section
// "1 トークン、三者の分担" (the experts resident on the card run on the GPU)
// and section "予測してから検証する" (a verify batch reads each expert once,
// so each bucket's weights are streamed once for all of its tokens).
//
// These are the stand-alone kernels behind moe_expert_ffn for small T (and
// the building blocks of the unfused moe_layer path); the row arithmetic is
// in gemv_core.h.
#include "gemv_core.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kNV = 8;        // tokens per gate/up pass
constexpr int kNVd = 16;      // vectors per down pass (8 pairs x hi/lo)
constexpr int kLdsBudget = 64 * 1024;

struct Unit {
  int slot, p0, n;
  bool shared;
};

__device__ __forceinline__ Unit unit_of(const FfnArgs& a, int u, int n_act) {
  Unit r;
  r.shared = u >= n_act;
  if (!r.shared) {
    r.slot = a.act.slot[u];
    r.p0 = a.act.start[u];
    r.n = a.act.start[u + 1] - r.p0;
  } else {
    r.slot = 0;
    r.p0 = 0;
    r.n = a.T;
  }
  return r;
}

// gate/up + SwiGLU.  Work unit = (bucket, block of rows of G and U); the
// shared expert is one more bucket holding every token.
template <int FMT, int LPR>
__global__ __launch_bounds__(256) void ffn_gateup_kernel(FfnArgs a, int units_per_expert, int nv) {
  extern __shared__ uint32_t smem[];
  const int K = a.H;
  const int vstride = vec_dwords<FMT>(K);
  const int sstride = K / 32;
  uint32_t* vec = smem;
  float* sums = reinterpret_cast<float*>(smem + nv * vstride);
  int* items = reinterpret_cast<int*>(sums + nv * sstride);
  const int n_act = *a.act.count;
  const bool has_sh = a.sg.codes != nullptr;
  const int total = (n_act + (has_sh ? 1 : 0)) * units_per_expert;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lane_g = lane % LPR;
  constexpr int kRowsPerUnit = 4 * (64 / LPR);
  const int chunks = chunks_per_row<FMT>(K);
  const int64_t row_bytes = int64_t(K) * fmt_bits(FMT) / 8;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const Unit un = unit_of(a, w / units_per_expert, n_act);
    const int i = (w % units_per_expert) * kRowsPerUnit + wave * (64 / LPR) + lane / LPR;
    const MatView G = un.shared ? a.sg : a.g;
    const MatView U = un.shared ? a.su : a.u;
    const uint8_t* gc = G.codes + un.slot * G.mat_bytes + i * row_bytes;
    const uint8_t* uc = U.codes + un.slot * U.mat_bytes + i * row_bytes;
    const uint16_t* gs = G.scale + un.slot * G.mat_blocks + int64_t(i) * sstride;
    const uint16_t* gm = G.mn + un.slot * G.mat_blocks + int64_t(i) * sstride;
    const uint16_t* us = U.scale + un.slot * U.mat_blocks + int64_t(i) * sstride;
    const uint16_t* um = U.mn + un.slot * U.mat_blocks + int64_t(i) * sstride;
    for (int g0 = 0; g0 < un.n; g0 += nv) {
      const int n = min(nv, un.n - g0);
      __syncthreads();
      if (threadIdx.x < n)
        items[threadIdx.x] = un.shared ? g0 + threadIdx.x : a.bucket_pair[un.p0 + g0 + threadIdx.x];
      __syncthreads();
      for (int v = 0; v < n; ++v) {
        const int tok = un.shared ? items[v] : items[v] / a.k;
        stage_bf16<FMT>(vec + v * vstride, sums + v * sstride, a.x + int64_t(tok) * K, K);
      }
      __syncthreads();
      float ag[kNV], au[kNV];
#pragma unroll
      for (int v = 0; v < kNV; ++v) ag[v] = au[v] = 0.f;
      if (i < a.I) {
        row_dot<FMT, kNV>(gc, gs, gm, chunks, lane_g, LPR, vec, vstride, sums, sstride, n, ag);
        row_dot<FMT, kNV>(uc, us, um, chunks, lane_g, LPR, vec, vstride, sums, sstride, n, au);
      }
#pragma unroll
      for (int v = 0; v < kNV; ++v) {
        if (v < n) {
          const float g = group_sum<LPR>(ag[v]);
          const float uu = group_sum<LPR>(au[v]);
          if (i < a.I && lane_g == 0) {
            float* out = un.shared ? a.h_sh : a.h;
            out[int64_t(items[v]) * a.I + i] = silu_f32(g) * uu;
          }
        }
      }
    }
  }
}

// down projection: o = D h for every pair of a bucket (and the shared
// expert), written to pair_out / shared_out, or (accumulate mode) added
// into y with the pair's gate.
template <int FMT, int LPR>
__global__ __launch_bounds__(256) void ffn_down_kernel(FfnArgs a, int units_per_expert, int np) {
  extern __shared__ uint32_t smem[];
  constexpr bool kSplit = FMT != MOE_W_F32;   // hi/lo bf16 vectors per pair
  constexpr int kVPP = kSplit ? 2 : 1;       // vectors per pair
  const int K = a.I;
  const int vstride = vec_dwords<FMT>(K);
  const int sstride = K / 32;
  const int nvec = np * kVPP;
  uint32_t* vec = smem;
  float* sums = reinterpret_cast<float*>(smem + nvec * vstride);
  int* items = reinterpret_cast<int*>(sums + nvec * sstride);
  const int n_act = *a.act.count;
  const bool has_sh = a.sd.codes != nullptr;
  const int total = (n_act + (has_sh ? 1 : 0)) * units_per_expert;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lane_g = lane % LPR;
  constexpr int kRowsPerUnit = 4 * (64 / LPR);
  const int chunks = chunks_per_row<FMT>(K);
  const int64_t row_bytes = int64_t(K) * fmt_bits(FMT) / 8;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const Unit un = unit_of(a, w / units_per_expert, n_act);
    const int r = (w % units_per_expert) * kRowsPerUnit + wave * (64 / LPR) + lane / LPR;
    const MatView D = un.shared ? a.sd : a.d;
    const uint8_t* dc = D.codes + un.slot * D.mat_bytes + r * row_bytes;
    const uint16_t* ds = D.scale + un.slot * D.mat_blocks + int64_t(r) * sstride;
    const uint16_t* dm = D.mn + un.slot * D.mat_blocks + int64_t(r) * sstride;
    for (int g0 = 0; g0 < un.n; g0 += np) {
      const int n = min(np, un.n - g0);
      __syncthreads();
      if (threadIdx.x < n)
        items[threadIdx.x] = un.shared ? g0 + threadIdx.x : a.bucket_pair[un.p0 + g0 + threadIdx.x];
      __syncthreads();
      for (int v = 0; v < n; ++v) {
        const float* src = (un.shared ? a.h_sh : a.h) + int64_t(items[v]) * K;
        stage_f32<FMT>(vec + (kVPP * v) * vstride, sums + (kVPP * v) * sstride,
                       vec + (kVPP * v + kVPP - 1) * vstride, sums + (kVPP * v + kVPP - 1) * sstride,
                       src, K);
      }
      __syncthreads();
      float acc[kNVd];
#pragma unroll
      for (int v = 0; v < kNVd; ++v) acc[v] = 0.f;
      if (r < a.H)
        row_dot<FMT, kNVd>(dc, ds, dm, chunks, lane_g, LPR, vec, vstride, sums, sstride,
                           n * kVPP, acc);
#pragma unroll
      for (int v = 0; v < kNVd / kVPP; ++v) {
        if (v < n) {
          float o = group_sum<LPR>(acc[kVPP * v]);
          if (kSplit) o += group_sum<LPR>(acc[kVPP * v + 1]);
          if (r < a.H && lane_g == 0) {
            if (a.y_acc) {   // the combine, fused: y[t] += gate * o
              const int t = un.shared ? items[v] : items[v] / a.k;
              const float g = un.shared ? 1.f : a.gate[items[v]];
              __hip_atomic_fetch_add(a.y_acc + int64_t(t) * a.H + r, g * o, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            } else {
              float* out = un.shared ? a.shared_out : a.pair_out;
              out[int64_t(items[v]) * a.H + r] = o;
            }
          }
        }
      }
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const FfnArgs& a, hipStream_t st) {
  constexpr int kLprGU = 8, kLprD = 4;
  const bool has_sh = a.sg.codes != nullptr;
  // gate/up
  {
    const int rows = 4 * (64 / kLprGU);
    const int upe = (a.I + rows - 1) / rows;
    const int per_vec = vec_dwords<FMT>(a.H) * 4 + (a.H / 32) * 4;
    int nv = (kLdsBudget - 64) / per_vec;
    nv = nv > kNV ? kNV : nv;
    if (nv < 1) return hipErrorInvalidValue;
    const size_t lds = size_t(nv) * per_vec + 64;
    const int units = (a.active_cap + (has_sh ? 1 : 0)) * upe;
    const int grid = units < 8192 ? units : 8192;
    if (grid > 0)
      hipLaunchKernelGGL((ffn_gateup_kernel<FMT, kLprGU>), dim3(grid), dim3(256), lds, st, a, upe,
                         nv);
  }
  // down
  {
    const int rows = 4 * (64 / kLprD);
    const int upe = (a.H + rows - 1) / rows;
    constexpr int kVPP = FMT != MOE_W_F32 ? 2 : 1;
    const int per_pair = kVPP * (vec_dwords<FMT>(a.I) * 4 + (a.I / 32) * 4);
    int np = (kLdsBudget - 64) / per_pair;
    np = np > kNVd / kVPP ? kNVd / kVPP : np;
    if (np < 1) return hipErrorInvalidValue;
    const size_t lds = size_t(np) * per_pair + 64;
    const int units = (a.active_cap + (has_sh ? 1 : 0)) * upe;
    const int grid = units < 8192 ? units : 8192;
    if (grid > 0)
      hipLaunchKernelGGL((ffn_down_kernel<FMT, kLprD>), dim3(grid), dim3(256), lds, st, a, upe, np);
  }
  return hipGetLastError();
}

// y[t] = shared_out[t] + sum_j (slot >= 0) gate[t][j] * pair_out[t*k+j]
__global__ __launch_bounds__(256) void combine_kernel(int T, int k, int H,
                                                      const int32_t* __restrict__ slot_idx,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ pair_out,
                                                      const float* __restrict__ shared_out,
                                                      float* __restrict__ y) {
  const int H4 = H / 4;
  const int64_t total = int64_t(T) * H4;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t t = i / H4;
    const int64_t r4 = i % H4;
    float4 s = shared_out ? reinterpret_cast<const float4*>(shared_out + t * H)[r4]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int64_t p = t * k + j;
      if (slot_idx[p] >= 0) {
        const float g = gate[p];
        const float4 o = reinterpret_cast<const float4*>(pair_out + p * H)[r4];
        s.x += g * o.x;
        s.y += g * o.y;
        s.z += g * o.z;
        s.w += g * o.w;
      }
    }
    reinterpret_cast<float4*>(y + t * H)[r4] = s;
  }
}

}  // namespace

hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t st) {
  switch (a.fmt) {
    case MOE_W_Q2B32: return launch_fmt<MOE_W_Q2B32>(a, st);
    case MOE_W_Q4B32: return launch_fmt<MOE_W_Q4B32>(a, st);
    case MOE_W_F32: return launch_fmt<MOE_W_F32>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(int T, int k, int H, const int32_t* slot_idx, const float* gate,
                          const float* pair_out, const float* shared_out, float* y,
                          hipStream_t st) {
  const int64_t total = int64_t(T) * (H / 4);
  int64_t grid = (total + 255) / 256;
  grid = grid > 4096 ? 4096 : grid;
  if (grid > 0)
    hipLaunchKernelGGL(combine_kernel, dim3(unsigned(grid)), dim3(256), 0, st, T, k, H, slot_idx,
                       gate, pair_out, shared_out, y);
  return hipGetLastError();
}

}  // namespace moe
