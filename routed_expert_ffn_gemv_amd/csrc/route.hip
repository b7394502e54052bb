// Router GEMV and top-k selection with gate weights.
//
// [MD] = ModelDock, "Strata はなぜ少ない VRAM でも速いのか": section "問題"
// (each layer's router picks 10 of 512 experts per token) and section
// "1 トークン、三者の分担" (the router runs on the GPU before the chosen ids
// are dispatched).
#include "kernels.h"

namespace moe {

// logits[t][e] = sum_h x[t][h] * W[e][h] + bias[e], fp32 accumulation.
// One wave per expert row (64 lanes stream the row with 16-byte loads), a
// block of 2 waves, tokens staged in LDS in groups of up to kRouterNT.
// grid = (ceil(E/2), ceil(T/ntok)); dynamic LDS = ntok * H * xbytes.
template <int RFMT>
__global__ __launch_bounds__(128) void router_gemv_kernel(const uint16_t* __restrict__ x, int T,
                                                          int H, int E, const void* __restrict__ W,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int ntok) {
  extern __shared__ uint32_t smem[];
  const int t0 = blockIdx.y * ntok;
  const int n = min(ntok, T - t0);
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 2 + (threadIdx.x >> 6);
  // stage tokens: bf16 pairs (BF16 weights) or fp32 (F32 weights)
  if (RFMT == MOE_W_BF16) {
    const uint32_t* xs = reinterpret_cast<const uint32_t*>(x + int64_t(t0) * H);
    for (int i = threadIdx.x; i < n * H / 2; i += blockDim.x) smem[i] = xs[i];
  } else {
    float* xf = reinterpret_cast<float*>(smem);
    for (int i = threadIdx.x; i < n * H; i += blockDim.x)
      xf[i] = bf16_to_f32(x[int64_t(t0) * H + i]);
  }
  __syncthreads();
  if (e >= E) return;
  float acc[kRouterNT];
#pragma unroll
  for (int v = 0; v < kRouterNT; ++v) acc[v] = 0.f;
  if (RFMT == MOE_W_BF16) {
    const u32x4* row = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) +
                                                      int64_t(e) * H);
    const int chunks = H / 8;  // 8 bf16 per 16 bytes
    for (int c = lane; c < chunks; c += 64) {
      const u32x4 w = row[c];
#pragma unroll
      for (int v = 0; v < kRouterNT; ++v) {
        if (v < n) {
          const uint32_t* xv = smem + v * (H / 2) + c * 4;
          float a = acc[v];
          a = dot2_bf16(w[0], xv[0], a);
          a = dot2_bf16(w[1], xv[1], a);
          a = dot2_bf16(w[2], xv[2], a);
          a = dot2_bf16(w[3], xv[3], a);
          acc[v] = a;
        }
      }
    }
  } else {
    const float4* row = reinterpret_cast<const float4*>(static_cast<const float*>(W) +
                                                        int64_t(e) * H);
    const float* xf = reinterpret_cast<const float*>(smem);
    const int chunks = H / 4;
    for (int c = lane; c < chunks; c += 64) {
      const float4 w = row[c];
#pragma unroll
      for (int v = 0; v < kRouterNT; ++v) {
        if (v < n) {
          const float* xv = xf + v * H + c * 4;
          acc[v] = fmaf(w.x, xv[0], fmaf(w.y, xv[1], fmaf(w.z, xv[2], fmaf(w.w, xv[3], acc[v]))));
        }
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int v = 0; v < kRouterNT; ++v) {
    if (v < n) {
      const float s = group_sum<64>(acc[v]);
      if (lane == 0) logits[int64_t(t0 + v) * E + e] = s + b;
    }
  }
}

// Top-k of each token's logits and softmax gates over the selected ones.
// One wave per token; lane l holds experts l, l+64, ...  Keys are
// (order-preserving logit bits << 32) | ~expert, so the wave maximum is the
// largest logit and, among equal logits, the lowest expert id.  k rounds of
// a wave-wide max extract the experts in order.
template <int KPL>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ logits, int T,
                                                        int E, int k, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + int64_t(t) * E;
  uint64_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? (uint64_t(ordered_bits(l[e])) << 32) | uint64_t(~uint32_t(e)) : 0ull;
  }
  int my_e = 0;
  float my_v = 0.f;
  float vmax = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) m = key[i] > m ? key[i] : m;
    m = wave_max_u64(m);
    const int e = int(~uint32_t(m));
    const uint32_t ob = uint32_t(m >> 32);
    const float v = __uint_as_float((ob & 0x80000000u) ? (ob & 0x7FFFFFFFu) : ~ob);
    if (j == 0) vmax = v;
    if (lane == j) {
      my_e = e;
      my_v = v;
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (lane == (e & 63) && i == (e >> 6)) key[i] = 0ull;
  }
  const float ex = lane < k ? expf(my_v - vmax) : 0.f;
  const float z = group_sum<64>(ex);
  if (lane < k) {
    idx[int64_t(t) * k + lane] = my_e;
    gate[int64_t(t) * k + lane] = ex / z;
  }
}

hipError_t launch_router(const uint16_t* x, int T, int H, int E, int rfmt, const void* W,
                         const float* bias, float* logits, hipStream_t st) {
  const int xbytes = rfmt == MOE_W_BF16 ? 2 : 4;
  int ntok = kRouterLdsBytes / (H * xbytes);
  ntok = ntok > kRouterNT ? kRouterNT : ntok;
  dim3 grid((E + 1) / 2, (T + ntok - 1) / ntok);
  const size_t lds = size_t(ntok) * H * xbytes;
  if (rfmt == MOE_W_BF16)
    hipLaunchKernelGGL(router_gemv_kernel<MOE_W_BF16>, grid, dim3(128), lds, st, x, T, H, E, W,
                       bias, logits, ntok);
  else
    hipLaunchKernelGGL(router_gemv_kernel<MOE_W_F32>, grid, dim3(128), lds, st, x, T, H, E, W,
                       bias, logits, ntok);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                       hipStream_t st) {
  dim3 grid((T + 3) / 4);
  if (E <= 64)
    hipLaunchKernelGGL(topk_gate_kernel<1>, grid, dim3(256), 0, st, logits, T, E, k, idx, gate);
  else if (E <= 256)
    hipLaunchKernelGGL(topk_gate_kernel<4>, grid, dim3(256), 0, st, logits, T, E, k, idx, gate);
  else if (E <= 512)
    hipLaunchKernelGGL(topk_gate_kernel<8>, grid, dim3(256), 0, st, logits, T, E, k, idx, gate);
  else
    hipLaunchKernelGGL(topk_gate_kernel<16>, grid, dim3(256), 0, st, logits, T, E, k, idx, gate);
  return hipGetLastError();
}

}  // namespace moe
