// Acceptance of a verify pass on the GPU.
//
// [MD] ModelDock, "Strata はなぜ少ない VRAM でも速いのか", section
// "予測してから検証する": a draft layer proposes up to 3 next tokens, one pass
// of the 48 layers checks them all, keeps the drafts the model agrees with
// and adds one token of its own, so the output is token for token the
// greedy decode.  Row i of the pass's logits is the model's prediction
// after input i (input 0 = the last accepted token, input i = draft i).
//
// 1. partial argmax: block (p, i) scans slice p of row i; keys are
//    (order-preserving bits << 32) | ~index, so the largest key is the
//    largest logit and, among equal logits (-0 equals +0), the lowest index;
// 2. one block: the largest key of each row gives g_i; drafts are kept while
//    draft i+1 equals g_i; out = g_0 .. g_a, n_out = a + 1.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace moe {
namespace {

constexpr int kVThreads = 256;

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor(uint32_t(v), o, 64), hi = __shfl_xor(uint32_t(v >> 32), o, 64);
    v = max_u64(v, (uint64_t(hi) << 32) | lo);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint64_t m = 0;
  for (int w = 0; w < int(blockDim.x >> 6); ++w) m = max_u64(m, red[w]);
  return m;
}

__global__ __launch_bounds__(kVThreads) void argmax_part_kernel(const float* __restrict__ logits,
                                                                int V, int P,
                                                                uint64_t* __restrict__ part) {
  __shared__ uint64_t red[kVThreads / 64];
  const int p = blockIdx.x, row = blockIdx.y;
  const int per = (V + P - 1) / P;
  const int v0 = p * per, v1 = min(V, v0 + per);
  const float* l = logits + int64_t(row) * V;
  uint64_t best = 0;   // below every key (a key's low word ~v is never 0 for v < 2^31 - 1)
  for (int v = v0 + int(threadIdx.x); v < v1; v += kVThreads)
    best = max_u64(best, (uint64_t(ordered_bits(l[v])) << 32) | uint64_t(~uint32_t(v)));
  best = block_max_u64(best, red);
  if (threadIdx.x == 0) part[int64_t(row) * P + p] = best;
}

__global__ __launch_bounds__(kVThreads) void accept_kernel(const uint64_t* __restrict__ part,
                                                           int T, int P,
                                                           const int32_t* __restrict__ draft,
                                                           int32_t* __restrict__ out,
                                                           int32_t* __restrict__ n_out) {
  __shared__ uint64_t red[kVThreads / 64];
  __shared__ int32_t g[64];
  for (int row = 0; row < T; ++row) {
    uint64_t best = 0;
    for (int p = threadIdx.x; p < P; p += kVThreads) best = max_u64(best, part[int64_t(row) * P + p]);
    best = block_max_u64(best, red);
    if (threadIdx.x == 0) g[row] = int32_t(~uint32_t(best));
    __syncthreads();   // red is reused by the next row
  }
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < T - 1 && draft[a] == g[a]) ++a;
    for (int i = 0; i < T; ++i) out[i] = g[i];
    *n_out = a + 1;
  }
}

}  // namespace

int verify_parts(int T, int V) {
  // about 2 blocks per CU over the whole pass, at least 2048 logits per block
  const int want = max(1, 512 / max(T, 1));
  return max(1, min(want, (V + 2047) / 2048));
}

hipError_t launch_verify_accept(const float* logits, int T, int V, const int32_t* draft,
                                int32_t* out, int32_t* n_out, void* ws, hipStream_t st) {
  const int P = verify_parts(T, V);
  uint64_t* part = static_cast<uint64_t*>(ws);
  argmax_part_kernel<<<dim3(P, T), kVThreads, 0, st>>>(logits, V, P, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  accept_kernel<<<1, kVThreads, 0, st>>>(part, T, P, draft, out, n_out);
  return hipGetLastError();
}

}  // namespace moe
