// Adaptive slot table: usage counts and the refresh that swaps the most-used
// non-resident experts into the pool.
//
// [MD] = ModelDock, "Strata はなぜ少ない VRAM でも速いのか", section
// "粗から細へ" and its placement figure: every card fills its expert slots by
// a usage ranking, and an adaptive tier swaps a bounded number of experts
// (at most 96 every 4 rounds) toward the experts the conversation uses.
//
// Three stream-ordered launches:
//  1. plan (one workgroup): the best max_swaps candidates and victims by a
//     radix select over 32-bit keys (4 passes of 8 bits with LDS
//     histograms), each list then sorted in LDS (bitonic), and paired;
//  2. copy: one group of workgroups per swap streams the expert's planes
//     from the store into its slot (16-byte accesses where aligned);
//  3. tables + decay: slot_of / expert_of updated, every count halved.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kMaxSwaps = 1024;   // MOE_REFRESH_MAX_SWAPS
constexpr uint32_t kUsageCap = 65535u;

__device__ __forceinline__ uint32_t capped(uint32_t u) { return u < kUsageCap ? u : kUsageCap; }

// Candidate key of expert j (0: not a candidate).  Larger = better: higher
// count, then lower j.
__device__ __forceinline__ uint32_t cand_key(const RefreshArgs& a, int j) {
  const uint32_t u = capped(a.usage[j]);
  return (a.slot_of[j] < 0 && u > 0u) ? (u << 16) | (65535u - uint32_t(j)) : 0u;
}
// Victim key of slot s (never 0).  Larger = better: free slots first (by s
// ascending), then lower count of the held expert, then lower s.
__device__ __forceinline__ uint32_t vict_key(const RefreshArgs& a, int s) {
  const int j = a.expert_of[s];
  if (j < 0) return 0x80000000u | (65535u - uint32_t(s));
  return 1u + (((kUsageCap - capped(a.usage[j])) << 14) | (16383u - uint32_t(s)));
}

// The (at most) m largest nonzero keys of items 0..n-1, in descending
// order, into out[]; returns how many.  Radix select from the top byte:
// after each pass the keys above the chosen digit are certainly in, and the
// search narrows to the digit's keys.  Keys are unique, so the threshold
// key found after four passes closes the set exactly.  Called by every
// thread of the block.
template <typename KeyFn>
__device__ int select_top(KeyFn key, int n, int m, uint32_t* hist, uint32_t* out, int* cnt) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int need = m;
  for (int d = 3; d >= 0; --d) {
    for (int i = tid; i < 256; i += kPlanThreads) hist[i] = 0;
    __syncthreads();
    const int sh = 8 * d;
    for (int i = tid; i < n; i += kPlanThreads) {
      const uint32_t k = key(i);
      if (k != 0u && (k & mask) == prefix) atomicAdd(&hist[(k >> sh) & 255u], 1u);
    }
    __syncthreads();
    // digit b: the largest with (keys in digits >= b) >= need
    if (tid == 0) {
      int above = 0, b = 255;
      for (; b >= 0; --b) {
        if (above + int(hist[b]) >= need) break;
        above += int(hist[b]);
      }
      if (b < 0) {   // fewer than need keys left: take them all
        cnt[0] = -1;
      } else {
        cnt[0] = b;
        cnt[1] = need - above;
      }
    }
    __syncthreads();
    const int b = cnt[0];
    if (b < 0) {   // every remaining key qualifies: threshold = lowest nonzero
      prefix = 0;
      mask = 0;
      break;
    }
    need = cnt[1];
    prefix |= uint32_t(b) << sh;
    mask |= 255u << sh;
    __syncthreads();
  }
  // gather keys >= threshold (prefix; 0 and mask 0 mean "every nonzero key"
  // when the select ended early)
  if (tid == 0) cnt[2] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kPlanThreads) {
    const uint32_t k = key(i);
    if (k != 0u && k >= prefix) {
      const int p = atomicAdd(&cnt[2], 1);
      if (p < kMaxSwaps) out[p] = k;
    }
  }
  __syncthreads();
  const int got = min(cnt[2], m);
  // bitonic sort of out[0 .. 1024) descending (padding with 0)
  for (int i = tid; i < kMaxSwaps; i += kPlanThreads)
    if (i >= cnt[2]) out[i] = 0u;
  __syncthreads();
  for (int size = 2; size <= kMaxSwaps; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < kMaxSwaps; i += kPlanThreads) {
        const int p = i ^ stride;
        if (p > i) {
          const bool desc = (i & size) == 0;
          const uint32_t x = out[i], y = out[p];
          if (desc ? (x < y) : (x > y)) {
            out[i] = y;
            out[p] = x;
          }
        }
      }
      __syncthreads();
    }
  return got;
}

__global__ __launch_bounds__(kPlanThreads) void refresh_plan_kernel(RefreshArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t cand[kMaxSwaps], vict[kMaxSwaps];
  __shared__ int cnt[4];
  __shared__ int n_ok;
  const int tid = threadIdx.x;
  const int nc = select_top([&](int j) { return cand_key(a, j); }, a.N, a.max_swaps, hist, cand, cnt);
  const int nv = select_top([&](int s) { return vict_key(a, s); }, a.S, a.max_swaps, hist, vict, cnt);
  const int n = min(nc, nv);
  if (tid == 0) n_ok = n;
  __syncthreads();
  // the pairing condition holds for a prefix of the lists
  if (tid < n) {
    const uint32_t kc = cand[tid], kv = vict[tid];
    const uint32_t uc = kc >> 16;
    const bool free_slot = (kv & 0x80000000u) != 0u;
    const uint32_t uv = kUsageCap - (((kv - 1u) >> 14) & 0xFFFFu);
    if (!free_slot && !(uc > uv)) atomicMin(&n_ok, tid);
  }
  __syncthreads();
  const int ns = n_ok;
  if (tid < ns) {
    const uint32_t kc = cand[tid], kv = vict[tid];
    const int j = int(65535u - (kc & 0xFFFFu));
    const bool free_slot = (kv & 0x80000000u) != 0u;
    const int s = free_slot ? int(65535u - (kv & 0xFFFFu)) : int(16383u - ((kv - 1u) & 0x3FFFu));
    a.swaps[3 * tid] = s;
    a.swaps[3 * tid + 1] = j;
    a.swaps[3 * tid + 2] = a.expert_of[s];
  }
  if (tid == 0) *a.n_swaps = ns;
}

// Copies plane bytes [lo, hi) of one matrix (16-byte steps when both ends
// are 16-byte aligned, else 4-byte steps; sizes are multiples of 4).
__device__ __forceinline__ void copy_bytes(uint8_t* dst, const uint8_t* src, int64_t n, int part,
                                           int parts) {
  const bool v16 =
      ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) | uintptr_t(n)) & 15u) == 0u;
  const int64_t unit = v16 ? 16 : 4;
  const int64_t nu = n / unit;
  const int64_t per = (nu + parts - 1) / parts;
  const int64_t u0 = int64_t(part) * per, u1 = min(u0 + per, nu);
  if (v16) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    for (int64_t i = u0 + threadIdx.x; i < u1; i += blockDim.x) d4[i] = s4[i];
  } else {
    const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src);
    uint32_t* d1 = reinterpret_cast<uint32_t*>(dst);
    for (int64_t i = u0 + threadIdx.x; i < u1; i += blockDim.x) d1[i] = s1[i];
  }
}

// grid: (max_swaps, parts).  Block (i, part) copies its share of swap i's
// nine planes (three for fp32).
__global__ __launch_bounds__(256) void refresh_copy_kernel(RefreshArgs a) {
  const int i = blockIdx.x;
  if (i >= *a.n_swaps) return;
  const int s = a.swaps[3 * i], j = a.swaps[3 * i + 1];
  const int part = blockIdx.y, parts = gridDim.y;
  for (int m = 0; m < 3; ++m) {
    const RefreshMat& M = a.mats[m];
    copy_bytes(M.pool_codes + s * M.mat_bytes, M.store_codes + j * M.mat_bytes, M.mat_bytes, part,
               parts);
    if (M.pool_scale) {
      const int64_t nb = M.mat_blocks * 2;   // fp16 bytes
      copy_bytes(reinterpret_cast<uint8_t*>(M.pool_scale + s * M.mat_blocks),
                 reinterpret_cast<const uint8_t*>(M.store_scale + j * M.mat_blocks), nb, part, parts);
      copy_bytes(reinterpret_cast<uint8_t*>(M.pool_min + s * M.mat_blocks),
                 reinterpret_cast<const uint8_t*>(M.store_min + j * M.mat_blocks), nb, part, parts);
    }
  }
}

// Tables, then the halving of every count (one workgroup for the tables;
// every workgroup halves a share of the counts).
__global__ __launch_bounds__(256) void refresh_tables_kernel(RefreshArgs a) {
  if (blockIdx.x == 0) {
    const int ns = *a.n_swaps;
    for (int i = threadIdx.x; i < ns; i += blockDim.x) {
      const int old = a.swaps[3 * i + 2];
      if (old >= 0) a.slot_of[old] = -1;
    }
    __syncthreads();   // a new expert is never an old one, but keep the order plain
    for (int i = threadIdx.x; i < ns; i += blockDim.x) {
      const int s = a.swaps[3 * i], j = a.swaps[3 * i + 1];
      a.slot_of[j] = s;
      a.expert_of[s] = j;
    }
  }
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < a.N; j += gridDim.x * blockDim.x)
    a.usage[j] >>= 1;
}

__global__ __launch_bounds__(256) void count_usage_kernel(int P, int E, const int32_t* idx,
                                                          uint32_t* usage) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p < P) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(usage + e, 1u);
  }
}

}  // namespace

hipError_t launch_count_usage(int P, int E, const int32_t* idx, uint32_t* usage, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  hipLaunchKernelGGL(count_usage_kernel, dim3((P + 255) / 256), dim3(256), 0, st, P, E, idx,
                     usage);
  return hipGetLastError();
}

hipError_t launch_slot_refresh(const RefreshArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(refresh_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.max_swaps > 0) {
    hipLaunchKernelGGL(refresh_copy_kernel, dim3(a.max_swaps, 16), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int blocks = (a.N + 255) / 256;
  hipLaunchKernelGGL(refresh_tables_kernel, dim3(blocks < 64 ? blocks : 64), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
