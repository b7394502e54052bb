// Slot resolution, compacted miss list and stable bucketing by slot.
//
// [MD] = ModelDock, "Strata はなぜ少ない VRAM でも速いのか": section
// "1 トークン、三者の分担" (each chosen expert id is looked up: experts already
// resident go to the GPU, the rest are handled elsewhere) and the placement
// figure of section "粗から細へ" (a per-card table of resident experts).
// Bucketing by slot lets each distinct resident expert be read once for all
// of its tokens (section "予測してから検証する": verifying extra tokens only
// costs the extra experts they route to).
#include "kernels.h"

namespace moe {

__device__ __forceinline__ int resolve_slot(int e, int E, int S, const int32_t* slot_of) {
  if (e < 0 || e >= E) return -1;
  const int s = slot_of ? slot_of[e] : e;
  return (s >= 0 && s < S) ? s : -1;
}

// Everything in one block of 256 threads for P = T*k <= 256 pairs.
//  - miss list: exclusive scan of the miss flags in pair order;
//  - bucket position of a hit pair = number of hit pairs with a smaller
//    slot, or the same slot and a smaller pair id (a stable counting sort
//    written as ranks);
//  - bucket_off[s] = lower bound of s in the sorted slots;
//  - active list = first pair of each distinct slot.
__global__ __launch_bounds__(256) void resolve_small_kernel(
    int T, int k, int E, int S, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ slot_of, int32_t* __restrict__ slot_idx,
    int32_t* __restrict__ bucket_off, int32_t* __restrict__ bucket_pair,
    moe_miss* __restrict__ miss, int32_t* __restrict__ miss_off, ActiveList act) {
  __shared__ int sl[kResolveSmallMax];
  __shared__ int sorted_s[kResolveSmallMax];
  __shared__ int tmp[32];
  const int P = T * k;
  const int p = threadIdx.x;
  int e = -1, s = -1;
  if (p < P) {
    e = idx[p];
    s = resolve_slot(e, E, S, slot_of);
    if (slot_idx) slot_idx[p] = s;
  }
  sl[p] = s;
  const int is_miss = (p < P && s < 0) ? 1 : 0;
  int n_miss;
  const int mpos = block_exclusive_scan(is_miss, tmp, &n_miss);
  if (is_miss && miss) {
    moe_miss m;
    m.expert = e;
    m.token = p / k;
    m.gate = gate[p];
    miss[mpos] = m;
  }
  if (miss_off) {
    if (p < P && p % k == 0) miss_off[p / k] = mpos;
    if (p == 0) miss_off[T] = n_miss;
  }
  __syncthreads();
  const int n_hit = P - n_miss;
  if (p < P && s >= 0) {
    int pos = 0;
    for (int q = 0; q < P; ++q) {
      const int sq = sl[q];
      pos += (sq >= 0 && (sq < s || (sq == s && q < p))) ? 1 : 0;
    }
    if (bucket_pair) bucket_pair[pos] = p;
    sorted_s[pos] = s;
  }
  __syncthreads();
  if (bucket_off) {
    for (int q = threadIdx.x; q <= S; q += blockDim.x) {
      int lo = 0, hi = n_hit;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sorted_s[mid] < q) lo = mid + 1; else hi = mid;
      }
      bucket_off[q] = lo;
    }
  }
  const int first = (p < n_hit && (p == 0 || sorted_s[p] != sorted_s[p - 1])) ? 1 : 0;
  int n_act;
  const int apos = block_exclusive_scan(first, tmp, &n_act);
  if (act.slot) {
    if (first) {
      act.slot[apos] = sorted_s[p];
      act.start[apos] = p;
    }
    if (p == 0) {
      act.start[n_act] = n_hit;
      *act.count = n_act;
    }
  }
}

hipError_t launch_resolve_small(int T, int k, int E, int S, const int32_t* idx,
                                const float* gate, const int32_t* slot_of, int32_t* slot_idx,
                                int32_t* bucket_off, int32_t* bucket_pair, moe_miss* miss,
                                int32_t* miss_off, ActiveList act, hipStream_t st) {
  hipLaunchKernelGGL(resolve_small_kernel, dim3(1), dim3(kResolveSmallMax), 0, st, T, k, E, S,
                     idx, gate, slot_of, slot_idx, bucket_off, bucket_pair, miss, miss_off, act);
  return hipGetLastError();
}

// ---------------------------------------------------------------- large P
// Pairs are cut into chunks of kResolveChunk consecutive pairs.
//  1. count:   per chunk, slot of each pair, per-slot counts (slot-major
//              table cnt[s][chunk]) and the chunk's miss count;
//  2. scan:    (a) per slot, the exclusive prefix of its counts over the
//              chunks (each chunk's first position inside the bucket,
//              relative to the bucket's start) and the slot's total, slots
//              and chunk ranges spread over blocks and waves; (b) one block
//              scans the chunk miss counts and the slot totals (bucket
//              starts, bucket_off, the active list);
//  3. scatter: per chunk, a pair's rank among the chunk's earlier pairs of
//              the same slot (or among its earlier misses) places it.

struct LargeWs {
  int32_t* cnt;        // [nchunk][S]: chunk-major, so a pass over slots is coalesced
  int32_t* cmiss;      // [nchunk + 1]
  int32_t* stot;       // [S] pairs per slot
  int32_t* sbase;      // [S] first position of the slot's bucket
};

static inline LargeWs large_ws_layout(void* ws, int nchunk, int S) {
  LargeWs w;
  w.cnt = static_cast<int32_t*>(ws);
  w.cmiss = w.cnt + size_t(S) * nchunk;
  w.stot = w.cmiss + nchunk + 1;
  w.sbase = w.stot + S;
  return w;
}

size_t resolve_large_ws(int T, int k, int S) {
  const int64_t P = int64_t(T) * k;
  const int64_t nchunk = (P + kResolveChunk - 1) / kResolveChunk;
  return size_t((int64_t(S) * nchunk + nchunk + 1 + 2 * int64_t(S)) * 4);
}

__global__ __launch_bounds__(256) void resolve_count_kernel(int P, int E, int S, int nchunk,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ slot_of,
                                                            int32_t* __restrict__ slot_idx,
                                                            LargeWs w) {
  extern __shared__ int hist[];  // [S]
  const int c = blockIdx.x;
  for (int s = threadIdx.x; s < S; s += blockDim.x) hist[s] = 0;
  __shared__ int nm;
  if (threadIdx.x == 0) nm = 0;
  __syncthreads();
  const int p0 = c * kResolveChunk;
  int my_miss = 0;
  for (int i = threadIdx.x; i < kResolveChunk; i += blockDim.x) {
    const int p = p0 + i;
    if (p >= P) break;
    const int s = resolve_slot(idx[p], E, S, slot_of);
    slot_idx[p] = s;
    if (s >= 0) atomicAdd(&hist[s], 1); else ++my_miss;
  }
  if (my_miss) atomicAdd(&nm, my_miss);
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) w.cnt[int64_t(c) * S + s] = hist[s];
  if (threadIdx.x == 0) w.cmiss[c] = nm;
}

// 2a. 64 slots per block (a lane each), the chunks split among the 16
// waves: each wave sums its range, the ranges before it give its start, and
// a second pass writes the exclusive prefixes in place.
constexpr int kColWaves = 16;
__global__ __launch_bounds__(64 * kColWaves) void resolve_colscan_kernel(int S, int nchunk,
                                                                         LargeWs w) {
  __shared__ int part[kColWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int s = blockIdx.x * 64 + lane;
  const int per = (nchunk + kColWaves - 1) / kColWaves;
  const int c0 = min(nchunk, wv * per), c1 = min(nchunk, c0 + per);
  int sum = 0;
  if (s < S) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) sum += w.cnt[int64_t(c) * S + s];
  }
  part[wv][lane] = sum;
  __syncthreads();
  int r = 0;
  for (int q = 0; q < wv; ++q) r += part[q][lane];
  if (s < S) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
      const int v = w.cnt[int64_t(c) * S + s];
      w.cnt[int64_t(c) * S + s] = r;
      r += v;
    }
    if (wv == kColWaves - 1) w.stot[s] = r;
  }
}

// 2b. One block of 1024 threads: chunk miss counts and slot totals.
__global__ __launch_bounds__(1024) void resolve_scan_kernel(int T, int S, int nchunk, LargeWs w,
                                                            int32_t* __restrict__ bucket_off,
                                                            int32_t* __restrict__ miss_off,
                                                            ActiveList act) {
  __shared__ int tmp[32];
  int run = 0;
  for (int base = 0; base < nchunk; base += blockDim.x) {
    const int i = base + threadIdx.x;
    const int v = i < nchunk ? w.cmiss[i] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, tmp, &tot);
    if (i < nchunk) w.cmiss[i] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0) {
    w.cmiss[nchunk] = run;
    if (miss_off) miss_off[T] = run;
  }
  int hits_before = 0, act_before = 0;
  for (int base = 0; base < S; base += blockDim.x) {
    const int s = base + threadIdx.x;
    const int tot_s = s < S ? w.stot[s] : 0;
    int tot_all;
    const int off = hits_before + block_exclusive_scan(tot_s, tmp, &tot_all);
    if (s < S) {
      w.sbase[s] = off;
      if (bucket_off) bucket_off[s] = off;
    }
    const int nonempty = (s < S && tot_s > 0) ? 1 : 0;
    int n_ne;
    const int apos = act_before + block_exclusive_scan(nonempty, tmp, &n_ne);
    if (nonempty && act.slot) {
      act.slot[apos] = s;
      act.start[apos] = off;
    }
    hits_before += tot_all;
    act_before += n_ne;
  }
  if (threadIdx.x == 0) {
    if (bucket_off) bucket_off[S] = hits_before;
    if (act.slot) {
      act.start[act_before] = hits_before;
      *act.count = act_before;
    }
  }
}

// 3. One wave per chunk, 64 pairs at a time in pair order.  A pair's place
// among the chunk's pairs of its slot is the slot's running count plus the
// earlier lanes with the same slot; the lanes with equal slots are found by
// one ballot per key bit (misses take the key S).  Misses are ranked by
// their own ballot.
__global__ __launch_bounds__(64) void resolve_scatter_kernel(
    int P, int k, int S, int nchunk, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ slot_idx, LargeWs w, int32_t* __restrict__ bucket_pair,
    moe_miss* __restrict__ miss, int32_t* __restrict__ miss_off) {
  extern __shared__ int run[];   // [S] pairs of each slot placed so far in the chunk
  const int c = blockIdx.x, lane = threadIdx.x;
  const int p0 = c * kResolveChunk;
  const int n = min(kResolveChunk, P - p0);
  for (int q = lane; q < S; q += 64) run[q] = 0;
  __syncthreads();
  const int nbits = 32 - __clz(S);   // keys 0 .. S
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int cmiss = w.cmiss[c];
  int mbase = 0;                     // misses in the earlier groups
  for (int g = 0; g < n; g += 64) {
    const int i = g + lane;
    const bool valid = i < n;
    const int p = p0 + i;
    const int sl = valid ? slot_idx[p] : -1;
    const int key = sl >= 0 ? sl : S;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t set = __ballot(bit);
      same &= bit ? set : ~set;
    }
    const uint64_t missm = __ballot(valid && sl < 0);
    const int rm = mbase + __popcll(missm & below);
    if (valid && sl >= 0) {
      const int within = __popcll(same & below);
      const int base = run[sl];
      // every lane has read its count before the first lane of each slot
      // (program order within the wave) adds the group's pairs
      if (within == 0) run[sl] = base + __popcll(same);
      if (bucket_pair) bucket_pair[w.sbase[sl] + w.cnt[int64_t(c) * S + sl] + base + within] = p;
    } else if (valid && miss) {
      moe_miss m;
      m.expert = idx[p];
      m.token = p / k;
      m.gate = gate[p];
      miss[cmiss + rm] = m;
    }
    if (valid && miss_off && p % k == 0) miss_off[p / k] = cmiss + rm;
    mbase += __popcll(missm);
  }
}

hipError_t launch_resolve_large(int T, int k, int E, int S, const int32_t* idx,
                                const float* gate, const int32_t* slot_of, int32_t* slot_idx,
                                int32_t* bucket_off, int32_t* bucket_pair, moe_miss* miss,
                                int32_t* miss_off, ActiveList act, void* ws, hipStream_t st) {
  const int P = T * k;
  const int nchunk = (P + kResolveChunk - 1) / kResolveChunk;
  LargeWs w = large_ws_layout(ws, nchunk, S);
  hipLaunchKernelGGL(resolve_count_kernel, dim3(nchunk), dim3(256), size_t(S) * 4, st, P, E, S,
                     nchunk, idx, slot_of, slot_idx, w);
  hipLaunchKernelGGL(resolve_colscan_kernel, dim3((S + 63) / 64), dim3(64 * kColWaves), 0, st, S,
                     nchunk, w);
  hipLaunchKernelGGL(resolve_scan_kernel, dim3(1), dim3(1024), 0, st, T, S, nchunk, w,
                     bucket_off, miss_off, act);
  hipLaunchKernelGGL(resolve_scatter_kernel, dim3(nchunk), dim3(64), size_t(S) * 4, st, P, k, S,
                     nchunk, idx, gate, slot_idx, w, bucket_pair, miss, miss_off);
  return hipGetLastError();
}

// Active list from caller-provided bucket offsets (one block).
__global__ __launch_bounds__(1024) void active_from_offsets_kernel(
    int S, const int32_t* __restrict__ bucket_off, ActiveList act) {
  __shared__ int tmp[32];
  int before = 0;
  for (int base = 0; base < S; base += blockDim.x) {
    const int s = base + threadIdx.x;
    const int ne = (s < S && bucket_off[s + 1] > bucket_off[s]) ? 1 : 0;
    int tot;
    const int pos = before + block_exclusive_scan(ne, tmp, &tot);
    if (ne) {
      act.slot[pos] = s;
      act.start[pos] = bucket_off[s];
    }
    before += tot;
  }
  if (threadIdx.x == 0) {
    act.start[before] = bucket_off[S];
    *act.count = before;
  }
}

hipError_t launch_active_from_offsets(int S, const int32_t* bucket_off, ActiveList act,
                                      hipStream_t st) {
  hipLaunchKernelGGL(active_from_offsets_kernel, dim3(1), dim3(1024), 0, st, S, bucket_off, act);
  return hipGetLastError();
}

}  // namespace moe
