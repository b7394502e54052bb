// The whole routed-MoE layer for decode and verify batches in one persistent
// launch (T <= 16 tokens, T*k <= 256 pairs).
//
// [MD] = ModelDock, "Strata はなぜ少ない VRAM でも速いのか":
//  - section "1 トークン、三者の分担": per layer the GPU runs the router, the
//    chosen expert ids are resolved against the resident set, resident
//    experts are computed on the GPU, and the GPU sums the results before the
//    next layer starts;
//  - section "予測してから検証する": a verify step of 1 + up to 3 draft tokens
//    costs only the extra experts those tokens route to, so every distinct
//    expert is streamed once for all of its tokens;
//  - section "問題": the shared expert and the router are among the weights
//    every token uses.
//
// A decode layer moves ~21.6 MB in a dependent chain (router -> top-k ->
// gate/up -> down -> sum).  At ~1-2 us per HBM round trip the chain, not the
// bandwidth, sets the time, so it runs in one launch, every step issues all
// of its loads before it consumes any, and each hand-off between
// workgroups costs one round trip:
//  A  each wave issues the loads of its first task (router rows, or
//     shared-expert gate/up rows: neither depends on the routing) before the
//     tokens are staged in LDS; router waves zero their share of y first.
//     Logits and shared h are published as tagged words (below);
//  B  every workgroup polls all logits (and one arrival word per
//     workgroup) until they carry this call's number, then takes the
//     routing decisions itself (top-k, gates, slots, miss list, buckets) --
//     the same deterministic result everywhere, so nothing is broadcast;
//     workgroup 0 writes the routing outputs;
//  C  the workgroup's first down unit issues its weight loads; routed
//     gate/up + SwiGLU, a few rows of one expert per wave task, publishes
//     tagged h;
//  D  down units (expert, block of rows) poll their expert's h, stage it
//     and add gate * output into y with device-scope float atomics (the
//     shared expert adds with weight 1).  The summation order over experts
//     is not fixed, so y may differ from run to run in the last bits.
// Hand-offs are 64-bit words {value, call number} written with one store:
// a reader that sees this call's number has the value, so no flag, fence
// or reset is needed (this is the flag-in-data idea of low-latency
// collective protocols).  Loads and stores of them are device-scope (sc1),
// which bypasses the per-XCD L2 caches.  The grid never exceeds the
// workgroups the device holds at once, so every producer a poll waits for
// is running, and no producer waits on anything.
#include "gemv_core.h"
#include "kernels.h"
#include "layer.h"

namespace moe {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTMax = MOE_LAYER_MAX_T;
constexpr int kPMax = kLayerMaxPairs;
constexpr int kEMax = 1024;
// 16-byte chunks a lane holds of one weight row: gate/up rows (K = H) and
// down rows (K = I).  2-bit gate/up rows take two (H <= 2048), so the
// registers of several rows in flight stay small.
constexpr int kNChD = 4;
template <int FMT>
constexpr int nch_gu() { return FMT == MOE_W_Q2B32 ? 2 : 4; }

// Lanes per weight row: a lane holds at most 2 (Q2) or 4 (Q4) chunks of a
// 2048-wide gate/up row and 3 of a 768-wide down row.
template <int FMT>
struct Lanes {
  static constexpr int kGU = FMT == MOE_W_F32 ? 8 : 16;     // gate/up
  static constexpr int kD = FMT == MOE_W_Q4B32 ? 8 : 4;     // down
  static constexpr int kRowsGU = 64 / kGU;                  // rows per wave task
  static constexpr int kRowsD = kWaves * (64 / kD);         // rows per down unit
};

// Global-memory views of pointers.  Pointers read back from the LDS copy of
// the arguments carry no address space, so the compiler would access them
// with flat instructions -- and a flat access also counts against the LDS
// wait counter, which makes every later LDS wait wait for HBM too.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
  return (const __attribute__((address_space(1))) T*)(p);
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem_w(T* p) {
  return (__attribute__((address_space(1))) T*)(p);
}
__device__ __forceinline__ void store_miss(moe_miss* p, const moe_miss& m) {
  *gmem_w(&p->expert) = m.expert;
  *gmem_w(&p->token) = m.token;
  *gmem_w(&p->gate) = m.gate;
}
template <typename V>
__device__ __forceinline__ V ld_dev(const V* p) {
  return __hip_atomic_load(gmem(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void st_dev(V* p, V v) {
  __hip_atomic_store(gmem_w(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fadd_dev(float* p, float v) {
  __hip_atomic_fetch_add(gmem_w(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Marks a register as rewritten here, so work derived from it is redone at
// this point instead of being hoisted out of the enclosing loop (emits no
// instruction).
__device__ __forceinline__ u32x4 fresh(u32x4 w) {
  asm volatile("" : "+v"(w));
  return w;
}

// Wait until this wave's memory operations have completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Parts of the hand-off region.
__device__ __forceinline__ uint32_t* region_calls(const LayerArgs& a) {
  return reinterpret_cast<uint32_t*>(a.region);
}
__device__ __forceinline__ uint64_t* region_arrive(const LayerArgs& a) {
  return reinterpret_cast<uint64_t*>(a.region + 256);
}
__device__ __forceinline__ uint64_t* region_lg(const LayerArgs& a) {
  return region_arrive(a) + kLayerMaxGrid;
}
__device__ __forceinline__ uint64_t* region_h(const LayerArgs& a) {
  return region_lg(a) + kTMax * a.E;
}
__device__ __forceinline__ uint64_t* region_h_sh(const LayerArgs& a) {
  return region_h(a) + int64_t(layer_h_rows(a.k) - kTMax) * a.I;
}

// Tagged words: value bits low, call number high.
__device__ __forceinline__ uint64_t tag_word(float v, uint32_t epoch) {
  return (uint64_t(epoch) << 32) | __float_as_uint(v);
}
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t epoch) {
  return uint32_t(w >> 32) == epoch;
}
__device__ __forceinline__ float tag_val(uint64_t w) { return __uint_as_float(uint32_t(w)); }

// Wave reductions: DPP steps within quads, half rows and rows of 16 lanes
// (fused into the max/add), then the four row results read as scalars.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));   // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ float wave_sum_f32(float f) {
  f += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(f)));
  f += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(f)));
  f += __uint_as_float(dpp_u32<0x141>(__float_as_uint(f)));
  f += __uint_as_float(dpp_u32<0x140>(__float_as_uint(f)));
  const uint32_t v = __float_as_uint(f);
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(v, 15));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(v, 31));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(v, 47));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(v, 63));
  return (r0 + r1) + (r2 + r3);
}

// One selection round over the lanes' head keys (logit bits hv, ~expert
// lo): the largest logit, and among equal logits the lowest expert id.
// Keys are unique, so exactly one lane owns the winner.
struct Pick {
  uint32_t hv, lo;
  int owner;
};
__device__ __forceinline__ Pick wave_pick(uint32_t hv, uint32_t lo) {
  Pick p;
  p.hv = wave_max_u32(hv);
  uint64_t own = __ballot(hv == p.hv);
  if (__popcll(own) > 1) {   // equal logits: the lowest expert id has the largest ~id
    const uint32_t ml = wave_max_u32(hv == p.hv ? lo : 0u);
    own = __ballot(hv == p.hv && lo == ml);
  }
  p.owner = __ffsll(static_cast<unsigned long long>(own)) - 1;
  p.lo = __builtin_amdgcn_readlane(lo, p.owner);
  return p;
}

// Logit of an order-preserving key.
__device__ __forceinline__ float key_value(uint32_t ob) {
  return __uint_as_float((ob & 0x80000000u) ? (ob & 0x7FFFFFFFu) : ~ob);
}

__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b) {
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// Top-k of one token's logits (LDS, E <= 64 * KPL) by one wave.  Keys are
// (order-preserving logit bits << 32) | ~expert, unique, so the largest key
// is the largest logit and, among equal logits, the lowest expert id.  Each
// lane sorts its KPL keys once; each round picks the best head (wave_pick)
// and the owning lane drops it.  Lane j < k returns the j-th choice.
template <int KPL>
__device__ __forceinline__ void wave_topk(const float* l, int E, int k, int lane, int* e_out,
                                          float* v_out) {
  uint64_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? (uint64_t(ordered_bits(l[e])) << 32) | uint64_t(~uint32_t(e)) : 0ull;
  }
  // descending sort: 19-comparator network for 8 keys, applied per 8
#pragma unroll
  for (int o = 0; o < KPL; o += 8) {
    if (KPL - o >= 8) {
      uint64_t* q = key + o;
      cas_desc(q[0], q[2]); cas_desc(q[1], q[3]); cas_desc(q[4], q[6]); cas_desc(q[5], q[7]);
      cas_desc(q[0], q[4]); cas_desc(q[1], q[5]); cas_desc(q[2], q[6]); cas_desc(q[3], q[7]);
      cas_desc(q[0], q[1]); cas_desc(q[2], q[3]); cas_desc(q[4], q[5]); cas_desc(q[6], q[7]);
      cas_desc(q[2], q[4]); cas_desc(q[3], q[5]);
      cas_desc(q[1], q[4]); cas_desc(q[3], q[6]);
      cas_desc(q[1], q[2]); cas_desc(q[3], q[4]); cas_desc(q[5], q[6]);
    }
  }
  if (KPL == 16) {   // bitonic merge of the two sorted halves
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // reverse the second half
      const uint64_t t = key[8 + i];
      key[8 + i] = key[15 - i];
      key[15 - i] = t;
    }
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i & d) == 0) cas_desc(key[i], key[i + d]);
  }
  int my_e = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    const Pick pk = wave_pick(uint32_t(key[0] >> 32), uint32_t(key[0]));
    if (lane == j) {
      my_e = int(~pk.lo);
      my_v = key_value(pk.hv);
    }
    if (lane == pk.owner) {
#pragma unroll
      for (int i = 0; i < KPL - 1; ++i) key[i] = key[i + 1];
      key[KPL - 1] = 0ull;
    }
  }
  *e_out = my_e;
  *v_out = my_v;
}

// Largest k that the threshold selection serves (k <= 32 is required by its
// threshold step; the per-wave selection takes larger k).
constexpr int kTopkListMax = 16;

struct Lds {
  int idx[kPMax];        // choices (token-major); logits until the gates are made
  float gate[kPMax];
  int bpair[kPMax];      // hit pairs grouped by bucket
  int tok[kPMax];        // their tokens
  int act_slot[kPMax];   // the buckets' slots
  int act_start[kPMax + 1];
  int slot_of[kEMax];    // the slot table (when the layer has one)
  uint32_t emask[kEMax]; // per expert: tokens that chose it | bucket start << 16
  alignas(16) uint64_t rkey[kThreads + 8];   // segment maxima, then candidates (top-k)
  uint64_t tau[kTMax];       // per-token thresholds
  int ncand[kTMax];          // per-token candidate counts
  alignas(16) uint32_t tmp[32];
  int cstart[kWaves + 1];   // this workgroup's waves' gate/up task ranges
  int dstart[2];            // this workgroup's down unit range
  int n_act;
  uint32_t calls;
};

// --------------------------------------------------------------- staging
// Tokens into the expert format's LDS layout, with 32-byte loads per
// thread (16 columns of one token) issued before any is used.  psum holds
// each 16-column group's sum; block sums add two groups in a fixed order.
// The caller synchronises before reading xs or psum.
template <int FMT>
__device__ __forceinline__ void stage_tokens(const uint16_t* __restrict__ x, int T, int H, uint32_t* xs,
                                             float* psum, int vstride) {
  const int per_tok = H / 16;
  const int n_items = T * per_tok;
  constexpr int kR = 4;
  for (int base = 0; base < n_items; base += kR * kThreads) {
    u32x4 w[kR][2];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int it = base + r * kThreads + threadIdx.x;
      if (it < n_items) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + int64_t(it) * 16);
        w[r][0] = src[0];
        w[r][1] = src[1];
      }
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int it = base + r * kThreads + threadIdx.x;
      if (it >= n_items) continue;
      const int t = it / per_tok, g16 = it % per_tok;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s += bf16_to_f32(w[r][q][e] & 0xFFFFu) + bf16_to_f32(w[r][q][e] >> 16);
      psum[t * per_tok + g16] = s;
      if constexpr (FMT == MOE_W_F32) {
        float* xf = reinterpret_cast<float*>(xs) + t * vstride + g16 * 16;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xf[q * 8 + 2 * e] = bf16_to_f32(w[r][q][e] & 0xFFFFu);
            xf[q * 8 + 2 * e + 1] = bf16_to_f32(w[r][q][e] >> 16);
          }
      } else if constexpr (FMT == MOE_W_Q2B32) {
        // pairs (s, s+8), s < 8, of this 16-column group
        uint32_t* d = xs + t * vstride + (g16 >> 2) * Fmt<FMT>::kCS + (g16 & 3) * 8;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          d[2 * m] = __builtin_amdgcn_perm(w[r][1][m], w[r][0][m], 0x05040100u);
          d[2 * m + 1] = __builtin_amdgcn_perm(w[r][1][m], w[r][0][m], 0x07060302u);
        }
      } else {
        // two 8-column groups, pairs (s, s+4), s < 4
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t* d = xs + t * vstride + (g16 >> 1) * Fmt<FMT>::kCS + ((g16 & 1) * 2 + q) * 4;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            d[2 * m] = __builtin_amdgcn_perm(w[r][q][2 + m], w[r][q][m], 0x05040100u);
            d[2 * m + 1] = __builtin_amdgcn_perm(w[r][q][2 + m], w[r][q][m], 0x07060302u);
          }
        }
      }
    }
  }
}

// Block sums of the staged tokens (after a barrier that follows stage_tokens).
__device__ __forceinline__ void token_block_sums(int T, int H, float* xsum, const float* psum) {
  const int nb = H / 32, per_tok = H / 16;
  for (int i = threadIdx.x; i < T * nb; i += kThreads) {
    const int t = i / nb, b = i % nb;
    xsum[t * nb + b] = psum[t * per_tok + 2 * b] + psum[t * per_tok + 2 * b + 1];
  }
}


// Tagged fp32 vectors published by other workgroups (h), staged for the
// down projection, 16 columns per item.  Quantised formats: fp16 in the pair
// layout, each 32-column block scaled by a power of two that brings its
// largest |h| into [0.5, 1) (bsc keeps the inverse, psum the sums of the
// stored values), so no block overflows fp16 and each keeps 11 bits
// relative to its largest value.  F32 format: plain fp32.
// All loads of a batch are issued first; words that do not yet carry this
// call's number are read again until they do (their producers never wait
// on anything, so this ends).  Every thread calls it (the block maxima pass
// between neighbouring lanes).
template <int FMT>
__device__ __forceinline__ void stage_h(const uint64_t* const* srcs, int n, int K, uint32_t* xd,
                                        float* sd, float* psum, float* bsc, int vs,
                                        uint32_t epoch) {
  const int per_vec = K / 16;
  const int n_items = n * per_vec;
  constexpr int kIt = 2;   // items per thread and batch
  for (int base = 0; base < n_items; base += kIt * kThreads) {
    uint64_t wv[kIt][16];
    const uint64_t* src[kIt];
#pragma unroll
    for (int r = 0; r < kIt; ++r) {
      const int it = base + r * kThreads + threadIdx.x;
      src[r] = it < n_items ? srcs[it / per_vec] + (it % per_vec) * 16 : nullptr;
      if (src[r]) {
#pragma unroll
        for (int c = 0; c < 16; ++c) wv[r][c] = ld_dev(src[r] + c);
      }
    }
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int r = 0; r < kIt; ++r)
#pragma unroll
        for (int c = 0; c < 16; ++c) ok = ok && (!src[r] || tag_ok(wv[r][c], epoch));
      if (ok) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int r = 0; r < kIt; ++r)
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (src[r] && !tag_ok(wv[r][c], epoch)) wv[r][c] = ld_dev(src[r] + c);
    }
#pragma unroll
    for (int r = 0; r < kIt; ++r) {
      const int it = base + r * kThreads + threadIdx.x;
      float v[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) v[c] = src[r] ? tag_val(wv[r][c]) : 0.f;
      if constexpr (FMT == MOE_W_F32) {
        if (it < n_items) {
          const int p = it / per_vec, g16 = it % per_vec;
          float* xf = reinterpret_cast<float*>(xd) + p * vs + g16 * 16;
#pragma unroll
          for (int c = 0; c < 16; ++c) xf[c] = v[c];
        }
      } else {
        // block maximum: items 2b and 2b + 1 of a vector sit in lanes 2j and
        // 2j + 1 (per_vec is even and batches start at multiples of 512)
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(v[c]));
        amax = fmaxf(amax, dpp_f32<0xB1>(amax));   // quad_perm [1,0,3,2]
        uint32_t ex = (__float_as_uint(amax) >> 23) & 0xFFu;
        ex = ex > 253u ? 253u : ex;
        // amax in [2^(ex-127), 2^(ex-126)): scale by 2^(126-ex); zero and
        // subnormal maxima keep scale 1
        const float sc = ex == 0u ? 1.f : __uint_as_float((253u - ex) << 23);
        const float inv = ex == 0u ? 1.f : __uint_as_float((ex + 1u) << 23);
        if (it < n_items) {
          const int p = it / per_vec, g16 = it % per_vec;
          uint32_t hv[16];
          float sum = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const _Float16 hh = static_cast<_Float16>(v[c] * sc);
            hv[c] = __builtin_bit_cast(uint16_t, hh);
            sum += static_cast<float>(hh);
          }
          psum[p * per_vec + g16] = sum;
          if ((g16 & 1) == 0) bsc[p * (K / 32) + (g16 >> 1)] = inv;
          uint32_t* dh = xd + p * vs;
          if constexpr (FMT == MOE_W_Q2B32) {
            const int off = (g16 >> 2) * Fmt<FMT>::kCS + (g16 & 3) * 8;
#pragma unroll
            for (int q = 0; q < 8; ++q) dh[off + q] = hv[q] | (hv[q + 8] << 16);
          } else {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int off = (g16 >> 1) * Fmt<FMT>::kCS + ((g16 & 1) * 2 + q) * 4;
#pragma unroll
              for (int t = 0; t < 4; ++t) dh[off + t] = hv[8 * q + t] | (hv[8 * q + t + 4] << 16);
            }
          }
        }
      }
    }
  }
  __syncthreads();
  if (FMT != MOE_W_F32) {
    const int nb = K / 32;
    for (int i = threadIdx.x; i < n * nb; i += kThreads) {
      const int v = i / nb, b = i % nb;
      sd[v * nb + b] = psum[v * per_vec + 2 * b] + psum[v * per_vec + 2 * b + 1];
    }
  }
}

// --------------------------------------------------------------- row tiles
// A lane's share of one weight row, loaded before use: chunk j of the lane
// is chunk lane_g + j * lpr of the row.
template <int FMT, int NCH>
struct RowRegs {
  u32x4 w[NCH];
  uint32_t sc[NCH];   // Q2: two fp16 scales; Q4: one (low half)
  uint32_t mn[NCH];
};

template <int FMT, int NCH>
__device__ __forceinline__ void load_row(RowRegs<FMT, NCH>& R, const uint8_t* __restrict__ codes,
                                         const uint16_t* __restrict__ sc,
                                         const uint16_t* __restrict__ mn, int nch, int lane_g,
                                         int lpr) {
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j < nch) {
      const int c = lane_g + j * lpr;
      R.w[j] = *gmem(reinterpret_cast<const u32x4*>(codes + 16 * c));
      if constexpr (FMT == MOE_W_Q2B32) {
        R.sc[j] = *gmem(reinterpret_cast<const uint32_t*>(sc + 2 * c));
        R.mn[j] = *gmem(reinterpret_cast<const uint32_t*>(mn + 2 * c));
      } else if constexpr (FMT == MOE_W_Q4B32) {
        R.sc[j] = *gmem(sc + c);
        R.mn[j] = *gmem(mn + c);
      }
    }
  }
}

// Block dot products of one 16-byte code chunk with one staged vector.
// Q2: 64 codes = two 32-weight blocks, pairs (s, s+8) of each code dword;
// Q4: 32 codes = one block, pairs (s, s+4).  Returns sum (128 + q) x per
// block in p[0..1]; independent accumulators keep the dot2 chains short.
template <int FMT>
__device__ __forceinline__ void chunk_dot(u32x4 w, const uint32_t* xv, float* p) {
  w = fresh(w);   // unpack per vector; keeping every unpacked pair costs more registers
  const u32x4* x4 = reinterpret_cast<const u32x4*>(xv);
#pragma unroll
  for (int bb = 0; bb < (FMT == MOE_W_Q2B32 ? 2 : 1); ++bb) {
    u32x4 xx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xx[q] = x4[4 * bb + q];
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pr = FMT == MOE_W_Q2B32 ? q2_pair(w[2 * bb + (q >> 1)], (q & 1) * 4 + e)
                                                : q4_pair(w[q], e);
        a[e] = dot2_bf16(pr, xx[q][e], a[e]);
      }
    p[bb] = (a[0] + a[1]) + (a[2] + a[3]);
  }
}

// The same for two code chunks (gate and up rows) against one vector chunk.
template <int FMT>
__device__ __forceinline__ void chunk_dot2(u32x4 wg, u32x4 wu, const uint32_t* xv,
                                           float* pg, float* pu) {
  wg = fresh(wg);
  wu = fresh(wu);
  const u32x4* x4 = reinterpret_cast<const u32x4*>(xv);
#pragma unroll
  for (int bb = 0; bb < (FMT == MOE_W_Q2B32 ? 2 : 1); ++bb) {
    u32x4 xx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xx[q] = x4[4 * bb + q];
    float a[4] = {0.f, 0.f, 0.f, 0.f}, c[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s2 = (q & 1) * 4 + e;
        const uint32_t prg = FMT == MOE_W_Q2B32 ? q2_pair(wg[2 * bb + (q >> 1)], s2)
                                                 : q4_pair(wg[q], e);
        const uint32_t pru = FMT == MOE_W_Q2B32 ? q2_pair(wu[2 * bb + (q >> 1)], s2)
                                                 : q4_pair(wu[q], e);
        a[e] = dot2_bf16(prg, xx[q][e], a[e]);
        c[e] = dot2_bf16(pru, xx[q][e], c[e]);
      }
    pg[bb] = (a[0] + a[1]) + (a[2] + a[3]);
    pu[bb] = (c[0] + c[1]) + (c[2] + c[3]);
  }
}

// This lane's part of one row . one staged vector (at xv_base + chunk
// offsets, block sums at sv_base), over the lane's NCH chunks.
template <int FMT, int NCH>
__device__ __forceinline__ float row_vec_dot(const RowRegs<FMT, NCH>& R, int nch, int lane_g,
                                             int lpr, const uint32_t* xv_base,
                                             const float* sv_base) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j >= nch) continue;
    const int c = lane_g + j * lpr;
    if constexpr (FMT == MOE_W_F32) {
      const float4 wf = __builtin_bit_cast(float4, R.w[j]);
      const float* xv = reinterpret_cast<const float*>(xv_base) + 4 * c;
      acc = fmaf(wf.x, xv[0], fmaf(wf.y, xv[1], fmaf(wf.z, xv[2], fmaf(wf.w, xv[3], acc))));
    } else if constexpr (FMT == MOE_W_Q2B32) {
      float p[2];
      chunk_dot<FMT>(R.w[j], xv_base + c * Fmt<FMT>::kCS, p);
      const float d0 = f16_to_f32(uint16_t(R.sc[j] & 0xFFFFu));
      const float d1 = f16_to_f32(uint16_t(R.sc[j] >> 16));
      const float m0 = f16_to_f32(uint16_t(R.mn[j] & 0xFFFFu)) - 128.f * d0;
      const float m1 = f16_to_f32(uint16_t(R.mn[j] >> 16)) - 128.f * d1;
      acc += (d0 * p[0] + m0 * sv_base[2 * c]) + (d1 * p[1] + m1 * sv_base[2 * c + 1]);
    } else {
      float p[2];
      chunk_dot<FMT>(R.w[j], xv_base + c * Fmt<FMT>::kCS, p);
      const float d = f16_to_f32(uint16_t(R.sc[j]));
      const float m = f16_to_f32(uint16_t(R.mn[j])) - 128.f * d;
      acc += d * p[0] + m * sv_base[c];
    }
  }
  return acc;
}

// Gate and up rows . one vector in one pass (one set of LDS reads for both).
template <int FMT, int NCH>
__device__ __forceinline__ void row_pair_vec_dot(const RowRegs<FMT, NCH>& RG,
                                                 const RowRegs<FMT, NCH>& RU, int nch, int lane_g,
                                                 int lpr, const uint32_t* xv_base,
                                                 const float* sv_base, float& g, float& u) {
  if constexpr (FMT == MOE_W_F32) {
    g = row_vec_dot<FMT, NCH>(RG, nch, lane_g, lpr, xv_base, sv_base);
    u = row_vec_dot<FMT, NCH>(RU, nch, lane_g, lpr, xv_base, sv_base);
  } else {
    g = 0.f;
    u = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (j >= nch) continue;
      const int c = lane_g + j * lpr;
      const uint32_t* xv = xv_base + c * Fmt<FMT>::kCS;
      float pg[2], pu[2];
      chunk_dot2<FMT>(RG.w[j], RU.w[j], xv, pg, pu);
      if constexpr (FMT == MOE_W_Q2B32) {
        const float s0 = sv_base[2 * c], s1 = sv_base[2 * c + 1];
        const float dg0 = f16_to_f32(uint16_t(RG.sc[j] & 0xFFFFu));
        const float dg1 = f16_to_f32(uint16_t(RG.sc[j] >> 16));
        const float du0 = f16_to_f32(uint16_t(RU.sc[j] & 0xFFFFu));
        const float du1 = f16_to_f32(uint16_t(RU.sc[j] >> 16));
        g += (dg0 * pg[0] + (f16_to_f32(uint16_t(RG.mn[j] & 0xFFFFu)) - 128.f * dg0) * s0) +
             (dg1 * pg[1] + (f16_to_f32(uint16_t(RG.mn[j] >> 16)) - 128.f * dg1) * s1);
        u += (du0 * pu[0] + (f16_to_f32(uint16_t(RU.mn[j] & 0xFFFFu)) - 128.f * du0) * s0) +
             (du1 * pu[1] + (f16_to_f32(uint16_t(RU.mn[j] >> 16)) - 128.f * du1) * s1);
      } else {
        const float s0 = sv_base[c];
        const float dg = f16_to_f32(uint16_t(RG.sc[j])), du = f16_to_f32(uint16_t(RU.sc[j]));
        g += dg * pg[0] + (f16_to_f32(uint16_t(RG.mn[j])) - 128.f * dg) * s0;
        u += du * pu[0] + (f16_to_f32(uint16_t(RU.mn[j])) - 128.f * du) * s0;
      }
    }
  }
}

// Up to NG tokens at once: the code pairs of a block are unpacked once for
// the group.  Block scale d and min m enter as d * sum (128 + q) x +
// (m - 128 d) * sum x, with the block sums of the vectors staged beside them.
template <int FMT>
__device__ __forceinline__ void block_scales(uint32_t sc, uint32_t mn, int bb, float& d, float& m) {
  const uint32_t dsh = FMT == MOE_W_Q2B32 ? 16u * uint32_t(bb) : 0u;
  d = f16_to_f32(uint16_t((sc >> dsh) & 0xFFFFu));
  m = f16_to_f32(uint16_t((mn >> dsh) & 0xFFFFu)) - 128.f * d;
}
template <int FMT>
__device__ __forceinline__ void unpack_block(u32x4 w, int bb, uint32_t (&pr)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pr[q * 4 + e] = FMT == MOE_W_Q2B32 ? q2_pair(w[2 * bb + (q >> 1)], (q & 1) * 4 + e)
                                         : q4_pair(w[q], e);
}
// sum over one block of the code pairs . the vector's pairs (4 chains)
__device__ __forceinline__ float block_dot(const uint32_t (&pr)[16], const u32x4* x4) {
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 xx = x4[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = dot2_bf16(pr[q * 4 + e], xx[e], a[e]);
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// Gate and up rows . the vectors xv[v] (block sums sv[v]) of tokens v < nv.
template <int FMT, int NCH, int NG>
__device__ __forceinline__ void row_pair_vecs_dot(const RowRegs<FMT, NCH>& RG,
                                                  const RowRegs<FMT, NCH>& RU, int nch, int lane_g,
                                                  int lpr, const uint32_t* const (&xv)[NG],
                                                  const float* const (&sv)[NG], int nv,
                                                  float (&g)[NG], float (&u)[NG]) {
#pragma unroll
  for (int v = 0; v < NG; ++v) {
    g[v] = 0.f;
    u[v] = 0.f;
  }
  if constexpr (FMT == MOE_W_F32) {
#pragma unroll
    for (int v = 0; v < NG; ++v)
      if (v < nv) {
        g[v] = row_vec_dot<FMT, NCH>(RG, nch, lane_g, lpr, xv[v], sv[v]);
        u[v] = row_vec_dot<FMT, NCH>(RU, nch, lane_g, lpr, xv[v], sv[v]);
      }
  } else {
    constexpr int kBlk = FMT == MOE_W_Q2B32 ? 2 : 1;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (j >= nch) continue;
      const int c = lane_g + j * lpr;
      // unpacked here, once per call: not hoisted out of the caller's loops
      const u32x4 wg = fresh(RG.w[j]), wu = fresh(RU.w[j]);
#pragma unroll
      for (int bb = 0; bb < kBlk; ++bb) {
        float dg, mg, du, mu;
        block_scales<FMT>(RG.sc[j], RG.mn[j], bb, dg, mg);
        block_scales<FMT>(RU.sc[j], RU.mn[j], bb, du, mu);
        uint32_t pg[16], pu[16];
        unpack_block<FMT>(wg, bb, pg);
        unpack_block<FMT>(wu, bb, pu);
#pragma unroll
        for (int v = 0; v < NG; ++v) {
          if (v >= nv) continue;
          const u32x4* x4 = reinterpret_cast<const u32x4*>(xv[v] + c * Fmt<FMT>::kCS) + 4 * bb;
          const float sx = sv[v][kBlk * c + bb];
          g[v] += dg * block_dot(pg, x4) + mg * sx;
          u[v] += du * block_dot(pu, x4) + mu * sx;
        }
        __builtin_amdgcn_sched_barrier(0);   // one block's pairs live at a time
      }
    }
  }
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// a.lo*b.lo + a.hi*b.hi + c with fp16 pairs and fp32 accumulation
// (v_dot2_f32_f16).  The pairs come in as scalars: a bit cast of a vector
// element in place reads the wrong element.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}

// fp16 code pairs (1024 + q) of a block, for the fp16-staged h: OR-ing a
// code below 1024 into the mantissa of fp16(1024) = 0x6400 gives 1024 + q.
template <int FMT>
__device__ __forceinline__ void unpack_block_f16(u32x4 w, int bb, uint32_t (&pr)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pr[q * 4 + e] = FMT == MOE_W_Q2B32
                          ? ((w[2 * bb + (q >> 1)] >> (2 * ((q & 1) * 4 + e))) & 0x00030003u) | 0x64006400u
                          : ((w[q] >> (4 * e)) & 0x000F000Fu) | 0x64006400u;
}
__device__ __forceinline__ float block_dot_f16(const uint32_t (&pr)[16], const u32x4* x4) {
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 xx = x4[q];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a[e] = dot2_f16(pr[q * 4 + e], xx[e], a[e]);
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// One row . h of tokens v0 .. v0 + nv - 1, staged by stage_h (token t's
// vector at xd + t * vs, block sums at sd + t * ss, block scales at
// bsc + t * ss).  Per block: 2^e * (d * sum (1024 + q) h' + (m - 1024 d) *
// sum h'), with h' the scaled fp16 values.
template <int FMT, int NCH, int NG>
__device__ __forceinline__ void row_vecs_dot_f16(const RowRegs<FMT, NCH>& R, int nch, int lane_g,
                                                 int lpr, const uint32_t* xd, const float* sd,
                                                 const float* bsc, int vs, int ss, int v0, int nv,
                                                 float (&o)[NG]) {
#pragma unroll
  for (int v = 0; v < NG; ++v) o[v] = 0.f;
  constexpr int kBlk = FMT == MOE_W_Q2B32 ? 2 : 1;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j >= nch) continue;
    const int c = lane_g + j * lpr;
    const u32x4 w = fresh(R.w[j]);
#pragma unroll
    for (int bb = 0; bb < kBlk; ++bb) {
      const uint32_t dsh = FMT == MOE_W_Q2B32 ? 16u * uint32_t(bb) : 0u;
      const float d = f16_to_f32(uint16_t((R.sc[j] >> dsh) & 0xFFFFu));
      const float m = f16_to_f32(uint16_t((R.mn[j] >> dsh) & 0xFFFFu)) - 1024.f * d;
      uint32_t pr[16];
      unpack_block_f16<FMT>(w, bb, pr);
#pragma unroll
      for (int v = 0; v < NG; ++v) {
        if (v >= nv) continue;
        const int t = v0 + v, blk = kBlk * c + bb;
        const u32x4* h4 = reinterpret_cast<const u32x4*>(xd + t * vs + c * Fmt<FMT>::kCS) + 4 * bb;
        o[v] += bsc[t * ss + blk] * (d * block_dot_f16(pr, h4) + m * sd[t * ss + blk]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int FMT>
__host__ __device__ __forceinline__ int chunks_of(int K) {
  return FMT == MOE_W_F32 ? K / 4 : K / Fmt<FMT>::kWPC;
}

// gate/up rows i of one expert: this lane's chunks (loads only).
template <int FMT>
__device__ __forceinline__ void gateup_load(RowRegs<FMT, nch_gu<FMT>()>& rg,
                                            RowRegs<FMT, nch_gu<FMT>()>& ru,
                                            const LayerArgs& a, const Planes& G, const Planes& U,
                                            int slot, int i, int lane_g) {
  constexpr int kLprGU = Lanes<FMT>::kGU;
  const int K = a.H, sstride = K / 32;
  const int nch = chunks_of<FMT>(K) / kLprGU;
  const int64_t row_bytes = int64_t(K) * fmt_bits(FMT) / 8;
  const int64_t blk = int64_t(slot) * a.mat_blocks + int64_t(i) * sstride;
  const int64_t off = slot * a.mat_bytes + i * row_bytes;
  load_row<FMT, nch_gu<FMT>()>(rg, G.codes + off, G.scale + blk, G.mn + blk, nch, lane_g, kLprGU);
  load_row<FMT, nch_gu<FMT>()>(ru, U.codes + off, U.scale + blk, U.mn + blk, nch, lane_g, kLprGU);
}

// SwiGLU of row i for the expert's n tokens (vid: their staged vectors,
// or tokens t0 + v when vid is null); h of token v is published at
// out[ids(v)][i] (ids = pair ids, or the token itself when ids is null).
template <int FMT, int NG>
__device__ __forceinline__ void gateup_compute(const RowRegs<FMT, nch_gu<FMT>()>& rg,
                                               const RowRegs<FMT, nch_gu<FMT>()>& ru,
                                               const LayerArgs& a,
                                               int i, int n, const int* vid, const int* ids,
                                               int t0, uint64_t* out, const uint32_t* xs,
                                               const float* xsum, int vstride, int lane_g,
                                               uint32_t epoch) {
  constexpr int kLprGU = Lanes<FMT>::kGU;
  const int K = a.H, sstride = K / 32;
  const int nch = chunks_of<FMT>(K) / kLprGU;
  for (int v0 = 0; v0 < n; v0 += NG) {
    const int nv = min(NG, n - v0);
    const uint32_t* xv[NG];
    const float* sv[NG];
#pragma unroll
    for (int v = 0; v < NG; ++v) {
      const int id = v < nv ? (vid ? vid[v0 + v] : t0 + v0 + v) : 0;
      xv[v] = xs + id * vstride;
      sv[v] = xsum + id * sstride;
    }
    float g[NG], u[NG];
    row_pair_vecs_dot<FMT, nch_gu<FMT>(), NG>(rg, ru, nch, lane_g, kLprGU, xv, sv, nv, g, u);
#pragma unroll
    for (int v = 0; v < NG; ++v) {
      if (v >= nv) continue;
      const float gs = group_sum<kLprGU>(g[v]);
      const float us = group_sum<kLprGU>(u[v]);
      if (lane_g == 0)
        st_dev(out + int64_t(ids ? ids[v0 + v] : t0 + v0 + v) * a.I + i,
               tag_word(silu_f32(gs) * us, epoch));
    }
  }
}

// Router wave tasks: 64 / LPR rows of W (E x H) against the T tokens.
// Quantised expert formats keep the tokens in the expert pair layout, so
// W's natural bf16 pairs are regrouped with v_perm; their router is bf16
// with one 16-byte-aligned chunk of kWPC columns per lane (LPR = chunks).
template <int FMT>
__host__ __device__ __forceinline__ int router_lpr(int H) {
  if (FMT == MOE_W_F32) return 64;
  const int chunks = H / Fmt<FMT>::kWPC;
  return chunks < 64 ? chunks : 64;
}

template <int FMT>
struct RouterRegs {
  static constexpr int kQ = FMT == MOE_W_F32 ? 1 : Fmt<FMT>::kWPC / 8;   // 16-byte loads
  u32x4 w[kQ];
  float bias;
};

// Router task = (row group rg of 64 / lpr rows, token group).  Issues the
// task's loads: zeroes its share of y (every router task has one; they
// cover y), then loads this lane's router chunk and bias.
template <int FMT>
__device__ __forceinline__ void router_load(RouterRegs<FMT>& R, const LayerArgs& a, int task,
                                            int rg, int n_router, int lane) {
  const int TH = a.T * a.H, per = (TH + n_router - 1) / n_router;
  const int y0 = task * per, y1 = min(y0 + per, TH);
  for (int i = y0 + lane; i < y1; i += 64) st_dev(a.y + i, 0.f);
  const int lpr = router_lpr<FMT>(a.H);
  const int e = rg * (64 / lpr) + lane / lpr;
  if constexpr (FMT != MOE_W_F32) {
    if (e < a.E) {
      const u32x4* row = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.W) +
                                                        int64_t(e) * a.H);
      const int c = lane % lpr;
#pragma unroll
      for (int q = 0; q < RouterRegs<FMT>::kQ; ++q) R.w[q] = gmem(row)[c * RouterRegs<FMT>::kQ + q];
    }
  }
  R.bias = (e < a.E && a.bias) ? *gmem(a.bias + e) : 0.f;
}

// Logits of the row group's rows for tokens [t0, t0 + TG), published as
// tagged words once this wave's zeroes of y have landed (a workgroup adds
// into y only after it has seen every logit).
template <int FMT, int TG>
__device__ __forceinline__ void router_compute(const RouterRegs<FMT>& R, const LayerArgs& a,
                                               int rg, int t0, const uint32_t* xs, int vstride,
                                               int lane, uint32_t epoch) {
  constexpr int TB = TG;
  const int lpr = router_lpr<FMT>(a.H);
  const int e = rg * (64 / lpr) + lane / lpr;
  const int lane_g = lane % lpr;
  const int nt = min(TG, a.T - t0);
  xs += t0 * vstride;
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.f;
  if (e < a.E) {
    if constexpr (FMT == MOE_W_Q2B32 || FMT == MOE_W_Q4B32) {
      constexpr int kQ = RouterRegs<FMT>::kQ;
      uint32_t w[kQ * 4];
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        w[q * 4 + 0] = R.w[q][0];
        w[q * 4 + 1] = R.w[q][1];
        w[q * 4 + 2] = R.w[q][2];
        w[q * 4 + 3] = R.w[q][3];
      }
      constexpr int kG = 4, kS = FMT == MOE_W_Q2B32 ? 8 : 4;
      uint32_t pr[kG * kS];
#pragma unroll
      for (int g = 0; g < kG; ++g)
#pragma unroll
        for (int m = 0; m < kS / 2; ++m) {
          const uint32_t lo_w = w[g * kS + m], hi_w = w[g * kS + kS / 2 + m];
          pr[g * kS + 2 * m] = __builtin_amdgcn_perm(hi_w, lo_w, 0x05040100u);
          pr[g * kS + 2 * m + 1] = __builtin_amdgcn_perm(hi_w, lo_w, 0x07060302u);
        }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t < nt) {
          const uint32_t* xv = xs + t * vstride + lane_g * Fmt<FMT>::kCS;
          float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < kG * kS; ++j) s4[j & 3] = dot2_bf16(pr[j], xv[j], s4[j & 3]);
          acc[t] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
      }
    } else {
      const float* xf = reinterpret_cast<const float*>(xs);
      for (int col = lane_g; col < a.H; col += lpr) {
        const float wv = a.rfmt == MOE_W_F32
                             ? *gmem(static_cast<const float*>(a.W) + int64_t(e) * a.H + col)
                             : bf16_to_f32(*gmem(static_cast<const uint16_t*>(a.W) + int64_t(e) * a.H + col));
#pragma unroll
        for (int t = 0; t < TB; ++t)
          if (t < nt) acc[t] = fmaf(wv, xf[t * vstride + col], acc[t]);
      }
    }
  }
  // sums over each row's lpr lanes (a power of two), the tokens side by side
  if (lpr >= 2)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] += dpp_f32<0xB1>(acc[t]);    // quad_perm [1,0,3,2]
  if (lpr >= 4)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] += dpp_f32<0x4E>(acc[t]);    // quad_perm [2,3,0,1]
  if (lpr >= 8)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] += dpp_f32<0x141>(acc[t]);   // row_half_mirror
  if (lpr >= 16)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] += dpp_f32<0x140>(acc[t]);   // row_mirror
  if (lpr >= 32)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] += __shfl_xor(acc[t], 16, 64);
  if (lpr >= 64)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] += __shfl_xor(acc[t], 32, 64);
  wait_mem();
  if (e < a.E && lane_g == 0) {
#pragma unroll
    for (int t = 0; t < TB; ++t)
      if (t < nt) st_dev(region_lg(a) + (t0 + t) * a.E + e, tag_word(acc[t] + R.bias, epoch));
  }
}

// Slot of a chosen expert: -1 when it is not resident (or out of range).
__device__ __forceinline__ int slot_of_choice(const LayerArgs& a, const Lds& L, int e) {
  int s = (e >= 0 && e < a.E) ? (a.slot_of ? L.slot_of[e] : e) : -1;
  return (s >= 0 && s < a.S) ? s : -1;
}

// ---- top-k of every token: threshold, candidates, ranks
// Keys are (order-preserving logit bits << 32) | ~expert: unique, so the
// largest key is the largest logit and, among equal logits, the lowest id.
__device__ __forceinline__ uint64_t logit_key(const float* l, int e) {
  return (uint64_t(ordered_bits(l[e])) << 32) | uint64_t(~uint32_t(e));
}
template <int CTRL>
__device__ __forceinline__ uint64_t key_max_dpp(uint64_t v) {
  const uint64_t p = (uint64_t(dpp_u32<CTRL>(uint32_t(v >> 32))) << 32) | dpp_u32<CTRL>(uint32_t(v));
  return p > v ? p : v;
}

// Token t < T is served by the GS = kThreads / TB threads [t*GS, (t+1)*GS);
// thread j of them holds the keys e = j + GS*i.  Three barriered steps, then
// the ranks:
//  1. the largest key of each of 32 segments (GS/32 neighbouring threads);
//  2. tau = the k-th largest of those 32 maxima.  k distinct keys (the
//     maxima of k segments) are >= tau, so all of the token's k best are;
//  3. the keys >= tau are appended to the token's candidate list (at most
//     CAP = kThreads / TB kept, the count in L.ncand);
//  4. a candidate's rank among the candidates is its place in the top-k.
// L.idx[t*k + r] and L.gate[t*k + r] receive the r-th choice and its logit.
// A token with more than CAP candidates (many equal logits) is left to the
// caller.  Called by every thread; k <= kTopkListMax.
template <int TB, int KPT>   // KPT: keys per thread, E <= KPT * kThreads / TB
__device__ __forceinline__ void topk_threshold_k(const float* lg, int T, int E, int k, Lds& L) {
  constexpr int GS = kThreads / TB, SL = GS / 32, CAP = kThreads / TB;
  const int tid = threadIdx.x, t = tid / GS, j = tid % GS;
  const bool on = t < T;
  const float* l = lg + (on ? t : 0) * E;
  // the thread's keys stay in registers for step 3 (0 past E)
  uint64_t key[KPT];
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int e = j + GS * i;
    const uint64_t kv = logit_key(l, e < E ? e : E - 1);
    key[i] = (on && e < E) ? kv : 0ull;
    m = key[i] > m ? key[i] : m;
  }
  if constexpr (SL >= 2) m = key_max_dpp<0xB1>(m);    // quad_perm [1,0,3,2]
  if constexpr (SL >= 4) m = key_max_dpp<0x4E>(m);    // quad_perm [2,3,0,1]
  if constexpr (SL >= 8) m = key_max_dpp<0x141>(m);   // row_half_mirror
  if constexpr (SL >= 16) m = key_max_dpp<0x140>(m);  // row_mirror
  if (on && j % SL == 0) L.rkey[t * 32 + j / SL] = m;
  __syncthreads();
  {
    const int tt = tid / 32, sg = tid % 32;
    if (tt < T) {
      const uint64_t* sk = L.rkey + tt * 32;
      const uint64_t my = sk[sg];
      int gt = 0, eq = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {   // two keys per 16-byte read
        const u32x4 o4 = reinterpret_cast<const u32x4*>(sk)[q];
        const uint64_t o0 = (uint64_t(o4[1]) << 32) | o4[0], o1 = (uint64_t(o4[3]) << 32) | o4[2];
        gt += (o0 > my ? 1 : 0) + (o1 > my ? 1 : 0);
        eq += (o0 == my ? 1 : 0) + (o1 == my ? 1 : 0);
      }
      // empty segments share the key 0; their writers agree
      if (gt <= k - 1 && k - 1 < gt + eq) L.tau[tt] = my;
    }
  }
  __syncthreads();
  if (on) {
    const uint64_t tau = L.tau[t];
    int c = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) c += (key[i] != 0ull && key[i] >= tau) ? 1 : 0;
    if (c > 0) {
      int pos = atomicAdd(&L.ncand[t], c);
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (key[i] != 0ull && key[i] >= tau) {
          if (pos < CAP) L.rkey[t * CAP + pos] = key[i];
          ++pos;
        }
    }
  }
  __syncthreads();
  if (on) {
    const int n = L.ncand[t];
    if (n <= CAP) {
      const uint64_t* ck = L.rkey + t * CAP;
      for (int c = j; c < n; c += GS) {
        const uint64_t my = ck[c];
        int r = 0;
        for (int q0 = 0; q0 < n; q0 += 8) {
#pragma unroll
          for (int h = 0; h < 4; ++h) {   // two keys per 16-byte read
            const u32x4 o4 = reinterpret_cast<const u32x4*>(ck + q0)[h];
            const uint64_t o0 = (uint64_t(o4[1]) << 32) | o4[0];
            const uint64_t o1 = (uint64_t(o4[3]) << 32) | o4[2];
            r += (q0 + 2 * h < n && o0 > my) ? 1 : 0;
            r += (q0 + 2 * h + 1 < n && o1 > my) ? 1 : 0;
          }
        }
        if (r < k) {
          L.idx[t * k + r] = int(~uint32_t(my));
          L.gate[t * k + r] = key_value(uint32_t(my >> 32));
        }
      }
    }
  }
}

template <int TB>
__device__ __forceinline__ void topk_threshold(const float* lg, int T, int E, int k, Lds& L) {
  constexpr int GS = kThreads / TB, KMAX = kEMax / GS;
  if (KMAX >= 2 && E <= GS * (KMAX / 2))
    topk_threshold_k<TB, (KMAX >= 2 ? KMAX / 2 : 1)>(lg, T, E, k, L);
  else
    topk_threshold_k<TB, KMAX>(lg, T, E, k, L);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// Exclusive scan of one value per thread over the workgroup: a DPP scan in
// each wave (row shifts, then the row broadcasts), wave totals through LDS.
// *total receives the sum.  Called by every thread; one barrier.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_shift(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ uint32_t block_scan_u32(uint32_t v, uint32_t* wtot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
  x += dpp_shift<0x111, 0xF>(x);   // row_shr:1
  x += dpp_shift<0x112, 0xF>(x);   // row_shr:2
  x += dpp_shift<0x114, 0xF>(x);   // row_shr:4
  x += dpp_shift<0x118, 0xF>(x);   // row_shr:8
  x += dpp_shift<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_shift<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t c = wtot[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  *total = all;
  return before + x - v;
}

// Resolution of one token's k choices by the wave that chose them (lane j
// holds choice j and its gate).  The choices are distinct experts, so the
// hits need no sorting: they stay in choice order, one bucket each.
__device__ __forceinline__ void resolve_one(const LayerArgs& a, Lds& L, int e, float g, int lane,
                                            bool writer) {
  const int k = a.k;
  const bool valid = lane < k;
  const int s = valid ? slot_of_choice(a, L, e) : -1;
  const bool hit = s >= 0;
  const uint64_t miss_mask = __ballot(valid && !hit);
  const uint64_t hit_mask = __ballot(hit);
  const int mpos = __builtin_amdgcn_mbcnt_hi(uint32_t(miss_mask >> 32),
                                             __builtin_amdgcn_mbcnt_lo(uint32_t(miss_mask), 0u));
  const int hpos = __builtin_amdgcn_mbcnt_hi(uint32_t(hit_mask >> 32),
                                             __builtin_amdgcn_mbcnt_lo(uint32_t(hit_mask), 0u));
  const int n_hit = __popcll(hit_mask);
  if (writer) {
    if (valid && a.slot_idx) *gmem_w(a.slot_idx + lane) = s;
    if (valid && !hit) {
      moe_miss m;
      m.expert = e;
      m.token = 0;
      m.gate = g;
      store_miss(a.miss + mpos, m);
    }
    if (lane == 0) *gmem_w(a.miss_off) = 0;
    if (lane == 1) *gmem_w(a.miss_off + 1) = __popcll(miss_mask);
  }
  if (hit) {
    L.bpair[hpos] = lane;
    L.tok[hpos] = 0;
    L.act_slot[hpos] = s;
    L.act_start[hpos] = hpos;
  }
  if (lane == 0) {
    L.act_start[n_hit] = n_hit;
    L.n_act = n_hit;
  }
}

// Orders this wave's LDS accesses across its lanes (LDS operations of one
// wave complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Routing of one token, two barriers in all.  Thread j polls the logits of
// experts j and j + kThreads; the 32 segments of 16 neighbouring threads
// publish the logit bits of their largest key.  Then every wave, for itself:
//  - tau = the k-th largest of those 32 values: k segment maxima reach it,
//    so the k best keys all do (lane l counts the values above value l % 32
//    in half l / 32 of the list; the two halves are added);
//  - the wave's candidates, the keys whose logit bits reach tau, take slots
//    of one list through one LDS add per wave;
// and after the second barrier, again every wave for itself (the tables it
// writes are the same in every wave, so no further barrier is needed):
//  - a candidate's rank is the number of larger candidate keys (keys are
//    unique), and the candidate of rank r < k is choice r;
//  - the gates (softmax over the k chosen logits) and the resolution.
// More than 64 candidates (many equal logits) or k > kTopkListMax: the
// per-wave selection instead.  lg receives the logits.  Only wave 0 of a
// writer workgroup stores the outputs.
__device__ __forceinline__ void route_token(const LayerArgs& a, float* lg, int E, int k, Lds& L,
                                            uint32_t epoch, bool writer) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kR = kEMax / kThreads;
  uint64_t w[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r)
    if (tid + r * kThreads < E) w[r] = ld_dev(region_lg(a) + tid + r * kThreads);
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int r = 0; r < kR; ++r) ok = ok && (tid + r * kThreads >= E || tag_ok(w[r], epoch));
    if (ok) break;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int r = 0; r < kR; ++r)
      if (tid + r * kThreads < E && !tag_ok(w[r], epoch))
        w[r] = ld_dev(region_lg(a) + tid + r * kThreads);
  }
  uint64_t key[kR];   // 0: no expert
  uint32_t m = 0u;    // largest logit bits of the thread
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int e = tid + r * kThreads;
    key[r] = 0ull;
    if (e < E) {
      const float v = tag_val(w[r]);
      lg[e] = v;
      const uint32_t ob = ordered_bits(v);
      key[r] = (uint64_t(ob) << 32) | uint64_t(~uint32_t(e));
      m = max(m, ob);
    }
  }
  m = max(m, dpp_u32<0xB1>(m));    // quad_perm [1,0,3,2]
  m = max(m, dpp_u32<0x4E>(m));    // quad_perm [2,3,0,1]
  m = max(m, dpp_u32<0x141>(m));   // row_half_mirror
  m = max(m, dpp_u32<0x140>(m));   // row_mirror
  if ((tid & 15) == 0) L.tmp[tid >> 4] = m;
  if (tid < 64) L.rkey[tid] = 0ull;   // the candidate list's empty slots
  __syncthreads();
  const bool thresh = k <= kTopkListMax;
  if (thresh) {
    const uint32_t my = L.tmp[lane & 31];
    const u32x4* half = reinterpret_cast<const u32x4*>(L.tmp) + 4 * (lane >> 5);
    int gt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 o = half[q];
#pragma unroll
      for (int c = 0; c < 4; ++c) gt += o[c] > my ? 1 : 0;
    }
    gt += __shfl_xor(gt, 32, 64);
    // the smallest value with fewer than k larger ones (as ~max of ~value)
    const uint32_t tau = ~wave_max_u32(gt <= k - 1 ? ~my : 0u);
    uint64_t cm[kR];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      cm[r] = __ballot(key[r] != 0ull && uint32_t(key[r] >> 32) >= tau);
      cnt += __popcll(cm[r]);
    }
    int base = 0;
    if (cnt > 0) {
      if (lane == 0) base = atomicAdd(&L.ncand[0], cnt);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int pos = base + lanes_below(cm[r]);
        if (((cm[r] >> lane) & 1ull) && pos < 64) L.rkey[pos] = key[r];
        base += __popcll(cm[r]);
      }
    }
  }
  __syncthreads();
  // The count, this lane's candidate and the first eight candidates are
  // read together; list slots past the count hold key 0 (zeroed before the
  // first barrier), which is below every key.
  const int n = thresh ? L.ncand[0] : 65;
  const uint64_t ck = L.rkey[lane];
  auto rank_step = [&](int j0, int r) {   // candidates j0 .. j0 + 7 above ck
    u32x4 q[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) q[h] = reinterpret_cast<const u32x4*>(L.rkey + j0)[h];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      r += ((uint64_t(q[h][1]) << 32) | q[h][0]) > ck ? 1 : 0;
      r += ((uint64_t(q[h][3]) << 32) | q[h][2]) > ck ? 1 : 0;
    }
    return r;
  };
  int r = rank_step(0, 0);
  int my_e;
  float my_v;
  if (n <= 64) {
    for (int j0 = 8; j0 < n; j0 += 8) r = rank_step(j0, r);
    // choice r moves to lane r (k <= 16 < 63, the lane that takes the rest)
    const int to = 4 * ((lane < n && r < k) ? r : 63);
    const uint32_t hi = uint32_t(__builtin_amdgcn_ds_permute(to, int(uint32_t(ck >> 32))));
    const uint32_t lo = uint32_t(__builtin_amdgcn_ds_permute(to, int(uint32_t(ck))));
    my_e = int(~lo);
    my_v = key_value(hi);
  } else if (E <= 512) {
    wave_topk<8>(lg, E, k, lane, &my_e, &my_v);
  } else {
    wave_topk<16>(lg, E, k, lane, &my_e, &my_v);
  }
  // gates: softmax over the k chosen logits (choice 0 is the largest)
  if (lane >= k) {
    my_e = 0;
    my_v = 0.f;
  }
  const float vmax = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_v), 0));
  const float ex = lane < k ? __expf(my_v - vmax) : 0.f;
  const float g = ex * __frcp_rn(wave_sum_f32(ex));
  const bool out = writer && wave == 0;
  if (lane < k) {
    L.idx[lane] = my_e;
    L.gate[lane] = g;
    if (out) {
      *gmem_w(a.idx + lane) = my_e;
      *gmem_w(a.gate + lane) = g;
    }
  }
  resolve_one(a, L, my_e, g, lane, out);
  wave_lds_sync();
}

// Resolution of the P = T*k pairs of T >= 2 tokens (thread p = pair p).
// Misses keep pair order (a ballot scan).  Hits are bucketed by expert, the
// buckets in ascending expert order, each bucket's pairs in token order (a
// token chooses an expert at most once): every expert gathers the mask of
// the tokens that chose it, and one scan over the experts of (bucket
// exists, bucket size) places the buckets and their pairs.  L.emask must be
// zero on entry; three barriers.
__device__ __forceinline__ void resolve_multi(const LayerArgs& a, Lds& L, int P, bool writer) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k, E = a.E;
  const bool valid = tid < P;
  const int e = valid ? L.idx[tid] : 0;
  const int t = valid ? tid / k : 0;
  const int s = valid ? slot_of_choice(a, L, e) : -1;
  const bool hit = s >= 0;
  if (hit) atomicOr(&L.emask[e], 1u << t);
  const uint64_t mm = __ballot(valid && !hit);
  if (lane == 0) L.tmp[wave] = uint32_t(__popcll(mm));
  __syncthreads();
  int mpos = lanes_below(mm), n_miss = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = int(L.tmp[w]);
    mpos += w < wave ? c : 0;
    n_miss += c;
  }
  if (writer) {
    if (valid && a.slot_idx) *gmem_w(a.slot_idx + tid) = s;
    if (valid && !hit) {
      moe_miss m;
      m.expert = e;
      m.token = t;
      m.gate = L.gate[tid];
      store_miss(a.miss + mpos, m);
    }
    if (valid && tid % k == 0) *gmem_w(a.miss_off + t) = mpos;
    if (tid == 0) *gmem_w(a.miss_off + a.T) = n_miss;
  }
  // experts 2*tid and 2*tid + 1 (E <= 2 * kThreads)
  const int e0 = 2 * tid;
  const uint32_t m0 = e0 < E ? L.emask[e0] : 0u, m1 = e0 + 1 < E ? L.emask[e0 + 1] : 0u;
  const uint32_t v0 = m0 ? (1u << 16) | uint32_t(__popc(m0)) : 0u;
  const uint32_t v1 = m1 ? (1u << 16) | uint32_t(__popc(m1)) : 0u;
  uint32_t total;
  const uint32_t x0 = block_scan_u32(v0 + v1, L.tmp + 8, &total);
  const uint32_t x1 = x0 + v0;
  if (m0) {
    L.act_slot[x0 >> 16] = slot_of_choice(a, L, e0);
    L.act_start[x0 >> 16] = int(x0 & 0xFFFFu);
    L.emask[e0] = m0 | (x0 << 16);
  }
  if (m1) {
    L.act_slot[x1 >> 16] = slot_of_choice(a, L, e0 + 1);
    L.act_start[x1 >> 16] = int(x1 & 0xFFFFu);
    L.emask[e0 + 1] = m1 | (x1 << 16);
  }
  if (tid == 0) {
    L.act_start[total >> 16] = int(total & 0xFFFFu);
    L.n_act = int(total >> 16);
  }
  __syncthreads();
  if (hit) {
    const uint32_t w = L.emask[e];
    const int pos = int(w >> 16) + __popc(w & ((1u << t) - 1u));
    L.bpair[pos] = tid;
    L.tok[pos] = t;
  }
}

// --------------------------------------------------------------- kernel
// TB: the largest token count the instance serves (1, 4 or 16), so per-token
// loops are unrolled no further than needed.
template <int FMT, int TB>
__global__ __launch_bounds__(kThreads) void moe_layer_kernel(LayerArgs ka) {
  constexpr int kLprGU = Lanes<FMT>::kGU, kRowsGU = Lanes<FMT>::kRowsGU;
  constexpr int kLprD = Lanes<FMT>::kD, kRowsD = Lanes<FMT>::kRowsD;
  extern __shared__ uint32_t smem[];
  __shared__ Lds L;
  __shared__ const uint64_t* srcs[kTMax];
  // The arguments are copied to LDS: after the first loads every phase reads
  // the fields it needs from there, so they do not occupy scalar registers
  // for the whole launch.
  __shared__ LayerArgs sa;
  const int G = gridDim.x, b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid == 0) sa = ka;
  const int T = ka.T, k = ka.k, P = T * k, E = ka.E;
  const int K = ka.H;
  const int vstride = FMT == MOE_W_F32 ? K : (K / Fmt<FMT>::kWPC) * Fmt<FMT>::kCS;
  // LDS: tokens | block sums | group sums | logits
  uint32_t* xs = smem;
  float* xsum = reinterpret_cast<float*>(xs + T * vstride);
  float* psum = xsum + T * (K / 32);
  float* lg = psum + T * (K / 16);

  // ---- A: loads first (call counter, slot table, first task's rows)
  const uint32_t calls = tid == 0 ? ld_dev(region_calls(ka)) : 0u;
  int so[kEMax / kThreads];
#pragma unroll
  for (int r = 0; r < kEMax / kThreads; ++r) {
    const int e = tid + r * kThreads;
    so[r] = (ka.slot_of && e < E) ? ka.slot_of[e] : -1;
  }
  // router tasks: row groups x token groups of kTG (a row group's token
  // groups share a workgroup when there are at most G row groups)
  constexpr int kTG = TB == 1 ? 1 : TB == 4 ? 2 : 4;
  constexpr int kNG = TB == 1 ? 1 : 4;   // tokens per unpacked block
  constexpr int kNGC = TB == 1 ? 1 : 4;  // the same for routed gate/up
  const int n_rg = (E + (64 / router_lpr<FMT>(K)) - 1) / (64 / router_lpr<FMT>(K));
  const int n_router = n_rg * ((T + kTG - 1) / kTG);
  // shared-expert gate/up tasks: row blocks x token groups of kTG
  const int n_srb = ka.I / kRowsGU;
  const int n_shared = ka.has_sh ? n_srb * ((T + kTG - 1) / kTG) : 0;
  const int n_a = n_router + n_shared;
  const int task0 = b + wave * G;
  const int lane_gu = lane % kLprGU;
  RouterRegs<FMT> rr;
  RowRegs<FMT, nch_gu<FMT>()> rg, ru;
  if (task0 < n_router)
    router_load<FMT>(rr, ka, task0, task0 % n_rg, n_router, lane);
  else if (task0 < n_a)
    gateup_load<FMT>(rg, ru, ka, ka.sg, ka.su, 0,
                     ((task0 - n_router) % n_srb) * kRowsGU + lane / kLprGU, lane_gu);
  stage_tokens<FMT>(ka.x, T, K, xs, psum, vstride);
  if (tid == 0) L.calls = calls;
  for (int e = tid; e < kEMax; e += kThreads) L.emask[e] = 0u;
  if (tid < kTMax) L.ncand[tid] = 0;
#pragma unroll
  for (int r = 0; r < kEMax / kThreads; ++r)
    if (tid + r * kThreads < E) L.slot_of[tid + r * kThreads] = so[r];
  __syncthreads();
  const LayerArgs& a = sa;
  token_block_sums(T, K, xsum, psum);
  __syncthreads();
  const uint32_t epoch = L.calls + 1u;   // this call's number
  for (int task = task0; task < n_a; task += kWaves * G) {
    if (task < n_router) {
      if (task != task0) router_load<FMT>(rr, a, task, task % n_rg, n_router, lane);
      router_compute<FMT, kTG>(rr, a, task % n_rg, (task / n_rg) * kTG, xs, vstride, lane, epoch);
    } else {
      const int s = task - n_router, t0 = (s / n_srb) * kTG;
      const int i = (s % n_srb) * kRowsGU + lane / kLprGU;
      if (task != task0) gateup_load<FMT>(rg, ru, a, a.sg, a.su, 0, i, lane_gu);
      gateup_compute<FMT, kNG>(rg, ru, a, i, min(kTG, T - t0), nullptr, nullptr, t0, region_h_sh(a), xs,
                          xsum, vstride, lane_gu, epoch);
    }
  }

  // this workgroup has read the counter (workgroup 0 checks before it
  // advances the counter)
  if (tid == 0) st_dev(region_arrive(a) + b, tag_word(0.f, epoch));

  // ---- B: every logit of this call, then routing
  if constexpr (TB == 1) {
    route_token(a, lg, E, k, L, epoch, b == 0);
  } else {
    const int n_lg = T * E;
    constexpr int kR = TB * kEMax / kThreads > 16 ? 16 : TB * kEMax / kThreads;
    for (int base = 0; base < n_lg; base += kR * kThreads) {
      uint64_t w[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int i = base + r * kThreads + tid;
        if (i < n_lg) w[r] = ld_dev(region_lg(a) + i);
      }
      for (;;) {
        bool ok = true;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int i = base + r * kThreads + tid;
          ok = ok && (i >= n_lg || tag_ok(w[r], epoch));
        }
        if (ok) break;
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int i = base + r * kThreads + tid;
          if (i < n_lg && !tag_ok(w[r], epoch)) w[r] = ld_dev(region_lg(a) + i);
        }
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int i = base + r * kThreads + tid;
        if (i < n_lg) lg[i] = tag_val(w[r]);
      }
    }
  __syncthreads();
  const bool thresh = k <= kTopkListMax;
  if (thresh) topk_threshold<TB>(lg, T, E, k, L);
  // tokens the threshold selection did not take: one wave each
  for (int t = wave; t < T; t += kWaves) {
    if (thresh && L.ncand[t] <= kThreads / TB) continue;
    int my_e;
    float my_v;
    if (E <= 512) wave_topk<8>(lg + t * E, E, k, lane, &my_e, &my_v);
    else wave_topk<16>(lg + t * E, E, k, lane, &my_e, &my_v);
    if (lane < k) {
      L.idx[t * k + lane] = my_e;
      L.gate[t * k + lane] = my_v;
    }
  }
  __syncthreads();
  for (int t = wave; t < T; t += kWaves) {
    // gates: softmax over the k chosen logits (choice 0 is the largest)
    const int my_e = lane < k ? L.idx[t * k + lane] : 0;
    const float my_v = lane < k ? L.gate[t * k + lane] : 0.f;
    const float vmax = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_v), 0));
    const float ex = lane < k ? expf(my_v - vmax) : 0.f;
    const float z = wave_sum_f32(ex);
    const float g = ex / z;
    if (lane < k) {
      L.gate[t * k + lane] = g;
      if (b == 0) {
        *gmem_w(a.idx + t * k + lane) = my_e;
        *gmem_w(a.gate + t * k + lane) = g;
      }
    }
  }
  __syncthreads();
  resolve_multi(a, L, P, b == 0);   // T >= 2 here
  __syncthreads();
  }
  const int n_act = L.n_act;
  if (b == 0 && a.usage && tid < P)
    __hip_atomic_fetch_add(gmem_w(a.usage + L.idx[tid]), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);

  // ---- C: routed gate/up
  const int Kd = a.I;
  const int vs_d = FMT == MOE_W_F32 ? Kd : (Kd / Fmt<FMT>::kWPC) * Fmt<FMT>::kCS;
  const int ss_d = Kd / 32;
  const int nch_d = chunks_of<FMT>(Kd) / kLprD;
  const int64_t row_bytes_d = int64_t(Kd) * fmt_bits(FMT) / 8;
  const int nrb = (a.H + kRowsD - 1) / kRowsD;
  const int n_units = (n_act + (a.has_sh ? 1 : 0)) * nrb;
  const int tpe = a.I / kRowsGU;
  const int n_tasks = n_act * tpe;
  const int lane_gd = lane % kLprD;
  // Who does what.  One token: gate/up tasks (bucket, row block) dealt to
  // the waves in turn and down units (bucket, row block) to the workgroups
  // in turn -- every bucket has one token, so their costs are equal.  More
  // tokens: buckets differ in size, so each wave takes a contiguous range
  // of tasks and each workgroup a contiguous range of units with equal sums
  // of cost (a fixed part plus the bucket's tokens).  Thread u finds the
  // range bounds that fall inside bucket u's span of cumulative cost.
  int c_first = b + wave * G, c_end = n_tasks, c_step = kWaves * G;
  int d_first = b, d_end = n_units, d_step = G;
  if constexpr (TB > 1) {
    constexpr int kCostC = 2, kCostD = 1;
    const int n_db = n_act + (a.has_sh ? 1 : 0);
    // (costs stay below 2^20; a bound's exact quotient a * tot / W comes from
    // double arithmetic: the product is exact and no quotient lies within a
    // rounding error of an integer it does not equal)
    const int totC = tpe * (kCostC * n_act + L.act_start[n_act]);
    const int totD = nrb * (kCostD * n_db + L.act_start[n_act] + (a.has_sh ? T : 0));
    auto bound = [](int i, int tot, int parts) {
      return int(floor(double(i) * double(tot) / double(parts)));
    };
    // One thread per range bound (kWaves + 1 task bounds, 2 unit bounds):
    // a binary search for the bucket whose span of cumulative cost holds the
    // bound's target, then the first task / unit of that bucket at or past it.
    if (tid <= kWaves + 2) {
      const bool is_c = tid <= kWaves;
      const int n = is_c ? n_act : n_db;
      const int rows = is_c ? tpe : nrb, fixed = is_c ? kCostC : kCostD;
      const int bt = is_c ? bound(b * kWaves + tid, totC, G * kWaves)
                          : bound(b + tid - (kWaves + 1), totD, G);
      auto tokens_before = [&](int u) {   // tokens of buckets < u (the shared one last)
        return u <= n_act ? L.act_start[u] : L.act_start[n_act] + T;
      };
      auto cum = [&](int u) { return rows * (fixed * u + tokens_before(u)); };
      int lo = 0, hi = n;   // the largest u <= n with cum(u) <= bt
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cum(mid) <= bt) lo = mid;
        else hi = mid - 1;
      }
      int v;
      if (lo == n) {
        v = is_c ? n_tasks : n_units;
      } else {
        const int cost = fixed + (lo < n_act ? L.act_start[lo + 1] - L.act_start[lo] : T);
        v = lo * rows + (bt - cum(lo) + cost - 1) / cost;
      }
      if (is_c) L.cstart[tid] = v;
      else L.dstart[tid - (kWaves + 1)] = v;
    }
    __syncthreads();
    c_first = L.cstart[wave];
    c_end = L.cstart[wave + 1];
    c_step = 1;
    d_first = L.dstart[0];
    d_end = L.dstart[1];
    d_step = 1;
  }
  RowRegs<FMT, kNChD> rd;
  auto load_down = [&](int unit, RowRegs<FMT, kNChD>& rd) {
    const int u = unit / nrb, rb = unit % nrb;
    const bool shared = u >= n_act;
    const Planes D = shared ? a.sd : a.d;
    const int slot = shared ? 0 : L.act_slot[u];
    const int r = rb * kRowsD + wave * (64 / kLprD) + lane / kLprD;
    const int rr_ = r < a.H ? r : a.H - 1;
    const int64_t blk = int64_t(slot) * a.mat_blocks + int64_t(rr_) * ss_d;
    load_row<FMT, kNChD>(rd, D.codes + slot * a.mat_bytes + rr_ * row_bytes_d, D.scale + blk,
                           D.mn + blk, nch_d, lane_gd, kLprD);
  };
  // One load per 128-byte line of this wave's share of a unit's rows (codes,
  // then scales and minima), whose values are not used: it brings the lines
  // into this XCD's L2 for one address-unit slot per wave instead of one per
  // row chunk.  Lines past the wave's 64 lanes are left out.  Every lane
  // loads (spare lanes and unit < 0 read the hand-off region), so that the
  // load is issued on every path and waits for earlier loads need not wait
  // for it.
  auto prefetch_down = [&](int unit) -> uint32_t {
    uintptr_t p = reinterpret_cast<uintptr_t>(a.region);
    if (unit >= 0) {
      const int u = unit / nrb, rb = unit % nrb;
      const bool shared = u >= n_act;
      const Planes D = shared ? a.sd : a.d;
      const int slot = shared ? 0 : L.act_slot[u];
      const int r0 = rb * kRowsD + wave * (64 / kLprD);
      const int nr = max(0, min(64 / kLprD, a.H - r0));
      const int nl_c = int((nr * row_bytes_d + 127) / 128);
      const uintptr_t c0 = reinterpret_cast<uintptr_t>(D.codes + slot * a.mat_bytes + r0 * row_bytes_d);
      p = lane < nl_c ? c0 + uintptr_t(lane) * 128 : p;
      if constexpr (FMT != MOE_W_F32) {
        const int64_t blk = int64_t(slot) * a.mat_blocks + int64_t(r0) * ss_d;
        const int nl_s = (nr * ss_d * 2 + 127) / 128;
        const int l = lane - nl_c;
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(D.scale + blk);
        const uintptr_t m0 = reinterpret_cast<uintptr_t>(D.mn + blk);
        p = (l >= 0 && l < nl_s) ? s0 + uintptr_t(l) * 128 : p;
        p = (l >= nl_s && l < 2 * nl_s) ? m0 + uintptr_t(l - nl_s) * 128 : p;
      }
    }
    return *gmem(reinterpret_cast<const uint32_t*>(p & ~uintptr_t(3)));
  };
  uint32_t pf = 0u;
  uint64_t arr = 0;
  {
    // each wave's tasks in turn, the next task's rows loading while the
    // current one computes
    // With several tasks per wave (T > 1) the rows of the next two tasks
    // are in flight while one computes; one token has at most one task.
    constexpr int kAhead = TB > 1 ? 2 : 1;
    auto load_task = [&](int t, RowRegs<FMT, nch_gu<FMT>()>& g, RowRegs<FMT, nch_gu<FMT>()>& u) {
      gateup_load<FMT>(g, u, a, a.g, a.u, L.act_slot[t / tpe], (t % tpe) * kRowsGU + lane / kLprGU,
                       lane_gu);
    };
    int task = c_first;
    RowRegs<FMT, nch_gu<FMT>()> ng, nu;
    if (task < c_end) load_task(task, rg, ru);
    if (kAhead == 2 && task + c_step < c_end) load_task(task + c_step, ng, nu);
    // one token: the first down unit's lines head for the L2 meanwhile
    if constexpr (TB == 1) pf = prefetch_down(d_first < d_end ? d_first : -1);
    auto compute_task = [&](int t, const RowRegs<FMT, nch_gu<FMT>()>& g,
                            const RowRegs<FMT, nch_gu<FMT>()>& up) {
      const int u = t / tpe;
      const int i = (t % tpe) * kRowsGU + lane / kLprGU;
      const int st = L.act_start[u];
      const int n = L.act_start[u + 1] - st;
      gateup_compute<FMT, kNGC>(g, up, a, i, n, L.tok + st, L.bpair + st, 0, region_h(a), xs,
                                xsum, vstride, lane_gu, epoch);
    };
    // At most one task (one token, the usual case): no loop, so no load is
    // issued on one path and not on another, which would make the waits
    // for the rows also wait for the prefetch.
    if (TB == 1 && task + c_step >= c_end) {
      if (task < c_end) compute_task(task, rg, ru);
      task = c_end;
    }
    for (; task < c_end; task += c_step) {
      const int ahead = task + kAhead * c_step;
      RowRegs<FMT, nch_gu<FMT>()> mg, mu;
      if (ahead < c_end) load_task(ahead, mg, mu);
      compute_task(task, rg, ru);
      if constexpr (kAhead == 2) {
        rg = ng;
        ru = nu;
        ng = mg;
        nu = mu;
      } else {
        rg = mg;
        ru = mu;
      }
    }
  }

  // ---- D: down units (expert or shared, block of rows), y += gate * D h
  {
    uint32_t* xd = smem;                                    // reuses the token area
    float* sd = reinterpret_cast<float*>(xd + kTMax * vs_d);
    float* pd = sd + kTMax * ss_d;
    float* bsc = pd + kTMax * (Kd / 16);
    // The first unit's rows load here, not during gate/up: there they would
    // queue ahead of other waves' gate/up rows in the CU's address unit,
    // which would then finish later.
    if (d_first < d_end) load_down(d_first, rd);
    // the arrival words, read while the first unit's activations are polled
    // for (issued here, no later register reuse has to wait for them)
    if (b == 0 && tid < G) arr = ld_dev(region_arrive(a) + tid);
    int staged = -1;   // bucket whose activations are in the LDS
    for (int unit = d_first; unit < d_end; unit += d_step) {
      RowRegs<FMT, kNChD> nd;   // the next unit's rows load meanwhile
      if (unit + d_step < d_end) load_down(unit + d_step, nd);
      const int u = unit / nrb, rb = unit % nrb;
      const bool shared = u >= n_act;
      const int st = shared ? 0 : L.act_start[u];
      const int n = shared ? T : L.act_start[u + 1] - st;
      const int r = rb * kRowsD + wave * (64 / kLprD) + lane / kLprD;
      if (u != staged) {
        __syncthreads();   // gate/up tasks and the previous unit are done with the LDS
        if (tid < n)
          srcs[tid] = shared ? region_h_sh(a) + int64_t(tid) * Kd
                             : region_h(a) + int64_t(L.bpair[st + tid]) * Kd;
        __syncthreads();
        stage_h<FMT>(srcs, n, Kd, xd, sd, pd, bsc, vs_d, epoch);
        __syncthreads();
        staged = u;
      }
      for (int v0 = 0; v0 < n; v0 += kNG) {
        const int nv = min(kNG, n - v0);
        float o[kNG];
        if constexpr (FMT != MOE_W_F32) {
          row_vecs_dot_f16<FMT, kNChD, kNG>(rd, nch_d, lane_gd, kLprD, xd, sd, bsc, vs_d, ss_d, v0,
                                            nv, o);
        } else {
#pragma unroll
          for (int v = 0; v < kNG; ++v)
            o[v] = v < nv ? row_vec_dot<FMT, kNChD>(rd, nch_d, lane_gd, kLprD,
                                                     xd + (v0 + v) * vs_d, sd + (v0 + v) * ss_d)
                          : 0.f;
        }
#pragma unroll
        for (int v = 0; v < kNG; ++v) {
          if (v >= nv) continue;
          const float os = group_sum<kLprD>(o[v]);
          if (r < a.H && lane_gd == 0) {
            const int t = shared ? v0 + v : L.tok[st + v0 + v];
            const float g = shared ? 1.f : L.gate[L.bpair[st + v0 + v]];
            fadd_dev(a.y + int64_t(t) * a.H + r, g * os);
          }
        }
      }
      rd = nd;
    }
  }
  // Workgroup 0 advances the call counter once every workgroup has read it.
  if (b == 0) {
    if (tid < G)
      while (!tag_ok(arr, epoch)) {
        __builtin_amdgcn_s_sleep(1);
        arr = ld_dev(region_arrive(a) + tid);
      }
    __syncthreads();
    if (tid == 0) st_dev(region_calls(a), epoch);
  }
  asm volatile("" ::"v"(pf));   // the prefetch's value counts as used
}

struct Occ {
  size_t lds = 0;
  int device = -1;
  int grid = 0;
};

template <int FMT, int TB>
hipError_t launch_fmt(const LayerArgs& a, size_t lds, hipStream_t st, int* grid_out) {
  static thread_local Occ c;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (c.lds != lds || c.device != dev) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_layer_kernel<FMT, TB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_layer_kernel<FMT, TB>, kThreads,
                                                     lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // one arrival word per workgroup; the block-wide scans take <= 512 threads
    if (per_cu < 1 || cus > kLayerMaxGrid || cus > kThreads) return hipErrorInvalidConfiguration;
    c.lds = lds;
    c.device = dev;
    c.grid = cus;   // one workgroup of 8 waves per CU
  }
  if (grid_out) *grid_out = c.grid;
  hipLaunchKernelGGL((moe_layer_kernel<FMT, TB>), dim3(c.grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_tb(const LayerArgs& a, size_t lds, hipStream_t st, int* grid_out) {
  if (a.T <= 1) return launch_fmt<FMT, 1>(a, lds, st, grid_out);
  if (a.T <= 4) return launch_fmt<FMT, 4>(a, lds, st, grid_out);
  return launch_fmt<FMT, kTMax>(a, lds, st, grid_out);
}

size_t vec_bytes(int fmt, int K) {
  if (fmt == MOE_W_F32) return size_t(K) * 4;
  const int wpc = fmt == MOE_W_Q2B32 ? 64 : 32, cs = fmt == MOE_W_Q2B32 ? 36 : 20;
  return size_t(K / wpc) * cs * 4;
}

}  // namespace

size_t layer_fused_lds(int fmt, int T, int E, int H, int I) {
  // A-C: tokens, block sums, group sums, logits
  const size_t a = size_t(T) * (vec_bytes(fmt, H) + (H / 32) * 4 + (H / 16) * 4) +
                   size_t(T) * E * 4;
  // D: a vector per token, block sums, group sums, block scales (16 tokens)
  const size_t d = size_t(kTMax) * (vec_bytes(fmt, I) + (I / 32) * 4 + (I / 16) * 4 + (I / 32) * 4);
  return a > d ? a : d;
}

bool layer_fused_ok(int fmt, int T, int k, int E, int H, int I) {
  if (T < 1 || T > kTMax || T * k > kPMax) return false;
  if (fmt != MOE_W_F32 && fmt != MOE_W_Q2B32 && fmt != MOE_W_Q4B32) return false;
  if (H % 32 || I % 32 || E > kEMax) return false;
  const int wpc = fmt == MOE_W_Q2B32 ? 64 : fmt == MOE_W_Q4B32 ? 32 : 4;
  const int lgu = fmt == MOE_W_Q4B32 ? Lanes<MOE_W_Q4B32>::kGU : Lanes<MOE_W_Q2B32>::kGU;
  const int ld = fmt == MOE_W_Q4B32 ? Lanes<MOE_W_Q4B32>::kD : Lanes<MOE_W_Q2B32>::kD;
  const int chunks = H / wpc, chunks_d = I / wpc;
  const int ngu = fmt == MOE_W_Q2B32 ? nch_gu<MOE_W_Q2B32>() : 4;
  if (chunks % lgu || chunks / lgu > ngu) return false;
  if (chunks_d % ld || chunks_d / ld > kNChD) return false;
  if (fmt != MOE_W_F32 && (chunks > 64 ? (chunks % 64) != 0 : (chunks & (chunks - 1)) != 0))
    return false;
  // dynamic LDS beside the static routing tables (~19 KB) within 160 KB
  return layer_fused_lds(fmt, T, E, H, I) <= 140 * 1024;
}

hipError_t launch_layer_fused(const LayerArgs& a, int fmt, hipStream_t st, int* grid) {
  const size_t lds = layer_fused_lds(fmt, a.T, a.E, a.H, a.I);
  switch (fmt) {
    case MOE_W_Q2B32: return launch_tb<MOE_W_Q2B32>(a, lds, st, grid);
    case MOE_W_Q4B32: return launch_tb<MOE_W_Q4B32>(a, lds, st, grid);
    case MOE_W_F32: return launch_fmt<MOE_W_F32, kTMax>(a, lds, st, grid);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
