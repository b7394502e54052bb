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
//     tokens are staged in LDS; router waves zero their share of y before
//     they publish their logits.
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
// Every wait is bounded: a workgroup that has polled for longer than the
// budget since its start (another kernel holding some CUs would keep
// producers from running) marks the call failed in the region header and
// goes on without the data; the call's outputs are then unspecified (every
// access still stays in bounds), and later calls on the workspace return at
// once until the caller zeroes it again (moe_layer_check reports it).
#include <mutex>
#include <type_traits>

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
__device__ __forceinline__ uint32_t* region_err(const LayerArgs& a) {
  return reinterpret_cast<uint32_t*>(a.region + kRegionErr);
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
// down-projection rows for the fixed-order sum: pair p at row p, the shared
// expert's row of token t at row layer_h_rows(k) - 16 + t
__device__ __forceinline__ uint64_t* region_part(const LayerArgs& a) {
  return region_h(a) + int64_t(layer_h_rows(a.k)) * a.I;
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
  uint64_t hmask[kTMax];     // per token: the choices j that hit a resident slot (bit j)
  alignas(16) uint32_t tmp[32];
  int dstart[2];            // this workgroup's down unit range (contiguous split)
  int dalign[2];            // the same, bucket-aligned split
  int dzero;                // 1: no bound fits the aligned split (more buckets than workgroups)
  int dhist[kTMax + 1];     // down buckets by tokens
  int n_act;
  uint32_t calls;
  int failed;               // 1: this workgroup gave up a wait; 2: the workspace was poisoned
  unsigned long long t_gu;  // trace: latest gate/up end over the waves
  unsigned long long t_a;   // trace: latest router / shared-expert task end over the waves
};

// Phase stamp (thread 0 of the workgroup; nothing when tracing is off).
__device__ __forceinline__ void stamp(uint64_t* trace, int slot, uint64_t v) {
  if (trace && threadIdx.x == 0) trace[blockIdx.x * kTraceSlots + slot] = v;
}
__device__ __forceinline__ void stamp_now(uint64_t* trace, int slot) {
  if (trace) stamp(trace, slot, __builtin_amdgcn_s_memrealtime());
}

// Bounded waits.  Returns true while a poll may go on.  Once the launch has
// run for the budget (t0: the thread's start time), or another thread of
// the workgroup has given up, it returns false; the first to give up marks
// the workgroup and the call (error word) failed.
__device__ __forceinline__ bool keep_waiting(const LayerArgs& a, Lds& L, uint64_t t0) {
  if (*reinterpret_cast<volatile int*>(&L.failed)) return false;
  if (__builtin_amdgcn_s_memrealtime() - t0 < a.wait_ticks) return true;
  *reinterpret_cast<volatile int*>(&L.failed) = 1;
  st_dev(region_err(a), L.calls + 1u);
  return false;
}

// --------------------------------------------------------------- staging
// Code pairs of a 2-bit code dword by class.  Pair s (codes s and s + 8)
// is taken from the dword shifted right by 6 * (s / 3), masked to its two
// fields at bits 2c and 16 + 2c, c = s % 3, and OR-ed into the mantissa of
// bf16(128): the pair is 128 + q * 4^c, exact, from one shift per three
// pairs and one AND-OR per pair.  The staged tokens carry the matching
// factor: pair s of a token is x * 4^-c (exact), so a block dot product of
// the pairs is sum q x + 128 * sum x', x' the staged values.
__device__ __forceinline__ int q2_class(int s) { return s % 3; }
// (a & m) | c as one v_and_or_b32.  Written out because with a literal mask
// and a literal c the compiler splits it into an AND and an OR (a
// three-operand VALU instruction takes no literal on this architecture);
// here the mask sits in a scalar register and c in a vector register, both
// set up once.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t q2_pair_cls(uint32_t w, int s) {
  return and_or(w >> (6 * (s / 3)), 0x00030003u << (2 * q2_class(s)), kMagic128x2);
}
// fp16 code pairs by class, for the class-staged h (fp16 1024 = 0x6400 has
// ten mantissa bits of weight 1 .. 512).  2-bit codes, pair s (codes s and
// s + 8): class c = s for s < 5 (fields at bits 2c, 16 + 2c), else s - 5
// from the dword shifted right by 10; the pair is 1024 + q * 4^c.  4-bit
// codes, pair s (codes s and s + 4): class c = s & 1 from the dword shifted
// right by 8 * (s >> 1); the pair is 1024 + q * 16^c.  One shift per five
// (two) pairs and one AND-OR per pair; h is staged as h * 4^-c (16^-c).
template <int FMT>
__device__ __forceinline__ int f16_class(int s) {
  return FMT == MOE_W_Q2B32 ? (s < 5 ? s : s - 5) : (s & 1);
}
template <int FMT>
__device__ __forceinline__ uint32_t f16_pair_cls(uint32_t w, int s) {
  if constexpr (FMT == MOE_W_Q2B32)
    return and_or(w >> (s < 5 ? 0 : 10), 0x00030003u << (2 * f16_class<FMT>(s)), 0x64006400u);
  else
    return and_or(w >> (8 * (s >> 1)), 0x000F000Fu << (4 * (s & 1)), 0x64006400u);
}
// A bf16 pair times 2^-e2 (both halves).  The fp32 products are exact, so
// their top halves are the bf16 results (for results below the normal
// range, truncated).
__device__ __forceinline__ uint32_t bf16x2_scaled(uint32_t p, int e2) {
  const float f = __uint_as_float(uint32_t(127 - e2) << 23);
  const uint32_t lo = __float_as_uint(__uint_as_float(p << 16) * f);
  const uint32_t hi = __float_as_uint(__uint_as_float(p & 0xFFFF0000u) * f);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Tokens into the expert format's LDS layout, with 32-byte loads per
// thread (16 columns of one token) issued before any is used.  xsum gets
// each 32-column block's sum of the token's values, xsum2 (2-bit codes)
// -128 times the sum of the values as staged (x'); the two 16-column groups of a
// block sit in lanes 2j and 2j + 1 and add in that order.  The caller
// synchronises before reading xs or the sums.
// mid() runs once, after the first batch's loads are issued and before they
// are used.
template <int FMT, typename Mid>
__device__ __forceinline__ void stage_tokens(const uint16_t* __restrict__ x, int T, int H, uint32_t* xs,
                                             float* xsum, float* xsum2, int vstride, Mid mid) {
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
      } else {
        w[r][0] = u32x4{0u, 0u, 0u, 0u};
        w[r][1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (base == 0) mid();
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int it = base + r * kThreads + threadIdx.x;
      const bool on = it < n_items;   // the same for lanes 2j and 2j + 1
      const int t = it / per_tok, g16 = it % per_tok;
      float s = 0.f, s2 = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s += bf16_to_f32(w[r][q][e] & 0xFFFFu) + bf16_to_f32(w[r][q][e] >> 16);
      if constexpr (FMT == MOE_W_F32) {
        if (on) {
          float* xf = reinterpret_cast<float*>(xs) + t * vstride + g16 * 16;
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              xf[q * 8 + 2 * e] = bf16_to_f32(w[r][q][e] & 0xFFFFu);
              xf[q * 8 + 2 * e + 1] = bf16_to_f32(w[r][q][e] >> 16);
            }
        }
      } else if constexpr (FMT == MOE_W_Q2B32) {
        // pairs (s, s+8), s < 8, of this 16-column group, pair s times 4^-(s % 3)
        uint32_t pr[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          pr[2 * m] = __builtin_amdgcn_perm(w[r][1][m], w[r][0][m], 0x05040100u);
          pr[2 * m + 1] = __builtin_amdgcn_perm(w[r][1][m], w[r][0][m], 0x07060302u);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (q2_class(q) != 0) pr[q] = bf16x2_scaled(pr[q], 2 * q2_class(q));
          s2 += bf16_to_f32(pr[q] & 0xFFFFu) + bf16_to_f32(pr[q] >> 16);
        }
        if (on) {
          uint32_t* d = xs + t * vstride + (g16 >> 2) * Fmt<FMT>::kCS + (g16 & 3) * 8;
#pragma unroll
          for (int q = 0; q < 8; ++q) d[q] = pr[q];
        }
      } else {
        // two 8-column groups, pairs (s, s+4), s < 4
        if (on) {
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
      // block sums: group 2b (even lane) + group 2b + 1 (odd lane)
      const float sp = dpp_f32<0xB1>(s), sp2 = dpp_f32<0xB1>(s2);   // quad_perm [1,0,3,2]
      if (on && (g16 & 1) == 0) {
        xsum[t * (H / 32) + (g16 >> 1)] = s + sp;
        if constexpr (FMT == MOE_W_Q2B32) xsum2[t * (H / 32) + (g16 >> 1)] = -128.f * (s2 + sp2);
      }
    }
  }
}

// Tagged fp32 vectors published by other workgroups (h), staged for the
// down projection, 16 columns per item.  Quantised formats: fp16 in the pair
// layout, each 32-column block scaled by a power of two that brings its
// largest |h| into [128, 256) (bsc keeps the inverse), so no block
// overflows fp16 and each keeps 11 bits relative to its largest value; pair
// s is stored times 4^-c (2-bit codes) or 16^-c (4-bit codes), c its code
// class, so even the smallest class factor leaves the block maximum a
// normal fp16 number.  sd gets the block sums of h (the scaled values
// times bsc), sd2 -1024 bsc times the block sums of the values as stored.
// F32 format: plain fp32.
// All loads of a batch are issued first; words that do not yet carry this
// call's number are read again until they do (their producers never wait
// on anything, so this ends).  Every thread calls it (the block sums and
// maxima pass between neighbouring lanes).
template <int FMT>
__device__ __forceinline__ void stage_h(const uint64_t* const* srcs, int n, int K, uint32_t* xd,
                                        float* sd, float* sd2, float* bsc, int vs,
                                        uint32_t epoch, const LayerArgs& a, Lds& L, uint64_t t0,
                                        uint64_t* trc) {
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
    auto all_here = [&]() {
      bool ok = true;
#pragma unroll
      for (int r = 0; r < kIt; ++r)
#pragma unroll
        for (int c = 0; c < 16; ++c) ok = ok && (!src[r] || tag_ok(wv[r][c], epoch));
      return ok;
    };
    int rounds = 1;
    while (!all_here() && keep_waiting(a, L, t0)) {
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int r = 0; r < kIt; ++r)
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (src[r] && !tag_ok(wv[r][c], epoch)) wv[r][c] = ld_dev(src[r] + c);
      ++rounds;
    }
    if (base == 0 && trc) {
      stamp_now(trc, kTrHPolled);
      stamp(trc, kTrHPolls, uint64_t(rounds));
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
        ex = ex < 8u ? 8u : (ex > 253u ? 253u : ex);
        // amax in [2^(ex-127), 2^(ex-126)): scale by 2^(134-ex) (zero and
        // tiny maxima take the smallest exponent, 8)
        const float sc = __uint_as_float((261u - ex) << 23);
        const float inv = __uint_as_float((ex - 7u) << 23);
        // pair q: columns (q, q + 8) (2-bit codes) or (8g + e, 8g + e + 4)
        // (4-bit codes, q = 4g + e); stored times 2^-cls
        uint32_t hp[8];
        float sum = 0.f, sum2 = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int lo = FMT == MOE_W_Q2B32 ? q : 8 * (q >> 2) + (q & 3);
          const int hi = FMT == MOE_W_Q2B32 ? q + 8 : lo + 4;
          const int cls = FMT == MOE_W_Q2B32 ? 2 * f16_class<FMT>(q) : 4 * f16_class<FMT>(q & 3);
          const float scq = sc * __uint_as_float(uint32_t(127 - cls) << 23);
          const _Float16 h0 = static_cast<_Float16>(v[lo] * scq);
          const _Float16 h1 = static_cast<_Float16>(v[hi] * scq);
          hp[q] = uint32_t(__builtin_bit_cast(uint16_t, h0)) |
                  (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
          const float p2 = static_cast<float>(h0) + static_cast<float>(h1);
          sum2 += p2;
          sum += p2 * __uint_as_float(uint32_t(127 + cls) << 23);
        }
        // block sums: group 2b (even lane) + group 2b + 1 (odd lane)
        const float sp = dpp_f32<0xB1>(sum), sp2 = dpp_f32<0xB1>(sum2);
        if (it < n_items) {
          const int p = it / per_vec, g16 = it % per_vec;
          if ((g16 & 1) == 0) {
            bsc[p * (K / 32) + (g16 >> 1)] = inv;
            sd[p * (K / 32) + (g16 >> 1)] = inv * (sum + sp);
            sd2[p * (K / 32) + (g16 >> 1)] = -1024.f * inv * (sum2 + sp2);
          }
          uint32_t* dh = xd + p * vs;
          if constexpr (FMT == MOE_W_Q2B32) {
            const int off = (g16 >> 2) * Fmt<FMT>::kCS + (g16 & 3) * 8;
#pragma unroll
            for (int q = 0; q < 8; ++q) dh[off + q] = hp[q];
          } else {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int off = (g16 >> 1) * Fmt<FMT>::kCS + ((g16 & 1) * 2 + q) * 4;
#pragma unroll
              for (int t = 0; t < 4; ++t) dh[off + t] = hp[4 * q + t];
            }
          }
        }
      }
    }
  }
  if (trc) stamp_now(trc, kTrHConv);
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

// A global load; NT: with the non-temporal hint (data read once per call,
// such as a routed expert's rows, so that it does not displace what every
// call reuses: the router and the shared expert).
template <bool NT, typename T>
__device__ __forceinline__ T ldg(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(gmem(p));
  else return *gmem(p);
}

template <int FMT, int NCH, bool NT = false>
__device__ __forceinline__ void load_row(RowRegs<FMT, NCH>& R, const uint8_t* __restrict__ codes,
                                         const uint16_t* __restrict__ sc,
                                         const uint16_t* __restrict__ mn, int nch, int lane_g,
                                         int lpr) {
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j < nch) {
      const int c = lane_g + j * lpr;
      R.w[j] = ldg<NT>(reinterpret_cast<const u32x4*>(codes + 16 * c));
      if constexpr (FMT == MOE_W_Q2B32) {
        R.sc[j] = ldg<NT>(reinterpret_cast<const uint32_t*>(sc + 2 * c));
        R.mn[j] = ldg<NT>(reinterpret_cast<const uint32_t*>(mn + 2 * c));
      } else if constexpr (FMT == MOE_W_Q4B32) {
        R.sc[j] = uint32_t(ldg<NT>(sc + c));
        R.mn[j] = uint32_t(ldg<NT>(mn + c));
      }
    }
  }
}

// This lane's part of one fp32 row . one staged fp32 vector (at xv_base +
// chunk offsets), over the lane's NCH chunks of 4 columns.
template <int FMT, int NCH>
__device__ __forceinline__ float row_vec_dot(const RowRegs<FMT, NCH>& R, int nch, int lane_g,
                                             int lpr, const uint32_t* xv_base) {
  static_assert(FMT == MOE_W_F32, "fp32 rows only");
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j >= nch) continue;
    const int c = lane_g + j * lpr;
    const float4 wf = __builtin_bit_cast(float4, R.w[j]);
    const float* xv = reinterpret_cast<const float*>(xv_base) + 4 * c;
    acc = fmaf(wf.x, xv[0], fmaf(wf.y, xv[1], fmaf(wf.z, xv[2], fmaf(wf.w, xv[3], acc))));
  }
  return acc;
}

// Up to NG tokens at once: the code pairs of a block are unpacked once for
// the group.  Block scale d and min m (w = d q + m):
//  2-bit codes (class-staged x'): d * (sum (128 + q 4^c) x' - 128 sum x') + m * sum x;
//  4-bit codes: d * sum (128 + q) x + (m - 128 d) * sum x,
// with the block sums of the vectors (sum x, and sum x' for 2-bit codes)
// staged beside them.
template <int FMT>
__device__ __forceinline__ void block_scales(uint32_t sc, uint32_t mn, int bb, float& d, float& m) {
  const uint32_t dsh = FMT == MOE_W_Q2B32 ? 16u * uint32_t(bb) : 0u;
  d = f16_to_f32(uint16_t((sc >> dsh) & 0xFFFFu));
  m = f16_to_f32(uint16_t((mn >> dsh) & 0xFFFFu));
}
template <int FMT>
__device__ __forceinline__ void unpack_block(u32x4 w, int bb, uint32_t (&pr)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pr[q * 4 + e] = FMT == MOE_W_Q2B32 ? q2_pair_cls(w[2 * bb + (q >> 1)], (q & 1) * 4 + e)
                                         : and_or(w[q] >> (4 * e), 0x000F000Fu, kMagic128x2);
}
// sum over one block of the code pairs . the vector's pairs (4 chains)
// c + the block's 16 pairs . x, as one chain of dot2 instructions (a
// dependent dot2 issues right behind the one it waits for).
__device__ __forceinline__ float block_dot(const uint32_t (&pr)[16], const u32x4* x4, float c) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 xx = x4[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) c = dot2_bf16(pr[q * 4 + e], xx[e], c);
  }
  return c;
}

// Gate and up rows . the vectors xv[v] (block sums sv[v]; -128 times the
// block sums of the staged values sv2[v]) of tokens v < nv.
template <int FMT, int NCH, int NG>
__device__ __forceinline__ void row_pair_vecs_dot(const RowRegs<FMT, NCH>& RG,
                                                  const RowRegs<FMT, NCH>& RU, int nch, int lane_g,
                                                  int lpr, const uint32_t* const (&xv)[NG],
                                                  const float* const (&sv)[NG],
                                                  const float* const (&sv2)[NG], int nv,
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
        g[v] = row_vec_dot<FMT, NCH>(RG, nch, lane_g, lpr, xv[v]);
        u[v] = row_vec_dot<FMT, NCH>(RU, nch, lane_g, lpr, xv[v]);
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
        if constexpr (FMT == MOE_W_Q4B32) {
          mg -= 128.f * dg;
          mu -= 128.f * du;
        }
        uint32_t pg[16], pu[16];
        unpack_block<FMT>(wg, bb, pg);
        unpack_block<FMT>(wu, bb, pu);
#pragma unroll
        for (int v = 0; v < NG; ++v) {
          if (v >= nv) continue;
          const u32x4* x4 = reinterpret_cast<const u32x4*>(xv[v] + c * Fmt<FMT>::kCS) + 4 * bb;
          const float sx = sv[v][kBlk * c + bb];
          if constexpr (FMT == MOE_W_Q2B32) {
            const float sx2 = sv2[v][kBlk * c + bb];   // -128 sum x'
            g[v] = fmaf(dg, block_dot(pg, x4, sx2), fmaf(mg, sx, g[v]));
            u[v] = fmaf(du, block_dot(pu, x4, sx2), fmaf(mu, sx, u[v]));
          } else {
            g[v] += dg * block_dot(pg, x4, 0.f) + mg * sx;
            u[v] += du * block_dot(pu, x4, 0.f) + mu * sx;
          }
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

template <int FMT>
__device__ __forceinline__ void unpack_block_f16(u32x4 w, int bb, uint32_t (&pr)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pr[q * 4 + e] = FMT == MOE_W_Q2B32 ? f16_pair_cls<FMT>(w[2 * bb + (q >> 1)], (q & 1) * 4 + e)
                                         : f16_pair_cls<FMT>(w[q], e);
}
__device__ __forceinline__ float block_dot_f16(const uint32_t (&pr)[16], const u32x4* x4) {
  float c = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 xx = x4[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) c = dot2_f16(pr[q * 4 + e], xx[e], c);
  }
  return c;
}

// One row . h of tokens v0 .. v0 + nv - 1, staged by stage_h (token t's
// vector at xd + t * vs, block scales 2^e at bsc + t * ss, and per block
// 2^e * sum h and -1024 * 2^e * sum h' at sd + t * ss and sd2 + t * ss).
// Per block: d * (2^e * sum (1024 + q 4^c) h' - 1024 * 2^e * sum h') +
// m * 2^e * sum h, with h the block-scaled fp16 values and h' = h * 4^-c as
// staged.
template <int FMT, int NCH, int NG>
__device__ __forceinline__ void row_vecs_dot_f16(const RowRegs<FMT, NCH>& R, int nch, int lane_g,
                                                 int lpr, const uint32_t* xd, const float* sd,
                                                 const float* sd2, const float* bsc, int vs,
                                                 int ss, int v0, int nv, float (&o)[NG]) {
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
      const float m = f16_to_f32(uint16_t((R.mn[j] >> dsh) & 0xFFFFu));
      uint32_t pr[16];
      unpack_block_f16<FMT>(w, bb, pr);
#pragma unroll
      for (int v = 0; v < NG; ++v) {
        if (v >= nv) continue;
        const int t = v0 + v, blk = kBlk * c + bb;
        const u32x4* h4 = reinterpret_cast<const u32x4*>(xd + t * vs + c * Fmt<FMT>::kCS) + 4 * bb;
        const float p = fmaf(bsc[t * ss + blk], block_dot_f16(pr, h4), sd2[t * ss + blk]);
        o[v] = fmaf(d, p, fmaf(m, sd[t * ss + blk], o[v]));
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
template <int FMT, bool NT = false>
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
  load_row<FMT, nch_gu<FMT>(), NT>(rg, G.codes + off, G.scale + blk, G.mn + blk, nch, lane_g, kLprGU);
  load_row<FMT, nch_gu<FMT>(), NT>(ru, U.codes + off, U.scale + blk, U.mn + blk, nch, lane_g, kLprGU);
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
                                               const float* xsum, const float* xsum2, int vstride,
                                               int lane_g, uint32_t epoch) {
  constexpr int kLprGU = Lanes<FMT>::kGU;
  const int K = a.H, sstride = K / 32;
  const int nch = chunks_of<FMT>(K) / kLprGU;
  for (int v0 = 0; v0 < n; v0 += NG) {
    const int nv = min(NG, n - v0);
    const uint32_t* xv[NG];
    const float* sv[NG];
    const float* sv2[NG];
#pragma unroll
    for (int v = 0; v < NG; ++v) {
      const int id = v < nv ? (vid ? vid[v0 + v] : t0 + v0 + v) : 0;
      xv[v] = xs + id * vstride;
      sv[v] = xsum + id * sstride;
      sv2[v] = xsum2 + id * sstride;
    }
    float g[NG], u[NG];
    row_pair_vecs_dot<FMT, nch_gu<FMT>(), NG>(rg, ru, nch, lane_g, kLprGU, xv, sv, sv2, nv, g, u);
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

// Every router task zeroes its share of y (they cover y) before it
// publishes its logits: a workgroup adds into y only after it has seen
// every logit.
__device__ __forceinline__ void zero_y_share(const LayerArgs& a, int task, int n_router,
                                             int lane) {
  const int TH = a.T * a.H, per = (TH + n_router - 1) / n_router;
  const int y0 = task * per, y1 = min(y0 + per, TH);
  for (int i = y0 + lane; i < y1; i += 64) st_dev(a.y + i, 0.f);
}

// Router task = (row group rg of 64 / lpr rows, token group).  Issues the
// task's loads: this lane's router chunk and bias.
template <int FMT>
__device__ __forceinline__ void router_load(RouterRegs<FMT>& R, const LayerArgs& a, int task,
                                            int rg, int n_router, int lane) {
  (void)task;
  (void)n_router;
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
          if constexpr (FMT == MOE_W_Q2B32) {
            // pair s of each group is staged times 4^-(s % 3): sums per
            // class (and group parity, for shorter chains)
            float s6[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kG * kS; ++j) {
              const int a6 = 2 * q2_class(j % kS) + (j / kS) % 2;
              s6[a6] = dot2_bf16(pr[j], xv[j], s6[a6]);
            }
            acc[t] = fmaf(16.f, s6[4] + s6[5], fmaf(4.f, s6[2] + s6[3], s6[0] + s6[1]));
          } else {
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kG * kS; ++j) s4[j & 3] = dot2_bf16(pr[j], xv[j], s4[j & 3]);
            acc[t] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
          }
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
__device__ __forceinline__ void topk_threshold_k(const float* lg, int T, int E, int k, Lds& L,
                                                 uint64_t* trc) {
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
  stamp_now(trc, kTrTkSeg);
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
  stamp_now(trc, kTrTkTau);
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
  stamp_now(trc, kTrTkCand);
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
__device__ __forceinline__ void topk_threshold(const float* lg, int T, int E, int k, Lds& L,
                                               uint64_t* trc) {
  constexpr int GS = kThreads / TB, KMAX = kEMax / GS;
  if (KMAX >= 2 && E <= GS * (KMAX / 2))
    topk_threshold_k<TB, (KMAX >= 2 ? KMAX / 2 : 1)>(lg, T, E, k, L, trc);
  else
    topk_threshold_k<TB, KMAX>(lg, T, E, k, L, trc);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// v of the lane CTRL names (a DPP row shift or broadcast), 0 where none or
// outside the rows ROWS.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_shift(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROWS, 0xF, true));
}
// Inclusive sum over the lanes of the wave up to this one: row shifts, then
// the row broadcasts.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  uint32_t x = v;
  x += dpp_shift<0x111, 0xF>(x);   // row_shr:1
  x += dpp_shift<0x112, 0xF>(x);   // row_shr:2
  x += dpp_shift<0x114, 0xF>(x);   // row_shr:4
  x += dpp_shift<0x118, 0xF>(x);   // row_shr:8
  x += dpp_shift<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_shift<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
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
    L.hmask[0] = hit_mask;
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
template <typename OnChoices>
__device__ __forceinline__ void route_token(const LayerArgs& a, float* lg, int E, int k, Lds& L,
                                            uint32_t epoch, bool writer, uint64_t t0,
                                            uint64_t* trc, OnChoices on_choices) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kR = kEMax / kThreads;
  uint64_t w[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r)
    if (tid + r * kThreads < E) w[r] = ld_dev(region_lg(a) + tid + r * kThreads);
  int rounds = 1;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int r = 0; r < kR; ++r) ok = ok && (tid + r * kThreads >= E || tag_ok(w[r], epoch));
    if (ok || !keep_waiting(a, L, t0)) break;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int r = 0; r < kR; ++r)
      if (tid + r * kThreads < E && !tag_ok(w[r], epoch))
        w[r] = ld_dev(region_lg(a) + tid + r * kThreads);
    ++rounds;
  }
  if (trc) {
    stamp_now(trc, kTrLogits);
    stamp(trc, kTrLgPolls, uint64_t(rounds));
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
  stamp_now(trc, kTrLogitsAll);
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
  stamp_now(trc, kTrRtCand);
  __syncthreads();
  stamp_now(trc, kTrRtBar2);
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
    stamp_now(trc, kTrRtRank);
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
  on_choices(my_e);   // lane r < k holds choice r
  const float vmax = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_v), 0));
  const float ex = lane < k ? __expf(my_v - vmax) : 0.f;
  const float g = ex * __frcp_rn(wave_sum_f32(ex));
  stamp_now(trc, kTrRtGate);
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
  stamp_now(trc, kTrRtResolved);
}

// Routing of up to four tokens (E <= 512, k <= kTopkListMax) in three
// barriers: the one-token scheme with two waves per token.  Token t owns
// the 128 threads of waves 2t and 2t + 1; thread j of them holds experts
// 4j .. 4j + 3, and each of the 32 segments of 16 experts (four
// neighbouring threads) publishes the logit bits of its largest key.
// After the first barrier each of the token's waves finds tau -- the
// smallest of those 32 values with fewer than k larger ones, so that at
// least k keys reach it and the k best all do -- and lists its keys that
// reach tau through one LDS add per wave.  After the second barrier the
// token's first wave ranks the candidates (keys are unique), moves choice r
// to lane r, makes the gates and writes the choices.  A token with more
// than 64 candidates (many equal logits) takes the exact per-wave
// selection instead.  L.idx and L.gate receive the choices and gates as
// from topk_threshold and the gate step; writer: also the outputs.
__device__ __forceinline__ void route_few(const LayerArgs& a, const float* lg, int T, int E, int k,
                                          Lds& L, bool writer, uint64_t* trc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = tid >> 7, j = tid & 127;
  const bool on = t < T;
  uint32_t* seg = reinterpret_cast<uint32_t*>(L.idx);   // [t][32], until the choices
  uint64_t key[4];   // 0: no expert
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * j + i;
    key[i] = 0ull;
    if (on && e < E) {
      const uint32_t ob = ordered_bits(lg[t * E + e]);
      key[i] = (uint64_t(ob) << 32) | uint64_t(~uint32_t(e));
      m = max(m, ob);
    }
  }
  m = max(m, dpp_u32<0xB1>(m));   // quad_perm [1,0,3,2]
  m = max(m, dpp_u32<0x4E>(m));   // quad_perm [2,3,0,1]
  if (on && (j & 3) == 0) seg[t * 32 + (j >> 2)] = m;
  if (tid < 4 * 64) L.rkey[tid] = 0ull;   // the candidate lists' empty slots
  __syncthreads();
  stamp_now(trc, kTrTkSeg);
  if (on) {
    const uint32_t my = seg[t * 32 + (lane & 31)];
    const u32x4* half = reinterpret_cast<const u32x4*>(seg + t * 32) + 4 * (lane >> 5);
    int gt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 o = half[q];
#pragma unroll
      for (int c = 0; c < 4; ++c) gt += o[c] > my ? 1 : 0;
    }
    gt += __shfl_xor(gt, 32, 64);
    const uint32_t tau = ~wave_max_u32(gt <= k - 1 ? ~my : 0u);
    uint64_t cm[4];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      cm[r] = __ballot(key[r] != 0ull && uint32_t(key[r] >> 32) >= tau);
      cnt += __popcll(cm[r]);
    }
    if (cnt > 0) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&L.ncand[t], cnt);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = base + lanes_below(cm[r]);
        if (((cm[r] >> lane) & 1ull) && pos < 64) L.rkey[t * 64 + pos] = key[r];
        base += __popcll(cm[r]);
      }
    }
  }
  __syncthreads();
  stamp_now(trc, kTrTkTau);
  if (on && (wave & 1) == 0) {
    const int n = L.ncand[t];
    int my_e = 0;
    float my_v = 0.f;
    if (n <= 64) {
      const uint64_t* list = L.rkey + t * 64;
      const uint64_t ck = list[lane];
      int r = 0;
      for (int j0 = 0; j0 < n; j0 += 8) {   // candidates j0 .. j0 + 7 above ck
        u32x4 q[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) q[h] = reinterpret_cast<const u32x4*>(list + j0)[h];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          r += ((uint64_t(q[h][1]) << 32) | q[h][0]) > ck ? 1 : 0;
          r += ((uint64_t(q[h][3]) << 32) | q[h][2]) > ck ? 1 : 0;
        }
      }
      // choice r moves to lane r (k <= 16 < 63, the lane that takes the rest)
      const int to = 4 * ((lane < n && r < k) ? r : 63);
      const uint32_t hi = uint32_t(__builtin_amdgcn_ds_permute(to, int(uint32_t(ck >> 32))));
      const uint32_t lo = uint32_t(__builtin_amdgcn_ds_permute(to, int(uint32_t(ck))));
      my_e = int(~lo);
      my_v = key_value(hi);
    } else {
      wave_topk<8>(lg + t * E, E, k, lane, &my_e, &my_v);
    }
    // gates: softmax over the k chosen logits (choice 0 is the largest)
    if (lane >= k) {
      my_e = 0;
      my_v = 0.f;
    }
    const float vmax = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_v), 0));
    const float ex = lane < k ? expf(my_v - vmax) : 0.f;
    const float z = wave_sum_f32(ex);
    const float g = ex / z;
    if (lane < k) {
      L.idx[t * k + lane] = my_e;
      L.gate[t * k + lane] = g;
      if (writer) {
        *gmem_w(a.idx + t * k + lane) = my_e;
        *gmem_w(a.gate + t * k + lane) = g;
      }
    }
  }
  __syncthreads();
}

// Resolution of the P = T*k <= 64 pairs of up to four tokens (lane p =
// pair p) by every wave for itself, with no barrier: the waves write the
// same values to the same places of the tables, and the LDS operations of
// one wave complete in order.  Misses keep pair order.  One bucket per hit
// expert, the buckets in the order of their first pairs, each bucket's
// pairs in token order: the tokens that chose an expert gather in
// L.emask[e] by OR (bits that any number of waves may set), a pair opens
// its bucket when its token is the lowest there, and a scan of the opened
// buckets' sizes over the wave places them.  L.emask must be zero on entry.
__device__ __forceinline__ void resolve_few(const LayerArgs& a, Lds& L, int P, bool writer) {
  const int lane = threadIdx.x & 63;
  const int k = a.k;
  const bool valid = lane < P;
  const int e = valid ? L.idx[lane] : 0;
  const int t = valid ? lane / k : 0;
  const int s = valid ? slot_of_choice(a, L, e) : -1;
  const bool hit = s >= 0;
  if (hit) atomicOr(&L.emask[e], 1u << t);
  const uint64_t hm = __ballot(hit), mm = __ballot(valid && !hit);
  wave_lds_sync();
  const uint32_t tm = hit ? (L.emask[e] & 0xFFFFu) : 0u;   // this wave's ORs cover every pair
  const bool first = hit && __builtin_ctz(tm) == t;
  const uint32_t size = first ? uint32_t(__popc(tm)) : 0u;
  const uint32_t x = wave_scan_u32(size) - size;   // the bucket's first place
  const uint64_t fm = __ballot(first);
  const int n_act = __popcll(fm), n_hit = __popcll(hm);
  if (first) {
    const int bi = lanes_below(fm);
    L.act_slot[bi] = s;
    L.act_start[bi] = int(x);
    L.emask[e] = tm | (x << 16);
  }
  if (lane == 0) {
    L.act_start[n_act] = n_hit;
    L.n_act = n_act;
  }
  if (lane < P / k) L.hmask[lane] = (hm >> (lane * k)) & ((1ull << k) - 1ull);
  wave_lds_sync();
  if (hit) {
    const int pos = int(L.emask[e] >> 16) + __popc(tm & ((1u << t) - 1u));
    L.bpair[pos] = lane;
    L.tok[pos] = t;
  }
  if (writer) {
    const int mpos = lanes_below(mm);
    if (valid && a.slot_idx) *gmem_w(a.slot_idx + lane) = s;
    if (valid && !hit) {
      moe_miss m;
      m.expert = e;
      m.token = t;
      m.gate = L.gate[lane];
      store_miss(a.miss + mpos, m);
    }
    if (valid && lane % k == 0) *gmem_w(a.miss_off + t) = mpos;
    if (lane == 0) *gmem_w(a.miss_off + a.T) = __popcll(mm);
  }
  wave_lds_sync();
}

// The same for up to kPMax pairs: lane l holds pairs 4l .. 4l + 3, so that
// pair order is lane order and then i.  Per lane counts of opened buckets,
// misses and bucket sizes are scanned over the wave in one packed word.
// L.emask and L.hmask must be zero on entry.
__device__ __forceinline__ void resolve_wave(const LayerArgs& a, Lds& L, int P, bool writer) {
  constexpr int kPL = kPMax / 64;   // pairs per lane
  const int lane = threadIdx.x & 63;
  const int k = a.k;
  int e[kPL], t[kPL], s[kPL];
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    const int p = kPL * lane + i;
    const bool valid = p < P;
    e[i] = valid ? L.idx[p] : 0;
    t[i] = valid ? p / k : 0;
    s[i] = valid ? slot_of_choice(a, L, e[i]) : -2;   // -2: no pair, -1: a miss
    if (s[i] >= 0) {
      atomicOr(&L.emask[e[i]], 1u << t[i]);
      atomicOr(reinterpret_cast<unsigned long long*>(&L.hmask[t[i]]), 1ull << (p - t[i] * k));
    }
  }
  wave_lds_sync();
  uint32_t tm[kPL], cnt = 0u;   // opened buckets | misses << 10 | hits in opened buckets << 20
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    tm[i] = s[i] >= 0 ? (L.emask[e[i]] & 0xFFFFu) : 0u;   // this wave's ORs cover every pair
    const bool first = s[i] >= 0 && __builtin_ctz(tm[i]) == t[i];
    cnt += first ? 1u + (uint32_t(__popc(tm[i])) << 20) : 0u;
    cnt += s[i] == -1 ? 1u << 10 : 0u;
  }
  const uint32_t incl = wave_scan_u32(cnt);
  const uint32_t all = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
  uint32_t before = incl - cnt;
  const int n_act = int(all & 0x3FFu), n_miss = int((all >> 10) & 0x3FFu);
  const int n_hit = int(all >> 20);
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    if (s[i] >= 0 && __builtin_ctz(tm[i]) == t[i]) {
      const int bi = int(before & 0x3FFu);
      const uint32_t x = before >> 20;
      L.act_slot[bi] = s[i];
      L.act_start[bi] = int(x);
      L.emask[e[i]] = tm[i] | (x << 16);
      before += 1u + (uint32_t(__popc(tm[i])) << 20);
    }
  }
  if (lane == 0) {
    L.act_start[n_act] = n_hit;
    L.n_act = n_act;
  }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    if (s[i] >= 0) {
      const int pos = int(L.emask[e[i]] >> 16) + __popc(tm[i] & ((1u << t[i]) - 1u));
      L.bpair[pos] = kPL * lane + i;
      L.tok[pos] = t[i];
    }
  }
  if (writer) {
    int mpos = int((before >> 10) & 0x3FFu);   // misses before this lane's pairs
#pragma unroll
    for (int i = 0; i < kPL; ++i) {
      const int p = kPL * lane + i;
      if (s[i] == -2) continue;
      if (a.slot_idx) *gmem_w(a.slot_idx + p) = s[i];
      if (p % k == 0) *gmem_w(a.miss_off + t[i]) = mpos;
      if (s[i] == -1) {
        moe_miss m;
        m.expert = e[i];
        m.token = t[i];
        m.gate = L.gate[p];
        store_miss(a.miss + mpos, m);
        ++mpos;
      }
    }
    if (lane == 0) *gmem_w(a.miss_off + a.T) = n_miss;
  }
  wave_lds_sync();
}

// --------------------------------------------------------------- kernel
// TB: the largest token count the instance serves (1, 4 or 16), so per-token
// loops are unrolled no further than needed.
template <int FMT, int TB, bool DET, bool TR>
__global__ __launch_bounds__(kThreads) void moe_layer_kernel(LayerArgs ka) {
  constexpr int kLprGU = Lanes<FMT>::kGU, kRowsGU = Lanes<FMT>::kRowsGU;
  constexpr int kLprD = Lanes<FMT>::kD, kRowsD = Lanes<FMT>::kRowsD;
  // One token: routed experts' rows load with the non-temporal hint (read
  // once per call; c2 18.6 -> 18.2 us).  Several tokens: plain loads (the
  // hint measured 5 % slower on c3).
  constexpr bool kRoutedNT = TB == 1;
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
  // Phase stamps only in the traced instance: with tracing off the kernel
  // carries none of their code (a few stamps measured 0.3-0.8 us per call
  // even when not taken).
  uint64_t* const trc = TR ? ka.trace : nullptr;
  const int T = ka.T, k = ka.k, P = T * k, E = ka.E;
  const int K = ka.H;
  const int vstride = FMT == MOE_W_F32 ? K : (K / Fmt<FMT>::kWPC) * Fmt<FMT>::kCS;
  // LDS: tokens | block sums of the values | of the staged values | logits
  uint32_t* xs = smem;
  float* xsum = reinterpret_cast<float*>(xs + T * vstride);
  float* xsum2 = xsum + T * (K / 32);
  float* lg = xsum2 + T * (K / 32);

  // ---- A: loads first (call counter and error word, slot table, first task's rows)
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();   // start of this workgroup's waits
  if (trc) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    stamp(trc, kTrStart, t0);
    stamp(trc, kTrXcd, xcc & 0xFu);
  }
  // every wave reads the header (its router task zeroes y only on a sound workspace)
  const uint64_t hdr = lane == 0 ? ld_dev(reinterpret_cast<const uint64_t*>(ka.region)) : 0ull;
  int so[kEMax / kThreads];
#pragma unroll
  for (int r = 0; r < kEMax / kThreads; ++r) {
    const int e = tid + r * kThreads;
    so[r] = (ka.slot_of && e < E) ? ka.slot_of[e] : -1;
  }
  // router tasks: row groups x token groups of kTG (a row group's token
  // groups share a workgroup when there are at most G row groups)
  constexpr int kTG = TB == 1 ? 1 : TB == 4 ? 2 : 4;
  // tokens per unpacked block (shared-expert gate/up, down) and the same
  // for routed gate/up: two for verify batches (most of their buckets hold
  // one token, and the smaller code measured faster: c3 38.4 -> 37.7 us),
  // four for larger ones
  constexpr int kNG = TB == 1 ? 1 : TB <= 4 ? 2 : 4;
  constexpr int kNGC = kNG;
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
  // Several tokens: the second gate/up task's rows, issued during routing
  // (an empty type for one token, so that its instance carries none of it).
  struct NoRegs {};
  using EarlyRegs = std::conditional_t<(TB > 1), RowRegs<FMT, nch_gu<FMT>()>, NoRegs>;
  EarlyRegs eg, eu;
  if (task0 < n_router)
    router_load<FMT>(rr, ka, task0, task0 % n_rg, n_router, lane);
  else if (task0 < n_a)
    gateup_load<FMT>(rg, ru, ka, ka.sg, ka.su, 0,
                     ((task0 - n_router) % n_srb) * kRowsGU + lane / kLprGU, lane_gu);
  // The first router task zeroes its share of y while the tokens load: the
  // stores land before the task publishes its logits, and the wait for the
  // header lets the row and token loads stay in flight.
  stage_tokens<FMT>(ka.x, T, K, xs, xsum, xsum2, vstride, [&]() {
    if (task0 < n_router && !DET && __builtin_amdgcn_readfirstlane(uint32_t(hdr >> 32)) == 0u)
      zero_y_share(ka, task0, n_router, lane);
  });
  if (tid == 0) {
    L.calls = uint32_t(hdr);
    L.failed = uint32_t(hdr >> 32) != 0u ? 2 : 0;   // a failed call left the workspace poisoned
  }
  for (int e = tid; e < kEMax; e += kThreads) L.emask[e] = 0u;
  if (tid < kTMax) {
    L.ncand[tid] = 0;
    L.hmask[tid] = 0ull;
  }
  if (tid <= kTMax) L.dhist[tid] = 0;
  if (tid == 0) {
    L.dzero = 0;
    L.dalign[0] = 0;
    L.dalign[1] = 0;
    L.t_gu = 0ull;
    L.t_a = 0ull;
  }
#pragma unroll
  for (int r = 0; r < kEMax / kThreads; ++r)
    if (tid + r * kThreads < E) L.slot_of[tid + r * kThreads] = so[r];
  __syncthreads();
  if (L.failed == 2) return;   // every thread: nothing is written
  const LayerArgs& a = sa;
  stamp_now(trc, kTrStaged);
  const uint32_t epoch = L.calls + 1u;   // this call's number
  if (a.debug_hold && b == 0 && tid == 0) {
    // test hook: wait for a word nothing writes until the budget is spent
    const uint32_t* hold = reinterpret_cast<const uint32_t*>(a.region + kRegionHold);
    while (ld_dev(hold) != epoch && keep_waiting(a, L, t0)) __builtin_amdgcn_s_sleep(1);
  }
  for (int task = task0; task < n_a; task += kWaves * G) {
    if (task < n_router) {
      if (task != task0) {
        router_load<FMT>(rr, a, task, task % n_rg, n_router, lane);
        if (!DET) zero_y_share(a, task, n_router, lane);   // after the workspace check, before the logits
      }
      router_compute<FMT, kTG>(rr, a, task % n_rg, (task / n_rg) * kTG, xs, vstride, lane, epoch);
    } else {
      const int s = task - n_router, t0 = (s / n_srb) * kTG;
      const int i = (s % n_srb) * kRowsGU + lane / kLprGU;
      if (task != task0) gateup_load<FMT>(rg, ru, a, a.sg, a.su, 0, i, lane_gu);
      gateup_compute<FMT, kNG>(rg, ru, a, i, min(kTG, T - t0), nullptr, nullptr, t0, region_h_sh(a), xs,
                               xsum, xsum2, vstride, lane_gu, epoch);
    }
  }

  stamp_now(trc, kTrTasksA);
  if (trc && lane == 0)
    atomicMax(&L.t_a, static_cast<unsigned long long>(__builtin_amdgcn_s_memrealtime()));
  // this workgroup has read the counter (workgroup 0 checks before it
  // advances the counter)
  if (tid == 0) st_dev(region_arrive(a) + b, tag_word(0.f, epoch));

  // ---- B: every logit of this call, then routing
  if constexpr (TB == 1) {
    // The wave's gate/up task needs only its expert's slot, known once the
    // choices are: its rows load from there, before the gates and the
    // resolution (which build the same bucket list: hits in choice order).
    const int tpe1 = a.I / kRowsGU, c1 = b + wave * G;
    route_token(a, lg, E, k, L, epoch, b == 0, t0, trc, [&](int my_e) {
      const int s = lane < k ? slot_of_choice(a, L, my_e) : -1;
      const uint64_t hm = __ballot(s >= 0);
      const int u = c1 / tpe1;
      if (u < __popcll(hm)) {
        const int hpos = __builtin_amdgcn_mbcnt_hi(uint32_t(hm >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(uint32_t(hm), 0u));
        const uint64_t at = __ballot(s >= 0 && hpos == u);
        const int slot = __builtin_amdgcn_readlane(s, __builtin_ctzll(at));
        gateup_load<FMT, kRoutedNT>(rg, ru, a, a.g, a.u, slot, (c1 % tpe1) * kRowsGU + lane / kLprGU,
                                    lane_gu);
      }
    });
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
        if (ok || !keep_waiting(a, L, t0)) break;
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
  stamp_now(trc, kTrLogits);
  __syncthreads();
  stamp_now(trc, kTrLogitsAll);
  if (TB == 4 && E <= 512 && k <= kTopkListMax) {
    route_few(a, lg, T, E, k, L, b == 0, trc);
    stamp_now(trc, kTrRtGate);
    resolve_few(a, L, P, b == 0 && wave == 0);
  } else {
  const bool thresh = k <= kTopkListMax;
  if (thresh) topk_threshold<TB>(lg, T, E, k, L, trc);
  stamp_now(trc, kTrRtCand);
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
  stamp_now(trc, kTrRtRank);
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
  stamp_now(trc, kTrRtGate);
  resolve_wave(a, L, P, b == 0 && wave == 0);
  }
  stamp_now(trc, kTrRtResolved);
  // This wave's first two gate/up tasks load now, ahead of the work split
  // and its barrier: the wave's own tables are complete.
  const int tpe1 = a.I / kRowsGU, nt1 = L.n_act * tpe1, c1 = b + wave * G;
  if (c1 < nt1)
    gateup_load<FMT, kRoutedNT>(rg, ru, a, a.g, a.u, L.act_slot[c1 / tpe1],
                                (c1 % tpe1) * kRowsGU + lane / kLprGU, lane_gu);
  const int c2 = c1 + kWaves * G;
  if (c2 < nt1)
    gateup_load<FMT, kRoutedNT>(eg, eu, a, a.g, a.u, L.act_slot[c2 / tpe1],
                                (c2 % tpe1) * kRowsGU + lane / kLprGU, lane_gu);
  }
  stamp_now(trc, kTrRouted);
  if (trc) stamp(trc, kTrTasksAAll, L.t_a);
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
  // The shared expert's down work is split into token groups of at most
  // kShG tokens, each a bucket of its own: one unit of all 16 tokens of a
  // batch would cost more than a workgroup's whole share of the phase.
  constexpr int kShG = 4;
  const int n_shg = a.has_sh ? (TB > kShG ? (T + kShG - 1) / kShG : 1) : 0;
  const int n_units = (n_act + n_shg) * nrb;
  const int tpe = a.I / kRowsGU;
  const int n_tasks = n_act * tpe;
  const int lane_gd = lane % kLprD;
  // Who does what.  Gate/up tasks (bucket, row block) are dealt to the waves
  // in turn, consecutive tasks to consecutive workgroups, so each bucket's
  // tasks spread over the whole grid (for several tokens this measured
  // faster than contiguous ranges of equal cost: c3 39.4 -> 38.7 us, c4
  // 76.1 -> 75.3 us).  Down units (bucket, row block): one token -- every
  // bucket costs the same -- dealt to the workgroups in turn; several
  // tokens, by cost (a fixed part plus the bucket's tokens), in the
  // bucket-aligned split below, else a contiguous range of equal cost per
  // workgroup, whose bounds thread u finds inside bucket u's span of
  // cumulative cost.
  const int c_first = b + wave * G, c_end = n_tasks, c_step = kWaves * G;
  int d_first = b, d_end = n_units, d_step = G;
  if constexpr (TB > 1) {
    constexpr int kCostD = 1;
    const int n_db = n_act + n_shg;
    auto tokens_of = [&](int u) {   // tokens of down bucket u (the shared groups last)
      return u < n_act ? L.act_start[u + 1] - L.act_start[u]
                       : (TB > kShG ? min(kShG, T - (u - n_act) * kShG) : T);
    };
    // (costs stay below 2^20; a bound's exact quotient a * tot / W comes from
    // double arithmetic: the product is exact and no quotient lies within a
    // rounding error of an integer it does not equal)
    const int totD = nrb * (kCostD * n_db + L.act_start[n_act] + (a.has_sh ? T : 0));
    auto bound = [](int i, int tot, int parts) {
      return int(floor(double(i) * double(tot) / double(parts)));
    };
    // One thread per range bound (2 unit bounds): a binary search for the
    // bucket whose span of cumulative cost holds the bound's target, then
    // the first unit of that bucket at or past it.
    if (tid < 2) {
      const int n = n_db;
      const int rows = nrb, fixed = kCostD;
      const int bt = bound(b + tid, totD, G);
      auto tokens_before = [&](int u) {   // tokens of buckets < u (the shared groups last)
        return u <= n_act ? L.act_start[u] : L.act_start[n_act] + min(T, (u - n_act) * kShG);
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
        v = n_units;
      } else {
        const int cost =
            fixed + (lo < n_act ? L.act_start[lo + 1] - L.act_start[lo] : min(kShG, T - (lo - n_act) * kShG));
        v = lo * rows + (bt - cum(lo) + cost - 1) / cost;
      }
      L.dstart[tid] = v;
    }
    // Down units, bucket-aligned, by a min-max split: the smallest cost
    // bound C such that every bucket's units fit on its own run of
    // workgroups, each with at most C of cost, where bucket u (cost c per
    // unit) takes w(u) = ceil(nrb / min(nrb, floor(C / c))) workgroups and
    // its units spread evenly over them -- so a workgroup stages the
    // activations of one bucket only (a second staging costs a poll round
    // trip and a conversion, more than a unit).  The runs follow the bucket
    // order; workgroups past the last run take no down unit.  With more
    // buckets than workgroups no bound fits, and every workgroup keeps the
    // contiguous split above.  Wave 1 alone: a histogram of the bucket sizes
    // (one wave's LDS operations complete in order), then each lane tries a
    // bound, 64 consecutive bounds per round from a lower limit; at C =
    // nrb * (largest cost) every bucket takes one workgroup, so the search
    // ends there at the latest.
    if (wave == 1) {
      for (int u = lane; u < n_db; u += 64) atomicAdd(&L.dhist[tokens_of(u)], 1);
      int nmax = TB;
      while (nmax > 1 && L.dhist[nmax] == 0) --nmax;
      // floor(p / q) for small positive integers: the exact quotient's
      // fraction lies at least 0.5 / q away from an integer, far beyond the
      // reciprocal's rounding error
      auto fdiv = [](int p, int q) {
        return int((float(p) + 0.5f) * __builtin_amdgcn_rcpf(float(q)));
      };
      // workgroups a bucket of cost c takes under bound C (0 if a unit does
      // not fit)
      auto wgs = [&](int C, int c) {
        const int m = min(nrb, fdiv(C, c));
        return m == 0 ? 0 : fdiv(nrb - 1, m) + 1;
      };
      int cs = -1;
      if (n_db <= G) {
        for (int c0 = max(kCostD + nmax, (totD + G - 1) / G);; c0 += 64) {
          const int C = c0 + lane;
          int need = 0;
          for (int n = 1; n <= nmax; ++n) {
            const int h = L.dhist[n];
            if (h == 0) continue;
            const int w = wgs(C, kCostD + n);
            need += w == 0 ? G + 1 : h * w;
          }
          const uint64_t ok = __ballot(need <= G);
          if (ok != 0ull) {
            cs = c0 + __builtin_ctzll(ok);
            break;
          }
        }
      }
      if (cs < 0) {
        if (lane == 0) L.dzero = 1;
      } else {
        int before = 0;   // workgroups taken by the buckets of earlier groups of 64
        for (int u0 = 0; u0 < n_db; u0 += 64) {
          const int u = u0 + lane;
          const int w = u < n_db ? wgs(cs, kCostD + tokens_of(u)) : 0;
          int incl = w;   // inclusive prefix sum over the wave
          for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
          }
          const int s0 = before + incl - w;
          if (b >= s0 && b < s0 + w) {
            const int j = b - s0;
            L.dalign[0] = u * nrb + j * nrb / w;
            L.dalign[1] = u * nrb + (j + 1) * nrb / w;
          }
          before += __shfl(incl, 63);
        }
      }
    }
    __syncthreads();
    const bool aligned = L.dzero == 0;
    d_first = aligned ? L.dalign[0] : L.dstart[0];
    d_end = aligned ? L.dalign[1] : L.dstart[1];
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
    if (!kRoutedNT || shared)
      load_row<FMT, kNChD>(rd, D.codes + slot * a.mat_bytes + rr_ * row_bytes_d, D.scale + blk,
                           D.mn + blk, nch_d, lane_gd, kLprD);
    else
      load_row<FMT, kNChD, true>(rd, D.codes + slot * a.mat_bytes + rr_ * row_bytes_d, D.scale + blk,
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
      gateup_load<FMT, kRoutedNT>(g, u, a, a.g, a.u, L.act_slot[t / tpe],
                                  (t % tpe) * kRowsGU + lane / kLprGU, lane_gu);
    };
    int task = c_first;
    // (the first task's rows, and with several tokens the second's, were
    // issued during routing)
    RowRegs<FMT, nch_gu<FMT>()> ng, nu;
    if constexpr (TB > 1) {
      ng = eg;
      nu = eu;
    }
    // one token: the first down unit's lines head for the L2 meanwhile
    if constexpr (TB == 1) pf = prefetch_down(d_first < d_end ? d_first : -1);
    auto compute_task = [&](int t, const RowRegs<FMT, nch_gu<FMT>()>& g,
                            const RowRegs<FMT, nch_gu<FMT>()>& up) {
      const int u = t / tpe;
      const int i = (t % tpe) * kRowsGU + lane / kLprGU;
      const int st = L.act_start[u];
      const int n = L.act_start[u + 1] - st;
      gateup_compute<FMT, kNGC>(g, up, a, i, n, L.tok + st, L.bpair + st, 0, region_h(a), xs,
                                xsum, xsum2, vstride, lane_gu, epoch);
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

  if (trc) {   // this wave's gate/up end
    const uint64_t t = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) atomicMax(&L.t_gu, static_cast<unsigned long long>(t));
    if (wave == 0) stamp(trc, kTrGateUp0, t);
  }
  // ---- D: down units (expert or shared, block of rows), y += gate * D h
  stamp_now(trc, kTrDStart);
  {
    uint32_t* xd = smem;                                    // reuses the token area
    float* sd = reinterpret_cast<float*>(xd + kTMax * vs_d);
    float* sd2 = sd + kTMax * ss_d;
    float* bsc = sd2 + kTMax * ss_d;
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
      // (a shared group's first token, else the bucket's first position)
      const int st = shared ? (TB > kShG ? (u - n_act) * kShG : 0) : L.act_start[u];
      const int n = shared ? (TB > kShG ? min(kShG, T - st) : T) : L.act_start[u + 1] - st;
      const int r = rb * kRowsD + wave * (64 / kLprD) + lane / kLprD;
      if (u != staged) {
        __syncthreads();   // gate/up tasks and the previous unit are done with the LDS
        if (staged < 0) stamp_now(trc, kTrDBar1);
        if (tid < n)
          srcs[tid] = shared ? region_h_sh(a) + int64_t(st + tid) * Kd
                             : region_h(a) + int64_t(L.bpair[st + tid]) * Kd;
        __syncthreads();
        if (staged < 0) stamp_now(trc, kTrDBar2);
        stage_h<FMT>(srcs, n, Kd, xd, sd, sd2, bsc, vs_d, epoch, a, L, t0,
                     staged < 0 ? trc : nullptr);
        __syncthreads();
        if (staged < 0 && trc) {
          stamp(trc, kTrHBar, __builtin_amdgcn_s_memrealtime());
          stamp(trc, kTrStagedH, __builtin_amdgcn_s_memrealtime());
          stamp(trc, kTrGateUpAll, L.t_gu);
        }
        staged = u;
      }
      for (int v0 = 0; v0 < n; v0 += kNG) {
        const int nv = min(kNG, n - v0);
        float o[kNG];
        if constexpr (FMT != MOE_W_F32) {
          row_vecs_dot_f16<FMT, kNChD, kNG>(rd, nch_d, lane_gd, kLprD, xd, sd, sd2, bsc, vs_d,
                                            ss_d, v0, nv, o);
        } else {
#pragma unroll
          for (int v = 0; v < kNG; ++v)
            o[v] = v < nv ? row_vec_dot<FMT, kNChD>(rd, nch_d, lane_gd, kLprD, xd + (v0 + v) * vs_d)
                          : 0.f;
        }
#pragma unroll
        for (int v = 0; v < kNG; ++v) {
          if (v >= nv) continue;
          const float os = group_sum<kLprD>(o[v]);
          if (r < a.H && lane_gd == 0) {
            const int t = shared ? st + v0 + v : L.tok[st + v0 + v];
            const int pr = shared ? 0 : L.bpair[st + v0 + v];
            const float g = shared ? 1.f : L.gate[pr];
            if constexpr (DET) {
              const int row = shared ? layer_h_rows(a.k) - kTMax + t : pr;
              st_dev(region_part(a) + int64_t(row) * a.H + r, tag_word(g * os, epoch));
            } else {
              fadd_dev(a.y + int64_t(t) * a.H + r, g * os);
            }
          }
        }
      }
      rd = nd;
    }
  }
  stamp_now(trc, kTrDown);
  if constexpr (DET) {
    // Fixed-order sums: this workgroup's share of y, each element by one
    // thread: the hit choices j = 0 .. k-1 in order, then the shared expert
    // (index k), their rows read once every unit has published them (16
    // words in flight per thread; words not yet of this call are read again).
    const int TH = T * a.H, per = (TH + G - 1) / G;
    const int i0 = b * per, i1 = min(i0 + per, TH);
    const uint64_t* part = region_part(a);
    const int sh_row = layer_h_rows(k) - kTMax;
    for (int i = i0 + tid; i < i1; i += kThreads) {
      const int t = i / a.H, r = i - t * a.H;
      const uint64_t m = L.hmask[t];
      float acc = 0.f;
      for (int j0 = 0; j0 <= k; j0 += 16) {
        uint64_t w[16];
        const uint64_t* src[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int j = j0 + q;
          const bool want = j < k ? ((m >> j) & 1ull) != 0ull : (j == k && a.has_sh != 0);
          src[q] = want ? part + int64_t(j < k ? t * k + j : sh_row + t) * a.H + r : nullptr;
          if (src[q]) w[q] = ld_dev(src[q]);
        }
        auto all_here = [&]() {
          bool ok = true;
#pragma unroll
          for (int q = 0; q < 16; ++q) ok = ok && (!src[q] || tag_ok(w[q], epoch));
          return ok;
        };
        while (!all_here() && keep_waiting(a, L, t0)) {
          __builtin_amdgcn_s_sleep(1);
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (src[q] && !tag_ok(w[q], epoch)) w[q] = ld_dev(src[q]);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (src[q]) acc += tag_val(w[q]);
      }
      *gmem_w(a.y + i) = acc;
    }
  }
  // Workgroup 0 advances the call counter once every workgroup has read it
  // (a failed call leaves it: the workspace is poisoned anyway).
  if (b == 0) {
    if (tid < G)
      while (!tag_ok(arr, epoch) && keep_waiting(a, L, t0)) {
        __builtin_amdgcn_s_sleep(1);
        arr = ld_dev(region_arrive(a) + tid);
      }
    __syncthreads();
    if (tid == 0 && !L.failed) st_dev(region_calls(a), epoch);
  }
  stamp_now(trc, kTrEnd);
  asm volatile("" ::"v"(pf));   // the prefetch's value counts as used
}

struct Occ {
  size_t lds = 0;
  int device = -1;
  int grid = 0;
};

template <int FMT, int TB, bool DET, bool TR>
hipError_t launch_det(const LayerArgs& a, size_t lds, hipStream_t st, int* grid_out) {
  static thread_local Occ c;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (c.lds != lds || c.device != dev) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_layer_kernel<FMT, TB, DET, TR>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_layer_kernel<FMT, TB, DET, TR>, kThreads,
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
  hipLaunchKernelGGL((moe_layer_kernel<FMT, TB, DET, TR>), dim3(c.grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

// The fixed-order sums and the phase stamps are separate instances: the
// plain instance carries none of their code.  (The fixed-order instance is
// not traced.)
template <int FMT, int TB>
hipError_t launch_fmt(const LayerArgs& a, size_t lds, hipStream_t st, int* grid_out) {
  if (a.det) return launch_det<FMT, TB, true, false>(a, lds, st, grid_out);
  return a.trace ? launch_det<FMT, TB, false, true>(a, lds, st, grid_out)
                 : launch_det<FMT, TB, false, false>(a, lds, st, grid_out);
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
  // A-C: tokens, two sets of block sums, logits
  const size_t a = size_t(T) * (vec_bytes(fmt, H) + 2 * (H / 32) * 4) + size_t(T) * E * 4;
  // D: a vector per token, two sets of block sums, block scales (16 tokens)
  const size_t d = size_t(kTMax) * (vec_bytes(fmt, I) + 3 * (I / 32) * 4);
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

// ---------------------------------------------------------------- no-alloc
// Hand-off region of moe_layer_noalloc: one static array, which every GPU
// the library runs on holds at its own address until the process ends.  In
// host code the array's name is not a device address: the address comes
// from hipGetSymbolAddress, taken once per device with that device current,
// and only that address is used (kernel arguments, the clear below).
static __device__ __align__(256) uint8_t scratch[MOE_LAYER_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices] = {};

__global__ __launch_bounds__(256) void clear_words_kernel(u32x4* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t clear_region(uint8_t* p, hipStream_t st) {
  // a fill kernel rather than a memset node, so that a captured first call
  // records a kernel
  hipLaunchKernelGGL(clear_words_kernel, dim3(256), dim3(256), 0, st, reinterpret_cast<u32x4*>(p),
                     int64_t(MOE_LAYER_SCRATCH_BYTES / 16));
  return hipGetLastError();
}

// The current device's region: its address on first use (then cleared on
// st, ahead of the call that follows on st).
hipError_t scratch_of_device(hipStream_t st, uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    e = clear_region(static_cast<uint8_t*>(p), st);
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_layer_noalloc(LayerArgs a, int fmt, hipStream_t st) {
  uint8_t* region = nullptr;
  const hipError_t e = scratch_of_device(st, &region);
  if (e != hipSuccess) return e;
  a.region = region;
  return launch_layer_fused(a, fmt, st, nullptr);
}

hipError_t layer_scratch_address(uint8_t** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t layer_scratch_clear(hipStream_t st) {
  uint8_t* p = nullptr;
  const hipError_t e = layer_scratch_address(&p);
  if (e != hipSuccess || !p) return e;
  return clear_region(p, st);
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
