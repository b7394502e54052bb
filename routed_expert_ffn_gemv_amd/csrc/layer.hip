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
// bandwidth, sets the time, so it runs in one launch and every step issues
// all of its loads before it consumes any:
//  A  stage the tokens in LDS; router rows and shared-expert gate/up rows
//     (independent of the routing); zero y; grid barrier (each workgroup
//     stores its arrival, every workgroup polls all arrivals);
//  B  every workgroup reads all logits and takes the routing decisions
//     itself (top-k, gates, slots, miss list, buckets) -- the same
//     deterministic result everywhere, so nothing has to be broadcast;
//     workgroup 0 writes the routing outputs;
//  C  routed gate/up + SwiGLU, a few rows of one expert per wave task; each
//     task raises its own flag when its rows of h are out;
//  D  down projection units (expert, block of rows): the unit loads its
//     weight rows, then waits for its expert's task flags, stages h, and adds
//     gate * output into y with device-scope float atomics (the shared
//     expert adds with weight 1).  The summation order over experts is not
//     fixed, so y may differ from run to run in the last bits.
// The grid never exceeds the number of workgroups the device holds at once,
// so every workgroup a wait depends on is running.  Data one workgroup hands
// to another goes through device-scope (sc1) loads and stores, which bypass
// the per-XCD L2 caches; a wave waits for its own stores (s_waitcnt) before
// the flag that publishes them, so no cache-wide write-back or invalidate
// is needed, and flags carry the call number so none is ever reset.
#include "gemv_core.h"
#include "kernels.h"
#include "layer.h"

namespace moe {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTMax = MOE_LAYER_MAX_T;
constexpr int kPMax = 256;
constexpr int kNChMax = 4;                      // 16-byte chunks per lane and weight row

// Lanes per weight row: a lane holds at most 2 (Q2) or 4 (Q4) chunks of a
// 2048-wide gate/up row and 3 of a 768-wide down row.
template <int FMT>
struct Lanes {
  static constexpr int kGU = FMT == MOE_W_F32 ? 8 : 16;     // gate/up
  static constexpr int kD = FMT == MOE_W_Q4B32 ? 8 : 4;     // down
  static constexpr int kRowsGU = 64 / kGU;                  // rows per wave task
  static constexpr int kRowsD = kWaves * (64 / kD);         // rows per down unit
};

template <typename V>
__device__ __forceinline__ V ld_dev(const V* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void st_dev(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fadd_dev(float* p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// 64-bit wave maximum with DPP row operations; every lane gets the result.
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
#define MOE_DPP_STEP(ctrl, rmask)                                                              \
  {                                                                                            \
    const uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);                                   \
    const uint32_t olo = __builtin_amdgcn_update_dpp(lo, lo, ctrl, rmask, 0xF, false);         \
    const uint32_t ohi = __builtin_amdgcn_update_dpp(hi, hi, ctrl, rmask, 0xF, false);         \
    const uint64_t o = (uint64_t(ohi) << 32) | olo;                                            \
    v = o > v ? o : v;                                                                         \
  }
  MOE_DPP_STEP(0xB1, 0xF)    // quad_perm [1,0,3,2]
  MOE_DPP_STEP(0x4E, 0xF)    // quad_perm [2,3,0,1]
  MOE_DPP_STEP(0x141, 0xF)   // row_half_mirror
  MOE_DPP_STEP(0x140, 0xF)   // row_mirror
  MOE_DPP_STEP(0x142, 0xA)   // row_bcast:15
  MOE_DPP_STEP(0x143, 0xC)   // row_bcast:31
#undef MOE_DPP_STEP
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(v >> 32), 63);
  return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b) {
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// Top-k of one token's logits (LDS, E <= 64 * KPL) by one wave.  Keys are
// (order-preserving logit bits << 32) | ~expert, unique, so the largest key
// is the largest logit and, among equal logits, the lowest expert id.  Each
// lane sorts its KPL keys once; each round takes the wave maximum of the
// lane heads and the owning lane drops its head.  Lane j < k returns the
// j-th choice.
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
    const uint64_t m = wave_max_u64_dpp(key[0]);
    const int e = int(~uint32_t(m));
    const uint32_t ob = uint32_t(m >> 32);
    if (lane == j) {
      my_e = e;
      my_v = __uint_as_float((ob & 0x80000000u) ? (ob & 0x7FFFFFFFu) : ~ob);
    }
    if (lane == (e & 63)) {
#pragma unroll
      for (int i = 0; i < KPL - 1; ++i) key[i] = key[i + 1];
      key[KPL - 1] = 0ull;
    }
  }
  *e_out = my_e;
  *v_out = my_v;
}

struct Lds {
  int idx[kPMax];
  float gate[kPMax];
  int slot[kPMax];
  int sorted[kPMax];
  int bpair[kPMax];      // hit pairs sorted by (slot, t, j)
  int tok[kPMax];        // their tokens
  int act_slot[kPMax];   // distinct hit slots, ascending
  int act_start[kPMax + 1];
  int tmp[32];
  int n_act;
  uint32_t flag0;
};

// --------------------------------------------------------------- staging
// Tokens into the expert format's LDS layout, with 32-byte loads per
// thread (16 columns of one token) issued before any is used.  psum holds
// each 16-column group's sum; block sums add two groups in a fixed order.
template <int FMT>
__device__ __forceinline__ void stage_tokens(const uint16_t* __restrict__ x, int T, int H, uint32_t* xs,
                             float* xsum, float* psum, int vstride) {
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
  __syncthreads();
  const int nb = H / 32;
  for (int i = threadIdx.x; i < T * nb; i += kThreads) {
    const int t = i / nb, b = i % nb;
    xsum[t * nb + b] = psum[t * per_tok + 2 * b] + psum[t * per_tok + 2 * b + 1];
  }
}

// fp32 vectors written by other workgroups (h) into hi/lo bf16 vectors of
// the pair layout (F32 format: plain fp32), 16 columns per item, loads first.
template <int FMT>
__device__ __forceinline__ void stage_h(const float* const* srcs, int n, int K, uint32_t* xd, float* sd,
                        float* psum, int vs) {
  const int per_vec = K / 16;
  const int n_items = n * per_vec;
  constexpr int kVPP = FMT == MOE_W_F32 ? 1 : 2;
  for (int base = 0; base < n_items; base += kThreads) {
    const int it = base + threadIdx.x;
    float v[16];
    if (it < n_items) {
      const float* src = srcs[it / per_vec] + (it % per_vec) * 16;
#pragma unroll
      for (int c = 0; c < 16; ++c) v[c] = ld_dev(src + c);
    }
    if (it < n_items) {
      const int p = it / per_vec, g16 = it % per_vec;
      if constexpr (FMT == MOE_W_F32) {
        float* xf = reinterpret_cast<float*>(xd) + p * vs + g16 * 16;
#pragma unroll
        for (int c = 0; c < 16; ++c) xf[c] = v[c];
      } else {
        uint32_t hi[16], lo[16];
        float shi = 0.f, slo = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          hi[c] = f32_to_bf16_bits(v[c]);
          const float hf = bf16_to_f32(hi[c]);
          lo[c] = f32_to_bf16_bits(v[c] - hf);
          shi += hf;
          slo += bf16_to_f32(lo[c]);
        }
        psum[(kVPP * p) * per_vec + g16] = shi;
        psum[(kVPP * p + 1) * per_vec + g16] = slo;
        uint32_t* dh = xd + (kVPP * p) * vs;
        uint32_t* dl = xd + (kVPP * p + 1) * vs;
        if constexpr (FMT == MOE_W_Q2B32) {
          const int off = (g16 >> 2) * Fmt<FMT>::kCS + (g16 & 3) * 8;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            dh[off + s] = hi[s] | (hi[s + 8] << 16);
            dl[off + s] = lo[s] | (lo[s + 8] << 16);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int off = (g16 >> 1) * Fmt<FMT>::kCS + ((g16 & 1) * 2 + q) * 4;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              dh[off + s] = hi[8 * q + s] | (hi[8 * q + s + 4] << 16);
              dl[off + s] = lo[8 * q + s] | (lo[8 * q + s + 4] << 16);
            }
          }
        }
      }
    }
  }
  __syncthreads();
  if (FMT != MOE_W_F32) {
    const int nb = K / 32;
    for (int i = threadIdx.x; i < kVPP * n * nb; i += kThreads) {
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
      R.w[j] = *reinterpret_cast<const u32x4*>(codes + 16 * c);
      if constexpr (FMT == MOE_W_Q2B32) {
        R.sc[j] = *reinterpret_cast<const uint32_t*>(sc + 2 * c);
        R.mn[j] = *reinterpret_cast<const uint32_t*>(mn + 2 * c);
      } else if constexpr (FMT == MOE_W_Q4B32) {
        R.sc[j] = sc[c];
        R.mn[j] = mn[c];
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

template <int FMT>
__host__ __device__ __forceinline__ int chunks_of(int K) {
  return FMT == MOE_W_F32 ? K / 4 : K / Fmt<FMT>::kWPC;
}

// gate/up + SwiGLU for one row per lane group (64 / LPR rows per wave) of
// one expert, for its n tokens; h[t] goes to out[ids(t)][i] (ids = pair ids,
// or the tokens themselves when ids is null).
template <int FMT>
__device__ __forceinline__ void gateup_task(const LayerArgs& a, const MatView& G, const MatView& U,
                                            int slot, int i, int n, const int* vid,
                                            const int* ids, float* out, const uint32_t* xs,
                                            const float* xsum, int vstride, int lane_g) {
  constexpr int kLprGU = Lanes<FMT>::kGU;
  const int K = a.H, sstride = K / 32;
  const int nch = chunks_of<FMT>(K) / kLprGU;
  const int64_t row_bytes = int64_t(K) * fmt_bits(FMT) / 8;
  const int64_t blk = int64_t(slot) * G.mat_blocks + int64_t(i) * sstride;
  RowRegs<FMT, kNChMax> rg, ru;
  load_row<FMT, kNChMax>(rg, G.codes + slot * G.mat_bytes + i * row_bytes, G.scale + blk,
                         G.mn + blk, nch, lane_g, kLprGU);
  load_row<FMT, kNChMax>(ru, U.codes + slot * U.mat_bytes + i * row_bytes, U.scale + blk,
                         U.mn + blk, nch, lane_g, kLprGU);
  for (int v = 0; v < n; ++v) {
    const int id = vid ? vid[v] : v;
    float g, u;
    row_pair_vec_dot<FMT, kNChMax>(rg, ru, nch, lane_g, kLprGU, xs + id * vstride,
                                   xsum + id * sstride, g, u);
    g = group_sum<kLprGU>(g);
    u = group_sum<kLprGU>(u);
    if (lane_g == 0) st_dev(out + int64_t(ids ? ids[v] : v) * a.I + i, silu_f32(g) * u);
  }
}

// One router wave task: 64 / LPR rows of W (E x H) against the T tokens.
// Quantised formats keep the tokens in the expert pair layout, so W's
// natural bf16 pairs are regrouped with v_perm.
template <int FMT>
__host__ __device__ __forceinline__ int router_lpr(int H) {
  if (FMT == MOE_W_F32) return 64;
  const int chunks = H / Fmt<FMT>::kWPC;
  return chunks < 64 ? chunks : 64;
}

template <int FMT>
__device__ __forceinline__ void router_task(const LayerArgs& a, int task, const uint32_t* xs, int vstride,
                            int lane) {
  const int lpr = router_lpr<FMT>(a.H);
  const int e = task * (64 / lpr) + lane / lpr;
  const int lane_g = lane % lpr;
  float acc[kTMax];
#pragma unroll
  for (int t = 0; t < kTMax; ++t) acc[t] = 0.f;
  if (e < a.E) {
    if constexpr (FMT == MOE_W_Q2B32 || FMT == MOE_W_Q4B32) {
      constexpr int kWPC = Fmt<FMT>::kWPC;
      const int chunks = a.H / kWPC;
      const u32x4* row = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.W) +
                                                        int64_t(e) * a.H);
      constexpr int kQ = kWPC / 8;          // 16-byte loads of W per chunk
      for (int c = lane_g; c < chunks; c += lpr) {
        uint32_t w[kQ * 4];
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const u32x4 v = row[c * kQ + q];
          w[q * 4 + 0] = v[0];
          w[q * 4 + 1] = v[1];
          w[q * 4 + 2] = v[2];
          w[q * 4 + 3] = v[3];
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
        for (int t = 0; t < kTMax; ++t) {
          if (t < a.T) {
            const uint32_t* xv = xs + t * vstride + c * Fmt<FMT>::kCS;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kG * kS; ++j) s4[j & 3] = dot2_bf16(pr[j], xv[j], s4[j & 3]);
            acc[t] += (s4[0] + s4[1]) + (s4[2] + s4[3]);
          }
        }
      }
    } else {
      const float* xf = reinterpret_cast<const float*>(xs);
      for (int col = lane_g; col < a.H; col += lpr) {
        const float wv = a.rfmt == MOE_W_F32
                             ? static_cast<const float*>(a.W)[int64_t(e) * a.H + col]
                             : bf16_to_f32(static_cast<const uint16_t*>(a.W)[int64_t(e) * a.H + col]);
#pragma unroll
        for (int t = 0; t < kTMax; ++t)
          if (t < a.T) acc[t] = fmaf(wv, xf[t * vstride + col], acc[t]);
      }
    }
  }
  const float b = (e < a.E && a.bias) ? a.bias[e] : 0.f;
#pragma unroll
  for (int t = 0; t < kTMax; ++t) {
    if (t < a.T) {
      float s = acc[t];
      for (int m = 1; m < lpr; m <<= 1) s += __shfl_xor(s, m, 64);
      if (e < a.E && lane_g == 0) st_dev(a.logits + t * a.E + e, s + b);
    }
  }
}

// --------------------------------------------------------------- kernel
template <int FMT>
__global__ __launch_bounds__(kThreads) void moe_layer_kernel(LayerArgs a) {
  constexpr int kLprGU = Lanes<FMT>::kGU, kRowsGU = Lanes<FMT>::kRowsGU;
  constexpr int kLprD = Lanes<FMT>::kD, kRowsD = Lanes<FMT>::kRowsD;
  extern __shared__ uint32_t smem[];
  __shared__ Lds L;
  __shared__ const float* srcs[kTMax];
  const int G = gridDim.x, b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int T = a.T, k = a.k, P = T * k, E = a.E;
  const int K = a.H;
  const int vstride = FMT == MOE_W_F32 ? K : (K / Fmt<FMT>::kWPC) * Fmt<FMT>::kCS;
  const int sstride = K / 32;
  // LDS: tokens | block sums | group sums | logits
  uint32_t* xs = smem;
  float* xsum = reinterpret_cast<float*>(xs + T * vstride);
  float* psum = xsum + T * sstride;
  float* lg = psum + T * (K / 16);

  if (tid == 0) L.flag0 = ld_dev(a.sync + kSyncCalls);
  stage_tokens<FMT>(a.x, T, K, xs, xsum, psum, vstride);
  __syncthreads();
  const uint32_t epoch = L.flag0 + 1u;     // this call's number
  uint32_t* task_flag = a.sync + kSyncTasks;

  // ---- A: router rows, shared gate/up rows, zero y
  {
    const int lpr = router_lpr<FMT>(K);
    const int n_router = (E + (64 / lpr) - 1) / (64 / lpr);
    const int n_shared = a.has_sh ? a.I / kRowsGU : 0;
    for (int task = b + wave * G; task < n_router + n_shared; task += kWaves * G) {
      if (task < n_router) {
        router_task<FMT>(a, task, xs, vstride, lane);
      } else {
        const int i = (task - n_router) * kRowsGU + lane / kLprGU;
        gateup_task<FMT>(a, a.sg, a.su, 0, i, T, nullptr, nullptr, a.h_sh, xs, xsum, vstride,
                         lane % kLprGU);
      }
    }
    for (int i = b * kThreads + tid; i < T * K; i += G * kThreads) st_dev(a.y + i, 0.f);
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) st_dev(a.sync + kSyncArrive + b, epoch);
  while (!__syncthreads_and(tid >= G || ld_dev(a.sync + kSyncArrive + tid) == epoch))
    __builtin_amdgcn_s_sleep(1);
  if (b == 0 && tid == 0) st_dev(a.sync + kSyncCalls, epoch);   // every workgroup has read it

  // ---- B: routing, in every workgroup
  {
    constexpr int kR = 8;
    for (int base = 0; base < T * E; base += kR * kThreads) {
      float v[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int i = base + r * kThreads + tid;
        if (i < T * E) v[r] = ld_dev(a.logits + i);
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int i = base + r * kThreads + tid;
        if (i < T * E) lg[i] = v[r];
      }
    }
  }
  __syncthreads();
  for (int t = wave; t < T; t += kWaves) {
    int my_e;
    float my_v;
    if (E <= 512) wave_topk<8>(lg + t * E, E, k, lane, &my_e, &my_v);
    else wave_topk<16>(lg + t * E, E, k, lane, &my_e, &my_v);
    const float vmax = __shfl(my_v, 0, 64);
    const float ex = lane < k ? expf(my_v - vmax) : 0.f;
    float z = ex;
    for (int m = 1; m < 64; m <<= 1) z += __shfl_xor(z, m, 64);
    if (lane < k) {
      const float g = ex / z;
      L.idx[t * k + lane] = my_e;
      L.gate[t * k + lane] = g;
      if (b == 0) {
        a.idx[t * k + lane] = my_e;
        a.gate[t * k + lane] = g;
      }
    }
  }
  __syncthreads();
  {
    const int p = tid;
    int s = -1;
    if (p < P) {
      const int e = L.idx[p];
      s = (e >= 0 && e < E) ? (a.slot_of ? a.slot_of[e] : e) : -1;
      s = (s >= 0 && s < a.S) ? s : -1;
      if (b == 0 && a.slot_idx) a.slot_idx[p] = s;
    }
    if (p < kPMax) L.slot[p] = s;
    const int is_miss = (p < P && s < 0) ? 1 : 0;
    int n_miss;
    const int mpos = block_exclusive_scan(is_miss, L.tmp, &n_miss);
    if (b == 0) {
      if (is_miss) {
        moe_miss m;
        m.expert = L.idx[p];
        m.token = p / k;
        m.gate = L.gate[p];
        a.miss[mpos] = m;
      }
      if (p < P && p % k == 0) a.miss_off[p / k] = mpos;
      if (p == 0) a.miss_off[T] = n_miss;
    }
    __syncthreads();
    const int n_hit = P - n_miss;
    if (p < P && s >= 0) {
      int pos = 0;
      for (int q = 0; q < P; ++q) {
        const int sq = L.slot[q];
        pos += (sq >= 0 && (sq < s || (sq == s && q < p))) ? 1 : 0;
      }
      L.bpair[pos] = p;
      L.tok[pos] = p / k;
      L.sorted[pos] = s;
    }
    __syncthreads();
    const int first = (p < n_hit && (p == 0 || L.sorted[p] != L.sorted[p - 1])) ? 1 : 0;
    int n_act;
    const int apos = block_exclusive_scan(first, L.tmp, &n_act);
    if (first) {
      L.act_slot[apos] = L.sorted[p];
      L.act_start[apos] = p;
    }
    if (p == 0) {
      L.act_start[n_act] = n_hit;
      L.n_act = n_act;
    }
    __syncthreads();
  }
  const int n_act = L.n_act;

  // ---- C: routed gate/up, 8 rows of one expert per wave task
  {
    const int tasks_per_expert = a.I / kRowsGU;
    const int n_tasks = n_act * tasks_per_expert;
    for (int task = b + wave * G; task < n_tasks; task += kWaves * G) {
      const int u = task / tasks_per_expert;
      const int i = (task % tasks_per_expert) * kRowsGU + lane / kLprGU;
      const int st = L.act_start[u];
      const int n = L.act_start[u + 1] - st;
      gateup_task<FMT>(a, a.g, a.u, L.act_slot[u], i, n, L.tok + st, L.bpair + st, a.h, xs, xsum,
                       vstride, lane % kLprGU);
      wait_mem();
      if (lane == 0) st_dev(task_flag + u * tasks_per_expert + task % tasks_per_expert, epoch);
    }
  }

  // ---- D: down units (expert or shared, 128-row block), y += gate * D h
  {
    const int Kd = a.I;
    constexpr int kVPP = FMT == MOE_W_F32 ? 1 : 2;
    const int vs_d = FMT == MOE_W_F32 ? Kd : (Kd / Fmt<FMT>::kWPC) * Fmt<FMT>::kCS;
    const int ss_d = Kd / 32;
    const int nch = chunks_of<FMT>(Kd) / kLprD;
    const int64_t row_bytes = int64_t(Kd) * fmt_bits(FMT) / 8;
    const int nrb = (a.H + kRowsD - 1) / kRowsD;
    const int contributors = n_act + (a.has_sh ? 1 : 0);
    const int n_units = contributors * nrb;
    uint32_t* xd = smem;                                    // reuses the token area
    float* sd = reinterpret_cast<float*>(xd + kVPP * kTMax * vs_d);
    float* pd = sd + kVPP * kTMax * ss_d;
    const int lane_g = lane % kLprD;
    for (int unit = b; unit < n_units; unit += G) {
      const int u = unit / nrb, rb = unit % nrb;
      const bool shared = u >= n_act;
      const int st = shared ? 0 : L.act_start[u];
      const int n = shared ? T : L.act_start[u + 1] - st;
      const MatView D = shared ? a.sd : a.d;
      const int slot = shared ? 0 : L.act_slot[u];
      const int r = rb * kRowsD + wave * (64 / kLprD) + lane / kLprD;
      const int rr = r < a.H ? r : a.H - 1;
      RowRegs<FMT, kNChMax> rd;
      const int64_t blk = int64_t(slot) * D.mat_blocks + int64_t(rr) * ss_d;
      load_row<FMT, kNChMax>(rd, D.codes + slot * D.mat_bytes + rr * row_bytes, D.scale + blk,
                              D.mn + blk, nch, lane_g, kLprD);
      // wait for this expert's gate/up tasks (also the barrier for LDS reuse)
      const int tpe = a.I / kRowsGU;
      while (!__syncthreads_and(shared || tid >= tpe ||
                                ld_dev(task_flag + u * tpe + tid) == epoch))
        __builtin_amdgcn_s_sleep(1);
      if (tid < n)
        srcs[tid] = shared ? a.h_sh + int64_t(tid) * Kd : a.h + int64_t(L.bpair[st + tid]) * Kd;
      __syncthreads();
      stage_h<FMT>(srcs, n, Kd, xd, sd, pd, vs_d);
      __syncthreads();
      for (int v = 0; v < n; ++v) {
        float o = row_vec_dot<FMT, kNChMax>(rd, nch, lane_g, kLprD, xd + (kVPP * v) * vs_d,
                                            sd + (kVPP * v) * ss_d);
        if (kVPP == 2)
          o += row_vec_dot<FMT, kNChMax>(rd, nch, lane_g, kLprD, xd + (kVPP * v + 1) * vs_d,
                                         sd + (kVPP * v + 1) * ss_d);
        o = group_sum<kLprD>(o);
        if (r < a.H && lane_g == 0) {
          const int t = shared ? v : L.tok[st + v];
          const float g = shared ? 1.f : L.gate[L.bpair[st + v]];
          fadd_dev(a.y + int64_t(t) * a.H + r, g * o);
        }
      }
    }
  }
}

struct Occ {
  size_t lds = 0;
  int device = -1;
  int grid = 0;
};

template <int FMT>
hipError_t launch_fmt(const LayerArgs& a, size_t lds, hipStream_t st, int* grid_out) {
  static thread_local Occ cache[3];
  Occ& c = cache[FMT == MOE_W_F32 ? 0 : FMT == MOE_W_Q2B32 ? 1 : 2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (c.lds != lds || c.device != dev) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_layer_kernel<FMT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_layer_kernel<FMT>, kThreads,
                                                     lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus > kThreads) return hipErrorInvalidConfiguration;
    c.lds = lds;
    c.device = dev;
    c.grid = cus;   // one workgroup of 8 waves per CU
  }
  if (grid_out) *grid_out = c.grid;
  hipLaunchKernelGGL(moe_layer_kernel<FMT>, dim3(c.grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
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
  // D: 2 vectors per token (hi, lo), block sums, group sums (sized for 16 tokens)
  const int vpp = fmt == MOE_W_F32 ? 1 : 2;
  const size_t d = size_t(vpp) * kTMax * (vec_bytes(fmt, I) + (I / 32) * 4 + (I / 16) * 4);
  return a > d ? a : d;
}

bool layer_fused_ok(int fmt, int T, int k, int E, int H, int I) {
  if (T < 1 || T > kTMax || T * k > kPMax) return false;
  if (fmt != MOE_W_F32 && fmt != MOE_W_Q2B32 && fmt != MOE_W_Q4B32) return false;
  if (H % 32 || I % 32 || E > 1024) return false;
  const int wpc = fmt == MOE_W_Q2B32 ? 64 : fmt == MOE_W_Q4B32 ? 32 : 4;
  const int lgu = fmt == MOE_W_Q4B32 ? Lanes<MOE_W_Q4B32>::kGU : Lanes<MOE_W_Q2B32>::kGU;
  const int ld = fmt == MOE_W_Q4B32 ? Lanes<MOE_W_Q4B32>::kD : Lanes<MOE_W_Q2B32>::kD;
  const int chunks = H / wpc, chunks_d = I / wpc;
  if (chunks % lgu || chunks / lgu > kNChMax) return false;
  if (chunks_d % ld || chunks_d / ld > kNChMax) return false;
  if (I / (64 / lgu) > kThreads) return false;   // one thread per task flag
  if (fmt != MOE_W_F32 && (chunks > 64 ? (chunks % 64) != 0 : (chunks & (chunks - 1)) != 0))
    return false;
  return layer_fused_lds(fmt, T, E, H, I) <= 150 * 1024;
}

hipError_t launch_layer_fused(const LayerArgs& a, hipStream_t st, int* grid) {
  const size_t lds = layer_fused_lds(a.fmt, a.T, a.E, a.H, a.I);
  switch (a.fmt) {
    case MOE_W_Q2B32: return launch_fmt<MOE_W_Q2B32>(a, lds, st, grid);
    case MOE_W_Q4B32: return launch_fmt<MOE_W_Q4B32>(a, lds, st, grid);
    case MOE_W_F32: return launch_fmt<MOE_W_F32>(a, lds, st, grid);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
