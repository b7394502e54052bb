// Prefill: the expert FFN as grouped GEMMs on fp16 MFMA, and the router as
// a bf16 MFMA GEMM.
//
// [MD] = ModelDock, "Strata はなぜ少ない VRAM でも速いのか", section
// "長いプロンプトを読む": a long prompt routes to nearly every expert of every
// layer, and an expert's weights are used by every token of the chunk that
// routes to it -- so each expert bucket becomes one GEMM whose weights are
// read once per tile of tokens instead of once per token.
//
// Work split (C = A B^T, A = tokens or h rows, B = weight rows):
//  - A tiles of 128 rows x 64 K live in LDS (double-buffered, rows padded),
//    filled through registers two K steps ahead, 8 lanes per 128-byte row.
//    A is fp16 and stored in a K order permuted inside each 32-wide block
//    (perm_pos) -- the tokens by a conversion pass, h by the gate/up
//    epilogue.
//  - B never goes through LDS: each wave owns 64 weight rows, and each lane
//    builds its MFMA operands from the one 32-weight block it needs (16 or 8
//    code bytes, loaded two K steps ahead; scales and mins of 8 blocks at a
//    time go through a small LDS table).  v_perm puts each code byte under
//    the exponent byte of fp16 1024, giving two exact values 1024 + q;
//    v_pk_add_f16 removes the 1024 exactly and v_pk_fma_f16 applies
//    d * q + m with one rounding.  The next K step's operands are built while
//    the current step's MFMAs run.
//  - Waves: 4 per block, two blocks per CU, wave tile 128 rows x 64 columns
//    (4 x 2 MFMA 32x32x16 tiles, fp32 accumulation).  gate/up waves hold 32
//    gate rows and the 32 up rows of the same features, so SwiGLU happens in
//    registers; h goes through LDS and leaves as whole fp16 rows.  Down waves
//    hold 64 output columns; their fp32 rows go through LDS in 32-row slabs
//    and leave as whole row pieces to pair_out by pair id.
//  - A bucket's last tile runs only the 32-row MFMA tiles its rows fill (the
//    body is compiled for 1-4 row tiles and chosen once per tile).
//  - The K loop is unrolled over one scale group with the registers in
//    flight indexed by K-step parity: no register copy forces a wait.
//  - Tiles are ordered so that consecutive tiles of one expert run on the
//    same XCD and share its weights in that XCD's L2.
//  - fp16 range: a token row whose largest magnitude lies outside
//    [2^-6, 2^16) is converted as x * 2^-e, with e chosen so that its largest
//    magnitude lands in [2^14, 2^15); the gate/up epilogue multiplies that
//    row's products by 2^e (exact).  Likewise each h row slab of 128
//    features outside [2^-6, 2^15) is stored as h * 2^-e with its own e; a
//    small pass brings the slabs of a row to the row's largest e (rescaling
//    the others in place), and the down epilogue multiplies the row's
//    outputs by 2^e.  In range every e is 0 and nothing is rescaled; inside
//    the range every bf16 token value converts to fp16 exactly and h keeps
//    11 significant bits relative to the slab's largest value.
#include "gemv_core.h"
#include "kernels.h"

namespace moe {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;          // rows per router tile
constexpr int kQM = 128;          // rows per grouped-GEMM tile
constexpr int kBK = 64;           // K per step
constexpr int kLdsRow = kBK + 8;  // halves per LDS row (padding spreads banks)
constexpr int kXcds = 8;

// Position, inside its 32-wide block, at which the activation of K index
// j (0..31) is stored: the order in which the weight operand of one lane
// holds the block (w_operand below).
//   4-bit: dword i (weights 8i..8i+7) gives operand kk = i with elements
//          [0,2,4,6,1,3,5,7] + 8i;
//   2-bit: dword i (weights 16i..16i+15) gives operands kk = 2i + t, t = 0,1,
//          with elements r + 4b for r = 2t, 2t+1 (outer) and b = 0..3 (inner).
template <int FMT>
__host__ __device__ __forceinline__ int perm_pos(int j) {
  if (FMT == MOE_W_Q4B32) {
    const int g = j >> 3, r = j & 7;
    return 8 * g + ((r & 1) ? 4 + (r >> 1) : (r >> 1));
  } else {
    const int i = j >> 4, r = j & 3, b = (j >> 2) & 3;
    return 8 * (2 * i + (r >> 1)) + 4 * (r & 1) + b;
  }
}

// Scale exponent of a row (or row slab) whose largest magnitude is amax:
// 0 inside [lo, hi), else floor(log2 amax) - 14, which brings the largest
// magnitude into [2^14, 2^15).  An all-zero slab gets kZeroSlab, which
// takes no part in the row's common exponent.
constexpr int kZeroSlab = -128;
__device__ __forceinline__ int range_exp(float amax, float lo, float hi) {
  if (amax == 0.f) return kZeroSlab;
  if (amax >= lo && amax < hi) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 14;   // frexp: amax = m 2^f, m in [0.5, 1)
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
  const _Float16 a = _Float16(lo), b = _Float16(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Codes -> fp16 pairs (1024 + q, 1024 + q'): v_perm places a code byte (at
// most 15) under the exponent byte 0x64 of fp16 1024.  Selector bytes 0-3
// pick the code bytes, 4 the magic byte.
constexpr uint32_t kMagic = 0x64646464u;
constexpr uint32_t kSelB01 = 0x04010400u;   // code bytes 0, 1
constexpr uint32_t kSelB23 = 0x04030402u;   // code bytes 2, 3

__device__ __forceinline__ uint32_t dq_pair(uint32_t pr, f16x2 d2, f16x2 m2) {
  const f16x2 k1024 = {_Float16(1024.f), _Float16(1024.f)};
  const f16x2 q = __builtin_bit_cast(f16x2, pr) - k1024;                 // the codes, exact
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, d2, m2));   // d q + m, one rounding
}

// MFMA B operand kk (0..3) of a lane's block: 8 dequantised fp16 weights in
// the order perm_pos describes.
template <int FMT>
__device__ __forceinline__ f16x8 w_operand(const uint32_t* c, int kk, f16x2 d2, f16x2 m2) {
  uint32_t g0, g1;
  if constexpr (FMT == MOE_W_Q4B32) {
    g0 = c[kk] & 0x0F0F0F0Fu;
    g1 = (c[kk] >> 4) & 0x0F0F0F0Fu;
  } else {
    const uint32_t w = c[kk >> 1];
    const int t = kk & 1;
    g0 = (w >> (4 * t)) & 0x03030303u;
    g1 = (w >> (4 * t + 2)) & 0x03030303u;
  }
  const u32x4 v = {dq_pair(__builtin_amdgcn_perm(kMagic, g0, kSelB01), d2, m2),
                   dq_pair(__builtin_amdgcn_perm(kMagic, g0, kSelB23), d2, m2),
                   dq_pair(__builtin_amdgcn_perm(kMagic, g1, kSelB01), d2, m2),
                   dq_pair(__builtin_amdgcn_perm(kMagic, g1, kSelB23), d2, m2)};
  return __builtin_bit_cast(f16x8, v);
}

struct TileInfo {
  int bucket, m0;
};

// ---------------------------------------------------------------- schedule
// Tile list over the active buckets (and the shared expert as one more
// bucket holding every token): tiles[i] = (bucket, first row).
__global__ __launch_bounds__(1024) void gemm_schedule_kernel(ActiveList act, int T, int has_sh,
                                                             int2* tiles, int* n_tiles) {
  __shared__ int tmp[32];
  const int n_act = *act.count;
  const int nb = n_act + has_sh;
  int before = 0;
  for (int base = 0; base < nb; base += blockDim.x) {
    const int u = base + threadIdx.x;
    int cnt = 0;
    if (u < nb) {
      const int n = u < n_act ? act.start[u + 1] - act.start[u] : T;
      cnt = (n + kQM - 1) / kQM;
    }
    int tot;
    const int off = before + block_exclusive_scan(cnt, tmp, &tot);
    for (int i = 0; i < cnt; ++i) tiles[off + i] = make_int2(u, i * kQM);
    before += tot;
  }
  if (threadIdx.x == 0) *n_tiles = before;
}

// Grids are a multiple of kXcds so that xcd_item() is a bijection.
inline int round_xcd(int g) { return (g + kXcds - 1) / kXcds * kXcds; }

// Work item of this workgroup: workgroups are dealt to the XCDs in turn, so
// XCD x runs items [x * per, (x + 1) * per) and consecutive items share it.
__device__ __forceinline__ int xcd_item() {
  const int L = blockIdx.x, G = gridDim.x;
  const int per = (G + kXcds - 1) / kXcds;
  return (L % kXcds) * per + L / kXcds;
}

struct GemmArgs {
  const uint16_t* x16;      // fp16 [T][H], K-permuted
  int T, k, H, I;
  MatView g, u, d, sg, su, sd;
  ActiveList act;
  const int32_t* bucket_pair;
  const int2* tiles;
  const int* n_tiles;
  uint16_t* h;              // fp16 [n_hit][I] by bucket position, K-permuted
  uint16_t* h_sh;           // fp16 [T][I]
  float* pair_out;          // [T*k][H]
  float* shared_out;        // [T][H]
  // scale exponents (fp16 range): tokens [T]; h row slabs [P + T][I / 128]
  // and h rows [P + T] (routed rows at their bucket position, the shared
  // expert's rows at P + token)
  int8_t* xe;
  int8_t* he;
  int8_t* hr;
  int P;
  float* y_acc;             // accumulate mode: y [T][H] += gate * o (else null)
  const float* gate;        // [T*k]
};

// Rows of the tile: token (A source row) and output row id.
struct RowMap {
  int rows;          // valid rows in the tile
  int slot;
  bool shared;
  int pos0;          // bucket position of row 0 (routed)
};

__device__ __forceinline__ RowMap row_map(const GemmArgs& a, int2 t, int n_act) {
  RowMap r;
  r.shared = t.x >= n_act;
  if (!r.shared) {
    const int st = a.act.start[t.x], n = a.act.start[t.x + 1] - st;
    r.rows = min(kQM, n - t.y);
    r.slot = a.act.slot[t.x];
    r.pos0 = st + t.y;
  } else {
    r.rows = min(kQM, a.T - t.y);
    r.slot = 0;
    r.pos0 = t.y;
  }
  return r;
}

// ---------------------------------------------------------------- tokens
// x (bf16) -> x16 (fp16) with K permuted inside each 32-wide block, one wave
// per token (H <= 8192: at most 4 blocks of 32 per lane).  xe[t] receives
// the token's scale exponent (x16 = x * 2^-xe).
template <int FMT>
__global__ __launch_bounds__(256) void x16_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                  uint16_t* __restrict__ x16,
                                                  int8_t* __restrict__ xe) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const int nb = H / 32;
  const uint16_t* row = x + int64_t(t) * H;
  uint32_t w[4][16];
  uint32_t mbits = 0;   // largest |x| of the lane as bf16 bits (monotonic for finite values)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = lane + 64 * j;
    if (b < nb) {
      const u32x4* src = reinterpret_cast<const u32x4*>(row + b * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = src[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[j][4 * q + e] = v[e];
          mbits = max(mbits, max(v[e] & 0x7FFFu, (v[e] >> 16) & 0x7FFFu));
        }
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) mbits = max(mbits, uint32_t(__shfl_xor(int(mbits), m, 64)));
  int e = range_exp(__uint_as_float(mbits << 16), 0x1p-6f, 0x1p16f);
  e = e == kZeroSlab ? 0 : e;
  if (lane == 0) xe[t] = int8_t(e);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = lane + 64 * j;
    if (b >= nb) continue;
    uint16_t o[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t bits = (w[j][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const float f = __uint_as_float(bits << 16);
      o[perm_pos<FMT>(i)] = __builtin_bit_cast(uint16_t, _Float16(e ? ldexpf(f, -e) : f));
    }
    u32x4* dst = reinterpret_cast<u32x4*>(x16 + int64_t(t) * H + b * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dst[q] = u32x4{uint32_t(o[8 * q]) | (uint32_t(o[8 * q + 1]) << 16),
                     uint32_t(o[8 * q + 2]) | (uint32_t(o[8 * q + 3]) << 16),
                     uint32_t(o[8 * q + 4]) | (uint32_t(o[8 * q + 5]) << 16),
                     uint32_t(o[8 * q + 6]) | (uint32_t(o[8 * q + 7]) << 16)};
  }
}

// ---------------------------------------------------------------- GEMM
// One grouped-GEMM tile: 128 rows of one bucket x 128 * NJ weight rows
// (gate/up, NJ = 2: 128 gate + 128 up rows of 128 features; down: 128 * NJ
// output columns).  Each wave holds all 128 rows x 32 * NJ columns (4 x NJ
// MFMA tiles), so every dequantised weight feeds 4 MFMAs.
constexpr int kSdRow = 9;         // dwords per weight row in the scale table (8 + pad)
constexpr int kGroup = 4;         // K steps per scale group (8 blocks)

typedef uint16_t ATile[kQM * kLdsRow];

// One tile whose rows fit in MT MFMA row tiles (MT * 32 >= rows): the
// waves skip the row tiles of a bucket's last, partly filled tile.
template <int FMT, bool GU, int MT, int NJ>
__device__ __forceinline__ void qgemm_tile(const GemmArgs& a, const RowMap& rm, int nt, ATile* As,
                                           uint32_t* Sd0, const int* arow, const int* orow,
                                           const int* rsc, bool scaled) {
  constexpr int kBNt = 128 * NJ;   // weight rows of the tile (32 * NJ per wave)
  auto Sd = [&](int buf) { return Sd0 + buf * (kBNt * kSdRow); };
  constexpr int kCW = FMT == MOE_W_Q4B32 ? 4 : 2;   // code dwords of one block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = GU ? a.H : a.I;
  const int nk = K / kBK, nb = K / 32;
  const uint16_t* abase = GU ? a.x16 : (rm.shared ? a.h_sh : a.h);
  // A staging: 8 lanes per row (16 bytes each, a whole 128-byte K step);
  // this thread's rows q * 32 + tid / 8, q = 0..3
  const int achunk = tid & 7;
  uint32_t aoff[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) aoff[q] = uint32_t(arow[q * 32 + (tid >> 3)]) * uint32_t(K) + achunk * 8;
  // weight rows: tile row R = wave * 64 + j * 32 + col (j = MFMA column tile)
  const MatView W0 = GU ? (rm.shared ? a.sg : a.g) : (rm.shared ? a.sd : a.d);
  const MatView W1 = GU ? (rm.shared ? a.su : a.u) : W0;
  const int slot = rm.shared ? 0 : rm.slot;
  auto weight_row = [&](int R, const MatView*& Wm) {
    const int wv = R / (32 * NJ), j = (R >> 5) % NJ, c = R & 31;
    if (GU) {
      Wm = j ? &W1 : &W0;
      return nt * 128 + wv * 32 + c;
    }
    Wm = &W0;
    return nt * kBNt + R;
  };
  const int col = lane & 31, bh = lane >> 5;
  const int64_t row_bytes = int64_t(K) * fmt_bits(FMT) / 8;
  const uint8_t* cw[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const MatView* Wm;
    const int r = weight_row(wave * 32 * NJ + j * 32 + col, Wm);
    cw[j] = Wm->codes + slot * Wm->mat_bytes + r * row_bytes;
  }
  // scale group staging: thread tid loads weight row tid's 8 scales and mins
  const uint16_t *sg_sc, *sg_mn;
  {
    const MatView* Wm;
    const int r = weight_row(tid < kBNt ? tid : 0, Wm);
    const int64_t b = int64_t(slot) * Wm->mat_blocks + int64_t(r) * nb;
    sg_sc = Wm->scale + b;
    sg_mn = Wm->mn + b;
  }

  // Registers in flight are indexed by K-step parity and the K loop is
  // unrolled over one scale group, so no register copy ever forces a wait
  // for loads issued in the same step: A of step kt + 2 and its codes are
  // loaded into the parity-kt buffers at the start of step kt; A of step
  // kt + 1 (loaded one step earlier) goes to LDS at its end.  Loads past the
  // last step repeat the last step (in bounds, unused), so every step issues
  // the same loads and the wait counts stay exact.
  u32x4 ra[2][MT];              // A of K steps kt + 1 and kt + 2
  uint32_t wc[2][NJ][kCW];       // codes of K steps kt + 1 and kt + 2
  u32x4 gsc, gmn;                // scales / mins of the next group in flight
  auto load_a = [&](int kt, u32x4* r) {
#pragma unroll
    for (int q = 0; q < MT; ++q) r[q] = *reinterpret_cast<const u32x4*>(abase + aoff[q] + kt * kBK);
  };
  auto store_a = [&](const u32x4* r, int buf) {
#pragma unroll
    for (int q = 0; q < MT; ++q)
      *reinterpret_cast<u32x4*>(&As[buf][(q * 32 + (tid >> 3)) * kLdsRow + achunk * 8]) = r[q];
  };
  auto load_codes = [&](int kt, uint32_t (*c)[kCW]) {
    const int blk = 2 * kt + bh;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (FMT == MOE_W_Q4B32) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(cw[j] + blk * 16);
        c[j][0] = v[0]; c[j][1] = v[1]; c[j][2] = v[2]; c[j][3] = v[3];
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(cw[j] + blk * 8);
        c[j][0] = v.x; c[j][1] = v.y;
      }
    }
  };
  auto load_group = [&](int g) {
    gsc = *reinterpret_cast<const u32x4*>(sg_sc + 8 * g);
    gmn = *reinterpret_cast<const u32x4*>(sg_mn + 8 * g);
  };
  auto store_group = [&](int buf) {
    if (tid >= kBNt) return;
    uint32_t* d = Sd(buf) + tid * kSdRow;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d[2 * q] = (gsc[q] & 0xFFFFu) | (gmn[q] << 16);
      d[2 * q + 1] = (gsc[q] >> 16) | (gmn[q] & 0xFFFF0000u);
    }
  };
  f32x16 acc[MT][NJ];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

  // Scale group g sits in Sd[g & 1] from the K step before its first one
  // on; its loads are issued three K steps before that (the last group's
  // loads are repeated past the end, into a buffer nothing reads again).
  const int ngroups = nk / kGroup;
  auto scales = [&](int kt, int j, f16x2& d2, f16x2& m2) {
    const uint32_t dm = Sd((kt / kGroup) & 1)[(wave * 32 * NJ + j * 32 + col) * kSdRow + 2 * (kt % kGroup) + bh];
    d2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(dm, dm, 0x01000100u));
    m2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(dm, dm, 0x03020302u));
  };
  load_group(0);
  load_a(0, ra[0]);
  load_codes(0, wc[0]);
  load_a(min(1, nk - 1), ra[1]);
  load_codes(min(1, nk - 1), wc[1]);
  store_group(0);
  load_group(min(1, ngroups - 1));
  store_a(ra[0], 0);
  __syncthreads();
  // weight operands of K step 0
  f16x8 bv[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    f16x2 d2, m2;
    scales(0, j, d2, m2);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bv[j][kk] = w_operand<FMT>(wc[0][j], kk, d2, m2);
  }
  for (int kt0 = 0; kt0 < nk; kt0 += kGroup) {
    const int g = kt0 / kGroup;
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
      const int kt = kt0 + s, p = s & 1;   // kt0 is even: p is the parity of kt
      const int kl = min(kt + 2, nk - 1), kn = min(kt + 1, nk - 1);
      load_a(kl, ra[p]);
      load_codes(kl, wc[p]);
      f16x2 dn[NJ], mn[NJ];   // scales of the next K step
#pragma unroll
      for (int j = 0; j < NJ; ++j) scales(kn, j, dn[j], mn[j]);
      const uint16_t* Ab = As[p];
      // the next K step's weight operand kk is built while the MFMAs of kk
      // run, in the registers those MFMAs have just read (after the last
      // step the build repeats the last step's operands, unused)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f16x8 av[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
          av[i] = *reinterpret_cast<const f16x8*>(Ab + (i * 32 + col) * kLdsRow + bh * 32 + kk * 8);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j][kk], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bv[j][kk] = w_operand<FMT>(wc[p ^ 1][j], kk, dn[j], mn[j]);
      }
      store_a(ra[p ^ 1], p ^ 1);
      if (s == kGroup - 2) {
        store_group((g + 1) & 1);
        load_group(min(g + 2, ngroups - 1));
      }
      __syncthreads();
    }
  }
  // epilogue: element v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4 of
  // the 32 x 32 tile, column l % 32
  if constexpr (GU) {
    // h tile (128 rows x 128 features, fp16, features in the permuted order)
    // through LDS, then whole 256-byte rows to global memory
    constexpr int kHRow = 128 + 8;   // halves per LDS row
    static_assert(kQM * kHRow <= 2 * kQM * kLdsRow, "h tile fits in the A buffers");
    uint16_t* ht = &As[0][0];        // the A buffers are free after the last K step
    const int fl = wave * 32 + col;  // feature within the tile
    const int fcol = (fl & ~31) + perm_pos<FMT>(fl & 31);
    // h of element v of MFMA row tile i (the token's scale undone first)
    auto h_of = [&](int i, int v) {
      float ga = acc[i][0][v], ua = acc[i][1][v];
      if (scaled) {
        const int sc = rsc[i * 32 + 8 * (v >> 2) + 4 * bh + (v & 3)];
        ga = ldexpf(ga, sc);
        ua = ldexpf(ua, sc);
      }
      return silu_f32(ga) * ua;
    };
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = i * 32 + 8 * (v >> 2) + 4 * bh + (v & 3);
        ht[row * kHRow + fcol] = __builtin_bit_cast(uint16_t, _Float16(h_of(i, v)));
      }
    __syncthreads();
    // Range check of the slab: the 16 threads of a row (one 16-lane DPP row)
    // take the largest |h| of their pieces as fp16 bits.  Inside [2^-6, 2^15)
    // for every row of the tile: stored as is, exponent 0.
    constexpr int kQ = kQM * 16 / 256;
    bool off = false;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int c = q * 256 + tid, row = c >> 4, ch = c & 15;
      const u32x4 pc = *reinterpret_cast<const u32x4*>(ht + row * kHRow + ch * 8);
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) m = max(m, max(pc[e] & 0x7FFFu, (pc[e] >> 16) & 0x7FFFu));
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0xB1, 0xF, 0xF, true)));
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x4E, 0xF, 0xF, true)));
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x141, 0xF, 0xF, true)));
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x140, 0xF, 0xF, true)));
      // fp16 bits of 2^-6 and 2^15
      off = off || (row < rm.rows && (m < 0x2400u || m >= 0x7800u));
    }
    const bool slow = __syncthreads_or(off) != 0;
    int8_t* he = a.he + (int64_t(rm.shared ? a.P + rm.pos0 : rm.pos0)) * (a.I / 128) + nt;
    if (slow) {
      // exact per-row maxima of the fp32 h, then each row scaled into range
      uint32_t* rmax = reinterpret_cast<uint32_t*>(Sd0);   // the scale tables are free too
      if (tid < kQM) rmax[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          atomicMax(&rmax[i * 32 + 8 * (v >> 2) + 4 * bh + (v & 3)],
                    __float_as_uint(fabsf(h_of(i, v))));
      __syncthreads();
      int* rexp = reinterpret_cast<int*>(rmax) + kQM;
      if (tid < kQM) {
        const int e = range_exp(__uint_as_float(rmax[tid]), 0x1p-6f, 0x1p15f);
        rexp[tid] = e;
        if (tid < rm.rows) he[int64_t(tid) * (a.I / 128)] = int8_t(e);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = i * 32 + 8 * (v >> 2) + 4 * bh + (v & 3);
          const int e = rexp[row];
          const float hv = h_of(i, v);
          ht[row * kHRow + fcol] =
              __builtin_bit_cast(uint16_t, _Float16(e == kZeroSlab ? hv : ldexpf(hv, -e)));
        }
      __syncthreads();
    } else if (tid < rm.rows) {
      he[int64_t(tid) * (a.I / 128)] = 0;
    }
    uint16_t* out = (rm.shared ? a.h_sh : a.h) + int64_t(rm.pos0) * a.I + nt * 128;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int c = q * 256 + tid, row = c >> 4, ch = c & 15;
      if (row < rm.rows)
        *reinterpret_cast<u32x4*>(out + int64_t(row) * a.I + ch * 8) =
            *reinterpret_cast<const u32x4*>(ht + row * kHRow + ch * 8);
    }
  } else {
    // the fp32 tile in 32-row slabs through LDS, then whole 1 KB row pieces
    // to pair_out, 16 bytes per lane, as non-temporal stores (the combine
    // reads them much later; they would only displace weights and tokens
    // from the L2)
    constexpr int kORow = kBNt + 4;   // floats per LDS row
    static_assert(32 * kORow * 4 <= int(2 * sizeof(ATile)), "an output slab fits in the A buffers");
    float* ot = reinterpret_cast<float*>(&As[0][0]);
    float* out = (rm.shared ? a.shared_out : a.pair_out) + nt * kBNt;
    const int ocol = wave * 32 * NJ + col;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i > 0) __syncthreads();   // the previous slab has been read
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * bh + (v & 3);
#pragma unroll
        for (int j = 0; j < NJ; ++j) ot[r * kORow + ocol + 32 * j] = acc[i][j][v];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 32 / (1024 / kBNt); ++q) {
        const int r = q * (1024 / kBNt) + tid / (kBNt / 4), c4 = tid % (kBNt / 4);
        if (i * 32 + r < rm.rows) {
          f32x4 o4 = *reinterpret_cast<const f32x4*>(ot + r * kORow + 4 * c4);
          if (scaled) {   // the h row's scale undone
            const int e = rsc[i * 32 + r];
#pragma unroll
            for (int c = 0; c < 4; ++c) o4[c] = ldexpf(o4[c], e);
          }
          const int p = orow[i * 32 + r];
          if (a.y_acc) {   // the combine, fused: y[t] += gate * o
            const int t = rm.shared ? p : p / a.k;
            const float g = rm.shared ? 1.f : a.gate[p];
            float* yr = a.y_acc + int64_t(t) * a.H + nt * kBNt + 4 * c4;
#pragma unroll
            for (int c = 0; c < 4; ++c)
              __hip_atomic_fetch_add(yr + c, g * o4[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            __builtin_nontemporal_store(o4, reinterpret_cast<f32x4*>(out + int64_t(p) * a.H + 4 * c4));
          }
        }
      }
    }
  }
}

// Between the two GEMMs: brings the slabs of each h row to one exponent,
// the largest of the row's slabs (all-zero slabs take no part), rescaling
// the slabs stored with a smaller one in place by a power of two below 1,
// and records it in hr.  In range every slab has exponent 0 and the pass
// only reads the exponents.  One thread per row: routed rows are the bucket
// positions [0, n_hit), the shared expert's rows P + t.
__global__ __launch_bounds__(256) void h_range_kernel(GemmArgs a, int has_sh) {
  const int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool shared = r >= a.P;
  if (shared ? (!has_sh || r >= int64_t(a.P) + a.T) : r >= a.act.start[*a.act.count]) return;
  const int ns = a.I / 128;
  const int8_t* e = a.he + r * ns;
  int emax = kZeroSlab;
  for (int s = 0; s < ns; ++s) emax = max(emax, int(e[s]));
  if (emax == kZeroSlab) emax = 0;
  uint16_t* h = shared ? a.h_sh + (r - a.P) * a.I : a.h + r * a.I;
  for (int s = 0; s < ns; ++s) {
    const int es = e[s];
    if (es == kZeroSlab || es == emax) continue;
    for (int i = s * 128; i < (s + 1) * 128; ++i) {
      const float f = float(__builtin_bit_cast(_Float16, h[i]));
      h[i] = __builtin_bit_cast(uint16_t, _Float16(ldexpf(f, es - emax)));
    }
  }
  a.hr[r] = int8_t(emax);
}

template <int FMT, bool GU, int NJ>
__global__ __launch_bounds__(256, NJ == 1 ? 3 : 2) void qgemm_kernel(GemmArgs a, int n_ntiles) {
  __shared__ __align__(16) ATile As[2];
  __shared__ uint32_t Sd[2 * 128 * NJ * kSdRow];   // d | m << 16 per (weight row, block of the group)
  __shared__ int arow[kQM];
  __shared__ int orow[kQM];  // down: pair_out row of each tile row
  __shared__ int rsc[kQM];   // scale exponent of each tile row (gate/up: token; down: h row)
  const int w = xcd_item();
  const int total = *a.n_tiles * n_ntiles;
  if (w >= total) return;
  const int n_act = *a.act.count;
  const int2 tinfo = a.tiles[w / n_ntiles];
  const int nt = w % n_ntiles;
  const RowMap rm = row_map(a, tinfo, n_act);
  const int tid = threadIdx.x;
  // A source rows: gate/up gathers token rows of x16; down reads h rows at
  // the bucket positions.  Rows past the bucket read row 0 of the tile.
  int sc = 0;
  if (tid < kQM) {
    const int r = tid < rm.rows ? tid : 0;
    const int p = rm.shared ? rm.pos0 + r : a.bucket_pair[rm.pos0 + r];
    arow[tid] = GU ? (rm.shared ? p : p / a.k) : rm.pos0 + r;
    orow[tid] = p;
    sc = GU ? int(a.xe[rm.shared ? p : p / a.k])
            : int(a.hr[rm.shared ? a.P + rm.pos0 + r : rm.pos0 + r]);
    rsc[tid] = sc;
  }
  const bool scaled = __syncthreads_or(sc != 0) != 0;
  const int mt = (rm.rows + 31) >> 5;   // wave-uniform
  if (mt >= 4)
    qgemm_tile<FMT, GU, 4, NJ>(a, rm, nt, As, Sd, arow, orow, rsc, scaled);
  else if (mt == 3)
    qgemm_tile<FMT, GU, 3, NJ>(a, rm, nt, As, Sd, arow, orow, rsc, scaled);
  else if (mt == 2)
    qgemm_tile<FMT, GU, 2, NJ>(a, rm, nt, As, Sd, arow, orow, rsc, scaled);
  else
    qgemm_tile<FMT, GU, 1, NJ>(a, rm, nt, As, Sd, arow, orow, rsc, scaled);
}

// MFMA on one K step from LDS (bf16 router): wave tile = (MT x 32 rows) x
// (NT x 32 cols), A and B rows of kLdsRow halves.
template <int MT, int NT>
__device__ __forceinline__ void mma_step_bf16(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
                                              int lane, f32x16 (&acc)[MT][NT], int n_stride) {
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    u32x4 av[MT], bv[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      av[i] = *reinterpret_cast<const u32x4*>(As + (wm + i * 32 + (lane & 31)) * kLdsRow +
                                              kk * 16 + (lane >> 5) * 8);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      bv[j] = *reinterpret_cast<const u32x4*>(Bs + (wn + j * n_stride + (lane & 31)) * kLdsRow +
                                              kk * 16 + (lane >> 5) * 8);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                            __builtin_bit_cast(bf16x8, bv[j]),
                                                            acc[i][j], 0, 0, 0);
  }
}

// ---------------------------------------------------------------- router
// logits[t][e] = x[t] . W[e] + bias[e]; 128 tokens x 128 experts per tile.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x, int T,
                                                          int H, int E, const uint16_t* __restrict__ W,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int n_etiles) {
  __shared__ uint16_t As[2][kBM * kLdsRow];
  __shared__ uint16_t Bs[2][128 * kLdsRow];
  const int w = xcd_item();
  const int n_ttiles = (T + kBM - 1) / kBM;
  if (w >= n_ttiles * n_etiles) return;
  const int t0 = (w / n_etiles) * kBM, e0 = (w % n_etiles) * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ar = tid >> 1, ah = tid & 1;
  const int ta = min(t0 + ar, T - 1), eb = min(e0 + ar, E - 1);
  const uint16_t* xrow = x + int64_t(ta) * H + ah * 32;
  const uint16_t* wrow = W + int64_t(eb) * H + ah * 32;
  u32x4 ra[4], rb[4];
  auto load = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = reinterpret_cast<const u32x4*>(xrow + kt * kBK)[q];
      rb[q] = reinterpret_cast<const u32x4*>(wrow + kt * kBK)[q];
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      reinterpret_cast<u32x4*>(&As[buf][ar * kLdsRow + ah * 32])[q] = ra[q];
      reinterpret_cast<u32x4*>(&Bs[buf][ar * kLdsRow + ah * 32])[q] = rb[q];
    }
  };
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int nk = H / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    mma_step_bf16<2, 2>(As[kt & 1], Bs[kt & 1], wm, wn, lane, acc, 32);
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int e = e0 + wn + j * 32 + (lane & 31);
        if (t < T && e < E) logits[int64_t(t) * E + e] = acc[i][j][v] + (bias ? bias[e] : 0.f);
      }
}

template <int FMT>
hipError_t launch_gemm_fmt(const GemmArgs& ga, const uint16_t* x, int max_tiles, int has_sh,
                           hipStream_t st) {
  hipLaunchKernelGGL(x16_kernel<FMT>, dim3(unsigned((ga.T + 3) / 4)), dim3(256), 0, st, x, ga.T,
                     ga.H, const_cast<uint16_t*>(ga.x16), ga.xe);
  // down tiles of 256 columns (2 MFMA column tiles per wave); 128-column
  // tiles (1 per wave, 160 registers, three workgroups per CU) measured slower
  constexpr int kNJD = 2;
  const int nt_gu = ga.I / 128, nt_d = ga.H / (128 * kNJD);
  hipLaunchKernelGGL((qgemm_kernel<FMT, true, 2>), dim3(round_xcd(max_tiles * nt_gu)), dim3(256), 0, st,
                     ga, nt_gu);
  const int64_t rows = int64_t(ga.P) + ga.T;
  hipLaunchKernelGGL(h_range_kernel, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, st, ga, has_sh);
  hipLaunchKernelGGL((qgemm_kernel<FMT, false, kNJD>), dim3(round_xcd(max_tiles * nt_d)), dim3(256), 0,
                     st, ga, nt_d);
  return hipGetLastError();
}

int gemm_max_tiles(int T, int k, int S) {
  const int64_t P = int64_t(T) * k;
  return int(P / kQM + (P < S ? P : S) + T / kQM + 2);
}

// Workspace: tile list, fp16 h (bucket positions, then the shared expert's
// rows), fp16 tokens, then the scale exponents: tokens, h row slabs, h rows.
struct GemmWs {
  size_t tiles, h, x16, xe, he, hr, total;
};
GemmWs gemm_ws(int T, int k, int H, int I, int S) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int64_t P = int64_t(T) * k;
  GemmWs w;
  size_t o = 0;
  w.tiles = o;
  o += up(size_t(gemm_max_tiles(T, k, S)) * 8 + 8);
  w.h = o;
  o += up(size_t(P + T) * I * 2);
  w.x16 = o;
  o += up(size_t(T) * H * 2);
  w.xe = o;
  o += up(size_t(T));
  w.he = o;
  o += up(size_t(P + T) * (I / 128));
  w.hr = o;
  o += up(size_t(P + T));
  w.total = o;
  return w;
}
}  // namespace

size_t ffn_gemm_ws(int T, int k, int H, int I, int S) { return gemm_ws(T, k, H, I, S).total; }

// The tile offsets are 32-bit: token rows T * H and h rows (T * k + T) * I
// stay below 2^31 elements.
bool ffn_gemm_fits(int T, int k, int H, int I) {
  const int64_t P = int64_t(T) * k;
  return int64_t(T) * H < (int64_t(1) << 31) && (P + T) * I < (int64_t(1) << 31);
}

// K of both GEMMs a multiple of 256 (whole groups of 8 scale blocks); the
// gate/up tile covers 128 features, the down tile 256 columns.
bool ffn_gemm_ok(int fmt, int H, int I) {
  return (fmt == MOE_W_Q2B32 || fmt == MOE_W_Q4B32) && H % 256 == 0 && I % 256 == 0;
}

hipError_t launch_ffn_gemm(const FfnArgs& f, int S, const int32_t* bucket_off, void* ws,
                           hipStream_t st) {
  (void)bucket_off;
  const int64_t P = int64_t(f.T) * f.k;
  const int max_tiles = gemm_max_tiles(f.T, f.k, S);
  const GemmWs w = gemm_ws(f.T, f.k, f.H, f.I, S);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int* n_tiles = reinterpret_cast<int*>(base + w.tiles);
  int2* tiles = reinterpret_cast<int2*>(base + w.tiles + 8);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + w.h);
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base + w.x16);
  GemmArgs ga;
  ga.xe = reinterpret_cast<int8_t*>(base + w.xe);
  ga.he = reinterpret_cast<int8_t*>(base + w.he);
  ga.hr = reinterpret_cast<int8_t*>(base + w.hr);
  ga.P = int(P);
  ga.x16 = x16;
  ga.T = f.T;
  ga.k = f.k;
  ga.H = f.H;
  ga.I = f.I;
  ga.g = f.g; ga.u = f.u; ga.d = f.d;
  ga.sg = f.sg; ga.su = f.su; ga.sd = f.sd;
  ga.act = f.act;
  ga.bucket_pair = f.bucket_pair;
  ga.tiles = tiles;
  ga.n_tiles = n_tiles;
  ga.h = h;
  ga.h_sh = h + P * f.I;
  ga.pair_out = f.pair_out;
  ga.shared_out = f.shared_out;
  ga.y_acc = f.y_acc;
  ga.gate = f.gate;
  const int has_sh = f.sg.codes != nullptr ? 1 : 0;
  hipLaunchKernelGGL(gemm_schedule_kernel, dim3(1), dim3(1024), 0, st, f.act, f.T, has_sh, tiles,
                     n_tiles);
  switch (f.fmt) {
    case MOE_W_Q4B32: return launch_gemm_fmt<MOE_W_Q4B32>(ga, f.x, max_tiles, has_sh, st);
    case MOE_W_Q2B32: return launch_gemm_fmt<MOE_W_Q2B32>(ga, f.x, max_tiles, has_sh, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_router_mfma(const uint16_t* x, int T, int H, int E, const uint16_t* W,
                              const float* bias, float* logits, hipStream_t st) {
  const int n_et = (E + 127) / 128, n_tt = (T + kBM - 1) / kBM;
  hipLaunchKernelGGL(router_gemm_kernel, dim3(round_xcd(n_tt * n_et)), dim3(256), 0, st, x, T, H, E,
                     W, bias, logits, n_et);
  return hipGetLastError();
}

}  // namespace moe
