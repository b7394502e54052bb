// Prefill: the expert FFN as grouped GEMMs on fp16 MFMA, and the router as
// a bf16 MFMA GEMM.
//
// [MD] = ModelDock, "Strata はなぜ少ない VRAM でも速いのか", section
// "長いプロンプトを読む": a long prompt routes to nearly every expert of every
// layer, and an expert's weights are used by every token of the chunk that
// routes to it -- so each expert bucket becomes one GEMM whose weights are
// read once per tile of tokens instead of once per token.
//
// Tiles: 128 rows (tokens of one bucket) x 64 output features x 64 K per
// step, 4 waves of 64 x 32.  gate/up tiles carry the 64 gate rows and the 64
// up rows of the same features, so SwiGLU happens in registers and h leaves
// as fp16; down tiles are 128 x 128 and scatter fp32 rows to pair_out by pair
// id.  Quantised weights are dequantised (d * q + m in fp32, rounded to fp16)
// into LDS one K step ahead; activations bf16 -> fp16 (exact for the
// magnitudes here).  Tiles are ordered so that consecutive tiles of one
// expert run on the same XCD and share its weights in that XCD's L2.
#include "gemv_core.h"
#include "kernels.h"

namespace moe {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;          // rows per tile
constexpr int kBK = 64;           // K per step
constexpr int kLdsRow = kBK + 8;  // halves per LDS row (padding spreads banks)
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  const float lo = __uint_as_float(v << 16), hi = __uint_as_float(v & 0xFFFF0000u);
  const _Float16 a = _Float16(lo), b = _Float16(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
  const _Float16 a = _Float16(lo), b = _Float16(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// One 32-weight block of a quantised row -> 32 fp16 in 4 x u32x4.
template <int FMT>
__device__ __forceinline__ void dequant_block(const uint32_t* codes, uint16_t sb, uint16_t mb,
                                              u32x4* out) {
  const float d = f16_to_f32(sb), m = f16_to_f32(mb);
  float w[32];
  if (FMT == MOE_W_Q4B32) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) w[i * 8 + j] = d * float((codes[i] >> (4 * j)) & 15u) + m;
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) w[i * 16 + j] = d * float((codes[i] >> (2 * j)) & 3u) + m;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    out[q] = u32x4{f32x2_to_f16x2(w[8 * q + 0], w[8 * q + 1]), f32x2_to_f16x2(w[8 * q + 2], w[8 * q + 3]),
                   f32x2_to_f16x2(w[8 * q + 4], w[8 * q + 5]), f32x2_to_f16x2(w[8 * q + 6], w[8 * q + 7])};
}

// Register stage of one K step: this thread's share of the A rows (64 B of
// one row) and of the B rows (one 32-weight block of one row).
template <int FMT>
struct Stage {
  u32x4 a[4];
  uint32_t b[4];      // codes of one block (Q4: 16 B, Q2: 8 B)
  uint16_t bs, bm;    // its scale and min
  u32x4 bw[4];        // bf16 weights (router)
};

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
      cnt = (n + kBM - 1) / kBM;
    }
    int tot;
    const int off = before + block_exclusive_scan(cnt, tmp, &tot);
    for (int i = 0; i < cnt; ++i) tiles[off + i] = make_int2(u, i * kBM);
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
  const uint16_t* x;        // bf16 [T][H]
  int T, k, H, I, fmt;
  MatView g, u, d, sg, su, sd;
  ActiveList act;
  const int32_t* bucket_pair;
  const int2* tiles;
  const int* n_tiles;
  _Float16* h;              // fp16 [n_hit][I] by bucket position
  _Float16* h_sh;           // fp16 [T][I]
  float* pair_out;          // [T*k][H]
  float* shared_out;        // [T][H]
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
    r.rows = min(kBM, n - t.y);
    r.slot = a.act.slot[t.x];
    r.pos0 = st + t.y;
  } else {
    r.rows = min(kBM, a.T - t.y);
    r.slot = 0;
    r.pos0 = t.y;
  }
  return r;
}

// MFMA on one K step from LDS: wave tile = (MT x 32 rows) x (NT x 32 cols).
template <int MT, int NT, bool BF16>
__device__ __forceinline__ void mma_step(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
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
      for (int j = 0; j < NT; ++j) {
        if constexpr (BF16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                              __builtin_bit_cast(bf16x8, bv[j]),
                                                              acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av[i]),
                                                             __builtin_bit_cast(f16x8, bv[j]),
                                                             acc[i][j], 0, 0, 0);
      }
  }
}

// ---------------------------------------------------------------- gate/up
// Tile: 128 rows x 64 features; B rows 0..63 = gate rows n0.., 64..127 = up.
template <int FMT>
__global__ __launch_bounds__(256) void gateup_gemm_kernel(GemmArgs a, int n_ntiles) {
  __shared__ uint16_t As[2][kBM * kLdsRow];
  __shared__ uint16_t Bs[2][128 * kLdsRow];
  __shared__ int tok[kBM];
  const int w = xcd_item();
  const int total = *a.n_tiles * n_ntiles;
  if (w >= total) return;
  const int n_act = *a.act.count;
  const int2 tinfo = a.tiles[w / n_ntiles];
  const int n0 = (w % n_ntiles) * 64;
  const RowMap rm = row_map(a, tinfo, n_act);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kBM) {
    int t = 0;
    if (tid < rm.rows) t = rm.shared ? rm.pos0 + tid : a.bucket_pair[rm.pos0 + tid] / a.k;
    tok[tid] = t;
  }
  __syncthreads();
  const bool up_row = (tid >> 1) >= 64;
  const uint8_t* wcodes = rm.shared ? (up_row ? a.su.codes : a.sg.codes)
                                    : (up_row ? a.u.codes : a.g.codes);
  const uint16_t* wscale = rm.shared ? (up_row ? a.su.scale : a.sg.scale)
                                     : (up_row ? a.u.scale : a.g.scale);
  const uint16_t* wmin = rm.shared ? (up_row ? a.su.mn : a.sg.mn) : (up_row ? a.u.mn : a.g.mn);
  const int64_t mat_bytes = a.g.mat_bytes, mat_blocks = a.g.mat_blocks;
  const int K = a.H;
  const int nk = K / kBK;
  // this thread's A row (64 B) and B row block
  const int ar = tid >> 1, ah = tid & 1;
  const uint16_t* xrow = a.x + int64_t(tok[ar]) * K + ah * 32;
  const int br = tid >> 1, bblk = tid & 1;          // B row 0..127, block 0..1 of the step
  const int wrow = n0 + (br & 63);
  const int64_t blk_base = int64_t(rm.slot) * mat_blocks + int64_t(wrow) * (K / 32);
  const uint8_t* code_row = wcodes + rm.slot * mat_bytes + int64_t(wrow) * (K * fmt_bits(FMT) / 8);
  Stage<FMT> st;
  auto load = [&](int kt) {
    const u32x4* src = reinterpret_cast<const u32x4*>(xrow + kt * kBK);
#pragma unroll
    for (int q = 0; q < 4; ++q) st.a[q] = src[q];
    const int blk = kt * 2 + bblk;
    if (FMT == MOE_W_Q4B32) {
      const u32x4 c = *reinterpret_cast<const u32x4*>(code_row + blk * 16);
      st.b[0] = c[0]; st.b[1] = c[1]; st.b[2] = c[2]; st.b[3] = c[3];
    } else {
      const uint2 c = *reinterpret_cast<const uint2*>(code_row + blk * 8);
      st.b[0] = c.x; st.b[1] = c.y;
    }
    st.bs = wscale[blk_base + blk];
    st.bm = wmin[blk_base + blk];
  };
  auto store = [&](int buf) {
    u32x4* da = reinterpret_cast<u32x4*>(&As[buf][ar * kLdsRow + ah * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      da[q] = u32x4{bf16x2_to_f16x2(st.a[q][0]), bf16x2_to_f16x2(st.a[q][1]),
                    bf16x2_to_f16x2(st.a[q][2]), bf16x2_to_f16x2(st.a[q][3])};
    u32x4 wv[4];
    dequant_block<FMT>(st.b, st.bs, st.bm, wv);
    u32x4* db = reinterpret_cast<u32x4*>(&Bs[buf][br * kLdsRow + bblk * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q) db[q] = wv[q];
  };
  // waves: 2 (rows) x 2 (features); each: 64 rows x (32 gate + 32 up)
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 32;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    mma_step<2, 2, false>(As[kt & 1], Bs[kt & 1], wm, wn, lane, acc, 64);
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }
  // epilogue: h = silu(gate) * up -> fp16
  _Float16* out = rm.shared ? a.h_sh : a.h;
  const int out_row0 = rm.pos0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int col = n0 + wn + (lane & 31);
      if (row < rm.rows) {
        const float g = acc[i][0][v], u = acc[i][1][v];
        out[int64_t(out_row0 + row) * a.I + col] = _Float16(silu_f32(g) * u);
      }
    }
}

// ---------------------------------------------------------------- down
// Tile: 128 rows x 128 output features over K = I.
template <int FMT>
__global__ __launch_bounds__(256) void down_gemm_kernel(GemmArgs a, int n_ntiles) {
  __shared__ uint16_t As[2][kBM * kLdsRow];
  __shared__ uint16_t Bs[2][128 * kLdsRow];
  __shared__ int orow[kBM];
  const int w = xcd_item();
  const int total = *a.n_tiles * n_ntiles;
  if (w >= total) return;
  const int n_act = *a.act.count;
  const int2 tinfo = a.tiles[w / n_ntiles];
  const int n0 = (w % n_ntiles) * 128;
  const RowMap rm = row_map(a, tinfo, n_act);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kBM) {
    int o = -1;
    if (tid < rm.rows) o = rm.shared ? rm.pos0 + tid : a.bucket_pair[rm.pos0 + tid];
    orow[tid] = o;
  }
  __syncthreads();
  const MatView D = rm.shared ? a.sd : a.d;
  const int K = a.I;
  const int nk = K / kBK;
  const int ar = tid >> 1, ah = tid & 1;
  const _Float16* hsrc = rm.shared ? a.h_sh : a.h;
  const int arow = ar < rm.rows ? rm.pos0 + ar : rm.pos0;   // rows past the bucket read a valid row
  const _Float16* hrow = hsrc + int64_t(arow) * K + ah * 32;
  const int br = tid >> 1, bblk = tid & 1;
  const int wrow = n0 + br;
  const int64_t blk_base = int64_t(rm.slot) * D.mat_blocks + int64_t(wrow) * (K / 32);
  const uint8_t* code_row = D.codes + rm.slot * D.mat_bytes + int64_t(wrow) * (K * fmt_bits(FMT) / 8);
  Stage<FMT> st;
  auto load = [&](int kt) {
    const u32x4* src = reinterpret_cast<const u32x4*>(hrow + kt * kBK);
#pragma unroll
    for (int q = 0; q < 4; ++q) st.a[q] = src[q];
    const int blk = kt * 2 + bblk;
    if (FMT == MOE_W_Q4B32) {
      const u32x4 c = *reinterpret_cast<const u32x4*>(code_row + blk * 16);
      st.b[0] = c[0]; st.b[1] = c[1]; st.b[2] = c[2]; st.b[3] = c[3];
    } else {
      const uint2 c = *reinterpret_cast<const uint2*>(code_row + blk * 8);
      st.b[0] = c.x; st.b[1] = c.y;
    }
    st.bs = D.scale[blk_base + blk];
    st.bm = D.mn[blk_base + blk];
  };
  auto store = [&](int buf) {
    u32x4* da = reinterpret_cast<u32x4*>(&As[buf][ar * kLdsRow + ah * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q) da[q] = st.a[q];
    u32x4 wv[4];
    dequant_block<FMT>(st.b, st.bs, st.bm, wv);
    u32x4* db = reinterpret_cast<u32x4*>(&Bs[buf][br * kLdsRow + bblk * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q) db[q] = wv[q];
  };
  // waves 2 x 2, each 64 rows x 64 features
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    mma_step<2, 2, false>(As[kt & 1], Bs[kt & 1], wm, wn, lane, acc, 32);
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }
  float* out = rm.shared ? a.shared_out : a.pair_out;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int col = n0 + wn + j * 32 + (lane & 31);
        if (row < rm.rows) out[int64_t(orow[row]) * a.H + col] = acc[i][j][v];
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
    mma_step<2, 2, true>(As[kt & 1], Bs[kt & 1], wm, wn, lane, acc, 32);
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
hipError_t launch_gemm_fmt(const GemmArgs& ga, int max_tiles, hipStream_t st) {
  const int nt_gu = ga.I / 64, nt_d = ga.H / 128;
  hipLaunchKernelGGL(gateup_gemm_kernel<FMT>, dim3(round_xcd(max_tiles * nt_gu)), dim3(256), 0, st,
                     ga, nt_gu);
  hipLaunchKernelGGL(down_gemm_kernel<FMT>, dim3(round_xcd(max_tiles * nt_d)), dim3(256), 0, st, ga,
                     nt_d);
  return hipGetLastError();
}

}  // namespace

// Workspace: tile list then fp16 h (positions) then fp16 shared h.
size_t ffn_gemm_ws(int T, int k, int H, int I, int S) {
  (void)H;
  const int64_t P = int64_t(T) * k;
  const int64_t max_tiles = P / kBM + (P < S ? P : S) + T / kBM + 2;
  return size_t(max_tiles * 8 + 8) + 256 + size_t(P + T) * I * 2 + 256;
}

bool ffn_gemm_ok(int fmt, int H, int I) {
  return (fmt == MOE_W_Q2B32 || fmt == MOE_W_Q4B32) && H % 128 == 0 && I % 64 == 0;
}

hipError_t launch_ffn_gemm(const FfnArgs& f, int S, const int32_t* bucket_off, void* ws,
                           hipStream_t st) {
  (void)bucket_off;
  const int64_t P = int64_t(f.T) * f.k;
  const int max_tiles = int(P / kBM + (P < S ? P : S) + f.T / kBM + 2);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int* n_tiles = reinterpret_cast<int*>(base);
  int2* tiles = reinterpret_cast<int2*>(base + 8);
  size_t off = (size_t(max_tiles) * 8 + 8 + 255) / 256 * 256;
  _Float16* h = reinterpret_cast<_Float16*>(base + off);
  _Float16* h_sh = h + P * f.I;
  GemmArgs ga;
  ga.x = f.x;
  ga.T = f.T;
  ga.k = f.k;
  ga.H = f.H;
  ga.I = f.I;
  ga.fmt = f.fmt;
  ga.g = f.g; ga.u = f.u; ga.d = f.d;
  ga.sg = f.sg; ga.su = f.su; ga.sd = f.sd;
  ga.act = f.act;
  ga.bucket_pair = f.bucket_pair;
  ga.tiles = tiles;
  ga.n_tiles = n_tiles;
  ga.h = h;
  ga.h_sh = h_sh;
  ga.pair_out = f.pair_out;
  ga.shared_out = f.shared_out;
  const int has_sh = f.sg.codes != nullptr ? 1 : 0;
  hipLaunchKernelGGL(gemm_schedule_kernel, dim3(1), dim3(1024), 0, st, f.act, f.T, has_sh, tiles,
                     n_tiles);
  switch (f.fmt) {
    case MOE_W_Q4B32: return launch_gemm_fmt<MOE_W_Q4B32>(ga, max_tiles, st);
    case MOE_W_Q2B32: return launch_gemm_fmt<MOE_W_Q2B32>(ga, max_tiles, st);
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
