// Dequant-fused GEMV building blocks shared by the decode kernels.
//
// Each lane owns 16-byte chunks of a weight row (64 2-bit or 32 4-bit codes,
// or 4 fp32 weights), LPR lanes share a row, and the input vectors sit in
// LDS in the order the codes unpack into.  Codes become exact bf16 pairs
// (128 + q) with one shift and one and-or; v_dot2_f32_bf16 multiplies them
// with bf16 activation pairs and the 128 offset folds into the block's min:
//   sum_c (d q_c + m) x_c = d * sum_c (128 + q_c) x_c + (m - 128 d) * S_b,
// S_b = sum of the block's 32 inputs, precomputed when a vector is staged.
// fp32 inputs (the SwiGLU output h) enter as two bf16 vectors hi + lo
// (h - hi rounded again), which together carry 16 significant bits.
#pragma once

#include "common.h"

namespace moe {

template <int FMT>
struct Fmt;
template <>
struct Fmt<MOE_W_Q2B32> {
  static constexpr int kWPC = 64;   // weights per 16-byte chunk
  static constexpr int kCS = 36;    // LDS dwords per chunk (32 + 4 padding)
};
template <>
struct Fmt<MOE_W_Q4B32> {
  static constexpr int kWPC = 32;
  static constexpr int kCS = 20;    // 16 + 4 padding
};
template <>
struct Fmt<MOE_W_F32> {
  static constexpr int kWPC = 4;
  static constexpr int kCS = 4;     // 4 floats
};

// LDS dword holding the bf16 pair of columns (c, partner(c)) for column c
// with c < partner(c).  Q2: pairs (16g+s, 16g+s+8); Q4: (8g+s, 8g+s+4).
template <int FMT>
__device__ __forceinline__ int pair_slot(int c) {
  if (FMT == MOE_W_Q2B32) {
    const int chunk = c >> 6, g = (c >> 4) & 3, s = c & 7;
    return chunk * Fmt<FMT>::kCS + g * 8 + s;
  } else {
    const int chunk = c >> 5, g = (c >> 3) & 3, s = c & 3;
    return chunk * Fmt<FMT>::kCS + g * 4 + s;
  }
}
template <int FMT>
__device__ __forceinline__ int partner_offset() {
  return FMT == MOE_W_Q2B32 ? 8 : 4;
}
// the lower column of a pair slot index within the row (inverse of pair_slot)
template <int FMT>
__device__ __forceinline__ bool slot_low_column(int dw, int* c) {
  const int chunk = dw / Fmt<FMT>::kCS, r = dw % Fmt<FMT>::kCS;
  if (FMT == MOE_W_Q2B32) {
    if (r >= 32) return false;
    *c = chunk * 64 + (r >> 3) * 16 + (r & 7);
  } else {
    if (r >= 16) return false;
    *c = chunk * 32 + (r >> 2) * 8 + (r & 3);
  }
  return true;
}

// Stage one bf16 activation row of K values for format FMT.
template <int FMT>
__device__ __forceinline__ void stage_bf16(uint32_t* vec, float* sums, const uint16_t* src, int K) {
  if (FMT == MOE_W_F32) {
    float* vf = reinterpret_cast<float*>(vec);
    for (int c = threadIdx.x; c < K; c += blockDim.x) vf[c] = bf16_to_f32(src[c]);
  } else {
    const int ndw = (K / Fmt<FMT>::kWPC) * Fmt<FMT>::kCS;
    for (int dw = threadIdx.x; dw < ndw; dw += blockDim.x) {
      int c;
      if (slot_low_column<FMT>(dw, &c))
        vec[dw] = uint32_t(src[c]) | (uint32_t(src[c + partner_offset<FMT>()]) << 16);
    }
    for (int b = threadIdx.x; b < K / 32; b += blockDim.x) {
      float s = 0.f;
      for (int c = 0; c < 32; ++c) s += bf16_to_f32(src[32 * b + c]);
      sums[b] = s;
    }
  }
}

// fp32 load; kCoherent reads at device scope (bypassing the per-XCD L2),
// for data another workgroup of the same launch wrote.
template <bool kCoherent>
__device__ __forceinline__ float load_f32(const float* p) {
  if (kCoherent) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

// Stage one fp32 row (h) as bf16 hi and lo vectors (Q formats) or as fp32.
template <int FMT, bool kCoherent = false>
__device__ __forceinline__ void stage_f32(uint32_t* vhi, float* shi, uint32_t* vlo, float* slo,
                                          const float* src, int K) {
  if (FMT == MOE_W_F32) {
    float* vf = reinterpret_cast<float*>(vhi);
    for (int c = threadIdx.x; c < K; c += blockDim.x) vf[c] = load_f32<kCoherent>(src + c);
  } else {
    const int ndw = (K / Fmt<FMT>::kWPC) * Fmt<FMT>::kCS;
    for (int dw = threadIdx.x; dw < ndw; dw += blockDim.x) {
      int c;
      if (slot_low_column<FMT>(dw, &c)) {
        const float a = load_f32<kCoherent>(src + c);
        const float b = load_f32<kCoherent>(src + c + partner_offset<FMT>());
        const uint32_t ah = f32_to_bf16_bits(a), bh = f32_to_bf16_bits(b);
        const uint32_t al = f32_to_bf16_bits(a - bf16_to_f32(ah));
        const uint32_t bl = f32_to_bf16_bits(b - bf16_to_f32(bh));
        vhi[dw] = ah | (bh << 16);
        vlo[dw] = al | (bl << 16);
      }
    }
    for (int b = threadIdx.x; b < K / 32; b += blockDim.x) {
      float sh = 0.f, sl = 0.f;
      for (int c = 0; c < 32; ++c) {
        const float v = load_f32<kCoherent>(src + 32 * b + c);
        const float hi = bf16_to_f32(f32_to_bf16_bits(v));
        sh += hi;
        sl += bf16_to_f32(f32_to_bf16_bits(v - hi));
      }
      shi[b] = sh;
      slo[b] = sl;
    }
  }
}

// acc[v] += sum over this lane's chunks of one weight row times vector v,
// for v < n.  Vector v lives at vec + id(v) * vstride (sums likewise), with
// id(v) = vid[v] when vid is given, else v.
template <int FMT, int NV>
__device__ __forceinline__ void row_dot(const uint8_t* __restrict__ codes,
                                        const uint16_t* __restrict__ sc,
                                        const uint16_t* __restrict__ mn, int chunks, int lane_g,
                                        int lpr, const uint32_t* vec, int vstride,
                                        const float* sums, int sstride, int n, float (&acc)[NV],
                                        const int* vid = nullptr) {
  for (int c = lane_g; c < chunks; c += lpr) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(codes + 16 * c);
    if constexpr (FMT == MOE_W_Q2B32) {
      const uint32_t dd = *reinterpret_cast<const uint32_t*>(sc + 2 * c);
      const uint32_t mm = *reinterpret_cast<const uint32_t*>(mn + 2 * c);
      const float d0 = f16_to_f32(uint16_t(dd & 0xFFFFu)), d1 = f16_to_f32(uint16_t(dd >> 16));
      const float m0 = f16_to_f32(uint16_t(mm & 0xFFFFu)) - 128.f * d0;
      const float m1 = f16_to_f32(uint16_t(mm >> 16)) - 128.f * d1;
      uint32_t pr[32];
#pragma unroll
      for (int dw = 0; dw < 4; ++dw)
#pragma unroll
        for (int s = 0; s < 8; ++s) pr[dw * 8 + s] = q2_pair(w[dw], s);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if (v < n) {
          const int id = vid ? vid[v] : v;
          const u32x4* xv = reinterpret_cast<const u32x4*>(vec + id * vstride + c * Fmt<FMT>::kCS);
          float p0 = 0.f, p1 = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 xx = xv[q];
            p0 = dot2_bf16(pr[q * 4 + 0], xx[0], p0);
            p0 = dot2_bf16(pr[q * 4 + 1], xx[1], p0);
            p0 = dot2_bf16(pr[q * 4 + 2], xx[2], p0);
            p0 = dot2_bf16(pr[q * 4 + 3], xx[3], p0);
          }
#pragma unroll
          for (int q = 4; q < 8; ++q) {
            const u32x4 xx = xv[q];
            p1 = dot2_bf16(pr[q * 4 + 0], xx[0], p1);
            p1 = dot2_bf16(pr[q * 4 + 1], xx[1], p1);
            p1 = dot2_bf16(pr[q * 4 + 2], xx[2], p1);
            p1 = dot2_bf16(pr[q * 4 + 3], xx[3], p1);
          }
          const float* sv = sums + id * sstride + 2 * c;
          acc[v] += d0 * p0 + m0 * sv[0] + d1 * p1 + m1 * sv[1];
        }
      }
    } else if constexpr (FMT == MOE_W_Q4B32) {
      const float d = f16_to_f32(sc[c]);
      const float m = f16_to_f32(mn[c]) - 128.f * d;
      uint32_t pr[16];
#pragma unroll
      for (int dw = 0; dw < 4; ++dw)
#pragma unroll
        for (int s = 0; s < 4; ++s) pr[dw * 4 + s] = q4_pair(w[dw], s);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if (v < n) {
          const int id = vid ? vid[v] : v;
          const u32x4* xv = reinterpret_cast<const u32x4*>(vec + id * vstride + c * Fmt<FMT>::kCS);
          float p = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 xx = xv[q];
            p = dot2_bf16(pr[q * 4 + 0], xx[0], p);
            p = dot2_bf16(pr[q * 4 + 1], xx[1], p);
            p = dot2_bf16(pr[q * 4 + 2], xx[2], p);
            p = dot2_bf16(pr[q * 4 + 3], xx[3], p);
          }
          acc[v] += d * p + m * sums[id * sstride + c];
        }
      }
    } else {
      const float4 wf = __builtin_bit_cast(float4, w);
      const float* vf = reinterpret_cast<const float*>(vec);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if (v < n) {
          const float* xv = vf + (vid ? vid[v] : v) * vstride + 4 * c;
          acc[v] = fmaf(wf.x, xv[0], fmaf(wf.y, xv[1], fmaf(wf.z, xv[2], fmaf(wf.w, xv[3], acc[v]))));
        }
      }
    }
  }
}

template <int FMT>
__host__ __device__ inline int chunks_per_row(int K) {
  return K / Fmt<FMT>::kWPC;
}
template <int FMT>
__host__ __device__ inline int vec_dwords(int K) {
  return chunks_per_row<FMT>(K) * Fmt<FMT>::kCS;
}

}  // namespace moe
