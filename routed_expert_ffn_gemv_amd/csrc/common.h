// Device helpers shared by the gfx950 kernels of the routed-MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return float(__builtin_bit_cast(_Float16, b));
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs and fp32 accumulation
// (v_dot2_f32_bf16): products of bf16 values are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Code pairs -> bf16 pairs of (128 + q): OR-ing a code q < 128 into the
// mantissa of bf16(128) = 0x4300 gives 128 + q exactly.
constexpr uint32_t kMagic128x2 = 0x43004300u;

// Two 2-bit codes of a dword, columns s and s + 8 (s in 0..7), as bf16 pair.
__device__ __forceinline__ uint32_t q2_pair(uint32_t w, int s) {
  return ((w >> (2 * s)) & 0x00030003u) | kMagic128x2;
}
// Two 4-bit codes of a dword, columns s and s + 4 (s in 0..3), as bf16 pair.
__device__ __forceinline__ uint32_t q4_pair(uint32_t w, int s) {
  return ((w >> (4 * s)) & 0x000F000Fu) | kMagic128x2;
}

// Order-preserving unsigned image of an fp32 value; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

// Lane v's value moved by a DPP row permutation (every source lane valid).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G lanes (G a power of two, <= 64); every lane
// of the group receives the group sum.  Within a row of 16 lanes the steps
// are DPP permutations (quads, then the other quad of the half row, then
// the other half row); wider groups add lane shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror
  if constexpr (G >= 16) v += dpp_f32<0x140>(v);  // row_mirror
#pragma unroll
  for (int m = 16; m < G; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    uint64_t o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024,
// multiple of 64).  `tmp` is __shared__ int[32].  Returns the exclusive
// prefix; *total receives the block total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int s = lane < nw ? tmp[lane] : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      int y = __shfl_up(s, d, kWave);
      if (lane >= d) s += y;
    }
    if (lane < nw) tmp[lane] = s;
  }
  __syncthreads();
  const int before = wid > 0 ? tmp[wid - 1] : 0;
  if (total) *total = tmp[nw - 1];
  __syncthreads();
  return before + x - v;
}

// Byte offsets / element offsets of slot s in a matrix pool.
struct MatView {
  const uint8_t* codes;   // Q formats: codes; F32: fp32 data as bytes
  const uint16_t* scale;
  const uint16_t* mn;
  int64_t mat_bytes;      // bytes of one matrix's data plane
  int64_t mat_blocks;     // blocks of one matrix (Q formats)
};

__host__ __device__ inline int fmt_bits(int fmt) {
  return fmt == MOE_W_Q2B32 ? 2 : fmt == MOE_W_Q4B32 ? 4 : fmt == MOE_W_BF16 ? 16 : 32;
}

inline MatView make_view(const moe_mat& m, int rows, int cols) {
  MatView v;
  v.codes = static_cast<const uint8_t*>(m.data);
  v.scale = m.scale;
  v.mn = m.min;
  v.mat_bytes = int64_t(rows) * cols * fmt_bits(m.fmt) / 8;
  v.mat_blocks = int64_t(rows) * cols / 32;
  return v;
}

}  // namespace moe
