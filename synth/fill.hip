// GPU fill of the synthetic packed expert planes.
//
// Reproduces, byte for byte, the integer-only planes that synth/__init__.py
// draws on the host (packed codes, fp16 scale and fp16 min per 32-weight
// block), so that tens of GB of expert weights can be created in HBM in
// milliseconds.  Pure counter-based hashing: no part of the MoE layer's
// arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t stream_key(uint64_t seed, uint64_t tag,
                                               uint64_t layer, uint64_t idx) {
  uint64_t k = mix64(seed);
  k = mix64(k ^ tag);
  k = mix64(k ^ layer);
  return mix64(k ^ idx);
}

// fp16 bits of N * 2^-14 for N in [512, 2048).
__device__ __forceinline__ uint16_t f16_of_int(int64_t N) {
  int p = N >= 1024 ? 10 : 9;
  int64_t expo = p + 1;
  int64_t mant = (N - (int64_t(1) << p)) << (10 - p);
  return uint16_t((expo << 10) | mant);
}

__global__ void fill_codes(uint64_t seed, int matrix, int64_t words_per_slot,
                           const int32_t* slot_layer, const int32_t* slot_expert,
                           uint64_t* codes) {
  const int s = blockIdx.y;
  const uint64_t tag = 16 + 4 * matrix + 0;
  const uint64_t k = stream_key(seed, tag, uint64_t(int64_t(slot_layer[s])),
                                uint64_t(int64_t(slot_expert[s])));
  uint64_t* dst = codes + int64_t(s) * words_per_slot;
  for (int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; n < words_per_slot;
       n += int64_t(gridDim.x) * blockDim.x)
    dst[n] = mix64(k + uint64_t(n + 1) * kGolden);
}

__global__ void fill_blocks(uint64_t seed, int matrix, int bits, int64_t blocks_per_slot,
                            const int32_t* slot_layer, const int32_t* slot_expert,
                            uint16_t* scale, uint16_t* mn) {
  const int s = blockIdx.y;
  const uint64_t tag = 16 + 4 * matrix + 1;
  const uint64_t k = stream_key(seed, tag, uint64_t(int64_t(slot_layer[s])),
                                uint64_t(int64_t(slot_expert[s])));
  uint16_t* d = scale + int64_t(s) * blocks_per_slot;
  uint16_t* m = mn + int64_t(s) * blocks_per_slot;
  for (int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; n < blocks_per_slot;
       n += int64_t(gridDim.x) * blockDim.x) {
    const uint64_t w = mix64(k + uint64_t(n + 1) * kGolden);
    const int64_t v = int64_t((w >> 32) % 33ull) - 16;
    if (bits == 2) {
      const int64_t u = int64_t(w & 0xFFull);
      d[n] = uint16_t((10 << 10) | (u << 2));
      m[n] = uint16_t(f16_of_int(768 + 3 * u + v) | 0x8000u);
    } else {
      const int64_t u = int64_t(w & 0x3Full);
      d[n] = uint16_t((8 << 10) | (u << 4));
      m[n] = uint16_t(f16_of_int(960 + 15 * u + v) | 0x8000u);
    }
  }
}

}  // namespace

// Fill S slots of one quantised matrix pool.  matrix: 0 gate, 1 up, 2 down;
// bits 2 or 4; the matrix is [rows][cols] with cols a multiple of 32.
// slot_layer / slot_expert: device int32 [S].  codes: device [S][rows*cols*bits/8]
// bytes (8-byte aligned); scale, mn: device fp16 bits [S][rows*cols/32].
// Returns 0, or a hipError_t / -1 for invalid arguments.
extern "C" int synth_fill_q(uint64_t seed, int matrix, int bits, int rows, int cols,
                            int reserved, const int32_t* slot_layer,
                            const int32_t* slot_expert, int S, void* codes,
                            void* scale, void* mn, hipStream_t stream) {
  (void)reserved;
  if ((bits != 2 && bits != 4) || matrix < 0 || matrix > 2 || rows <= 0 || cols <= 0 ||
      cols % 32 != 0 || S < 0 || S > 65535)
    return -1;
  if (S == 0) return 0;
  if (!slot_layer || !slot_expert || !codes || !scale || !mn) return -1;
  if (reinterpret_cast<uintptr_t>(codes) % 8 != 0) return -1;
  const int64_t words = int64_t(rows) * cols * bits / 64;
  const int64_t blocks = int64_t(rows) * cols / 32;
  dim3 g1(unsigned((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024), unsigned(S));
  hipLaunchKernelGGL(fill_codes, g1, dim3(256), 0, stream, seed, matrix, words, slot_layer,
                     slot_expert, static_cast<uint64_t*>(codes));
  dim3 g2(unsigned((blocks + 255) / 256 < 1024 ? (blocks + 255) / 256 : 1024), unsigned(S));
  hipLaunchKernelGGL(fill_blocks, g2, dim3(256), 0, stream, seed, matrix, bits, blocks,
                     slot_layer, slot_expert, static_cast<uint16_t*>(scale),
                     static_cast<uint16_t*>(mn));
  return int(hipGetLastError());
}
