// Per-token offsets of the dithered randomized-Hadamard variant
// (thelatestinai.com paper page 2606.10458, third abstract: HD, then a random
// scalar offset subtracted before quantizing).  One offset per token, the same
// for all its coordinates:
//   delta = width * (u - 1/2),  width = c[L/2] - c[L/2 - 1] of the codebook,
//   u = ((z >> 11) + 1/2) 2^-53,  z = output number seq * 2^32 + t + 1 of the
//   SplitMix64 stream (Steele, Lea and Flood, OOPSLA 2014) that starts at
//   seed XOR (tag * 0xD1B54A32D192ED03), tag 3 for keys and 4 for values.
// Encoder and decoder regenerate it, so nothing is stored.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

constexpr int kDitherTagKeys = 3, kDitherTagValues = 4;

__host__ __device__ inline uint64_t dither_stream_start(uint64_t seed, int tag) {
  return seed ^ ((uint64_t)tag * 0xD1B54A32D192ED03ull);
}

__device__ __forceinline__ float dither_offset(uint64_t s0, int64_t seq, int64_t t, float width) {
  uint64_t z = s0 + (uint64_t)(((uint64_t)seq << 32) + (uint64_t)t + 1u) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  const float u = ((float)(z >> 11) + 0.5f) * 0x1p-53f;
  return width * (u - 0.5f);
}

}  // namespace tq
