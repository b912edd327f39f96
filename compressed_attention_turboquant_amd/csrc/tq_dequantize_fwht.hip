// Dequantize for the randomized Hadamard rotation (gfx950, vector ALU):
//   x_hat = n * (H D)^T c[idx] = n * D H c[idx]
// ([cuTile] listing, decompression function: codes -> centroids -> inverse
// rotation -> rescale; [Mobilint] "How JL Matrices Evolved" for H D with a
// normalised Sylvester H, which is its own inverse).  The inverse rotation is a
// fast Walsh-Hadamard transform: d log2(d) adds per row in fp32 instead of
// the d^2 multiply-adds of a general rotation, so the kernel is bound by HBM
// (d * bits / 8 bytes and a norm in, d outputs out per row).  The dithered
// variant reconstructs c[idx] + delta before the transform.
//
// Mapping to CDNA4 (one 64-lane wave per 8-token tile), the lane layout of the
// transform quantizer: lane l works on token t = (l>>2 & 1) | (l>>3 & 6) and
// holds the coordinates j = 8k + 64c + e (e < 8, c < d/64) with
// k = (l & 3) | (l>>1 & 4); index bits 0-2 and 6-7 of j live in registers,
// bits 3, 4 and 5 in lane bits 0, 1 and 3, so every cross-lane butterfly is one
// DPP move plus one FMA with a +-1 factor.
//  * The tile's packed codes (key rows or a coordinate-major value tile, d * bits
//    bytes either way) come in with 16-byte loads into the wave's LDS slice; each
//    lane then extracts the codes of its coordinates.
//  * Centroids come from a 16-entry fp32 table in LDS (every lane reads one of
//    16 words: no bank conflicts).
//  * Each lane stores its 8-coordinate chunks of the output row as 16- or
//    32-byte pieces.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <type_traits>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// DPP controls (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppXor8 = 0x128; // row_ror:8 (within a row of 16 lanes: lane ^ 8)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

struct FwhtDequantParams {
  const uint8_t* idx;
  const float* norm;
  int64_t seqs, n, cap, tiles;
  const float *dsign, *cent;
  void* out;
  uint64_t ds0;       // dithered variant: offset stream and width
  const float* dw;
};

// 32 bits of the little-endian byte string at LDS address base, starting at bit b.
__device__ __forceinline__ uint32_t bits_at(const uint8_t* base, int b) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(base) + (b >> 5);
  return __builtin_amdgcn_alignbit(w[1], w[0], b & 31);
}

template <int D, int BITS, int VALUES, int OUT16, int DITHER>
__global__ void __launch_bounds__(kThreads) dequant_fwht_kernel(FwhtDequantParams p) {
  constexpr int NC = D / 64, V = 8 * NC;
  constexpr int kTileBytes = D * BITS;  // packed codes of 8 tokens, either layout
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  // The wave's tile bytes, with 8 bytes of slack for the two-word reads of bits_at.
  __shared__ __align__(16) uint8_t raw[kWaves][kTileBytes + 16];
  __shared__ float ctab[16];

  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int k = (lane & 3) | ((lane >> 1) & 4);
  const int tl = ((lane >> 2) & 1) | ((lane >> 3) & 6);
  if (threadIdx.x < 16) ctab[threadIdx.x] = threadIdx.x < (1 << BITS) ? p.cent[threadIdx.x] : 0.f;
  __syncthreads();

  // Per lane coordinate factors D_j / sqrt(d).
  float dsc[V];
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) dsc[8 * c + e] = p.dsign[8 * k + 64 * c + e] * inv_sqrt_d;
  const float s1 = (lane & 1) ? -1.f : 1.f, s2 = (lane & 2) ? -1.f : 1.f, s8 = (lane & 8) ? -1.f : 1.f;
  const float dwidth = DITHER ? *p.dw : 0.f;

  const int64_t items = p.seqs * p.tiles;
  const int64_t wstride = (int64_t)gridDim.x * kWaves;
  const int64_t rowb = D * BITS / 8;
  for (int64_t item = (int64_t)blockIdx.x * kWaves + w; item < items; item += wstride) {
    const int64_t s = item / p.tiles, tile = item % p.tiles;
    // ---- the tile's packed codes into LDS ----
    const uint8_t* src = VALUES ? p.idx + (s * (p.cap / 8) + tile) * kTileBytes
                                : p.idx + (s * p.cap + tile * 8) * rowb;
#pragma unroll
    for (int o = 16 * lane; o < kTileBytes; o += 1024)
      *reinterpret_cast<u4*>(&raw[w][o]) = *reinterpret_cast<const u4*>(src + o);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int64_t t = tile * 8 + tl;
    const float delta = DITHER ? dither_offset(p.ds0, s, t, dwidth) : 0.f;
    // ---- centroids of the lane's coordinates ----
    float x[V];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int j0 = 8 * k + 64 * c;
      if constexpr (!VALUES) {
        // 8 consecutive codes of token tl's row, from bit BITS (tl D + j0)
        const uint32_t b = bits_at(raw[w], BITS * (tl * D + j0));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * c + e] = ctab[(b >> (BITS * e)) & kMask] + delta;
      } else {
        // code (j, tl) at bit BITS (8 j + tl) of the tile
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t b = bits_at(raw[w], BITS * (8 * (j0 + e) + tl));
          x[8 * c + e] = ctab[b & kMask] + delta;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();  // raw[w] is rewritten by the next item

    // ---- unnormalised Walsh-Hadamard transform: register bits, then lane bits ----
#pragma unroll
    for (int bb = 1; bb < V; bb <<= 1) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if (v & bb) continue;
        const float u = x[v], z = x[v + bb];
        x[v] = u + z;
        x[v + bb] = u - z;
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = fmaf(s1, x[v], dpp<kDppXor1>(x[v]));
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = fmaf(s2, x[v], dpp<kDppXor2>(x[v]));
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = fmaf(s8, x[v], dpp<kDppXor8>(x[v]));

    // ---- x_hat = n D H c / sqrt(d); the lane's 8-coordinate pieces of row t ----
    if (t < p.n) {
      const float nn = p.norm[s * p.cap + t];
      const int64_t o = (s * p.n + t) * D + 8 * k;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[8 * c + e] * (nn * dsc[8 * c + e]);
        if constexpr (OUT16) {
          u4 h;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const _Float16 a = (_Float16)y[2 * q], bh = (_Float16)y[2 * q + 1];
            h[q] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, bh) << 16);
          }
          *reinterpret_cast<u4*>(static_cast<__half*>(p.out) + o + 64 * c) = h;
        } else {
          f4* dst = reinterpret_cast<f4*>(static_cast<float*>(p.out) + o + 64 * c);
          dst[0] = f4{y[0], y[1], y[2], y[3]};
          dst[1] = f4{y[4], y[5], y[6], y[7]};
        }
      }
    }
  }
}

template <int D, int BITS, int VALUES, int OUT16>
hipError_t launch(const FwhtDequantParams& p, int dither, unsigned grid, hipStream_t st) {
  if (dither)
    hipLaunchKernelGGL((dequant_fwht_kernel<D, BITS, VALUES, OUT16, 1>), dim3(grid), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((dequant_fwht_kernel<D, BITS, VALUES, OUT16, 0>), dim3(grid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t dispatch_layout(const FwhtDequantParams& p, const DequantArgs& a, unsigned grid, hipStream_t st) {
  const bool h = a.out_dtype == TQ_F16;
  if (a.value_layout)
    return h ? launch<D, BITS, 1, 1>(p, a.dither, grid, st) : launch<D, BITS, 1, 0>(p, a.dither, grid, st);
  return h ? launch<D, BITS, 0, 1>(p, a.dither, grid, st) : launch<D, BITS, 0, 0>(p, a.dither, grid, st);
}

template <int D>
hipError_t dispatch_bits(const FwhtDequantParams& p, const DequantArgs& a, unsigned grid, hipStream_t st) {
  switch (a.bits) {
    case 1: return dispatch_layout<D, 1>(p, a, grid, st);
    case 2: return dispatch_layout<D, 2>(p, a, grid, st);
    case 3: return dispatch_layout<D, 3>(p, a, grid, st);
    default: return dispatch_layout<D, 4>(p, a, grid, st);
  }
}

}  // namespace

hipError_t launch_dequant_fwht(const DequantArgs& a, hipStream_t st) {
  if (a.n == 0 || a.seqs == 0) return hipSuccess;
  FwhtDequantParams p{};
  p.idx = a.idx;
  p.norm = a.norm;
  p.seqs = a.seqs;
  p.n = a.n;
  p.cap = a.cap;
  p.tiles = (a.n + 7) / 8;
  p.dsign = a.dsign;
  p.cent = a.cent;
  p.out = a.out;
  p.ds0 = a.dither_s0;
  p.dw = a.dither_w;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int64_t items = p.seqs * p.tiles;
  int64_t grid = (items + kWaves - 1) / kWaves;
  if (grid > (int64_t)cus * 8) grid = (int64_t)cus * 8;
  switch (a.d) {
    case 64: return dispatch_bits<64>(p, a, (unsigned)grid, st);
    case 128: return dispatch_bits<128>(p, a, (unsigned)grid, st);
    default: return dispatch_bits<256>(p, a, (unsigned)grid, st);
  }
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t st) {
  return a.rot == TQ_ROT_HADAMARD ? launch_dequant_fwht(a, st) : launch_dequant_mfma(a, st);
}

}  // namespace tq
