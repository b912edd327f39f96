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
// v_fmac_f32 whose multiplicand is read through DPP (own + s * partner, the
// upper lane's result negated; the lane's sign is folded into its output
// scale).
//  * The tile's packed codes (key rows or a coordinate-major value tile, d * bits
//    bytes either way) come in with one 16-byte load per lane, a tile ahead,
//    and go through the wave's LDS slice; each lane then reads the words that
//    hold its coordinates' codes (one per 8 coordinates of a key row; 2 bits
//    words per 8 coordinates of a value tile).
//  * Centroids come from a 16-entry fp32 table in LDS (every lane reads one of
//    16 words: no bank conflicts).
//  * The dithered variant's offset adds the same delta to every centroid; the
//    transform takes a constant vector to d delta at coordinate 0, so it is one
//    add on that coordinate.
//  * D is a sign flip of each output (an xor of the sign bit), after the
//    scale n / sqrt(d).
//  * Memory goes through buffer instructions on per-tile records, with an
//    out-of-range offset for what must not be accessed (a load returns 0, a
//    store is dropped), so each tile issues the same memory instructions and the
//    compiler's waits leave the next tile's loads in flight.
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
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;  // past every record used here
// Non-temporal cache policy (streamed past the caches) for the codes read and
// the rows written, each touched once (C5 K + V 4.41 -> 4.27 ms).
constexpr int kNT = 2;
__device__ __forceinline__ Rsrc record(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);  // raw buffer
}

// One cross-lane butterfly stage on 8 values: a[i] += s * a[i] of the partner
// lane, one v_fmac_f32 with its multiplicand read through DPP (the compiler
// does not fold a DPP move into an FMAC).  A DPP read of a VGPR needs two wait
// states after the VALU write of it, hence the s_nop; inside the block each
// instruction reads a different register.
#define TQ_BUTTERFLY8(NAME, MOD)                                                                    \
  __device__ __forceinline__ void NAME(float* a, float s) {                                       \
    asm volatile("s_nop 1\n\t"                                                                     \
                 "v_fmac_f32_dpp %0, %0, %8 " MOD " row_mask:0xf bank_mask:0xf\n\t"              \
                 "v_fmac_f32_dpp %1, %1, %8 " MOD " row_mask:0xf bank_mask:0xf\n\t"              \
                 "v_fmac_f32_dpp %2, %2, %8 " MOD " row_mask:0xf bank_mask:0xf\n\t"              \
                 "v_fmac_f32_dpp %3, %3, %8 " MOD " row_mask:0xf bank_mask:0xf\n\t"              \
                 "v_fmac_f32_dpp %4, %4, %8 " MOD " row_mask:0xf bank_mask:0xf\n\t"              \
                 "v_fmac_f32_dpp %5, %5, %8 " MOD " row_mask:0xf bank_mask:0xf\n\t"              \
                 "v_fmac_f32_dpp %6, %6, %8 " MOD " row_mask:0xf bank_mask:0xf\n\t"              \
                 "v_fmac_f32_dpp %7, %7, %8 " MOD " row_mask:0xf bank_mask:0xf"                    \
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),         \
                   "+v"(a[6]), "+v"(a[7])                                                          \
                 : "v"(s));                                                                        \
  }
TQ_BUTTERFLY8(butterfly8_xor1, "quad_perm:[1,0,3,2]")
TQ_BUTTERFLY8(butterfly8_xor2, "quad_perm:[2,3,0,1]")
TQ_BUTTERFLY8(butterfly8_xor8, "row_ror:8")
#undef TQ_BUTTERFLY8

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
  constexpr int kOsz = OUT16 ? 2 : 4;   // output bytes per coordinate
  // The wave's tile bytes, with 16 bytes of slack for the two-word reads of bits_at.
  __shared__ __align__(16) uint8_t raw[kWaves][kTileBytes + 16];
  __shared__ float ctab[16];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int k = (lane & 3) | ((lane >> 1) & 4);
  const int tl = ((lane >> 2) & 1) | ((lane >> 3) & 6);
  if (threadIdx.x < 16) ctab[threadIdx.x] = threadIdx.x < (1 << BITS) ? p.cent[threadIdx.x] : 0.f;
  __syncthreads();

  // D as sign-bit masks on the lane's outputs (fp16 pairs or fp32 words).
  constexpr int NM = OUT16 ? V / 2 : V;
  uint32_t dmask[NM];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool neg = p.dsign[8 * k + 64 * c + e] < 0.f;
      if constexpr (OUT16) {
        if (e % 2 == 0) dmask[4 * c + e / 2] = 0u;
        dmask[4 * c + e / 2] |= neg ? (e % 2 ? 0x80000000u : 0x8000u) : 0u;
      } else {
        dmask[8 * c + e] = neg ? 0x80000000u : 0u;
      }
    }
  const float s1 = (lane & 1) ? -1.f : 1.f, s2 = (lane & 2) ? -1.f : 1.f, s8 = (lane & 8) ? -1.f : 1.f;
  const float osc = s1 * s2 * s8 / sqrtf((float)D);  // the lane's transform sign and 1/sqrt(d)
  const float dwidth = DITHER ? *p.dw : 0.f;

  const int64_t items = p.seqs * p.tiles;
  const int64_t wstride = (int64_t)gridDim.x * kWaves;
  const int64_t rowb = D * BITS / 8;
  struct Cursor {
    int64_t item, s, tile;
  };
  const int64_t ds = wstride / p.tiles, dt = wstride % p.tiles;
  auto advance = [&](Cursor& c) {
    c.item += wstride;
    c.s += ds;
    c.tile += dt;
    if (c.tile >= p.tiles) {
      c.tile -= p.tiles;
      c.s += 1;
    }
  };
  struct In {
    u4 codes;  // 16 bytes of the tile's packed codes (lane l: bytes 16 l ..)
    float nn;  // the norm of the lane's token (0 past n)
  };
  const uint32_t coff = 16 * lane < kTileBytes ? 16u * lane : kOob;
  auto load = [&](const Cursor& cu, In& in) {
    const bool live = cu.item < items;  // uniform
    const uint8_t* src = VALUES ? p.idx + (cu.s * (p.cap / 8) + cu.tile) * kTileBytes
                                : p.idx + (cu.s * p.cap + cu.tile * 8) * rowb;
    in.codes = __builtin_amdgcn_raw_buffer_load_b128(record(src, live ? kTileBytes : 0), coff, 0, kNT);
    const int64_t rows = min(p.n - cu.tile * 8, (int64_t)8);
    in.nn = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        record(p.norm + cu.s * p.cap + cu.tile * 8, live ? 4 * rows : 0), 4 * tl, 0, 0));
  };

  auto process = [&](const Cursor& cu, const Cursor& ahead, In& in) {
    __builtin_amdgcn_sched_barrier(0);
    const int64_t s = cu.s, tile = cu.tile;
    // ---- the tile's packed codes into LDS, then the next tile's loads ----
    if (16 * lane < kTileBytes) *reinterpret_cast<u4*>(&raw[w][16 * lane]) = in.codes;
    const float nn = in.nn;
    load(ahead, in);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- centroids of the lane's coordinates ----
    float x[V];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int j0 = 8 * k + 64 * c;
      if constexpr (!VALUES) {
        // 8 consecutive codes of token tl's row, from bit BITS (tl D + j0)
        uint32_t b;
        if constexpr (BITS == 4) b = *reinterpret_cast<const uint32_t*>(&raw[w][(tl * D + j0) / 2]);
        else b = bits_at(raw[w], BITS * (tl * D + j0));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * c + e] = ctab[(b >> (BITS * e)) & kMask];
      } else if constexpr (BITS == 3) {
        // code (j, tl) at bit 3 (8 j + tl) of the tile
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * c + e] = ctab[bits_at(raw[w], 3 * (8 * (j0 + e) + tl)) & kMask];
      } else {
        // codes (j0 .. j0 + 7, t) are the 2 BITS words from byte BITS j0; code
        // (j0 + e, tl) at bit BITS (8 e + tl) of them
        uint32_t wd[2 * BITS];
        const uint32_t* src = reinterpret_cast<const uint32_t*>(&raw[w][BITS * j0]);
#pragma unroll
        for (int q = 0; q < 2 * BITS; ++q) wd[q] = src[q];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int bit = BITS * 8 * e;  // + BITS tl, inside one word
          x[8 * c + e] = ctab[(wd[bit / 32] >> ((bit % 32) + BITS * tl)) & kMask];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();  // raw[w] is rewritten by the next tile

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
    for (int v = 0; v < V; v += 8) butterfly8_xor1(x + v, s1);
#pragma unroll
    for (int v = 0; v < V; v += 8) butterfly8_xor2(x + v, s2);
#pragma unroll
    for (int v = 0; v < V; v += 8) butterfly8_xor8(x + v, s8);
    if constexpr (DITHER) {
      // c[idx] + delta for every coordinate: H takes delta 1 to (d delta, 0, ...)
      const float delta = dither_offset(p.ds0, s, tile * 8 + tl, dwidth);
      if (k == 0) x[0] += (float)D * delta;  // lanes k = 0 hold coordinate 0 with sign +1
    }

    // ---- x_hat = n D H c / sqrt(d): the lane's 8-coordinate pieces of row t ----
    const int64_t rows = min(p.n - tile * 8, (int64_t)8);
    const Rsrc orec = record(static_cast<uint8_t*>(p.out) + (s * p.n + tile * 8) * D * kOsz, rows * D * kOsz);
    const uint32_t ooff = tl < rows ? (uint32_t)((tl * D + 8 * k) * kOsz) : kOob;
    const float m = nn * osc;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (OUT16) {
        u4 h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          const h2 pr = h2{(_Float16)(x[8 * c + 2 * q] * m), (_Float16)(x[8 * c + 2 * q + 1] * m)};
          h[q] = __builtin_bit_cast(uint32_t, pr) ^ dmask[4 * c + q];
        }
        __builtin_amdgcn_raw_buffer_store_b128(h, orec, ooff + 64 * c * kOsz, 0, kNT);
      } else {
        u4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = __float_as_uint(x[8 * c + e] * m) ^ dmask[8 * c + e];
          hi[e] = __float_as_uint(x[8 * c + 4 + e] * m) ^ dmask[8 * c + 4 + e];
        }
        __builtin_amdgcn_raw_buffer_store_b128(lo, orec, ooff + 64 * c * kOsz, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b128(hi, orec, ooff + 64 * c * kOsz + 16, 0, kNT);
      }
    }
  };

  // Two tiles in flight per wave: rounds of two without an exit test inside
  // (so the loop is entered only from above and from its own end), then the
  // last tile if the count is odd.  Dropped stores to an empty record give the
  // path into the loop the same memory count as the loop's own end.
  const int64_t item0 = (int64_t)blockIdx.x * kWaves + w;
  Cursor cur{item0, item0 / p.tiles, item0 % p.tiles};
  Cursor ahead = cur;
  In in[2];
  load(ahead, in[0]);
  advance(ahead);
  load(ahead, in[1]);
  advance(ahead);
  const Rsrc none = record(p.norm, 0);
#pragma unroll
  for (int i = 0; i < 2 * NC * (OUT16 ? 1 : 2) + 4; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 64 * i, 0, 0);
  const int64_t mine = item0 < items ? (items - item0 + wstride - 1) / wstride : 0;
  for (int64_t r = mine / 2; r > 0; --r) {
    process(cur, ahead, in[0]);
    advance(cur);
    advance(ahead);
    process(cur, ahead, in[1]);
    advance(cur);
    advance(ahead);
  }
  if (mine % 2) process(cur, ahead, in[0]);
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
