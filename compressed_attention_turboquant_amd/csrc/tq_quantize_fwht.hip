// Key/value compression with the randomized Hadamard rotation, without QJL
// (gfx950, vector ALU).
//
// Per token x ([Mobilint] "How JL Matrices Evolved": the rotation H D with a
// normalised Sylvester H and random signs D; "Designing the Optimal Codebook
// Without Data" and "TurboQuant: Theoretical Optimality via Scalar
// Quantization" for the scalar quantizer):
//   n = ||x||;  y = H (D x) / n  (H with entries +-1/sqrt(d));
//   idx_j = #{i : beta_i < y_j};  pack idx.
// The rotation is a fast Walsh-Hadamard transform: d log2(d) adds per row,
// no matrix multiply, so the kernel is bound by HBM (d fp16 in, d*b/8 bytes +
// a norm out per row).
//
// Mapping to CDNA4 (one 64-lane wave per 8-token tile):
//  * Lane l works on token t = (l>>2 & 1) | (l>>3 & 6) of the tile and holds the
//    coordinates j = 8k + 64c + e (e < 8, c < d/64) with k = (l & 3) | (l>>1 & 4):
//    8 lanes share a token.  Index bits 0-2 and 6-7 of j live in registers,
//    bits 3, 4 and 5 in lane bits 0, 1 and 3, so every cross-lane butterfly is
//    one FMA whose multiplicand is read through DPP (quad_perm for lane xor 1
//    and 2, row_ror:8 for lane xor 8): own + s * partner with s = -1 on the
//    upper lane, which yields the upper output negated.  The negation is the
//    same for all of a lane's values, so it is carried as one sign per lane
//    (the product of its three s) and applied where the codes are taken.
//  * 3- and 4-bit codes come from a binned table in LDS instead of a search:
//    the coordinate on the codebook's N(0, 1) scale is cut into bins narrower
//    than any gap between boundaries, each bin holding the count of
//    boundaries below it and its own boundary, if any, so a code is one
//    lookup and one compare.
//  * Each chunk of 8 coordinates is one 16-byte load of fp16 input (a token's
//    8 lanes read 128 contiguous bytes per load).
//  * Codes go through LDS as bytes ([token][coordinate]) and leave as whole
//    dwords: keys as 32-coordinate pieces of a token's stream, values as
//    4-coordinate x 8-token pieces of the tile's coordinate-major stream.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <type_traits>

#include "tq_kernels.h"
#include "tq_quant_common.h"

namespace tq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Code table: kBins bins of width 1 / kBinScale on the codebook's N(0, 1) scale
// z = y sqrt(d) (y a coordinate of the unit vector), centred on 0, so they
// cover |z| < 4; the bins outside hold no boundary (the outermost boundary of
// the 4-bit codebooks is below 2.5), so values beyond them clamp to the end
// bins.  Every codebook's boundaries are more than one bin apart (the
// narrowest gap is about 0.25), so a bin holds at most one.  32 copies, one
// per lane of a half wave, keep the lookups free of bank conflicts.
constexpr int kBins = 64;
constexpr float kBinScale = 8.f;
constexpr int kBinCopies = 32;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// DPP controls (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppXor8 = 0x128; // row_ror:8 (within a row of 16 lanes: lane ^ 8)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
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

// BITS consecutive dwords to a 4-byte aligned address (16-byte aligned when
// BITS is 4), as one vector store.
template <int BITS>
__device__ __forceinline__ void store_words(uint8_t* dst, const uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    *reinterpret_cast<u4*>(dst) = u4{w[0], w[1], w[2], w[3]};
  } else if constexpr (BITS == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int q = 0; q < BITS; ++q) reinterpret_cast<uint32_t*>(dst)[q] = w[q];
  }
}

// Bytes per LDS code row: a multiple of 16 words plus 16 (mod 64 words), so the
// 8-byte writes of the 32 lanes of a half wave fall in distinct banks.
template <int D>
constexpr int lds_row() { return (D / 4) % 32 == 0 ? D + 64 : D; }

struct FwhtParams {
  const void* x;
  int64_t seqs, n, t0, cap;
  int64_t tile_first, tiles;  // tiles touched per sequence
  const float *dsign, *bnd;
  uint8_t* idx;
  float* norm;
  uint64_t ds0;       // dithered variant: offset stream and width
  const float* dw;
};

// DITHER: the dithered variant, codes of y - delta for the token's offset delta.
template <int D, int BITS, int VALUES, typename Tin, int DITHER>
__global__ void __launch_bounds__(kThreads) quantize_fwht_kernel(FwhtParams p) {
  constexpr int NC = D / 64, V = 8 * NC, ROW = lds_row<D>();
  constexpr int K = BITS > 1 ? (1 << (BITS - 1)) - 1 : 1;  // positive boundaries (array size)
  constexpr bool kHalf = std::is_same<Tin, _Float16>::value;
  constexpr int RW = kHalf ? 4 : 8;  // dwords per chunk of 8 inputs
  typedef uint32_t Raw __attribute__((ext_vector_type(RW)));
  constexpr bool kTable = BITS >= 3;
  __shared__ __align__(16) uint8_t codes[kWaves][8][ROW];
  __shared__ __align__(16) uint2 ctab[kTable ? kBins * kBinCopies : 1];  // {boundary in bin units, count below}

  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int k = (lane & 3) | ((lane >> 1) & 4);
  const int tl = ((lane >> 2) & 1) | ((lane >> 3) & 6);

  // D as sign-bit masks on the raw input words of this lane's coordinates.
  Raw dm[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      if constexpr (kHalf) {
        const float* sg = p.dsign + 8 * k + 64 * c + 2 * q;
        dm[c][q] = (sg[0] < 0.f ? 0x8000u : 0u) | (sg[1] < 0.f ? 0x80000000u : 0u);
      } else {
        dm[c][q] = p.dsign[8 * k + 64 * c + q] < 0.f ? 0x80000000u : 0u;
      }
    }
  // +1 where this lane is the lower partner of a cross-lane butterfly; the
  // lane's transform outputs come out multiplied by sgn = s1 s2 s8.
  const float s1 = (lane & 1) ? -1.f : 1.f, s2 = (lane & 2) ? -1.f : 1.f, s8 = (lane & 8) ? -1.f : 1.f;
  const float sgn = s1 * s2 * s8;
  float beta[K];
#pragma unroll
  for (int i = 0; i < K; ++i) beta[i] = BITS > 1 ? p.bnd[(1 << (BITS - 1)) + i] : 0.f;
  const float sqrt_d = sqrtf((float)D);
  // Boundary b in bin units: u = z kBinScale + kBins / 2 with z = b sqrt(d).
  const float ubin = sqrt_d * kBinScale;
  if constexpr (kTable) {
    constexpr int L = 1 << BITS;
    for (int e = threadIdx.x; e < kBins * kBinCopies; e += kThreads) {
      const int bin = e / kBinCopies;
      uint32_t below = 0;
      float inner = INFINITY;
      for (int i = 0; i + 1 < L; ++i) {
        const float ub = fmaf(p.bnd[i], ubin, 0.5f * kBins);
        if (ub < (float)bin) ++below;
        else if (ub < (float)(bin + 1)) inner = ub;
      }
      ctab[e] = make_uint2(__float_as_uint(inner), below);
    }
    __syncthreads();
  }
  const uint2* ctab_lane = ctab + (kTable ? lane % kBinCopies : 0);
  const float dwidth = DITHER ? *p.dw : 0.f;

  const int64_t items = p.seqs * p.tiles;
  const int64_t wstride = (int64_t)gridDim.x * kWaves;
  const int64_t t0 = p.t0, tend = p.t0 + p.n;
  constexpr int kRowB = D * BITS / 8;  // key stream bytes per token
  const bool small = items <= 0x7FFFFFFF;
  auto split = [&](int64_t item, int64_t& s, int64_t& tile) {  // item -> (sequence, tile), uniform
    if (small) {
      const uint32_t q = (uint32_t)item / (uint32_t)p.tiles;
      s = q;
      tile = p.tile_first + ((uint32_t)item - q * (uint32_t)p.tiles);
    } else {
      s = item / p.tiles;
      tile = p.tile_first + item % p.tiles;
    }
  };
  const int lane_off = tl * D + 8 * k;  // this lane's first input, relative to the tile's first row
  auto load = [&](int64_t item, Raw (&raw)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] = Raw{};
    if (item >= items) return;
    int64_t s, tile;
    split(item, s, tile);
    const int64_t t = tile * 8 + tl;
    if (t < t0 || t >= tend) return;
    const Tin* src = static_cast<const Tin*>(p.x) + (s * p.n + tile * 8 - t0) * D + lane_off;
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] = *reinterpret_cast<const Raw*>(src + 64 * c);
  };

  // Converts this tile's raw input, refills `raw` with the tile two steps
  // ahead (so its loads are in flight for two tiles of work), then quantizes.
  auto process = [&](int64_t item, Raw (&raw)[NC]) {
    int64_t s, tile;
    split(item, s, tile);
    float x[V];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const Raw r = raw[c] ^ dm[c];  // D applied to the input's sign bits
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (kHalf) {
          const uint32_t h = e % 2 ? r[e / 2] >> 16 : r[e / 2] & 0xFFFFu;
          x[8 * c + e] = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
        } else {
          x[8 * c + e] = __uint_as_float(r[e]);
        }
      }
    }
    load(item + 2 * wstride, raw);
    // norm over the token's 8 lanes (D does not change it)
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) ss = fmaf(x[v], x[v], ss);
    ss += dpp<kDppXor1>(ss);
    ss += dpp<kDppXor2>(ss);
    ss += dpp<kDppXor8>(ss);
    const float nn = sqrtf(ss);
    // thresholds in the unnormalised transform's units: beta * n * sqrt(d).  A
    // dithered zero row (y = 0) is compared at unit scale, so -delta decides.
    const float unit = DITHER && nn == 0.f ? 1.f : nn * sqrt_d;
    float th[K];
#pragma unroll
    for (int i = 0; i < K; ++i) th[i] = beta[i] * unit;
    // table search: bin units per transform unit, with the lane's sign (a zero
    // row without dither stays at u = kBins / 2, the lower middle code)
    const float su = unit > 0.f ? sgn * ubin / unit : 0.f;

    // unnormalised Walsh-Hadamard transform: register bits, then lane bits
#pragma unroll
    for (int b = 1; b < V; b <<= 1) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if (v & b) continue;
        const float u = x[v], z = x[v + b];
        x[v] = u + z;
        x[v + b] = u - z;
      }
    }
    // cross-lane stages: own + s * partner (the upper lane's result negated)
#pragma unroll
    for (int v = 0; v < V; v += 8) butterfly8_xor1(x + v, s1);
#pragma unroll
    for (int v = 0; v < V; v += 8) butterfly8_xor2(x + v, s2);
#pragma unroll
    for (int v = 0; v < V; v += 8) butterfly8_xor8(x + v, s8);
    // x = sgn * y from here on
    if constexpr (DITHER) {
      // y - delta in the unnormalised transform's units
      const float shift = sgn * dither_offset(p.ds0, s, tile * 8 + tl, dwidth) * unit;
#pragma unroll
      for (int v = 0; v < V; ++v) x[v] -= shift;
    }

    // codes into LDS, [token][coordinate]: code = #{i : beta_i < y}
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t wd[2] = {0u, 0u};
      if constexpr (kTable) {
        // all 8 lookups in flight before the first compare
        float u[8];
        uint2 ent[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u[e] = fmaf(x[8 * c + e], su, 0.5f * kBins);
          const int bin = (int)__builtin_amdgcn_fmed3f(u[e], 0.f, (float)(kBins - 1));
          ent[e] = ctab_lane[bin * kBinCopies];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          wd[e / 4] |= (ent[e].y + (u[e] > __uint_as_float(ent[e].x) ? 1u : 0u)) << (8 * (e % 4));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wd[e / 4] |= symmetric_code<BITS>(sgn * x[8 * c + e], th) << (8 * (e % 4));
      }
      *reinterpret_cast<uint2*>(&codes[w][tl][8 * k + 64 * c]) = make_uint2(wd[0], wd[1]);
    }
    const int64_t tok = tile * 8 + tl;
    if (k == 0 && tok >= t0 && tok < tend) p.norm[s * p.cap + tok] = nn;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // pack 32 codes per lane into BITS dwords and store
    if (lane < D / 4) {
      uint32_t cw[8];  // 32 code bytes, in stream order
      if constexpr (!VALUES) {
        const int t = lane / (D / 32), jb = lane % (D / 32);
        const u4 a = *reinterpret_cast<const u4*>(&codes[w][t][32 * jb]);
        const u4 b = *reinterpret_cast<const u4*>(&codes[w][t][32 * jb + 16]);
        cw[0] = a[0]; cw[1] = a[1]; cw[2] = a[2]; cw[3] = a[3];
        cw[4] = b[0]; cw[5] = b[1]; cw[6] = b[2]; cw[7] = b[3];
      } else {
        // stream positions 8 j + t, j = 4 lane + i: byte i of r[t] is code (j, t)
        uint32_t r[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) r[t] = *reinterpret_cast<const uint32_t*>(&codes[w][t][4 * lane]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t) lo |= ((r[t] >> (8 * i)) & 0xFFu) << (8 * t);
#pragma unroll
          for (int t = 0; t < 4; ++t) hi |= ((r[4 + t] >> (8 * i)) & 0xFFu) << (8 * t);
          cw[2 * i] = lo;
          cw[2 * i + 1] = hi;
        }
      }
      uint32_t out[BITS];
#pragma unroll
      for (int q = 0; q < BITS; ++q) out[q] = 0u;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t cd = (cw[i / 4] >> (8 * (i % 4))) & 0xFFu;
        const int bit = BITS * i;
        out[bit / 32] |= cd << (bit % 32);
        if (bit % 32 + BITS > 32) out[bit / 32 + 1] |= cd >> (32 - bit % 32);
      }
      if constexpr (!VALUES) {
        const int t = lane / (D / 32), jb = lane % (D / 32);
        const int64_t tk = tile * 8 + t;
        if (tk >= t0 && tk < tend) {
          store_words<BITS>(p.idx + (s * p.cap + tile * 8) * kRowB + t * kRowB + jb * 4 * BITS, out);
        }
      } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(p.idx + (s * (p.cap / 8) + tile) * (D * BITS) + lane * 4 * BITS);
        const int64_t first = tile * 8;
        if (first < t0 || first + 8 > tend) {
          // partial tile: keep the codes of tokens outside [t0, t0 + n)
          uint32_t keep[BITS];
#pragma unroll
          for (int q = 0; q < BITS; ++q) keep[q] = 0u;
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const int64_t tk = first + (i % 8);
            if (tk < t0 || tk >= tend) {
              const uint32_t m = (1u << BITS) - 1u;
              const int bit = BITS * i;
              keep[bit / 32] |= m << (bit % 32);
              if (bit % 32 + BITS > 32) keep[bit / 32 + 1] |= m >> (32 - bit % 32);
            }
          }
#pragma unroll
          for (int q = 0; q < BITS; ++q) out[q] = (out[q] & ~keep[q]) | (dst[q] & keep[q]);
        }
        store_words<BITS>(reinterpret_cast<uint8_t*>(dst), out);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Two tiles of loads in flight per wave.
  int64_t item = (int64_t)blockIdx.x * kWaves + w;
  Raw ra[NC], rb[NC];
  load(item, ra);
  load(item + wstride, rb);
  while (item < items) {
    process(item, ra);
    item += wstride;
    if (item >= items) break;
    process(item, rb);
    item += wstride;
  }
}

template <int D, int VALUES, typename Tin, int DITHER>
hipError_t launch_bits(const FwhtParams& p, int bits, unsigned grid, hipStream_t st) {
  switch (bits) {
    case 1: hipLaunchKernelGGL((quantize_fwht_kernel<D, 1, VALUES, Tin, DITHER>), dim3(grid), dim3(kThreads), 0, st, p); break;
    case 2: hipLaunchKernelGGL((quantize_fwht_kernel<D, 2, VALUES, Tin, DITHER>), dim3(grid), dim3(kThreads), 0, st, p); break;
    case 3: hipLaunchKernelGGL((quantize_fwht_kernel<D, 3, VALUES, Tin, DITHER>), dim3(grid), dim3(kThreads), 0, st, p); break;
    default: hipLaunchKernelGGL((quantize_fwht_kernel<D, 4, VALUES, Tin, DITHER>), dim3(grid), dim3(kThreads), 0, st, p); break;
  }
  return hipGetLastError();
}

template <int D, typename Tin>
hipError_t launch_in(const FwhtParams& p, const QuantizeArgs& a, unsigned grid, hipStream_t st) {
  if (a.dither)
    return a.value_layout ? launch_bits<D, 1, Tin, 1>(p, a.bits, grid, st) : launch_bits<D, 0, Tin, 1>(p, a.bits, grid, st);
  return a.value_layout ? launch_bits<D, 1, Tin, 0>(p, a.bits, grid, st) : launch_bits<D, 0, Tin, 0>(p, a.bits, grid, st);
}

template <int D>
hipError_t launch_d(const FwhtParams& p, const QuantizeArgs& a, unsigned grid, hipStream_t st) {
  return a.dtype == TQ_F16 ? launch_in<D, _Float16>(p, a, grid, st) : launch_in<D, float>(p, a, grid, st);
}

}  // namespace

bool fwht_quantize_supports(int d, int rot, int qjl) {
  return rot == TQ_ROT_HADAMARD && !qjl && (d == 64 || d == 128 || d == 256);
}

hipError_t launch_quantize_fwht(const QuantizeArgs& a, hipStream_t st) {
  if (a.n == 0 || a.seqs == 0) return hipSuccess;
  FwhtParams p{};
  p.x = a.x;
  p.seqs = a.seqs;
  p.n = a.n;
  p.t0 = a.t0;
  p.cap = a.cap;
  p.tile_first = a.t0 / 8;
  p.tiles = (a.t0 + a.n - 1) / 8 - p.tile_first + 1;
  p.dsign = a.dsign;
  p.bnd = a.bnd;
  p.idx = a.idx;
  p.norm = a.norm;
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
    case 64: return launch_d<64>(p, a, (unsigned)grid, st);
    case 128: return launch_d<128>(p, a, (unsigned)grid, st);
    default: return launch_d<256>(p, a, (unsigned)grid, st);
  }
}

}  // namespace tq
