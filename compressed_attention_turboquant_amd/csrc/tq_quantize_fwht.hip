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
#ifndef TQ_FWHT_AHEAD
#define TQ_FWHT_AHEAD 2
#endif
constexpr int kAhead = TQ_FWHT_AHEAD;  // tiles whose loads a wave keeps in flight


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

// Sum and difference of the two fp16 halves of w, in fp32 (exact conversions,
// one rounding each): v_fma_mix_f32 reads the halves directly, where the
// compiler would convert both first.
__device__ __forceinline__ void half_sum_diff(uint32_t w, float& sum, float& diff) {
  asm("v_fma_mix_f32 %0, %2, 1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %1, %2, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
      : "=&v"(sum), "=v"(diff)
      : "v"(w));
}

// Memory goes through buffer instructions on per-tile records: an access
// that must not happen gets an offset past the record (a load returns 0, a
// store is dropped) instead of a branch, so every tile issues the same memory
// instructions and the compiler can count them when it waits for the loads
// issued two tiles earlier.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;  // past every record used here
__device__ __forceinline__ Rsrc record(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);  // raw buffer
}

// BITS consecutive dwords at byte offset off of r (16-byte aligned when BITS is 4).
template <int BITS>
__device__ __forceinline__ void store_words(Rsrc r, uint32_t off, const uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(u4{w[0], w[1], w[2], w[3]}, r, off, 0, 0);
  } else if constexpr (BITS == 2) {
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u2v{w[0], w[1]}, r, off, 0, 0);
  } else {
#pragma unroll
    for (int q = 0; q < BITS; ++q) __builtin_amdgcn_raw_buffer_store_b32(w[q], r, off + 4 * q, 0, 0);
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
  __shared__ __align__(16) uint2 ctab[kTable ? kCodeTableEntries : 1];  // binned code table

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
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
    fill_code_table<BITS>(ctab, p.bnd, ubin, threadIdx.x, kThreads);
    __syncthreads();
  }
  const uint2* ctab_lane = ctab + (kTable ? lane % kBinCopies : 0);
  const float dwidth = DITHER ? *p.dw : 0.f;

  const int64_t items = p.seqs * p.tiles;
  const int64_t wstride = (int64_t)gridDim.x * kWaves;
  const int64_t t0 = p.t0, tend = p.t0 + p.n;
  constexpr int kRowB = D * BITS / 8;  // key stream bytes per token
  // Keys with 1, 2 or 4 bits: a lane's 8 consecutive coordinates make whole
  // bytes of the stream, packed in registers and stored directly.
  constexpr bool kDirect = !VALUES && BITS != 3;
  // The wave's items are item0 + i * wstride: (sequence, tile) advance by
  // (wstride / tiles, wstride % tiles) with one carry, so no division per tile.
  // Two cursors: the tile being quantized and the one whose loads are issued.
  struct Cursor {
    int64_t item, s, tile;  // tile relative to tile_first
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
  // Input of one tile: its rows in [t0, t0 + n) as one record (none past the
  // last item); rows outside read as 0.
  auto load = [&](const Cursor& cu, Raw (&raw)[NC]) {
    const int64_t tile = p.tile_first + cu.tile;
    const int64_t lo = max(tile * 8, t0), hi = min(tile * 8 + 8, tend);
    const Rsrc r = record(static_cast<const Tin*>(p.x) + (cu.s * p.n + lo - t0) * D,
                          cu.item < items ? (hi - lo) * D * (int64_t)sizeof(Tin) : 0);
    const int64_t t = tile * 8 + tl;
    const uint32_t off = t >= lo && t < hi ? (uint32_t)(((t - lo) * D + 8 * k) * sizeof(Tin)) : kOob;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t o = off + 64 * c * sizeof(Tin);
      if constexpr (kHalf) {
        raw[c] = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
      } else {
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
        const u4 b = __builtin_amdgcn_raw_buffer_load_b128(r, o + 16, 0, 0);
        raw[c] = Raw{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      }
    }
  };

  // Converts this tile's raw input, refills `raw` with the tile two steps
  // ahead (so its loads are in flight for two tiles of work), then quantizes.
  auto process = [&](const Cursor& cu, const Cursor& ahead, Raw (&raw)[NC]) {
    // (tiles stay in order: work of the next tile, in particular the wait for
    // its input, is not moved up into this one)
    __builtin_amdgcn_sched_barrier(0);
    const int64_t s = cu.s, tile = p.tile_first + cu.tile;
    // Values: the tile's record, and the old words a partial tile keeps (the
    // codes of tokens outside [t0, t0 + n)), read first so that waiting for
    // them does not wait for the next tiles' loads; a full tile reads them as
    // 0 without a memory access.
    const int ln = lane % (D / 4);
    const bool st_ok = lane < D / 4;  // lanes that store packed words
    const Rsrc vrec = record(p.idx + (s * (p.cap / 8) + tile) * (D * BITS), D * BITS);
    const uint32_t voff = st_ok ? (uint32_t)(ln * 4 * BITS) : kOob;
    const bool partial = tile * 8 < t0 || tile * 8 + 8 > tend;  // uniform
    uint32_t old[VALUES ? BITS : 1];
    if constexpr (VALUES) {
#pragma unroll
      for (int q = 0; q < BITS; ++q)
        old[q] = __builtin_amdgcn_raw_buffer_load_b32(vrec, partial ? voff + 4 * q : kOob, 0, 0);
    }
    float x[V];
    float ss = 0.f;  // squared norm of the lane's part (D does not change it)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const Raw r = raw[c] ^ dm[c];  // D applied to the input's sign bits
      if constexpr (kHalf) {
        // first butterfly stage (coordinate bit 0) fused with the conversion
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          // (through a scalar: a bit cast of a vector element reads element 0)
          const uint32_t wq = r[q];
          const h2 pr = __builtin_bit_cast(h2, wq);
          ss = __builtin_amdgcn_fdot2(pr, pr, ss, false);
          half_sum_diff(wq, x[8 * c + 2 * q], x[8 * c + 2 * q + 1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[8 * c + e] = __uint_as_float(r[e]);
          ss = fmaf(x[8 * c + e], x[8 * c + e], ss);
        }
      }
    }
    load(ahead, raw);
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
    // (bit 0 was done above for fp16 input)
#pragma unroll
    for (int b = kHalf ? 2 : 1; b < V; b <<= 1) {
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

    // code = #{i : beta_i < y}; keys of 1, 2 or 4 bits go straight to memory,
    // the others through LDS as bytes, [token][coordinate]
    const int64_t tok = tile * 8 + tl;
    const bool tok_ok = tok >= t0 && tok < tend;
    const Rsrc krec = record(p.idx + (s * p.cap + tile * 8) * kRowB, 8 * kRowB);  // the tile's key rows
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t cd[8];
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
        for (int e = 0; e < 8; ++e) cd[e] = ent[e].y + (u[e] > __uint_as_float(ent[e].x) ? 1u : 0u);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cd[e] = symmetric_code<BITS>(sgn * x[8 * c + e], th);
      }
      if constexpr (kDirect) {
        // coordinates 8 (k + 8 c) .. + 7: bytes BITS (k + 8 c) .. + BITS - 1 of the row
        uint32_t wd = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) wd |= cd[e] << (BITS * e);
        const uint32_t off = tok_ok ? (uint32_t)(tl * kRowB + BITS * (k + 8 * c)) : kOob;
        if constexpr (BITS == 4) __builtin_amdgcn_raw_buffer_store_b32(wd, krec, off, 0, 0);
        else if constexpr (BITS == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)wd, krec, off, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)wd, krec, off, 0, 0);
      } else {
        uint32_t wd[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) wd[e / 4] |= cd[e] << (8 * (e % 4));
        *reinterpret_cast<uint2*>(&codes[w][tl][8 * k + 64 * c]) = make_uint2(wd[0], wd[1]);
      }
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nn), record(p.norm + s * p.cap + tile * 8, 32),
                                          k == 0 && tok_ok ? (uint32_t)(4 * tl) : kOob, 0, 0);
    if constexpr (kDirect) return;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // pack 32 codes per lane into BITS dwords and store (lanes past D / 4
    // repeat lane % (D / 4) and store nothing)
    {
      uint32_t out[BITS];
      if constexpr (VALUES && BITS == 4) {
        // stream positions 8 j + t, j = 4 lane + i: dword i holds the codes of
        // coordinate j for tokens t = 0..7 at bits 4 t.  Nibble pairs of tokens
        // (2 m, 2 m + 1) first, then a 4 x 4 byte transpose with byte permutes.
        uint32_t r[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) r[t] = *reinterpret_cast<const uint32_t*>(&codes[w][t][4 * ln]);
        const uint32_t p0 = r[0] | (r[1] << 4), p1 = r[2] | (r[3] << 4);
        const uint32_t p2 = r[4] | (r[5] << 4), p3 = r[6] | (r[7] << 4);
        const uint32_t q0 = __builtin_amdgcn_perm(p1, p0, 0x05010400u);  // p0.b0 p1.b0 p0.b1 p1.b1
        const uint32_t q1 = __builtin_amdgcn_perm(p1, p0, 0x07030602u);  // p0.b2 p1.b2 p0.b3 p1.b3
        const uint32_t q2 = __builtin_amdgcn_perm(p3, p2, 0x05010400u);
        const uint32_t q3 = __builtin_amdgcn_perm(p3, p2, 0x07030602u);
        out[0] = __builtin_amdgcn_perm(q2, q0, 0x05040100u);  // byte i of p0 p1 p2 p3, i = 0
        out[1] = __builtin_amdgcn_perm(q2, q0, 0x07060302u);  // i = 1
        out[2] = __builtin_amdgcn_perm(q3, q1, 0x05040100u);  // i = 2
        out[3] = __builtin_amdgcn_perm(q3, q1, 0x07060302u);  // i = 3
      } else {
        uint32_t cw[8];  // 32 code bytes, in stream order
        if constexpr (!VALUES) {
          const int t = ln / (D / 32), jb = ln % (D / 32);
          const u4 a = *reinterpret_cast<const u4*>(&codes[w][t][32 * jb]);
          const u4 b = *reinterpret_cast<const u4*>(&codes[w][t][32 * jb + 16]);
          cw[0] = a[0]; cw[1] = a[1]; cw[2] = a[2]; cw[3] = a[3];
          cw[4] = b[0]; cw[5] = b[1]; cw[6] = b[2]; cw[7] = b[3];
        } else {
          // stream positions 8 j + t, j = 4 lane + i: byte i of r[t] is code (j, t)
          uint32_t r[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) r[t] = *reinterpret_cast<const uint32_t*>(&codes[w][t][4 * ln]);
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
#pragma unroll
        for (int q = 0; q < BITS; ++q) out[q] = 0u;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t cd = (cw[i / 4] >> (8 * (i % 4))) & 0xFFu;
          const int bit = BITS * i;
          out[bit / 32] |= cd << (bit % 32);
          if (bit % 32 + BITS > 32) out[bit / 32 + 1] |= cd >> (32 - bit % 32);
        }
      }
      if constexpr (!VALUES) {
        const int t = ln / (D / 32), jb = ln % (D / 32);
        const int64_t tk = tile * 8 + t;
        store_words<BITS>(krec, st_ok && tk >= t0 && tk < tend ? (uint32_t)(t * kRowB + jb * 4 * BITS) : kOob, out);
      } else {
        const int64_t first = tile * 8;
        {
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
          for (int q = 0; q < BITS; ++q) out[q] = (out[q] & ~keep[q]) | (old[q] & keep[q]);
        }
        store_words<BITS>(vrec, voff, out);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // kAhead tiles of loads in flight per wave.
  const int64_t item0 = (int64_t)blockIdx.x * kWaves + w;
  Cursor cur{item0, item0 / p.tiles, item0 % p.tiles};
  Cursor ahead = cur;
  Raw rbuf[kAhead][NC];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    load(ahead, rbuf[i]);
    advance(ahead);
  }
  // The memory counter is in order and counts stores too: inside the loop a
  // tile's loads are followed by the stores and loads of kAhead - 1 tiles
  // before they are waited for.  Stores to an empty record (dropped, no
  // memory access) give the path into the loop as many, so that the waits
  // the compiler places, which must hold on both paths, leave the loads of
  // the next tiles in flight.
  const Rsrc none = record(p.norm, 0);
#pragma unroll
  for (int i = 0; i < 16 * (kAhead - 1); ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 64 * i, 0, 0);
  // Whole rounds of kAhead tiles without an exit test inside (so the loop is
  // entered only from above and from its own end, and each buffer's wait sees
  // the same history), then the remaining tiles.
  const int64_t mine = item0 < items ? (items - item0 + wstride - 1) / wstride : 0;  // this wave's tiles
  for (int64_t r = mine / kAhead; r > 0; --r) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      process(cur, ahead, rbuf[i]);
      advance(cur);
      advance(ahead);
    }
  }
#pragma unroll
  for (int i = 0; i < kAhead - 1; ++i) {
    if (cur.item >= items) return;
    process(cur, ahead, rbuf[i]);
    advance(cur);
    advance(ahead);
  }
}

// Up to 8 workgroups per CU, each looping over its tiles: about twice what is
// resident at once, which measured a little faster than one round of exactly
// the resident workgroups (the second round fills in as the first finishes).
template <int D, int BITS, int VALUES, typename Tin, int DITHER>
hipError_t launch_k(const FwhtParams& p, int64_t groups, int cus, hipStream_t st) {
  const int64_t grid = groups < (int64_t)cus * 8 ? groups : (int64_t)cus * 8;
  hipLaunchKernelGGL((quantize_fwht_kernel<D, BITS, VALUES, Tin, DITHER>), dim3((unsigned)grid), dim3(kThreads), 0,
                     st, p);
  return hipGetLastError();
}

template <int D, int VALUES, typename Tin, int DITHER>
hipError_t launch_bits(const FwhtParams& p, int bits, int64_t groups, int cus, hipStream_t st) {
  switch (bits) {
    case 1: return launch_k<D, 1, VALUES, Tin, DITHER>(p, groups, cus, st);
    case 2: return launch_k<D, 2, VALUES, Tin, DITHER>(p, groups, cus, st);
    case 3: return launch_k<D, 3, VALUES, Tin, DITHER>(p, groups, cus, st);
    default: return launch_k<D, 4, VALUES, Tin, DITHER>(p, groups, cus, st);
  }
}

template <int D, typename Tin>
hipError_t launch_in(const FwhtParams& p, const QuantizeArgs& a, int64_t groups, int cus, hipStream_t st) {
  if (a.dither)
    return a.value_layout ? launch_bits<D, 1, Tin, 1>(p, a.bits, groups, cus, st)
                          : launch_bits<D, 0, Tin, 1>(p, a.bits, groups, cus, st);
  return a.value_layout ? launch_bits<D, 1, Tin, 0>(p, a.bits, groups, cus, st)
                        : launch_bits<D, 0, Tin, 0>(p, a.bits, groups, cus, st);
}

template <int D>
hipError_t launch_d(const FwhtParams& p, const QuantizeArgs& a, int64_t groups, int cus, hipStream_t st) {
  return a.dtype == TQ_F16 ? launch_in<D, _Float16>(p, a, groups, cus, st) : launch_in<D, float>(p, a, groups, cus, st);
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
  const int64_t groups = (p.seqs * p.tiles + kWaves - 1) / kWaves;  // workgroups with a tile per wave
  switch (a.d) {
    case 64: return launch_d<64>(p, a, groups, cus, st);
    case 128: return launch_d<128>(p, a, groups, cus, st);
    default: return launch_d<256>(p, a, groups, cus, st);
  }
}

}  // namespace tq
