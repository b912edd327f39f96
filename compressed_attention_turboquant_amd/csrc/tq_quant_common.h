// Device helpers shared by the quantize kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace tq {

// Magnitude index m = #{i : t_i < a} over the K = 2^(BITS-1) - 1 positive
// boundaries t (sorted), by a branchless binary search (value selects only).
template <int BITS>
__device__ __forceinline__ uint32_t magnitude(float a, const float (&t)[BITS > 1 ? (1 << (BITS - 1)) - 1 : 1]) {
  if constexpr (BITS == 1) {
    return 0u;
  } else if constexpr (BITS == 2) {
    return a > t[0] ? 1u : 0u;
  } else if constexpr (BITS == 3) {
    const float t0 = t[0], t1 = t[1], t2 = t[2];
    const bool c1 = a > t1;
    const float h = c1 ? t2 : t0;
    const bool c0 = a > h;
    return (c1 ? 2u : 0u) + (c0 ? 1u : 0u);
  } else {
    const float t0 = t[0], t1 = t[1], t2 = t[2], t3 = t[3], t4 = t[4], t5 = t[5], t6 = t[6];
    const bool c2 = a > t3;
    const float h1 = c2 ? t5 : t1;
    const float h04 = c2 ? t4 : t0;
    const float h26 = c2 ? t6 : t2;
    const bool c1 = a > h1;
    const float h0 = c1 ? h26 : h04;
    const bool c0 = a > h0;
    return (c2 ? 4u : 0u) + (c1 ? 2u : 0u) + (c0 ? 1u : 0u);
  }
}

// Code #{i : beta_i < y} of a value y for the symmetric boundaries whose
// positive half (scaled like y) is t: the magnitude index m, mirrored for y <= 0
// (y = 0 takes the lower middle code).
template <int BITS>
__device__ __forceinline__ uint32_t symmetric_code(float y, const float (&t)[BITS > 1 ? (1 << (BITS - 1)) - 1 : 1]) {
  constexpr uint32_t K = (1u << (BITS - 1)) - 1u;
  return magnitude<BITS>(fabsf(y), t) ^ (y > 0.f ? K + 1u : K);
}

// Binned code table for 3- and 4-bit codes.  The coordinate on the codebook's
// N(0, 1) scale, z = y sqrt(d) (y a coordinate of the unit vector), is cut into
// kBins bins of width 1 / kBinScale centred on 0, so they cover |z| < 4; the
// bins outside hold no boundary (the outermost boundary of the 4-bit codebooks
// is below 2.5), so values beyond them clamp to the end bins.  Every codebook's
// boundaries are more than one bin apart (the narrowest gap is about 0.25), so
// a bin holds at most one: its entry is {that boundary in bin units u = z
// kBinScale + kBins / 2, or +inf; the count of boundaries below the bin}, and a
// code is one lookup and one compare.  kBinCopies copies, one per lane of a
// half wave, keep the lookups free of bank conflicts.
constexpr int kBins = 64;
constexpr float kBinScale = 8.f;
constexpr int kBinCopies = 32;
constexpr int kCodeTableEntries = kBins * kBinCopies;

// Entry of bin `bin` for the 2^BITS - 1 sorted boundaries bnd (ubin =
// sqrt(d) * kBinScale, the table's bins starting at u = -offset): the boundary
// inside the bin in bin units, or +inf, and the count of boundaries below the bin.
template <int BITS>
__device__ __forceinline__ void bin_entry(const float* bnd, float ubin, float offset, int bin, float& inner,
                                          uint32_t& below) {
  constexpr int L = 1 << BITS;
  below = 0;
  inner = INFINITY;
  for (int i = 0; i + 1 < L; ++i) {
    const float ub = fmaf(bnd[i], ubin, offset);
    if (ub < (float)bin) ++below;
    else if (ub < (float)(bin + 1)) inner = ub;
  }
}

// Fills the table (kCodeTableEntries entries) from the 2^BITS - 1 sorted
// boundaries bnd; ubin = sqrt(d) * kBinScale.  Threads tid of nthreads share the work.
template <int BITS>
__device__ __forceinline__ void fill_code_table(uint2* tab, const float* bnd, float ubin, int tid, int nthreads) {
  for (int e = tid; e < kCodeTableEntries; e += nthreads) {
    float inner;
    uint32_t below;
    bin_entry<BITS>(bnd, ubin, 0.5f * kBins, e / kBinCopies, inner, below);
    tab[e] = make_uint2(__float_as_uint(inner), below);
  }
}

// Full-range tables for head dimension 128: a coordinate y of a unit vector
// has |z| = |y| sqrt(128) <= 11.32, i.e. |z| kBinScale <= 90.6, so kFullBins
// bins from u = -kFullOffset hold every value the rotation can produce (with
// two bins of margin for rounding).  The bin index then needs no clamp, only
// a float-to-unsigned conversion, which gives bin 0 for a negative value or
// NaN (the code of a row with a non-finite norm, whose scale is 0).
constexpr int kFullBins = 186;
constexpr float kFullOffset = 93.f;
__device__ __forceinline__ uint32_t full_bin(float u) {
  uint32_t b;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(b) : "v"(u));
  return b;
}

// COPIES copies of each full-range bin's entry (one per lane of the group of
// lanes one LDS cycle serves: 16 for 8-byte entries, 8 for 16-byte ones).
template <int BITS, int COPIES>
__device__ __forceinline__ void fill_full_code_table(uint2* tab, const float* bnd, float ubin, int tid,
                                                     int nthreads) {
  for (int e = tid; e < kFullBins * COPIES; e += nthreads) {
    float inner;
    uint32_t below;
    bin_entry<BITS>(bnd, ubin, kFullOffset, e / COPIES, inner, below);
    tab[e] = make_uint2(__float_as_uint(inner), below);
  }
}
template <int COPIES>
__device__ __forceinline__ uint32_t full_table_code(const uint2* lane_tab, float u) {
  const uint2 ent = lane_tab[full_bin(u) * COPIES];
  return ent.y + (u > __uint_as_float(ent.x) ? 1u : 0u);
}

// The full-range table with each entry also holding the centroids of its two
// possible codes, c[below] and c[below + 1], times cscale: a code's centroid is
// then a select on the code's own compare (no second lookup).
template <int BITS, int COPIES>
__device__ __forceinline__ void fill_full_code_cent_table(uint4* tab, const float* bnd, const float* cent, float ubin,
                                                          float cscale, int tid, int nthreads) {
  constexpr uint32_t L = 1u << BITS;
  for (int e = tid; e < kFullBins * COPIES; e += nthreads) {
    float inner;
    uint32_t below;
    bin_entry<BITS>(bnd, ubin, kFullOffset, e / COPIES, inner, below);
    const uint32_t above = below + 1 < L ? below + 1 : below;
    tab[e] = make_uint4(__float_as_uint(inner), below, __float_as_uint(cent[below] * cscale),
                        __float_as_uint(cent[above] * cscale));
  }
}
template <int COPIES>
__device__ __forceinline__ uint32_t full_table_code_cent(const uint4* lane_tab, float u, float& c) {
  const uint4 ent = lane_tab[full_bin(u) * COPIES];
  const bool up = u > __uint_as_float(ent.x);
  c = __uint_as_float(up ? ent.w : ent.z);
  return ent.y + (up ? 1u : 0u);
}

// Workgroup barrier that orders LDS only: global loads and stores stay in
// flight across it (a plain __syncthreads also waits for every outstanding
// global access, which drains prefetched loads and pending stores).  For
// barriers whose only purpose is to hand LDS data between waves.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace tq
