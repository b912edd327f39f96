// Key/value compression on the matrix cores (gfx950), head dimension 128.
//
// Per token x ([cuTile] listing, key and value compression functions, values
// without QJL; [Mobilint] "Coordinates Become Predictable After Rotation",
// "Designing the Optimal Codebook Without Data", "Two-Stage Approach"):
//   n = ||x||;  y = R x / n;  idx_j = #{i : beta_i < y_j};  pack idx;
//   keys with QJL: r = y - c[idx] (rotated residual), gamma = ||r||,
//                  sign bits of (S R^T) r = S (u - R^T c[idx]).
//
// Mapping to CDNA4:
//  * The rotation and the projection are [32 tokens x 128] x [128 x 128] GEMMs
//    on v_mfma_f32_16x16x32_f16.  fp16 inputs are exact; the weights sqrt(d) R
//    and S R^T are split into fp16 hi + lo (2 passes, ~2^-22 relative); the fp32
//    residual is split too (3 passes: hi*hi, hi*lo, lo*hi).
//  * Weights are stationary: each wave keeps the rows of 32 output coordinates
//    of its matrix in VGPRs for the whole kernel; tokens stream through LDS in
//    groups of 4 x 8 tokens (one 8-token value tile each), the workgroup
//    looping over groups (persistent grid).
//  * Keys with QJL split the work by role (quantize_keys_qjl_kernel): four
//    waves rotate and quantize, four project the residual, so that one SIMD
//    runs one role's vector work beside the other's matrix-core work.
//  * Operand roles are chosen per tensor so that each lane ends with exactly
//    what it stores: keys (row-major streams) use D = W * X^T, a lane holding 8
//    consecutive coordinates of a token; values (8-token coordinate-major
//    tiles) use D = X * W^T, a lane holding one coordinate of 8 tokens.
//  * The scalar quantizer takes 3- and 4-bit codes from the binned table of
//    tq_quant_common.h (one LDS lookup and one compare per value) and 1- and
//    2-bit codes from a branchless search of |y| over the positive half of the
//    symmetric boundaries.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <type_traits>

#include "tq_kernels.h"
#include "tq_lanes.h"
#include "tq_quant_common.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

// Raw buffer records: an access that must not happen gets an offset past the
// record (a load returns 0, a store is dropped) instead of a branch.
constexpr uint32_t kOob = 0x80000000u;  // past every record used here
__device__ __forceinline__ Rsrc record(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots = 32;  // tokens per tile: 4 value tiles of 8
// The role-split key kernel runs 4 waves per SIMD (two workgroups of 8 waves
// per CU: 128 VGPRs, and a code table small enough that both fit in LDS).
// Same-run timings of the C3 keys: 3.06 ms at 2 waves per SIMD, 2.76 ms at 4.
// Table copies: one per lane of the group one LDS cycle serves (8 lanes for
// the keys' 16-byte entries, 16 for the values' 8-byte entries).
constexpr int kKeyWaves = 4;
constexpr int kKeyCopies = 8;
constexpr int kValCopies = 16;

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The fp16 pair {a - hi.x, b - hi.y} for hi = {fp16(a), fp16(b)}: the lo
// halves of the two values' hi + lo split, one mixed-precision FMA each
// (a * 1.0 - hi.x in fp32, rounded to fp16 into the low or high half).
__device__ __forceinline__ uint32_t split_lo(float a, float b, uint32_t hi) {
  uint32_t lo;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(lo)
      : "v"(a), "v"(b), "v"(hi));
  return lo;
}

// Output coordinate held by weight row rho (0..15) of coordinate tile ct in
// wave w: lanes of group g = rho/4 get 8 consecutive coordinates 32w + 8g + 4ct + rho%4.
__device__ __forceinline__ int out_coord(int w, int ct, int rho) {
  return 32 * w + 8 * (rho / 4) + 4 * ct + (rho % 4);
}

// BITS code bits of 8 coordinates (BITS bytes) at byte offset off of r.
template <int BITS>
__device__ __forceinline__ void store_code_bits(uint32_t packed, Rsrc r, uint32_t off) {
  if constexpr (BITS == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(packed, r, off, 0, 0);
  } else if constexpr (BITS == 3) {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)packed, r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(packed >> 16), r, off + 2, 0, 0);
  } else if constexpr (BITS == 2) {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)packed, r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)packed, r, off, 0, 0);
  }
}

// Values, and keys without QJL: the rotation and the scalar quantizer.
template <int BITS, int VALUES>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
quantize_mfma_kernel(QuantMfmaParams p) {
  constexpr bool kTable = BITS >= 3;  // 3- and 4-bit codes from the binned table
  __shared__ __align__(16) _Float16 xs[kSlots][D + 8];  // token rows (padded)
  __shared__ float nrm[kSlots];
  __shared__ __align__(16) float nsc[kSlots];  // each slot's scale into the code step (0 for a zero row)
  __shared__ __align__(16) uint2 ctabl[kTable ? kFullBins * kValCopies : 1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;

  // Stationary weights: rows out_coord(w, ct, l16), columns 32 kb + 8 g4 + e.
  h8 wr[2][4][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = out_coord(w, ct, l16);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int col = 32 * kb + 8 * g4;
      wr[ct][kb][0] = *reinterpret_cast<const h8*>(p.rot_hi + row * D + col);
      wr[ct][kb][1] = *reinterpret_cast<const h8*>(p.rot_lo + row * D + col);
    }
  }
  // Positive half of the symmetric boundaries (1- and 2-bit codes).
  constexpr int KP = BITS > 1 ? (1 << (BITS - 1)) - 1 : 1;
  float beta[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) beta[i] = BITS > 1 ? p.bnd[(1 << (BITS - 1)) + i] : 0.f;
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float ubin = sqrtf((float)D) * kBinScale;  // unit-vector coordinate -> bin units
  if constexpr (kTable) fill_full_code_table<BITS, kValCopies>(ctabl, p.bnd, ubin, tid, kThreads);
  const uint2* ctab_lane = ctabl + (kTable ? lane % kValCopies : 0);

  // Work unit: 4 consecutive value tiles (32 token slots) of one sequence.
  // Group g is (sequence g / gps, group g % gps of it); the grid strides by
  // gridDim.x groups, i.e. by a fixed quotient and remainder, so the pair
  // advances with one carry instead of a 64-bit division per group.
  const int tiles = (int)(p.tile_last - p.tile_first + 1);  // tiles per sequence touched
  const int gps = (tiles + 3) / 4;                             // groups per sequence
  const int groups = (int)p.seqs * gps;  // < 2^31 (checked on the host)
  const int step_q = (int)gridDim.x / gps, step_r = (int)gridDim.x % gps;
  const int t0 = (int)p.t0, tend = (int)(p.t0 + p.n);
  const int tfirst = (int)p.tile_first * 8;
  const int rowb = D * BITS / 8;
  auto advance = [&](int& s_, int& g_) {
    s_ += step_q;
    g_ += step_r;
    if (g_ >= gps) {
      g_ -= gps;
      ++s_;
    }
  };

  // Loader role: 8 threads per token slot, 16 halves each.  The group's rows
  // load through a record starting at its first token slot; slots outside
  // [t0, t0 + n) (and every slot of a group past the end) get an offset past
  // the record, so the loads return 0 without a branch.
  const int lslot = tid / 8, lpart = tid % 8;
  auto load_x = [&](int gs, int gg, bool live, h8& v0, h8& v1) {
    const int tb = tfirst + 32 * gg;  // first token slot of the group
    const int t = tb + lslot;
    const Rsrc rec = record(p.x + ((int64_t)gs * p.n + (tb - t0)) * D, kSlots * D * 2);
    const uint32_t off = live && t >= t0 && t < tend ? (uint32_t)(lslot * D * 2 + lpart * 32) : kOob;
    v0 = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rec, off, 0, 0));
    v1 = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rec, off + 16, 0, 0));
  };
  int grp = (int)blockIdx.x;
  int cs = grp / gps, cg = grp % gps;  // sequence and group within it
  h8 nx0, nx1;
  load_x(cs, cg, grp < groups, nx0, nx1);
  __syncthreads();  // the code table is filled

  for (; grp < groups; grp += gridDim.x) {
    int ns = cs, ng = cg;
    advance(ns, ng);
    const int tb = tfirst + 32 * cg;  // first token slot of the group
    // ---- token rows into LDS, with their norms; prefetch the next group ----
    {
      const h8 v0 = nx0, v1 = nx1;
      *reinterpret_cast<h8*>(&xs[lslot][lpart * 16]) = v0;
      *reinterpret_cast<h8*>(&xs[lslot][lpart * 16 + 8]) = v1;
      // Sum of squares: fp16 products are exact in fp32; two independent
      // chains of packed dot products, then the slot's 8 lanes.
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const h2 a{v0[e], v0[e + 1]}, b{v1[e], v1[e + 1]};
        s0 = __builtin_amdgcn_fdot2(a, a, s0, false);
        s1 = __builtin_amdgcn_fdot2(b, b, s1, false);
      }
      const float ss = sum_over_8_lanes(s0 + s1);
      if (lpart == 0) {
        const float nn = __builtin_amdgcn_sqrtf(ss);
        const float inv = nn > 0.f ? inv_sqrt_d * __builtin_amdgcn_rcpf(nn) : 0.f;
        nrm[lslot] = nn;
        nsc[lslot] = kTable ? inv * ubin : inv;  // bin units, or unit-vector units for the search
      }
      load_x(ns, ng, grp + (int)gridDim.x < groups, nx0, nx1);
    }
    lds_barrier();

    // ---- rotation: acc[ct][tt] ----
    f4 acc[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[ct][tt] = f4{0.f, 0.f, 0.f, 0.f};
    // token operand: keys read slot 16 tt + l16; values read the slot that makes
    // lane group g4 hold value tile g4 (slot 8 (l16/4) + 4 tt + l16 % 4).  Steps
    // (kb, tt) run in order; each step's operand is read from LDS one step
    // ahead, so that the read overlaps the previous step's MFMAs.
    auto x_operand = [&](int st) {
      const int kb = st / 2, tt = st % 2;
      const int slot = VALUES ? 8 * (l16 / 4) + 4 * tt + (l16 % 4) : 16 * tt + l16;
      return *reinterpret_cast<const h8*>(&xs[slot][32 * kb + 8 * g4]);
    };
    h8 xv = x_operand(0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int kb = st / 2, tt = st % 2;
      const h8 xn = st < 7 ? x_operand(st + 1) : xv;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        if constexpr (VALUES) {
          acc[ct][tt] = mfma(xv, wr[ct][kb][0], acc[ct][tt]);
          acc[ct][tt] = mfma(xv, wr[ct][kb][1], acc[ct][tt]);
        } else {
          acc[ct][tt] = mfma(wr[ct][kb][0], xv, acc[ct][tt]);
          acc[ct][tt] = mfma(wr[ct][kb][1], xv, acc[ct][tt]);
        }
      }
      xv = xn;
    }
    // Order for the scheduler: two reads, then per step its four MFMAs and
    // the next read.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int st = 0; st < 7; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (st < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    if constexpr (!VALUES) {
      // Lane (g4, l16) holds coordinates 32w + 8g4 + 4ct + r of token slot
      // 16tt + l16.  Stores go through records from the group's first token
      // slot on; slots outside [t0, t0 + n) get an offset past the record.
      const int64_t row0 = (int64_t)cs * p.cap + tb;
      const Rsrc irec = record(p.idx + row0 * rowb, kSlots * rowb);
      const Rsrc nrec = record(p.norm + row0, kSlots * 4);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int slot = 16 * tt + l16;
        const int t = tb + slot;
        const bool ok = t >= t0 && t < tend;
        const uint32_t ioff = ok ? (uint32_t)(slot * rowb + (4 * w + g4) * BITS) : kOob;
        const float nn = nrm[slot], sc = nsc[slot];
        uint32_t packed = 0;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float a = acc[ct][tt][q];
            uint32_t code;
            if constexpr (kTable) code = full_table_code<kValCopies>(ctab_lane, fmaf(a, sc, kFullOffset));
            else code = symmetric_code<BITS>(a * sc, beta);
            packed |= code << (BITS * (4 * ct + q));
          }
        store_code_bits<BITS>(packed, irec, ioff);
        if (w == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nn), nrec, g4 == 0 && ok ? (uint32_t)(slot * 4) : kOob,
                                                0, 0);
      }
    } else {
      // Lane (g4, l16) holds, for coordinate tile ct, coordinate out_coord(w, ct, l16)
      // of the 8 tokens of value tile g4 (token 4 tt + r in D row 4 g4 + r of tile tt).
      const int s = cs;
      const int tile = (int)p.tile_first + 4 * cg + g4;
      // Tokens k of the tile inside [t0, t0 + n): lo <= k < hi (none for a
      // tile past the last one).
      const int lo = max(t0 - tile * 8, 0), hi = min(tend - tile * 8, 8);
      const bool tile_ok = hi > lo;
      uint32_t keep = 0;  // code bits of tokens outside [t0, t0+n) are left unchanged
      if (lo > 0 || hi < 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < lo || k >= hi) keep |= ((1u << BITS) - 1u) << (BITS * k);
      }
      const f4 sc0 = *reinterpret_cast<const f4*>(&nsc[8 * g4]), sc1 = *reinterpret_cast<const f4*>(&nsc[8 * g4 + 4]);
      const float inv[8] = {sc0[0], sc0[1], sc0[2], sc0[3], sc1[0], sc1[1], sc1[2], sc1[3]};
      // Norms: lane l16 < 8 of wave 0 stores token l16 of value tile g4.
      if (w == 0 && l16 < 8 && tile_ok) {
        const int t = tile * 8 + l16;
        if (t >= t0 && t < tend) p.norm[(int64_t)s * p.cap + t] = nrm[8 * g4 + l16];
      }
      uint8_t* tile_base = p.idx + (int64_t)s * (p.cap / 8) * (D * BITS) + (int64_t)tile * (D * BITS);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        uint32_t packed = 0;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = 4 * tt + q;
            if constexpr (kTable)
              packed |= full_table_code<kValCopies>(ctab_lane, fmaf(acc[ct][tt][q], inv[k], kFullOffset)) << (BITS * k);
            else
              packed |= symmetric_code<BITS>(acc[ct][tt][q] * inv[k], beta) << (BITS * k);
          }
        if (tile_ok) {
          uint8_t* dst = tile_base + out_coord(w, ct, l16) * BITS;
          if (keep) {
            uint32_t old = 0;
#pragma unroll
            for (int b = 0; b < BITS; ++b) old |= (uint32_t)dst[b] << (8 * b);
            packed = (packed & ~keep) | (old & keep);
          }
#pragma unroll
          for (int b = 0; b < BITS; ++b) dst[b] = (uint8_t)(packed >> (8 * b));
        }
      }
    }
    lds_barrier();
    cs = ns;
    cg = ng;
  }
}

// Keys with QJL, split by role.  Each SIMD holds one wave of each role:
//  * rotation waves (0-3): the rotation of group k from LDS, the scalar
//    quantizer, codes and norms to memory, the residual (hi + lo) and its
//    squared norm to LDS;
//  * projection waves (4-7): the projection of group k - 1's residual, its sign
//    bits and residual norm to memory, and the rows of group k + 1 into LDS
//    with their norms (loaded one iteration ahead).
// One SIMD then runs one wave's vector work beside the other's matrix-core
// work (a single wave issues vector instructions well below the SIMD's rate,
// and the two units only overlap across waves).  Rows, residuals and norms
// are double-buffered by group parity, so one barrier per group orders them.
template <int BITS>
__global__ void __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(kKeyWaves, kKeyWaves)))
quantize_keys_qjl_kernel(QuantMfmaParams p) {
  constexpr bool kTable = BITS >= 3;
  constexpr int kCopies = kKeyCopies;
  __shared__ __align__(16) _Float16 xs[2][kSlots][D + 8];     // token rows (padded)
  __shared__ __align__(16) _Float16 rs[2][2][kSlots][D + 8];  // [buffer][hi, lo] residual
  __shared__ float nrm[2][kSlots];
  __shared__ __align__(16) float2 nsc[2][kSlots];             // {scale into the code step, into kRes (y - c)}
  __shared__ __align__(16) float rsq[2][kSlots][kWaves];      // per-wave sums of r^2
  __shared__ __align__(16) uint4 ctabc[kTable ? kFullBins * kCopies : 1];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
  const int w = wv % kWaves;  // the wave's output coordinates: 32w .. 32w + 31
  const int lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;
  constexpr float kRes = 64.f;  // the residual is formed as kRes (y - c)
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float ubin = sqrtf((float)D) * kBinScale;
  if constexpr (kTable) fill_full_code_cent_table<BITS, kCopies>(ctabc, p.bnd, p.cent, ubin, kRes, tid, 2 * kThreads);

  const int tiles = (int)(p.tile_last - p.tile_first + 1);
  const int gps = (tiles + 3) / 4;
  const int groups = (int)p.seqs * gps;  // < 2^31 (checked on the host)
  const int step_q = (int)gridDim.x / gps, step_r = (int)gridDim.x % gps;
  const int t0 = (int)p.t0, tend = (int)(p.t0 + p.n);
  const int tfirst = (int)p.tile_first * 8;
  const int rowb = D * BITS / 8;
  auto advance = [&](int& s_, int& g_) {
    s_ += step_q;
    g_ += step_r;
    if (g_ >= gps) {
      g_ -= gps;
      ++s_;
    }
  };
  // Groups of this workgroup: blockIdx.x + k gridDim.x for k < nk.
  const int nk = (int)(((int64_t)groups - blockIdx.x + gridDim.x - 1) / gridDim.x);
  const int s0 = (int)blockIdx.x / gps, g0 = (int)blockIdx.x % gps;

  if (wv < kWaves) {
    // ---------------- rotation waves ----------------
    h8 wr[2][4][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int row = out_coord(w, ct, l16);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int col = 32 * kb + 8 * g4;
        wr[ct][kb][0] = *reinterpret_cast<const h8*>(p.rot_hi + row * D + col);
        wr[ct][kb][1] = *reinterpret_cast<const h8*>(p.rot_lo + row * D + col);
      }
    }
    constexpr int KP = BITS > 1 ? (1 << (BITS - 1)) - 1 : 1;
    float beta[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) beta[i] = BITS > 1 ? p.bnd[(1 << (BITS - 1)) + i] : 0.f;
    const int ctab = __float_as_int(p.cent[lane % 16] * kRes);  // 1- and 2-bit centroids (ds_bpermute)
    const uint4* ctabc_lane = ctabc + (kTable ? lane % kCopies : 0);
    lds_barrier();  // code table filled, rows of group 0 staged

    int cs = s0, cg = g0;
    for (int k = 0; k <= nk; ++k) {
      if (k < nk) {
        const int b = k & 1;
        const int tb = tfirst + 32 * cg;
        f4 acc[2][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) acc[ct][tt] = f4{0.f, 0.f, 0.f, 0.f};
        auto x_operand = [&](int st) {
          const int kb = st / 2, tt = st % 2;
          return *reinterpret_cast<const h8*>(&xs[b][16 * tt + l16][32 * kb + 8 * g4]);
        };
        h8 xv = x_operand(0);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int kb = st / 2, tt = st % 2;
          const h8 xn = st < 7 ? x_operand(st + 1) : xv;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            acc[ct][tt] = mfma(wr[ct][kb][0], xv, acc[ct][tt]);
            acc[ct][tt] = mfma(wr[ct][kb][1], xv, acc[ct][tt]);
          }
          xv = xn;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int st = 0; st < 7; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          if (st < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

        // Lane (g4, l16) holds coordinates 32w + 8g4 + 4ct + r of token slot
        // 16tt + l16.  Stores go through records from the group's first token
        // slot on; slots outside [t0, t0 + n) get an offset past the record.
        const int64_t row0 = (int64_t)cs * p.cap + tb;
        const Rsrc irec = record(p.idx + row0 * rowb, kSlots * rowb);
        const Rsrc nrec = record(p.norm + row0, kSlots * 4);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int slot = 16 * tt + l16;
          const int t = tb + slot;
          const bool ok = t >= t0 && t < tend;
          const uint32_t ioff = ok ? (uint32_t)(slot * rowb + (4 * w + g4) * BITS) : kOob;
          const float nn = nrm[b][slot];
          const float2 sc = nsc[b][slot];
          uint32_t packed = 0;
          float r[8];
          float rr = 0.f;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float a = acc[ct][tt][q];
              uint32_t code;
              float c;
              if constexpr (kTable) {
                code = full_table_code_cent<kCopies>(ctabc_lane, fmaf(a, sc.x, kFullOffset), c);
              } else {
                code = symmetric_code<BITS>(a * sc.x, beta);
                c = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(code << 2), ctab));
              }
              packed |= code << (BITS * (4 * ct + q));
              r[4 * ct + q] = fmaf(a, sc.y, -c);  // kRes (y - c)
              rr = fmaf(r[4 * ct + q], r[4 * ct + q], rr);
            }
          store_code_bits<BITS>(packed, irec, ioff);
          if (w == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nn), nrec,
                                                  g4 == 0 && ok ? (uint32_t)(slot * 4) : kOob, 0, 0);
          u4 hi, lo;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const h2 hv{(_Float16)r[2 * j], (_Float16)r[2 * j + 1]};
            hi[j] = __builtin_bit_cast(uint32_t, hv);
            lo[j] = split_lo(r[2 * j], r[2 * j + 1], hi[j]);
          }
          *reinterpret_cast<u4*>(&rs[b][0][slot][32 * w + 8 * g4]) = hi;
          *reinterpret_cast<u4*>(&rs[b][1][slot][32 * w + 8 * g4]) = lo;
          rr = sum_over_row_groups(rr);  // the wave's 32 coordinates of the slot
          if (g4 == 0) rsq[b][slot][w] = rr;
        }
        advance(cs, cg);
      }
      lds_barrier();
    }
  } else {
    // ---------------- projection waves ----------------
    h8 wp[2][4][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int row = out_coord(w, ct, l16);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int col = 32 * kb + 8 * g4;
        wp[ct][kb][0] = *reinterpret_cast<const h8*>(p.projr_hi + row * D + col);
        wp[ct][kb][1] = *reinterpret_cast<const h8*>(p.projr_lo + row * D + col);
      }
    }
    // Loader role: 8 threads per token slot, 16 halves each, through a record
    // from the group's first token slot (slots outside [t0, t0 + n), and
    // groups past the end, read 0 without touching memory).
    const int pt = tid - kThreads;
    const int lslot = pt / 8, lpart = pt % 8;
    auto load_x = [&](int gs, int gg, bool live, h8& v0, h8& v1) {
      const int tb = tfirst + 32 * gg;
      const int t = tb + lslot;
      const Rsrc rec = record(p.x + ((int64_t)gs * p.n + (tb - t0)) * D, kSlots * D * 2);
      const uint32_t off = live && t >= t0 && t < tend ? (uint32_t)(lslot * D * 2 + lpart * 32) : kOob;
      v0 = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rec, off, 0, 0));
      v1 = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rec, off + 16, 0, 0));
    };
    auto stage = [&](int b, const h8& v0, const h8& v1) {
      *reinterpret_cast<h8*>(&xs[b][lslot][lpart * 16]) = v0;
      *reinterpret_cast<h8*>(&xs[b][lslot][lpart * 16 + 8]) = v1;
      // Sum of squares: fp16 products are exact in fp32; then the slot's 8 lanes.
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const h2 a{v0[e], v0[e + 1]}, c{v1[e], v1[e + 1]};
        s0 = __builtin_amdgcn_fdot2(a, a, s0, false);
        s1 = __builtin_amdgcn_fdot2(c, c, s1, false);
      }
      const float ss = sum_over_8_lanes(s0 + s1);
      if (lpart == 0) {
        const float nn = __builtin_amdgcn_sqrtf(ss);
        const float inv = nn > 0.f ? inv_sqrt_d * __builtin_amdgcn_rcpf(nn) : 0.f;
        nrm[b][lslot] = nn;
        nsc[b][lslot] = make_float2(kTable ? inv * ubin : inv, inv * kRes);
      }
    };
    int ls = s0, lg = g0;  // next group to load
    h8 nx0, nx1;
    load_x(ls, lg, nk > 0, nx0, nx1);
    advance(ls, lg);
    stage(0, nx0, nx1);
    load_x(ls, lg, nk > 1, nx0, nx1);
    advance(ls, lg);
    lds_barrier();

    int ps = s0, pg = g0;  // group k - 1
    for (int k = 0; k <= nk; ++k) {
      if (k + 1 < nk) stage((k + 1) & 1, nx0, nx1);
      load_x(ls, lg, k + 2 < nk, nx0, nx1);
      advance(ls, lg);
      if (k >= 1) {
        const int b = (k - 1) & 1;
        const int tb = tfirst + 32 * pg;
        f4 pacc[2][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) pacc[ct][tt] = f4{0.f, 0.f, 0.f, 0.f};
        auto r_operand = [&](int st, int part) {
          const int kb = st / 2, tt = st % 2;
          return *reinterpret_cast<const h8*>(&rs[b][part][16 * tt + l16][32 * kb + 8 * g4]);
        };
        h8 rh = r_operand(0, 0), rl = r_operand(0, 1);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int kb = st / 2, tt = st % 2;
          const h8 nh = st < 7 ? r_operand(st + 1, 0) : rh;
          const h8 nl = st < 7 ? r_operand(st + 1, 1) : rl;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            pacc[ct][tt] = mfma(wp[ct][kb][0], rh, pacc[ct][tt]);
            pacc[ct][tt] = mfma(wp[ct][kb][0], rl, pacc[ct][tt]);
            pacc[ct][tt] = mfma(wp[ct][kb][1], rh, pacc[ct][tt]);
          }
          rh = nh;
          rl = nl;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int st = 0; st < 7; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
          if (st < 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        const int64_t row0 = (int64_t)ps * p.cap + tb;
        const Rsrc srec = record(p.sign + row0 * (D / 8), kSlots * (D / 8));
        const Rsrc grec = record(p.rnorm + row0, kSlots * 4);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int slot = 16 * tt + l16;
          const int t = tb + slot;
          const bool ok = t >= t0 && t < tend;
          // Bit 4ct + q is 1 for a projection >= +0: shift the float sign bits
          // in from the highest bit down (one funnel shift each), then invert.
          uint32_t bits = 0;
#pragma unroll
          for (int e = 7; e >= 0; --e)
            bits = __builtin_amdgcn_alignbit(bits, __float_as_uint(pacc[e / 4][tt][e % 4]), 31);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)~bits, srec,
                                               ok ? (uint32_t)(slot * (D / 8) + 4 * w + g4) : kOob, 0, 0);
          if (w == 0) {
            const f4 g = *reinterpret_cast<const f4*>(&rsq[b][slot][0]);
            const float gamma = __builtin_amdgcn_sqrtf((g[0] + g[1]) + (g[2] + g[3])) * (1.f / kRes);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gamma), grec,
                                                  g4 == 0 && ok ? (uint32_t)(slot * 4) : kOob, 0, 0);
          }
        }
        advance(ps, pg);
      }
      lds_barrier();
    }
  }
}

// Persistent grid: as many workgroups as the CUs hold at once (a second,
// partial round of workgroups would run the last share at low occupancy).
template <typename Kernel>
hipError_t launch_persistent(Kernel kernel, int threads, const QuantMfmaParams& p, int64_t groups, hipStream_t st) {
  int dev = 0, cus = 256, per_cu = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t slots = (int64_t)cus * per_cu;
  const int64_t grid = groups < slots ? groups : slots;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, st, p);
  return hipGetLastError();
}

template <int BITS, int QJL, int VALUES>
hipError_t launch(const QuantMfmaParams& p, int64_t groups, hipStream_t st) {
  if constexpr (QJL)
    return launch_persistent(quantize_keys_qjl_kernel<BITS>, 2 * kThreads, p, groups, st);
  else
    return launch_persistent(quantize_mfma_kernel<BITS, VALUES>, kThreads, p, groups, st);
}

template <int QJL, int VALUES>
hipError_t dispatch_bits(const QuantMfmaParams& p, int bits, int64_t groups, hipStream_t st) {
  switch (bits) {
    case 1: return launch<1, QJL, VALUES>(p, groups, st);
    case 2: return launch<2, QJL, VALUES>(p, groups, st);
    case 3: return launch<3, QJL, VALUES>(p, groups, st);
    default: return launch<4, QJL, VALUES>(p, groups, st);
  }
}

}  // namespace

bool mfma_quantize_supports(int d, int dtype) { return d == D && dtype == TQ_F16; }

hipError_t launch_quantize_mfma(const QuantizeArgs& a, hipStream_t st) {
  if (a.n == 0 || a.seqs == 0) return hipSuccess;
  QuantMfmaParams p{};
  p.x = static_cast<const _Float16*>(a.x);
  p.seqs = a.seqs;
  p.n = a.n;
  p.t0 = a.t0;
  p.cap = a.cap;
  p.tile_first = a.t0 / 8;
  p.tile_last = (a.t0 + a.n - 1) / 8;
  p.rot_hi = static_cast<const _Float16*>(a.rot_hi);
  p.rot_lo = static_cast<const _Float16*>(a.rot_lo);
  p.projr_hi = static_cast<const _Float16*>(a.projr_hi);
  p.projr_lo = static_cast<const _Float16*>(a.projr_lo);
  p.cent = a.cent;
  p.bnd = a.bnd;
  p.idx = a.idx;
  p.sign = a.sign;
  p.norm = a.norm;
  p.rnorm = a.rnorm;
  const int64_t groups = a.seqs * ((p.tile_last - p.tile_first + 1 + 3) / 4);
  if (a.value_layout) return dispatch_bits<0, 1>(p, a.bits, groups, st);
  if (a.qjl) return dispatch_bits<1, 0>(p, a.bits, groups, st);
  return dispatch_bits<0, 0>(p, a.bits, groups, st);
}

}  // namespace tq
