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
//  * Weights are stationary: wave w of a workgroup keeps the rows of 32 output
//    coordinates in VGPRs for the whole kernel; tokens stream through LDS in
//    tiles of 4 x 8 tokens (one 8-token value tile each), the workgroup looping
//    over tiles (persistent grid).
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
#include "tq_quant_common.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots = 32;  // tokens per tile: 4 value tiles of 8

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Output coordinate held by weight row rho (0..15) of coordinate tile ct in
// wave w: lanes of group g = rho/4 get 8 consecutive coordinates 32w + 8g + 4ct + rho%4.
__device__ __forceinline__ int out_coord(int w, int ct, int rho) {
  return 32 * w + 8 * (rho / 4) + 4 * ct + (rho % 4);
}

// Two waves per SIMD for keys (the stationary weights of the rotation and the
// projection take half the registers), three for values.
template <int BITS, int QJL, int VALUES>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(VALUES ? 3 : 2)))
quantize_mfma_kernel(QuantMfmaParams p) {
  __shared__ __align__(16) _Float16 xs[kSlots][D + 8];       // token rows (padded)
  __shared__ __align__(16) _Float16 rs[2][kSlots][D + 8];    // residual hi / lo
  __shared__ float nrm[kSlots];
  __shared__ float rsq[kSlots][16];
  constexpr bool kTable = BITS >= 3;  // 3- and 4-bit codes from the binned table
  __shared__ __align__(16) uint2 ctabl[kTable ? kCodeTableEntries : 1];

  const int tid = threadIdx.x;
  const int w = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;

  // Stationary weights: rows out_coord(w, ct, l16), columns 32 kb + 8 g4 + e.
  h8 wr[2][4][2], wp[QJL ? 2 : 1][4][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = out_coord(w, ct, l16);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int col = 32 * kb + 8 * g4;
      wr[ct][kb][0] = *reinterpret_cast<const h8*>(p.rot_hi + row * D + col);
      wr[ct][kb][1] = *reinterpret_cast<const h8*>(p.rot_lo + row * D + col);
      if constexpr (QJL) {
        wp[ct][kb][0] = *reinterpret_cast<const h8*>(p.projr_hi + row * D + col);
        wp[ct][kb][1] = *reinterpret_cast<const h8*>(p.projr_lo + row * D + col);
      }
    }
  }
  // Positive half of the symmetric boundaries, and the centroids as a register
  // table (lane i holds c[i mod 16]) read with ds_bpermute.
  constexpr int KP = BITS > 1 ? (1 << (BITS - 1)) - 1 : 1;
  float beta[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) beta[i] = BITS > 1 ? p.bnd[(1 << (BITS - 1)) + i] : 0.f;
  const int ctab = __float_as_int(p.cent[lane % 16]);
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float ubin = sqrtf((float)D) * kBinScale;  // unit-vector coordinate -> bin units
  if constexpr (kTable) {
    fill_code_table<BITS>(ctabl, p.bnd, ubin, tid, kThreads);
    __syncthreads();
  }
  const uint2* ctab_lane = ctabl + (kTable ? lane % kBinCopies : 0);

  // Work unit: 4 consecutive value tiles (32 token slots) of one sequence.
  const int tiles = (int)(p.tile_last - p.tile_first + 1);  // tiles per sequence touched
  const int gps = (tiles + 3) / 4;                             // groups per sequence
  const int groups = (int)p.seqs * gps;  // < 2^31 (checked on the host)
  const int t0 = (int)p.t0, tend = (int)(p.t0 + p.n);
  const int rowb = D * BITS / 8;

  // Loader role: 8 threads per token slot, 16 halves each.
  const int lslot = tid / 8, lpart = tid % 8;
  auto load_x = [&](int grp, h8& v0, h8& v1) {
    v0 = h8{0, 0, 0, 0, 0, 0, 0, 0};
    v1 = v0;
    if (grp >= groups) return;
    const int64_t s = grp / gps;  // uniform
    const int tile = (int)p.tile_first + 4 * (grp % gps) + lslot / 8;
    const int t = tile * 8 + lslot % 8;
    if (4 * (grp % gps) + lslot / 8 < tiles && t >= t0 && t < tend) {
      const _Float16* src = p.x + s * p.n * D + (t - t0) * D + lpart * 16;
      v0 = *reinterpret_cast<const h8*>(src);
      v1 = *reinterpret_cast<const h8*>(src + 8);
    }
  };
  h8 nx0, nx1;
  load_x((int)blockIdx.x, nx0, nx1);

  for (int grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t s = grp / gps;  // wave-uniform: scalar
    const int gt = 4 * (grp % gps);  // first tile of the group, relative to tile_first
    // ---- token rows into LDS, with their norms; prefetch the next group ----
    {
      const h8 v0 = nx0, v1 = nx1;
      *reinterpret_cast<h8*>(&xs[lslot][lpart * 16]) = v0;
      *reinterpret_cast<h8*>(&xs[lslot][lpart * 16 + 8]) = v1;
      // Sum of squares: fp16 products are exact in fp32; two independent
      // chains of packed dot products.
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const h2 a{v0[e], v0[e + 1]}, b{v1[e], v1[e + 1]};
        s0 = __builtin_amdgcn_fdot2(a, a, s0, false);
        s1 = __builtin_amdgcn_fdot2(b, b, s1, false);
      }
      float ss = s0 + s1;
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      if (lpart == 0) nrm[lslot] = __builtin_amdgcn_sqrtf(ss);
      load_x(grp + (int)gridDim.x, nx0, nx1);
    }
    __syncthreads();

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
      uint8_t* idx_s = p.idx + s * p.cap * rowb;
      // Lane (g4, l16) holds coordinates 32w + 8g4 + 4ct + r of token slot 16tt + l16.
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int slot = 16 * tt + l16;
        const int t = ((int)p.tile_first + gt + slot / 8) * 8 + slot % 8;
        const bool ok = gt + slot / 8 < tiles && t >= t0 && t < tend;
        const float nn = nrm[slot];
        const float inv = nn > 0.f ? inv_sqrt_d * __builtin_amdgcn_rcpf(nn) : 0.f;
        uint32_t packed = 0;
        float r[8];
        float rr = 0.f;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float y = acc[ct][tt][q] * inv;
            uint32_t code;
            if constexpr (kTable) code = table_code(ctab_lane, fmaf(acc[ct][tt][q], inv * ubin, 0.5f * kBins));
            else code = symmetric_code<BITS>(y, beta);
            const float c = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(code << 2), ctab));
            packed |= code << (BITS * (4 * ct + q));
            r[4 * ct + q] = y - c;
            rr = fmaf(r[4 * ct + q], r[4 * ct + q], rr);
          }
        if (ok) {
          uint8_t* dst = idx_s + t * rowb + (4 * w + g4) * BITS;
#pragma unroll
          for (int b = 0; b < BITS; ++b) dst[b] = (uint8_t)(packed >> (8 * b));
          if (w == 0 && g4 == 0) p.norm[s * p.cap + t] = nn;
        }
        if constexpr (QJL) {
          h8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = r[e] * 64.f;  // keep the lo half away from fp16 subnormals
            hi[e] = (_Float16)v;
            lo[e] = (_Float16)(v - (float)hi[e]);
          }
          *reinterpret_cast<h8*>(&rs[0][slot][32 * w + 8 * g4]) = hi;
          *reinterpret_cast<h8*>(&rs[1][slot][32 * w + 8 * g4]) = lo;
          rsq[slot][4 * w + g4] = rr;
        }
      }
      if constexpr (QJL) {
        __syncthreads();
        f4 pacc[2][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) pacc[ct][tt] = f4{0.f, 0.f, 0.f, 0.f};
        // Same one-step-ahead operand reads as the rotation.
        auto r_operand = [&](int st, int part) {
          const int kb = st / 2, tt = st % 2;
          return *reinterpret_cast<const h8*>(&rs[part][16 * tt + l16][32 * kb + 8 * g4]);
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
        uint8_t* sign_s = p.sign + s * p.cap * (D / 8);
        float* rn_s = p.rnorm + s * p.cap;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int slot = 16 * tt + l16;
          const int t = ((int)p.tile_first + gt + slot / 8) * 8 + slot % 8;
          const bool ok = gt + slot / 8 < tiles && t >= t0 && t < tend;
          uint32_t bits = 0;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int q = 0; q < 4; ++q)  // sign bit of the float, inverted: 1 for >= +0
              bits |= ((__float_as_uint(pacc[ct][tt][q]) >> 31) ^ 1u) << (4 * ct + q);
          if (ok) {
            sign_s[t * (D / 8) + 4 * w + g4] = (uint8_t)bits;
            if (w == 0 && g4 == 0) {
              float g = 0.f;
#pragma unroll
              for (int i = 0; i < 16; ++i) g += rsq[slot][i];
              rn_s[t] = __builtin_amdgcn_sqrtf(g);
            }
          }
        }
      }
    } else {
      // Lane (g4, l16) holds, for coordinate tile ct, coordinate out_coord(w, ct, l16)
      // of the 8 tokens of value tile g4 (token 4 tt + r in D row 4 g4 + r of tile tt).
      const bool tile_ok = gt + g4 < tiles;
      const int tile = (int)p.tile_first + gt + g4;
      uint32_t keep = 0;  // code bits of tokens outside [t0, t0+n) are left unchanged
      float inv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t = tile * 8 + k;
        const bool ok = t >= t0 && t < tend;
        if (!ok) keep |= ((1u << BITS) - 1u) << (BITS * k);
        const float nn = nrm[8 * g4 + k];
        inv[k] = nn > 0.f ? inv_sqrt_d * __builtin_amdgcn_rcpf(nn) : 0.f;
      }
      // Norms: lane l16 < 8 of wave 0 stores token l16 of value tile g4.
      if (w == 0 && l16 < 8 && tile_ok) {
        const int t = tile * 8 + l16;
        if (t >= t0 && t < tend) p.norm[s * p.cap + t] = nrm[8 * g4 + l16];
      }
      uint8_t* tile_base = p.idx + s * (p.cap / 8) * (D * BITS) + tile * (D * BITS);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        uint32_t packed = 0;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = 4 * tt + q;
            if constexpr (kTable)
              packed |= table_code(ctab_lane, fmaf(acc[ct][tt][q], inv[k] * ubin, 0.5f * kBins)) << (BITS * k);
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
    __syncthreads();
  }
}

// Persistent grid: as many workgroups as the CUs hold at once (a second,
// partial round of workgroups would run the last share at low occupancy).
template <int BITS, int QJL, int VALUES>
hipError_t launch(const QuantMfmaParams& p, int64_t groups, hipStream_t st) {
  int dev = 0, cus = 256, per_cu = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quantize_mfma_kernel<BITS, QJL, VALUES>, kThreads, 0) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t slots = (int64_t)cus * per_cu;
  const int64_t grid = groups < slots ? groups : slots;
  hipLaunchKernelGGL((quantize_mfma_kernel<BITS, QJL, VALUES>), dim3((unsigned)grid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
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
