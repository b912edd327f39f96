// Dequantize on the matrix cores: x_hat = n * R^T c[idx] per token
// ([cuTile] listing, decompression function: codes -> centroids -> inverse
// rotation -> rescale by the stored norm; [Mobilint] "Two-Stage Approach",
// reconstruction from the rotated-domain codes).
//
// A workgroup of D/32 waves steps through tiles of 64 tokens of one sequence.
// Per tile it decodes the codes into fp16 hi/lo centroid values in LDS
// (c = hi + lo to ~2^-22 relative), then computes the transposed tile
// X^T[j][t] = sum_k R^T[j][k] C[k][t] with v_mfma_f32_16x16x32_f16: output
// coordinates are the MFMA rows, tokens its columns.  Each wave keeps its 32
// rows of R^T (split hi + lo, likewise) in registers for the whole run and
// adds three products per fragment (hi*hi + hi*lo + lo*hi; the dropped lo*lo
// term is below 2^-22 relative).  Both factors are scaled by 16 (exact) so
// that their lo parts stay normal fp16 numbers; 1/256 is folded into the norm.
// A lane's accumulator holds 4 consecutive coordinates of one token, stored as
// one float4 (or 4 halves).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>
#include <type_traits>

#include "tq_kernels.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;        // tokens per workgroup step
constexpr float kFactor = 16.f;  // scale of R^T and of the centroids

__device__ __forceinline__ uint32_t hbits(_Float16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

// Bits [O, O + N) of the little-endian stream w[] (N <= 8).
template <int O, int N, int NW>
__device__ __forceinline__ uint32_t bits_at(const uint32_t (&w)[NW]) {
  constexpr int wi = O / 32, sh = O % 32;
  constexpr uint32_t mask = (1u << N) - 1u;
  if constexpr (sh + N <= 32)
    return (w[wi] >> sh) & mask;
  else
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
}

template <int I, int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor<I + 1, N>(f);
  }
}

template <int D, int BITS, int VALUES, int OUT16>
__global__ void __launch_bounds__(2 * D) dequant_mfma_kernel(DequantArgs a) {
  constexpr int W = D / 32;           // waves: each owns 32 output coordinates
  constexpr int T = 64 * W;           // threads: 2 D, one per 32 codes of a tile
  constexpr int NKB = D / 32;         // k-blocks of the MFMA
  constexpr int PITCH = D + 8;        // LDS row pitch (halves): rows 16 bytes apart in the banks
  constexpr int kPairs = 1 << (2 * BITS);
  // code pair -> {two fp16 hi parts, two fp16 lo parts} (first code in the low halves)
  __shared__ __align__(8) u2 tpair[kPairs];
  __shared__ __align__(16) _Float16 bhi[kTile][PITCH], blo[kTile][PITCH];
  __shared__ float nsh[kTile];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;

  for (int i = tid; i < kPairs; i += T) {
    const float c0 = a.cent[i & ((1 << BITS) - 1)] * kFactor, c1 = a.cent[i >> BITS] * kFactor;
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const _Float16 e0 = (_Float16)(c0 - (float)h0), e1 = (_Float16)(c1 - (float)h1);
    tpair[i] = u2{hbits(h0) | (hbits(h1) << 16), hbits(e0) | (hbits(e1) << 16)};
  }

  // This wave's rows of 16 R^T: row j = 32 wave + 16 jb + l16, k = 32 kb + 8 g4 + e.
  h8 ahi[2][NKB], alo[2][NKB];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const f4* src = reinterpret_cast<const f4*>(a.Rt + (size_t)(32 * wave + 16 * jb + l16) * D + 32 * kb + 8 * g4);
      const f4 x0 = src[0], x1 = src[1];
      h8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (e < 4 ? x0[e] : x1[e - 4]) * kFactor;
        hi[e] = (_Float16)v;
        lo[e] = (_Float16)(v - (float)hi[e]);
      }
      ahi[jb][kb] = hi;
      alo[jb][kb] = lo;
    }
  }

  const int64_t n = a.n, cap = a.cap;
  const int64_t tiles = (n + kTile - 1) / kTile;
  const int64_t items = a.seqs * tiles;
  // The thread's 32 codes of a tile (and, for threads < 64, a token's norm)
  // are loaded one tile ahead, so that the loads are in flight while the
  // matrix cores work on the previous tile.
  uint32_t w[BITS];
  float nrm = 0.f;
  auto load_codes = [&](int64_t item) {
    const int64_t seq = item / tiles, t0 = (item % tiles) * kTile;
    bool live;
    const uint32_t* src;
    if constexpr (VALUES) {
      // Value tiles of 8 tokens: code 8 k + i is coordinate k of token i, so
      // the thread's codes are coordinates 4q..4q+3 of the tile's 8 tokens.
      const int vt = tid / (D / 4), q = tid % (D / 4);
      live = t0 + 8 * vt < n;
      src = reinterpret_cast<const uint32_t*>(a.idx + (seq * (cap / 8) + t0 / 8 + vt) * (D * BITS) + q * 4 * BITS);
    } else {
      const int tt = tid / NKB, q = tid % NKB;
      live = t0 + tt < n;
      src = reinterpret_cast<const uint32_t*>(a.idx + (seq * cap + t0 + tt) * (D * BITS / 8) + q * 4 * BITS);
    }
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = live ? src[i] : 0u;
    if (tid < kTile) nrm = t0 + tid < n ? a.norm[seq * cap + t0 + tid] * (1.f / (kFactor * kFactor)) : 0.f;
  };
  if (blockIdx.x < items) load_codes(blockIdx.x);
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t seq = item / tiles;
    const int64_t t0 = (item % tiles) * kTile;
    __syncthreads();  // the previous tile's operands have been read
    // Decode: thread -> 32 consecutive codes of the packed stream.
    {
      uint32_t ph[16], pl[16];
      sfor<0, 16>([&](auto p) {
        const u2 e = tpair[bits_at<2 * BITS * p, 2 * BITS>(w)];
        ph[p] = e[0];
        pl[p] = e[1];
      });
      if constexpr (VALUES) {
        // Token i of the tile: pairs p = 4 kk + i / 2 (kk = 0..3), its half i % 2.
        const int vt = tid / (D / 4), q = tid % (D / 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t sel = i % 2 ? 0x07060302u : 0x05040100u;
          const int p0 = i / 2;
          const u2 vh = {__builtin_amdgcn_perm(ph[p0 + 4], ph[p0], sel), __builtin_amdgcn_perm(ph[p0 + 12], ph[p0 + 8], sel)};
          const u2 vl = {__builtin_amdgcn_perm(pl[p0 + 4], pl[p0], sel), __builtin_amdgcn_perm(pl[p0 + 12], pl[p0 + 8], sel)};
          *reinterpret_cast<u2*>(&bhi[8 * vt + i][4 * q]) = vh;
          *reinterpret_cast<u2*>(&blo[8 * vt + i][4 * q]) = vl;
        }
      } else {
        const int tt = tid / NKB, q = tid % NKB;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          *reinterpret_cast<u4*>(&bhi[tt][32 * q + 8 * c]) = u4{ph[4 * c], ph[4 * c + 1], ph[4 * c + 2], ph[4 * c + 3]};
          *reinterpret_cast<u4*>(&blo[tt][32 * q + 8 * c]) = u4{pl[4 * c], pl[4 * c + 1], pl[4 * c + 2], pl[4 * c + 3]};
        }
      }
      if (tid < kTile) nsh[tid] = nrm;
    }
    __syncthreads();
    if (item + gridDim.x < items) load_codes(item + gridDim.x);
    // Sixteen tokens at a time: B operand lane (token l16, k-group g4).
    const int64_t left = n - t0;
#pragma unroll
    for (int s = 0; s < kTile / 16; ++s) {
      if (16 * s >= left) break;
      h8 bh[NKB], bl[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        bh[kb] = *reinterpret_cast<const h8*>(&bhi[16 * s + l16][32 * kb + 8 * g4]);
        bl[kb] = *reinterpret_cast<const h8*>(&blo[16 * s + l16][32 * kb + 8 * g4]);
      }
      const int tok = 16 * s + l16;
      const float nt = nsh[tok];
      // Four independent accumulation chains (per row block: hi*hi, and the two
      // correction products) so that no product waits on the one before it.
      f4 acc[2], cor[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) acc[jb] = cor[jb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[jb][kb], bh[kb], acc[jb], 0, 0, 0);
          cor[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[jb][kb], bl[kb], cor[jb], 0, 0, 0);
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          cor[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[jb][kb], bh[kb], cor[jb], 0, 0, 0);
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        if (tok < left) {
          const int64_t o = (seq * n + t0 + tok) * D + 32 * wave + 16 * jb + 4 * g4;
          const f4 v = (acc[jb] + cor[jb]) * nt;
          if constexpr (OUT16) {
            const u2 hv = {hbits((_Float16)v[0]) | (hbits((_Float16)v[1]) << 16),
                           hbits((_Float16)v[2]) | (hbits((_Float16)v[3]) << 16)};
            *reinterpret_cast<u2*>(static_cast<__half*>(a.out) + o) = hv;
          } else {
            *reinterpret_cast<f4*>(static_cast<float*>(a.out) + o) = v;
          }
        }
      }
    }
  }
}

// Persistent grid: as many workgroups as the CUs hold at once, or one per
// tile if there are fewer.
template <int D, int BITS, int VALUES, int OUT16>
hipError_t launch(const DequantArgs& a, hipStream_t st) {
  auto kern = dequant_mfma_kernel<D, BITS, VALUES, OUT16>;
  int dev = 0, cus = 256, per_cu = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 2 * D, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t items = a.seqs * ((a.n + kTile - 1) / kTile);
  const int64_t slots = (int64_t)cus * per_cu;
  const int64_t grid = items < slots ? items : slots;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(2 * D), 0, st, a);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t dispatch_layout(const DequantArgs& a, hipStream_t st) {
  const bool h = a.out_dtype == TQ_F16;
  if (a.value_layout) return h ? launch<D, BITS, 1, 1>(a, st) : launch<D, BITS, 1, 0>(a, st);
  return h ? launch<D, BITS, 0, 1>(a, st) : launch<D, BITS, 0, 0>(a, st);
}

template <int D>
hipError_t dispatch_bits(const DequantArgs& a, hipStream_t st) {
  switch (a.bits) {
    case 1: return dispatch_layout<D, 1>(a, st);
    case 2: return dispatch_layout<D, 2>(a, st);
    case 3: return dispatch_layout<D, 3>(a, st);
    default: return dispatch_layout<D, 4>(a, st);
  }
}

}  // namespace

hipError_t launch_dequant_mfma(const DequantArgs& a, hipStream_t st) {
  if (a.n == 0 || a.seqs == 0) return hipSuccess;
  switch (a.d) {
    case 64: return dispatch_bits<64>(a, st);
    case 128: return dispatch_bits<128>(a, st);
    default: return dispatch_bits<256>(a, st);
  }
}

}  // namespace tq
