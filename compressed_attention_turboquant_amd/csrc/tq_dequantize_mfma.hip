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
// Rows written as fp16 take two products instead: R^T hi and lo times the
// centroids as single fp16 copies of s c, with the codebook factor s the
// decode tables use (chosen on the host so that every s c_i is within
// 1e-4 relative of its fp16 copy for every codebook built here, 2.3e-5 at
// 3 bits and 1e-6 at 1 and 2); the error before the output's rounding is
// then below 1.1e-4 of the norm, and 1/(16 s) goes into the norm.
// A lane's accumulator holds 4 consecutive coordinates of one token, stored as
// one float4 (or 4 halves).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>
#include <type_traits>

#include "tq_kernels.h"
#include "tq_quant_common.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;        // tokens per workgroup step
constexpr float kFactor = 16.f;  // scale of R^T and of the centroids

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;  // past every record used here
__device__ __forceinline__ Rsrc record(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);  // raw buffer
}

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

// QJL term of the two-stage reconstruction ([Mobilint] "Two-Stage Approach",
// stage 2 and the final reconstruction):
//   x_hat += n * sqrt(pi/2)/d * gamma * S^T sigma.
//
// Y^T[j][t] = sum_k S^T[j][k] sigma_t[k] runs on v_mfma_f32_16x16x32_f16 with
// output coordinates as rows and tokens as columns.  The B operand comes
// straight from the packed sign bits: a half whose only set bit is exponent
// bit p is 2^(2^(p-10) - 15), so rotating a token's 32 sign bits and masking
// bits 10+w and 26+w (w = 0..3) gives four dwords of such powers (or 0), one
// AND each.  The A operand carries S^T times the inverse powers (and 1/8, so
// that it stays inside the fp16 range), split hi + lo; the product is
// M = sum over sigma = +1 of S^T / 8, and S^T sigma = 16 M - sum_k S^T[j][k].
// Lane (row block, k-group g4) of k-block kb covers coordinate
// 32 kb + ((10 + w + 16 h + 4 g4) mod 32) with its element e = 2 w + h; the
// four k-groups together cover the block's 32 coordinates.
constexpr float kSignScale = 0.125f;

__device__ __forceinline__ float sign_power_inverse(int w) {  // 2^(15 - 2^w)
  return w == 0 ? 16384.f : w == 1 ? 8192.f : w == 2 ? 2048.f : 128.f;
}

// Stationary A operand of the QJL product for rows j = 32 wave + 16 jb + l16
// of S^T, in the coordinate order of the sign operand, and the row sums of S^T
// for the lane's accumulator rows (32 wave + 16 jb + 4 g4 + r).
template <int D>
__device__ __forceinline__ void sign_operand(const float* St, int wave, int l16, int g4, h8 (&shi)[2][D / 32],
                                             h8 (&slo)[2][D / 32], float (&rs)[2][4]) {
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int row = 32 * wave + 16 * jb + l16;
    float part = 0.f;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      h8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e / 2, h = e % 2;
        const int coord = 32 * kb + ((10 + w + 16 * h + 4 * g4) & 31);
        const float v = St[(size_t)row * D + coord];
        part += v;
        const float x = v * kSignScale * sign_power_inverse(w);
        hi[e] = (_Float16)x;
        lo[e] = (_Float16)(x - (float)hi[e]);
      }
      shi[jb][kb] = hi;
      slo[jb][kb] = lo;
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) rs[jb][r] = __shfl(part, 4 * g4 + r);
  }
}

// B operand of the QJL product from one sign dword of a token (k-group g4).
__device__ __forceinline__ h8 sign_b(uint32_t sw, int g4) {
  const uint32_t rot = __builtin_amdgcn_alignbit(sw, sw, 4 * g4);
  u4 b;
  sfor<0, 4>([&](auto w) {
    constexpr int W = decltype(w)::value;
    b[W] = rot & ((1u << (10 + W)) | (1u << (26 + W)));
  });
  return __builtin_bit_cast(h8, b);
}

// DITHER: the dithered variant, x_hat = n * R^T (c[idx] + delta): the offset
// term n * delta * (R^T 1)_j is added with the row sums of R^T.
// QJL: keys with QJL, the two-stage reconstruction in one pass: each tile's
// sign dwords go to LDS beside its codes, and the QJL product runs on the
// same accumulator rows with its own chain, so the rows are stored once.
// fp16 rows take S^T's hi part only: each element is then off by at most
// 2^-11 of itself, which over the d signs puts about 2^-11 sqrt(d) of
// sqrt(pi/2)/d gamma on a coordinate (near 1e-5 of the norm at 3 bits, d = 128),
// below the rounding of the fp16 output itself.  Instantiated for d = 64 and
// 128: at 256, S^T's registers beside R^T's would not fit.
template <int D, int BITS, int VALUES, int OUT16, int DITHER, int QJL>
__global__ void __launch_bounds__(2 * D) dequant_mfma_kernel(DequantArgs a) {
  constexpr int W = D / 32;           // waves: each owns 32 output coordinates
  constexpr int T = 64 * W;           // threads: 2 D, one per 32 codes of a tile
  constexpr int NKB = D / 32;         // k-blocks of the MFMA
  constexpr int PITCH = D + 8;        // LDS row pitch (halves): rows 16 bytes apart in the banks
  constexpr int kPairs = 1 << (2 * BITS);
  // code pair -> {two fp16 hi parts, two fp16 lo parts} (first code in the low
  // halves); fp16 rows: the two fp16 copies of s c only.
  using Pair = std::conditional_t<OUT16 != 0, uint32_t, u2>;
  __shared__ __align__(8) Pair tpair[kPairs];
  __shared__ __align__(16) _Float16 bhi[kTile][PITCH], blo[OUT16 ? 1 : kTile][OUT16 ? 8 : PITCH];
  __shared__ float nsh[kTile];
  __shared__ float dsh[DITHER ? kTile : 1];  // dithered variant: the tile's offsets, times kFactor^2
  // QJL: the tile's sign dwords (token, k-block) and n sqrt(pi/2)/d gamma.
  __shared__ __align__(16) uint32_t sgs[QJL ? kTile : 1][NKB];
  __shared__ float fsh[QJL ? kTile : 1];
  // fp16 rows: the finished tile is staged here and written back as whole
  // rows, 16 bytes per lane (the accumulator layout would write 8-byte pieces
  // of 16 rows per instruction, which measured at about half the HBM rate).
  __shared__ __align__(16) _Float16 ot[OUT16 ? kTile : 1][OUT16 ? PITCH : 8];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;

  const float cs = OUT16 ? *a.cscale : kFactor;  // factor of the centroid operand
  for (int i = tid; i < kPairs; i += T) {
    const float c0 = a.cent[i & ((1 << BITS) - 1)] * cs, c1 = a.cent[i >> BITS] * cs;
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    if constexpr (OUT16) {
      tpair[i] = hbits(h0) | (hbits(h1) << 16);
    } else {
      const _Float16 e0 = (_Float16)(c0 - (float)h0), e1 = (_Float16)(c1 - (float)h1);
      tpair[i] = u2{hbits(h0) | (hbits(h1) << 16), hbits(e0) | (hbits(e1) << 16)};
    }
  }
  const float nscale = 1.f / (kFactor * cs);  // the operands' factors, undone with the norm

  // This wave's rows of 16 R^T: row j = 32 wave + 16 jb + l16, k = 32 kb + 8 g4 + e.
  h8 ahi[2][NKB], alo[2][NKB];
  float rpart[2] = {0.f, 0.f};  // dithered variant: partial row sums of R^T
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
        if constexpr (DITHER) rpart[jb] += e < 4 ? x0[e] : x1[e - 4];
      }
      ahi[jb][kb] = hi;
      alo[jb][kb] = lo;
    }
  }
  // Row sums for the accumulator's rows 32 wave + 16 jb + 4 g4 + r: lane l16
  // of every k-group holds row 16 jb + l16 once the k-groups are summed.
  f4 rsum[2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    rsum[jb] = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (DITHER) {
      float r = rpart[jb];
      r += __shfl_xor(r, 16);
      r += __shfl_xor(r, 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) rsum[jb][i] = __shfl(r, 4 * g4 + i);
    }
  }
  const float dwidth = DITHER ? *a.dither_w : 0.f;
  h8 shi[2][NKB], slo[2][NKB];
  float qrs[2][4];
  if constexpr (QJL) sign_operand<D>(a.St, wave, l16, g4, shi, slo, qrs);
  const float kappa = sqrtf(0.5f * (float)M_PI) / (float)D;

  const int64_t n = a.n, cap = a.cap;
  const int64_t tiles = (n + kTile - 1) / kTile;
  const int64_t items = a.seqs * tiles;
  // Items item0 + i * gridDim.x: (sequence, tile) advance by a precomputed
  // step with one carry, no division per tile.
  const int64_t step_s = (int64_t)gridDim.x / tiles, step_t = (int64_t)gridDim.x % tiles;
  int64_t item = blockIdx.x, seq = item / tiles, tile = item % tiles;
  auto advance = [&](int64_t& it, int64_t& sq, int64_t& tl) {
    it += gridDim.x;
    sq += step_s;
    tl += step_t;
    if (tl >= tiles) {
      tl -= tiles;
      sq += 1;
    }
  };
  // The thread's 32 codes of a tile (and, for threads < 64, a token's norm)
  // are loaded one tile ahead, so that the loads are in flight while the
  // matrix cores work on the previous tile.  Loads and stores are buffer
  // instructions on per-tile records with out-of-range offsets (a load returns
  // 0, a store is dropped) instead of branches, so every tile issues the same
  // memory instructions and the compiler's waits can count them.
  uint32_t w[BITS];
  float nrm = 0.f;
  uint32_t sgw = 0;  // QJL: the thread's sign dword (token tid / NKB, k-block tid % NKB)
  float rn = 0.f;    // QJL: a token's gamma (threads < 64)
  auto load_codes = [&](int64_t it, int64_t sq, int64_t tl) {
    const bool live = it < items;  // uniform
    const int64_t t0 = tl * kTile;
    const int64_t rows = live ? min(n - t0, (int64_t)kTile) : 0;  // tokens of the tile
    uint32_t off;
    const uint8_t* base;
    int64_t bytes;
    if constexpr (VALUES) {
      // Value tiles of 8 tokens: code 8 k + i is coordinate k of token i, so
      // the thread's codes are coordinates 4q..4q+3 of the tile's 8 tokens.
      const int vt = tid / (D / 4), q = tid % (D / 4);
      base = a.idx + (sq * (cap / 8) + t0 / 8) * (D * BITS);
      bytes = (rows + 7) / 8 * (D * BITS);
      off = 8 * vt < rows ? (uint32_t)(vt * (D * BITS) + q * 4 * BITS) : kOob;
    } else {
      const int tt = tid / NKB, q = tid % NKB;
      base = a.idx + (sq * cap + t0) * (D * BITS / 8);
      bytes = rows * (D * BITS / 8);
      off = tt < rows ? (uint32_t)(tt * (D * BITS / 8) + q * 4 * BITS) : kOob;
    }
    const Rsrc rc = record(base, bytes);
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, off + 4 * i, 0, 0);
    nrm = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(record(a.norm + sq * cap + t0, 4 * rows),
                                                               tid < kTile ? 4u * tid : kOob, 0, 0));
    if constexpr (QJL) {
      const int tt = tid / NKB, q = tid % NKB;
      sgw = __builtin_amdgcn_raw_buffer_load_b32(record(a.sign + (sq * cap + t0) * (D / 8), rows * (D / 8)),
                                                 tt < rows ? (uint32_t)(tt * (D / 8) + 4 * q) : kOob, 0, 0);
      rn = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(record(a.rnorm + sq * cap + t0, 4 * rows),
                                                                tid < kTile ? 4u * tid : kOob, 0, 0));
    }
  };
  load_codes(item, seq, tile);
  if constexpr (!OUT16) {
    // The loop's own path to its top has the tile's stores after these loads;
    // as many dropped stores to an empty record give the path from here the
    // same count, so the wait at the top leaves the stores in flight.
    const Rsrc none = record(a.norm, 0);
#pragma unroll
    for (int i = 0; i < 2 * (kTile / 16); ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 64 * i, 0, 0);
  }
  // fp16 rows: the staged tile (sequence pseq, first token pt0, prows rows;
  // none before the first) is written back at the top of the next iteration,
  // beside that tile's decode.  Every thread stores 4 x 16 bytes; rows past
  // the tile's end (or no tile) get an offset past the record.
  int64_t pseq = 0, pt0 = 0, prows = 0;
  auto write_tile = [&]() {
    constexpr int kCpr = D / 8;  // 16-byte chunks per row
    const Rsrc prec = record(static_cast<uint8_t*>(a.out) + (pseq * n + pt0) * D * 2, prows * D * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + T * i, row = c / kCpr, part = c % kCpr;
      const u4 v = *reinterpret_cast<const u4*>(&ot[row][8 * part]);
      __builtin_amdgcn_raw_buffer_store_b128(v, prec, row < prows ? (uint32_t)(row * D * 2 + part * 16) : kOob, 0, 0);
    }
  };
  int64_t nitem = item, nseq = seq, ntile = tile;
  advance(nitem, nseq, ntile);
  for (; item < items; item = nitem, seq = nseq, tile = ntile, advance(nitem, nseq, ntile)) {
    const int64_t t0 = tile * kTile;
    lds_barrier();  // the previous tile's operands have been read (and its output staged)
    if constexpr (OUT16) write_tile();
    // Decode: thread -> 32 consecutive codes of the packed stream.
    {
      uint32_t ph[16], pl[16];
      sfor<0, 16>([&](auto p) {
        const Pair e = tpair[bits_at<2 * BITS * p, 2 * BITS>(w)];
        if constexpr (OUT16) {
          ph[p] = e;
        } else {
          ph[p] = e[0];
          pl[p] = e[1];
        }
      });
      if constexpr (VALUES) {
        // Token i of the tile: pairs p = 4 kk + i / 2 (kk = 0..3), its half i % 2.
        const int vt = tid / (D / 4), q = tid % (D / 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t sel = i % 2 ? 0x07060302u : 0x05040100u;
          const int p0 = i / 2;
          const u2 vh = {__builtin_amdgcn_perm(ph[p0 + 4], ph[p0], sel), __builtin_amdgcn_perm(ph[p0 + 12], ph[p0 + 8], sel)};
          *reinterpret_cast<u2*>(&bhi[8 * vt + i][4 * q]) = vh;
          if constexpr (!OUT16) {
            const u2 vl = {__builtin_amdgcn_perm(pl[p0 + 4], pl[p0], sel), __builtin_amdgcn_perm(pl[p0 + 12], pl[p0 + 8], sel)};
            *reinterpret_cast<u2*>(&blo[8 * vt + i][4 * q]) = vl;
          }
        }
      } else {
        const int tt = tid / NKB, q = tid % NKB;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          *reinterpret_cast<u4*>(&bhi[tt][32 * q + 8 * c]) = u4{ph[4 * c], ph[4 * c + 1], ph[4 * c + 2], ph[4 * c + 3]};
          if constexpr (!OUT16)
            *reinterpret_cast<u4*>(&blo[tt][32 * q + 8 * c]) = u4{pl[4 * c], pl[4 * c + 1], pl[4 * c + 2], pl[4 * c + 3]};
        }
      }
      if (tid < kTile) nsh[tid] = nrm * nscale;
      if constexpr (DITHER) {
        if (tid < kTile) dsh[tid] = dither_offset(a.dither_s0, seq, t0 + tid, dwidth) * (kFactor * cs);
      }
      if constexpr (QJL) {
        sgs[tid / NKB][tid % NKB] = sgw;
        if (tid < kTile) fsh[tid] = nrm * kappa * rn;
      }
    }
    lds_barrier();
    load_codes(nitem, nseq, ntile);
    // Sixteen tokens at a time: B operand lane (token l16, k-group g4); the
    // rows past n of the last tile are computed and not stored.
    const int64_t rows = min(n - t0, (int64_t)kTile);
    const Rsrc orec = record(static_cast<uint8_t*>(a.out) + (seq * n + t0) * D * (OUT16 ? 2 : 4),
                             rows * D * (OUT16 ? 2 : 4));
#pragma unroll
    for (int s = 0; s < kTile / 16; ++s) {
      h8 bh[NKB], bl[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        bh[kb] = *reinterpret_cast<const h8*>(&bhi[16 * s + l16][32 * kb + 8 * g4]);
        if constexpr (!OUT16) bl[kb] = *reinterpret_cast<const h8*>(&blo[16 * s + l16][32 * kb + 8 * g4]);
      }
      const int tok = 16 * s + l16;
      const float nt = nsh[tok];
      const float dl = DITHER ? dsh[tok] : 0.f;
      // Four independent accumulation chains (per row block: hi*hi, and the
      // correction products) so that no product waits on the one before it.
      f4 acc[2], cor[2], qacc[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) acc[jb] = cor[jb] = qacc[jb] = f4{0.f, 0.f, 0.f, 0.f};
      uint32_t sgv[NKB];  // the token's sign dwords
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sgv[kb] = QJL ? sgs[tok][kb] : 0u;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[jb][kb], bh[kb], acc[jb], 0, 0, 0);
          if constexpr (!OUT16) cor[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[jb][kb], bl[kb], cor[jb], 0, 0, 0);
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          cor[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[jb][kb], bh[kb], cor[jb], 0, 0, 0);
        if constexpr (QJL) {
          const h8 sb = sign_b(sgv[kb], g4);
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) {
            qacc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(shi[jb][kb], sb, qacc[jb], 0, 0, 0);
            if constexpr (!OUT16) qacc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(slo[jb][kb], sb, qacc[jb], 0, 0, 0);
          }
        }
      }
      const float fq = QJL ? fsh[tok] : 0.f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int col = 32 * wave + 16 * jb + 4 * g4;
        const uint32_t off = tok < rows ? (uint32_t)((tok * D + col) * (OUT16 ? 2 : 4)) : kOob;
        f4 v = acc[jb] + cor[jb];
        if constexpr (DITHER) v += dl * rsum[jb];
        v *= nt;
        if constexpr (QJL) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = fmaf(fq, fmaf(qacc[jb][r], 2.f / kSignScale, -qrs[jb][r]), v[r]);
        }
        if constexpr (OUT16) {
          const u2 hv = {hbits((_Float16)v[0]) | (hbits((_Float16)v[1]) << 16),
                         hbits((_Float16)v[2]) | (hbits((_Float16)v[3]) << 16)};
          *reinterpret_cast<u2*>(&ot[tok][col]) = hv;
          (void)off;
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), orec, off, 0, 0);
        }
      }
    }
    if constexpr (OUT16) {
      pseq = seq;
      pt0 = t0;
      prows = rows;
    }
  }
  if constexpr (OUT16) {
    lds_barrier();  // the last tile is staged
    write_tile();
  }
}

// Persistent grid: as many workgroups as the CUs hold at once, or one per
// tile if there are fewer.
template <int D, int BITS, int VALUES, int OUT16, int DITHER, int QJL = 0>
hipError_t launch(const DequantArgs& a, hipStream_t st) {
  auto kern = dequant_mfma_kernel<D, BITS, VALUES, OUT16, DITHER, QJL>;
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

template <int D, int BITS, int DITHER>
hipError_t dispatch_out(const DequantArgs& a, hipStream_t st) {
  const bool h = a.out_dtype == TQ_F16;
  if (a.value_layout) return h ? launch<D, BITS, 1, 1, DITHER>(a, st) : launch<D, BITS, 1, 0, DITHER>(a, st);
  return h ? launch<D, BITS, 0, 1, DITHER>(a, st) : launch<D, BITS, 0, 0, DITHER>(a, st);
}

template <int D, int BITS>
hipError_t dispatch_layout(const DequantArgs& a, hipStream_t st) {
  if (a.qjl) {
    // The fused pass: keys of undithered layers at d = 64 and 128 (at d = 256
    // the sign operand's registers beside R^T's do not fit).
    if constexpr (D <= 128) {
      if (a.value_layout || a.dither) return hipErrorInvalidValue;
      return a.out_dtype == TQ_F16 ? launch<D, BITS, 0, 1, 0, 1>(a, st) : launch<D, BITS, 0, 0, 0, 1>(a, st);
    }
    return hipErrorInvalidValue;
  }
  return a.dither ? dispatch_out<D, BITS, 1>(a, st) : dispatch_out<D, BITS, 0>(a, st);
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

// The QJL term alone, added to rows that dequant_mfma_kernel or
// dequant_fwht_kernel has written (the cases without the fused pass).
template <int D, int OUT16>
__global__ void __launch_bounds__(2 * D) dequant_qjl_kernel(DequantQjlArgs a) {
  constexpr int NKB = D / 32;      // k-blocks, = sign dwords per token
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;

  h8 shi[2][NKB], slo[2][NKB];
  float rs[2][4];
  sign_operand<D>(a.St, wave, l16, g4, shi, slo, rs);

  const float kappa = sqrtf(0.5f * (float)M_PI) / (float)D;
  const int64_t n = a.n, cap = a.cap;
  const int64_t tiles = (n + kTile - 1) / kTile;
  const int64_t items = a.seqs * tiles;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t seq = item / tiles;
    const int64_t t0 = (item % tiles) * kTile;
#pragma unroll
    for (int s = 0; s < kTile / 16; ++s) {
      if (t0 + 16 * s >= n) break;  // uniform
      const int64_t tok = t0 + 16 * s + l16;
      const bool live = tok < n;
      uint32_t sw[NKB];
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.sign + (seq * cap + tok) * (D / 8));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sw[kb] = live ? src[kb] : 0u;
      const float f = live ? a.norm[seq * cap + tok] * kappa * a.rnorm[seq * cap + tok] : 0.f;
      f4 acc[2];
      acc[0] = acc[1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const h8 bh = sign_b(sw[kb], g4);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(shi[jb][kb], bh, acc[jb], 0, 0, 0);
          acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(slo[jb][kb], bh, acc[jb], 0, 0, 0);
        }
      }
      if (live) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int64_t o = (seq * n + tok) * D + 32 * wave + 16 * jb + 4 * g4;
          f4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = f * (acc[jb][r] * (2.f / kSignScale) - rs[jb][r]);
          if constexpr (OUT16) {
            u2* dst = reinterpret_cast<u2*>(static_cast<__half*>(a.out) + o);
            const u2 old = *dst;
            const uint32_t v0 = old[0], v1 = old[1];
            const float x0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(v0 & 0xFFFFu)) + y[0];
            const float x1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(v0 >> 16)) + y[1];
            const float x2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(v1 & 0xFFFFu)) + y[2];
            const float x3 = (float)__builtin_bit_cast(_Float16, (uint16_t)(v1 >> 16)) + y[3];
            *dst = u2{hbits((_Float16)x0) | (hbits((_Float16)x1) << 16), hbits((_Float16)x2) | (hbits((_Float16)x3) << 16)};
          } else {
            f4* dst = reinterpret_cast<f4*>(static_cast<float*>(a.out) + o);
            *dst = *dst + y;
          }
        }
      }
    }
  }
}

template <int D, int OUT16>
hipError_t launch_qjl(const DequantQjlArgs& a, hipStream_t st) {
  auto kern = dequant_qjl_kernel<D, OUT16>;
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

}  // namespace

hipError_t launch_dequant_qjl(const DequantQjlArgs& a, hipStream_t st) {
  if (a.n == 0 || a.seqs == 0) return hipSuccess;
  const bool h = a.out_dtype == TQ_F16;
  switch (a.d) {
    case 64: return h ? launch_qjl<64, 1>(a, st) : launch_qjl<64, 0>(a, st);
    case 128: return h ? launch_qjl<128, 1>(a, st) : launch_qjl<128, 0>(a, st);
    default: return h ? launch_qjl<256, 1>(a, st) : launch_qjl<256, 0>(a, st);
  }
}

hipError_t launch_dequant_mfma(const DequantArgs& a, hipStream_t st) {
  if (a.n == 0 || a.seqs == 0) return hipSuccess;
  switch (a.d) {
    case 64: return dispatch_bits<64>(a, st);
    case 128: return dispatch_bits<128>(a, st);
    default: return dispatch_bits<256>(a, st);
  }
}

}  // namespace tq
