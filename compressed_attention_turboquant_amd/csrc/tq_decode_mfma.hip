// Decode attention on the compressed cache with the matrix cores (gfx950).
//
// What is computed is the asymmetric estimator and softmax of [cuTile]
// "Asymmetric estimator: term1 (MSE dot) + term2 (QJL correction)" and "Fused
// attention + online softmax, decompresses ... V on-chip", with the query
// rotated once ([Mobilint] "Two-Stage Approach": <q, x~> = <Pi q, y~>):
//   s_t = n_t * (<R q, c_k[idx_t]> + gamma_t sqrt(pi/2)/d <S q, sigma_t>) / sqrt(d)
//   out = R^T (sum_t softmax(s)_t * nv_t * c_v[idxv_t]).
//
// How it maps to CDNA4 (one 64-lane wave works on 32 keys at a time):
//  * Both contractions run on v_mfma_f32_16x16x32_f16.  Scores: the 16 MFMA rows
//    are 4 query rows x {R q hi, R q lo, S q hi, S q lo}; the key operand stacks
//    the decoded centroids (d values) over the sign bits (d values), so one
//    accumulator holds, per (query row, key), the hi/lo parts of both terms in
//    the 4 registers of a single lane.  P.V: rows are {p hi, p lo} per query row
//    against the decoded value centroids; the sum stays in the rotated domain.
//  * The fp32 query splits into hi + lo halves (exact to ~2^-22).  Centroids are
//    used as fp16 copies of s*c with a per-codebook factor s chosen at set-up so
//    every s*c_i is within 2e-5 (3-bit) / 1e-4 (4-bit) of an fp16 value; 1/s is
//    folded into the query side.
//  * Code -> fp16 decode is a table lookup through ds_bpermute: each lane holds
//    one table entry (the fp16 pair for a pair of codes), and the packed stream
//    shifted so the pair lands in address bits [2, 8) selects it (the
//    instruction ignores the other address bits; tables are replicated when
//    the index is shorter).  One VALU op + one bpermute per fp16 pair.
//  * Sign bits become fp16 B-operand halves by masking: a half whose only set
//    bit is exponent bit p is the power of two 2^(2^(p-10)-15); rotating the
//    32 sign bits by 0/4/8/12 and masking bits p and p+16 (p = 10..13) yields
//    16 dwords with one AND each.  The query side carries the matching 2^(15 -
//    2^(p-10)) factors, so the MFMA returns sum_{sigma=+1} S q and the sign term
//    is 2 * that - sum S q.
//  * Softmax runs in the log2 domain with a lazily updated running maximum: the
//    accumulators are rescaled only in the (rare) blocks where a score exceeds
//    the current maximum of its row.
//  * Split-K over keys: grid (sequence, split); 4 waves per workgroup take every
//    4th block of 32 keys; their partial (max, sum, acc) merge in LDS and one
//    partial per split goes to the workspace for the combine kernel.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <type_traits>

#include "tq_kernels.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

template <int I, int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor<I + 1, N>(f);
  }
}

// Bits [O, ...) of the little-endian stream in w[], moved to bit 2 of the
// result (bits above the field are don't-care): a ds_bpermute byte address.
template <int O, int NW>
__device__ __forceinline__ uint32_t at2(const uint32_t (&w)[NW]) {
  if constexpr (O == 0) {
    return w[0] << 2;
  } else {
    constexpr int b = O - 2, wi = b / 32, sh = b % 32;
    if constexpr (sh == 0)
      return w[wi];
    else if constexpr (wi + 1 < NW)
      return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
    else
      return w[wi] >> sh;
  }
}

__device__ __forceinline__ uint32_t bperm(uint32_t addr, uint32_t table) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)addr, (int)table);
}

// fp16 pair of centroids for codes 2i, 2i+1 of the stream (bit offset O0 + 2*BITS*i).
template <int BITS, int O0, int I, int NW>
__device__ __forceinline__ uint32_t decode_pair(const uint32_t (&w)[NW], uint32_t t0, uint32_t t1) {
  if constexpr (BITS < 4) {
    return bperm(at2<O0 + 2 * BITS * I>(w), t0);
  } else {
    return bperm(at2<O0 + 8 * I>(w), t0) | bperm(at2<O0 + 8 * I + 4>(w), t1);
  }
}

__device__ __forceinline__ uint32_t half_bits(float x) {
  return (uint32_t)__half_as_ushort(__float2half_rn(x));
}

// This lane's entries of the code -> fp16 tables (see decode_pair).
template <int BITS>
__device__ __forceinline__ void make_tables(const float* c, float s, int lane, uint32_t& t0,
                                            uint32_t& t1) {
  if constexpr (BITS == 4) {
    const uint32_t h = half_bits(s * c[lane & 15]);
    t0 = h;
    t1 = h << 16;
  } else {
    constexpr int L = 1 << BITS;
    const int idx = lane & (L * L - 1);
    t0 = half_bits(s * c[idx % L]) | (half_bits(s * c[idx / L]) << 16);
    t1 = 0;
  }
}

// Sign-term B operand: k-block kb, dword w selects exponent bit p = 10 + w of the
// sign word rotated left by 4*(kb % 4), in both halves.
template <int W>
__device__ __forceinline__ uint32_t sign_dword(uint32_t rotated) {
  return rotated & ((1u << (10 + W)) | (1u << (26 + W)));
}

// Coordinate offset (within the lane's 32 sign bits) and query-side factor of
// sign slot (kb % 4 = r, dword w, half h).
__device__ __forceinline__ int sign_coord(int r, int w, int h) {
  return (10 + w + 16 * h - 4 * r) & 31;
}
__device__ __forceinline__ float sign_comp(int w) {  // 2^(15 - 2^w)
  return w == 0 ? 16384.f : w == 1 ? 8192.f : w == 2 ? 2048.f : 128.f;
}

template <int D, int KB, int QJL, int VB>
struct Shape {
  static constexpr int KBLK = D / 32;         // k-blocks of 32 coordinates
  static constexpr int NWK = KB * D / 128;    // key-code dwords per lane per 16 keys
  static constexpr int NSW = D / 128;         // sign dwords per lane per 16 keys
  static constexpr int NWV = D * VB / 64;     // value-code dwords per lane per 32 keys
  static constexpr int CB = D / 16;           // 16-coordinate output blocks
  static constexpr int KROW = D * KB / 8;     // key-code bytes per token
  static constexpr int VTILE = D * VB;        // value-code bytes per 8-token tile
};

template <int D, int KB, int QJL, int VB>
struct Block {
  using S = Shape<D, KB, QJL, VB>;
  uint32_t kw[2][S::NWK];
  uint32_t sw[2][QJL ? S::NSW : 1];
  float kn[2], kg[2], vn[2];
  uint32_t vw[S::NWV];
};

template <int N>
__device__ __forceinline__ void load_words(uint32_t (&dst)[N], const uint32_t* src, bool ok) {
#pragma unroll
  for (int i = 0; i < N; ++i) dst[i] = ok ? src[i] : 0u;
}

template <int D, int KB, int QJL, int VB>
__device__ __forceinline__ void load_block(Block<D, KB, QJL, VB>& b, const DecodeMfmaParams& p,
                                           int64_t seq, int64_t k0, int l16, int g4) {
  using S = Shape<D, KB, QJL, VB>;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t key = k0 + 16 * t + l16;
    const bool in = key < p.cap;
    const int64_t row = seq * p.cap + key;
    load_words(b.kw[t], reinterpret_cast<const uint32_t*>(p.kidx + row * S::KROW + g4 * (S::KROW / 4)), in);
    if constexpr (QJL)
      load_words(b.sw[t], reinterpret_cast<const uint32_t*>(p.ksign + row * (D / 8) + g4 * (D / 32)), in);
    const bool valid = key < p.N;
    b.kn[t] = valid ? p.knorm[row] : 0.f;
    b.kg[t] = (QJL && valid) ? p.krnorm[row] : 0.f;
    b.vn[t] = valid ? p.vnorm[row] : 0.f;
  }
  const int64_t vt = k0 / 8 + g4;
  const bool vin = vt < p.cap / 8;
  load_words(b.vw, reinterpret_cast<const uint32_t*>(p.vidx + (seq * (p.cap / 8) + vt) * S::VTILE +
                                                     l16 * (S::VTILE / 16)), vin);
}

template <int D, int KB, int QJL, int VB>
__global__ void __launch_bounds__(kThreads) decode_mfma_kernel(DecodeMfmaParams p) {
  using S = Shape<D, KB, QJL, VB>;
  __shared__ __align__(16) _Float16 pbuf[kWaves][2][4][32];
  __shared__ float mrg_m[kWaves][4], mrg_l[kWaves][4];
  __shared__ float mrg_acc[kWaves][4][D];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;
  const int64_t seq = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t b_ = seq / p.Hkv;
  const int hkv = (int)(seq % p.Hkv);
  const int G = p.Hq / p.Hkv;
  const int rows = G * p.Tq;
  auto qrow_of = [&](int r) -> int64_t { return (b_ * p.Hq + (int64_t)hkv * G + r / p.Tq) * p.Tq + r % p.Tq; };

  const float* ck = p.cb;
  const float* cv = p.cb + 2 * kMaxLevels;
  uint32_t kt0, kt1, vt0, vt1;
  const float scale_k = p.scales[0], scale_v = p.scales[1];
  make_tables<KB>(ck, scale_k, lane, kt0, kt1);
  make_tables<VB>(cv, scale_v, lane, vt0, vt1);

  // Query operands: lane (row rho = l16, k-group g4).
  h8 Ak[S::KBLK], As[QJL ? S::KBLK : 1];
  {
    const int qr = l16 / 4, part = l16 % 4;
    const bool ok = qr < rows;
    const int64_t qrow = ok ? qrow_of(qr) : 0;
    sfor<0, S::KBLK>([&](auto kb) {
      h8 a;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = 0.f;
        if (ok && part < 2) x = p.qa[qrow * D + (D / 4) * g4 + 8 * kb + e];
        const _Float16 hi = (_Float16)x;
        const _Float16 lo = (_Float16)(x - (float)hi);
        a[e] = part == 0 ? hi : (part == 1 ? lo : (_Float16)0.f);
      }
      Ak[kb] = a;
      if constexpr (QJL) {
        h8 s;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e / 2, h = e % 2;
          float x = 0.f;
          if (ok && part >= 2)
            x = p.qb[qrow * D + (D / 4) * g4 + 32 * (kb / 4) + sign_coord(kb % 4, w, h)] * sign_comp(w);
          const _Float16 hi = (_Float16)x;
          const _Float16 lo = (_Float16)(x - (float)hi);
          s[e] = part == 2 ? hi : (part == 3 ? lo : (_Float16)0.f);
        }
        As[kb] = s;
      }
    });
  }

  // Score-side constants of this lane's query row g4.
  float ca = 0.f, cb2 = 0.f, c2 = 0.f, c0 = 0.f;
  int64_t limit = -1;
  int64_t srow = 0;
  if (g4 < rows) {
    srow = qrow_of(g4);
    const float* rc = p.rowc + srow * 4;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    ca = rc[0] * inv_sqrt_d * kLog2e;
    cb2 = sqrtf(0.5f * (float)M_PI) / (float)D * inv_sqrt_d * kLog2e;
    c2 = rc[1];
    c0 = rc[2];
    limit = p.causal ? p.N - p.Tq + (g4 % p.Tq) + 1 : p.N;
  }

  f4 acc[S::CB];
#pragma unroll
  for (int i = 0; i < S::CB; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, msafe = 0.f, lsum = 0.f;

  const int64_t nblk = (p.N + 31) / 32;
  const int64_t blk0 = (int64_t)split * (p.keys_per_split / 32);
  const int64_t blk1 = min(nblk, blk0 + p.keys_per_split / 32);

  Block<D, KB, QJL, VB> cur;
  int64_t blk = blk0 + wave;
  if (blk < blk1) load_block(cur, p, seq, blk * 32, l16, g4);
  for (; blk < blk1; blk += kWaves) {
    Block<D, KB, QJL, VB> nxt;
    const bool more = blk + kWaves < blk1;
    if (more) load_block(nxt, p, seq, (blk + kWaves) * 32, l16, g4);
    const int64_t k0 = blk * 32;

    float st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f4 sacc = f4{0.f, 0.f, 0.f, 0.f};
      sfor<0, S::KBLK>([&](auto kb) {
        u4 bw;
        sfor<0, 4>([&](auto w) { bw[decltype(w)::value] = decode_pair<KB, 0, 4 * kb + w>(cur.kw[t], kt0, kt1); });
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ak[kb], __builtin_bit_cast(h8, bw), sacc, 0, 0, 0);
      });
      if constexpr (QJL) {
        sfor<0, S::KBLK>([&](auto kb) {
          const uint32_t word = cur.sw[t][kb / 4];
          constexpr int r = kb % 4;
          const uint32_t rot = r == 0 ? word : __builtin_amdgcn_alignbit(word, word, 32 - 4 * r);
          u4 bw;
          sfor<0, 4>([&](auto w) { bw[decltype(w)::value] = sign_dword<decltype(w)::value>(rot); });
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(As[kb], __builtin_bit_cast(h8, bw), sacc, 0, 0, 0);
        });
      }
      // lane (query row g4, key l16)
      float s = (cur.kn[t] * ca) * (sacc[0] + sacc[1]);
      if constexpr (QJL) s = fmaf(cur.kn[t] * cur.kg[t] * cb2, fmaf(c2, sacc[2] + sacc[3], c0), s);
      const int64_t key = k0 + 16 * t + l16;
      s = key < limit ? s : -INFINITY;
      if (p.scores && g4 < rows && key < p.N) p.scores[srow * p.N + key] = s * kLn2;
      st[t] = s;
    }

    const float mx = fmaxf(st[0], st[1]);
    if (__any(mx > m)) {
      float rmax = mx;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o));
      const float mnew = fmaxf(m, rmax);
      const float alpha = mnew == -INFINITY ? 1.f : exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < S::CB; ++i) acc[i] *= alpha;
      m = mnew;
      msafe = m == -INFINITY ? 0.f : m;
    }
    const float p0 = exp2f(st[0] - msafe), p1 = exp2f(st[1] - msafe);
    lsum += p0 + p1;
    const float q0 = p0 * cur.vn[0], q1 = p1 * cur.vn[1];
    const _Float16 h0 = (_Float16)q0, h1 = (_Float16)q1;
    pbuf[wave][0][g4][l16] = h0;
    pbuf[wave][0][g4][16 + l16] = h1;
    pbuf[wave][1][g4][l16] = (_Float16)(q0 - (float)h0);
    pbuf[wave][1][g4][16 + l16] = (_Float16)(q1 - (float)h1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    h8 ap;
    {
      const int part = l16 % 4, qr = l16 / 4;
      if (part < 2)
        ap = *reinterpret_cast<const h8*>(&pbuf[wave][part][qr][8 * g4]);
      else
        ap = h8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    sfor<0, S::CB>([&](auto cb) {
      u4 bw;
      sfor<0, 4>([&](auto w) { bw[decltype(w)::value] = decode_pair<VB, 8 * VB * cb, w>(cur.vw, vt0, vt1); });
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(h8, bw), acc[cb], 0, 0, 0);
    });
    __builtin_amdgcn_wave_barrier();
    if (more) cur = nxt;
  }

  // Merge the waves of this workgroup.
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) lsum += __shfl_xor(lsum, o);
  if (l16 == 0) {
    mrg_m[wave][g4] = m;
    mrg_l[wave][g4] = lsum;
  }
  const float inv_sv = 1.0f / scale_v;
#pragma unroll
  for (int cb = 0; cb < S::CB; ++cb) mrg_acc[wave][g4][l16 * S::CB + cb] = (acc[cb][0] + acc[cb][1]) * inv_sv;
  __syncthreads();
  const int64_t rows_total = (int64_t)gridDim.x / p.Hkv * p.Hq * p.Tq;
  for (int idx = tid; idx < rows * D; idx += kThreads) {
    const int r = idx / D, j = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg_m[w][r]);
    float a = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(mrg_m[w][r] - M);
        a = fmaf(f, mrg_acc[w][r][j], a);
        L = fmaf(f, mrg_l[w][r], L);
      }
    }
    float* dst = p.part + ((int64_t)split * rows_total + qrow_of(r)) * (D + 2);
    dst[j] = a;
    if (j == 0) {
      dst[D] = M * kLn2;
      dst[D + 1] = L;
    }
  }
}

// Rotates every query row once and normalises it for the fp16 operand split.
// qa = (R q) / (s_k * c1), qb = (S q) / (c2 / 2), with c1, c2 powers of two
// that bring the largest entry into [1, 2); rowc = {c1, c2, -sum(S q), 0}.
__global__ void __launch_bounds__(256) prerotate_mfma_kernel(const void* __restrict__ q, int qdt, int d,
                                                              const float* __restrict__ R,
                                                              const float* __restrict__ Sm, int qjl,
                                                              const float* __restrict__ scales,
                                                              float* __restrict__ qa,
                                                              float* __restrict__ qb,
                                                              float* __restrict__ rowc) {
  __shared__ float qs[256];
  __shared__ float red[3][256];
  const int64_t row = blockIdx.x;
  const int j = threadIdx.x;
  if (j < d)
    qs[j] = qdt == TQ_F16 ? __half2float(static_cast<const __half*>(q)[row * d + j])
                          : static_cast<const float*>(q)[row * d + j];
  __syncthreads();
  float a = 0.f, b = 0.f;
  if (j < d) {
    for (int k = 0; k < d; ++k) {
      a = fmaf(R[(size_t)j * d + k], qs[k], a);
      if (qjl) b = fmaf(Sm[(size_t)j * d + k], qs[k], b);
    }
  }
  a /= scales[0];
  red[0][j] = j < d ? fabsf(a) : 0.f;
  red[1][j] = j < d ? fabsf(b) : 0.f;
  red[2][j] = j < d ? b : 0.f;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (j < o) {
      red[0][j] = fmaxf(red[0][j], red[0][j + o]);
      red[1][j] = fmaxf(red[1][j], red[1][j + o]);
      red[2][j] += red[2][j + o];
    }
    __syncthreads();
  }
  int e1 = 0, e2 = 0;
  frexpf(red[0][0], &e1);
  frexpf(red[1][0], &e2);
  const float c1 = red[0][0] > 0.f ? ldexpf(1.f, e1 - 1) : 1.f;
  const float c2 = red[1][0] > 0.f ? ldexpf(1.f, e2) : 2.f;
  if (j < d) {
    qa[row * d + j] = a / c1;
    qb[row * d + j] = b * 2.f / c2;
  }
  if (j == 0) {
    rowc[row * 4 + 0] = c1;
    rowc[row * 4 + 1] = c2;
    rowc[row * 4 + 2] = -red[2][0];
    rowc[row * 4 + 3] = 0.f;
  }
}

template <int D, int KB, int QJL, int VB>
hipError_t launch_split(const DecodeMfmaParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_mfma_kernel<D, KB, QJL, VB>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int D, int KB, int QJL>
hipError_t dispatch_vb(const DecodeMfmaParams& p, int vb, dim3 grid, hipStream_t st) {
  switch (vb) {
    case 1: return launch_split<D, KB, QJL, 1>(p, grid, st);
    case 2: return launch_split<D, KB, QJL, 2>(p, grid, st);
    case 3: return launch_split<D, KB, QJL, 3>(p, grid, st);
    default: return launch_split<D, KB, QJL, 4>(p, grid, st);
  }
}

template <int D>
hipError_t dispatch_d(const DecodeMfmaParams& p, int kb, int qjl, int vb, dim3 grid, hipStream_t st) {
  if (qjl) {
    switch (kb) {
      case 1: return dispatch_vb<D, 1, 1>(p, vb, grid, st);
      case 2: return dispatch_vb<D, 2, 1>(p, vb, grid, st);
      case 3: return dispatch_vb<D, 3, 1>(p, vb, grid, st);
      default: return dispatch_vb<D, 4, 1>(p, vb, grid, st);
    }
  }
  switch (kb) {
    case 1: return dispatch_vb<D, 1, 0>(p, vb, grid, st);
    case 2: return dispatch_vb<D, 2, 0>(p, vb, grid, st);
    case 3: return dispatch_vb<D, 3, 0>(p, vb, grid, st);
    default: return dispatch_vb<D, 4, 0>(p, vb, grid, st);
  }
}

}  // namespace

bool mfma_decode_supports(int d, int rows) { return (d == 128 || d == 256) && rows >= 1 && rows <= 4; }

hipError_t launch_decode_mfma(const DecodeArgs& a, const float* scales, float* rowc, hipStream_t st) {
  const int64_t qrows = (int64_t)a.B * a.Hq * a.Tq;
  hipLaunchKernelGGL(prerotate_mfma_kernel, dim3((unsigned)qrows), dim3(256), 0, st, a.q, a.q_dtype,
                     a.d, a.R, a.S, a.qjl, scales, a.q_rot, a.q_proj, rowc);
  DecodeMfmaParams p{};
  p.qa = a.q_rot;
  p.qb = a.q_proj;
  p.rowc = rowc;
  p.scales = scales;
  p.kidx = a.kidx;
  p.ksign = a.ksign;
  p.knorm = a.knorm;
  p.krnorm = a.krnorm;
  p.vidx = a.vidx;
  p.vnorm = a.vnorm;
  p.cb = a.cb;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Tq = a.Tq;
  p.N = a.N;
  p.cap = a.cap;
  p.causal = a.causal;
  p.keys_per_split = a.keys_per_split;
  p.part = a.part;
  p.scores = a.scores;
  const dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)a.nsplit);
  hipError_t e = a.d == 128 ? dispatch_d<128>(p, a.kb, a.qjl, a.vb, grid, st)
                            : dispatch_d<256>(p, a.kb, a.qjl, a.vb, grid, st);
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, st);
}

}  // namespace tq
