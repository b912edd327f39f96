// Decode on the matrix cores: the combine kernel and the launcher.  The split
// kernel (tq_decode_mfma_impl.h) is instantiated by tq_decode_mfma_inst.hip.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// Matrix-vector products with 256 threads: thread (jq, sl) owns outputs
// 4jq..4jq+3 and the k-slice sl, reading one float4 of a matrix row per k (so
// a wave reads whole rows) with every load of the slice in flight at once.
template <int D>
struct MatVec {
  static constexpr int kJ = D / 4;           // threads per k-slice
  static constexpr int kSlices = 256 / kJ;   // 8 (D = 128) or 4 (D = 256)
  static constexpr int kSpan = D / kSlices;  // k per slice
};

// sum over the thread's k-slice of M[k][4jq..4jq+3] * x[k]; M row-major D x D
// (global), x in LDS.  Slices start at row k0 (even), which blocks vary so that
// they do not all read the same rows at once.
template <int D>
__device__ __forceinline__ f4 matvec_part(const float* __restrict__ M, const float* x, int jq, int sl, int k0) {
  using V = MatVec<D>;
  const f4* m = reinterpret_cast<const f4*>(M) + jq;
  f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int kk = 0; kk < V::kSpan; kk += 2) {
    const int k = (sl * V::kSpan + kk + k0) & (D - 1);
    acc0 += m[(size_t)k * V::kJ] * x[k];
    acc1 += m[(size_t)(k + 1) * V::kJ] * x[k + 1];
  }
  return acc0 + acc1;
}

// Output j (thread j < D) of the slices' partial sums.
template <int D>
__device__ __forceinline__ float matvec_sum(const f4 (*part)[D / 4], int j) {
  float v = 0.f;
#pragma unroll
  for (int s = 0; s < MatVec<D>::kSlices; ++s) v += part[s][j / 4][j % 4];
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One block per query row: merges the splits' partial softmax sums (rows of D +
// kPartPad floats: accumulator, maximum in natural-log units, sum) and
// un-rotates the result, out = R^T (sum_s w_s acc_s / sum_s w_s L_s) with w_s =
// exp(m_s - max_s m_s).
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ part, int nsplit,
                                                      int64_t rows_total, const float* __restrict__ R,
                                                      float* __restrict__ out) {
  using V = MatVec<D>;
  constexpr int kStride = D + kPartPad;
  __shared__ float wts[1024];  // the plan keeps nsplit <= 1024
  __shared__ float os[D];
  __shared__ f4 acc[V::kSlices][V::kJ];
  __shared__ float red[2][4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const float* base = part + row * kStride;
  const int64_t sstride = rows_total * kStride;
  const int jq = tid % V::kJ, sl = tid / V::kJ;
  const int k0 = (int)(blockIdx.x * 6) & (D - 1);
  // The loads that do not depend on one another go out first: this thread's
  // (max, sum) of split tid, its first accumulator slice and, at d = 128, its
  // rows of R (16 float4) -- one memory round trip instead of three.
  float m_own = -INFINITY, l_own = 0.f;
  if (tid < nsplit) {
    m_own = base[tid * sstride + D];
    l_own = base[tid * sstride + D + 1];
  }
  f4 a_first = {0.f, 0.f, 0.f, 0.f};
  if (sl < nsplit) a_first = reinterpret_cast<const f4*>(base + sl * sstride)[jq];
  constexpr bool kPre = D == 128;
  f4 rrow[kPre ? V::kSpan : 1];
  if constexpr (kPre) {
    const f4* m = reinterpret_cast<const f4*>(R) + jq;
#pragma unroll
    for (int kk = 0; kk < V::kSpan; ++kk) rrow[kk] = m[(size_t)((sl * V::kSpan + kk + k0) & (D - 1)) * V::kJ];
  }
  float M = m_own;
  for (int s = tid + 256; s < nsplit; s += 256) M = fmaxf(M, base[s * sstride + D]);
  M = wave_max(M);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float L = 0.f;
  if (tid < nsplit) {
    const float w = m_own == -INFINITY ? 0.f : expf(m_own - M);
    wts[tid] = w;
    L = w * l_own;
  }
  for (int s = tid + 256; s < nsplit; s += 256) {
    const float m = base[s * sstride + D];
    const float w = m == -INFINITY ? 0.f : expf(m - M);
    wts[s] = w;
    L = fmaf(w, base[s * sstride + D + 1], L);
  }
  L = wave_sum(L);
  if (lane == 0) red[1][wave] = L;
  __syncthreads();
  const float invL = 1.0f / (red[1][0] + red[1][1] + red[1][2] + red[1][3]);
  f4 o = sl < nsplit ? a_first * wts[sl] : f4{0.f, 0.f, 0.f, 0.f};
  for (int s = sl + V::kSlices; s < nsplit; s += V::kSlices)
    o += reinterpret_cast<const f4*>(base + s * sstride)[jq] * wts[s];
  acc[sl][jq] = o;
  __syncthreads();
  if (tid < D) os[tid] = matvec_sum<D>(acc, tid) * invL;
  __syncthreads();
  if constexpr (kPre) {
    f4 r0 = {0.f, 0.f, 0.f, 0.f}, r1 = r0;
#pragma unroll
    for (int kk = 0; kk < V::kSpan; kk += 2) {
      r0 += rrow[kk] * os[(sl * V::kSpan + kk + k0) & (D - 1)];
      r1 += rrow[kk + 1] * os[(sl * V::kSpan + kk + 1 + k0) & (D - 1)];
    }
    acc[sl][jq] = r0 + r1;
  } else {
    acc[sl][jq] = matvec_part<D>(R, os, jq, sl, k0);
  }
  __syncthreads();
  if (tid < D) out[row * D + tid] = matvec_sum<D>(acc, tid);
}

// combine_kernel<128> for RB query rows per block: the R rows a thread needs
// (16 float4) are loaded once for all RB rows, and every row's first partial
// loads go out with them, so a block pays one memory round trip for RB rows
// and R is read RB times less often.
template <int RB>
__global__ void __launch_bounds__(256) combine_rows128_kernel(const float* __restrict__ part, int nsplit,
                                                              int64_t rows_total, const float* __restrict__ R,
                                                              float* __restrict__ out) {
  constexpr int D = 128;
  using V = MatVec<D>;
  constexpr int kStride = D + kPartPad;
  __shared__ float wts[RB][1024];  // the plan keeps nsplit <= 1024
  __shared__ float os[RB][D];
  __shared__ f4 acc[RB][V::kSlices][V::kJ];
  __shared__ float red[2][RB][4];
  const int64_t row0 = (int64_t)blockIdx.x * RB;
  const int rows = (int)min((int64_t)RB, rows_total - row0);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t sstride = rows_total * kStride;
  const int jq = tid % V::kJ, sl = tid / V::kJ;
  const int k0 = (int)(blockIdx.x * 6) & (D - 1);
  float m_own[RB], l_own[RB];
  f4 a_first[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    m_own[r] = -INFINITY;
    l_own[r] = 0.f;
    a_first[r] = f4{0.f, 0.f, 0.f, 0.f};
    if (r < rows) {
      const float* base = part + (row0 + r) * kStride;
      if (tid < nsplit) {
        m_own[r] = base[tid * sstride + D];
        l_own[r] = base[tid * sstride + D + 1];
      }
      if (sl < nsplit) a_first[r] = reinterpret_cast<const f4*>(base + sl * sstride)[jq];
    }
  }
  f4 rrow[V::kSpan];
  {
    const f4* m = reinterpret_cast<const f4*>(R) + jq;
#pragma unroll
    for (int kk = 0; kk < V::kSpan; ++kk) rrow[kk] = m[(size_t)((sl * V::kSpan + kk + k0) & (D - 1)) * V::kJ];
  }
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const float* base = part + (row0 + min(r, rows - 1)) * kStride;
    float M = m_own[r];
    if (r < rows)
      for (int s = tid + 256; s < nsplit; s += 256) M = fmaxf(M, base[s * sstride + D]);
    M = wave_max(M);
    if (lane == 0) red[0][r][wave] = M;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const float* base = part + (row0 + min(r, rows - 1)) * kStride;
    const float M = fmaxf(fmaxf(red[0][r][0], red[0][r][1]), fmaxf(red[0][r][2], red[0][r][3]));
    float L = 0.f;
    if (tid < nsplit) {
      const float w = m_own[r] == -INFINITY ? 0.f : expf(m_own[r] - M);
      wts[r][tid] = w;
      L = w * l_own[r];
    }
    if (r < rows)
      for (int s = tid + 256; s < nsplit; s += 256) {
        const float m = base[s * sstride + D];
        const float w = m == -INFINITY ? 0.f : expf(m - M);
        wts[r][s] = w;
        L = fmaf(w, base[s * sstride + D + 1], L);
      }
    L = wave_sum(L);
    if (lane == 0) red[1][r][wave] = L;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const float* base = part + (row0 + min(r, rows - 1)) * kStride;
    f4 o = sl < nsplit ? a_first[r] * wts[r][sl] : f4{0.f, 0.f, 0.f, 0.f};
    if (r < rows)
      for (int s = sl + V::kSlices; s < nsplit; s += V::kSlices)
        o += reinterpret_cast<const f4*>(base + s * sstride)[jq] * wts[r][s];
    acc[r][sl][jq] = o;
  }
  __syncthreads();
  for (int i = tid; i < RB * D; i += 256) {
    const int r = i / D, j = i % D;
    const float invL = 1.0f / (red[1][r][0] + red[1][r][1] + red[1][r][2] + red[1][r][3]);
    os[r][j] = r < rows ? matvec_sum<D>(acc[r], j) * invL : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    f4 r0 = {0.f, 0.f, 0.f, 0.f}, r1 = r0;
#pragma unroll
    for (int kk = 0; kk < V::kSpan; kk += 2) {
      r0 += rrow[kk] * os[r][(sl * V::kSpan + kk + k0) & (D - 1)];
      r1 += rrow[kk + 1] * os[r][(sl * V::kSpan + kk + 1 + k0) & (D - 1)];
    }
    acc[r][sl][jq] = r0 + r1;
  }
  __syncthreads();
  for (int i = tid; i < RB * D; i += 256) {
    const int r = i / D, j = i % D;
    if (r < rows) out[(row0 + r) * D + j] = matvec_sum<D>(acc[r], j);
  }
}

}  // namespace

// Key blocks of a CU's first-dispatched workgroup per block of its second one
// (x 1024), from the key-loop times of the two (split_blocks).
constexpr int kFirstShare = 1331;

bool mfma_decode_supports(int d, int rows) { return (d == 128 || d == 256) && rows >= 1; }

namespace {
// The merge of the splits' partials and the un-rotation.  Many query rows: 4
// per block (R read a quarter as often; C4's 16384 rows, -1.5%).  Fewer than
// 2048: one per block, which keeps more blocks in flight for the latency-bound
// small calls.
hipError_t launch_combine(const DecodeArgs& a, int64_t qrows, dim3 rgrid, hipStream_t st) {
  constexpr int kRB = 4;
  if (a.d == 128 && qrows >= 512 * kRB)
    hipLaunchKernelGGL(combine_rows128_kernel<kRB>, dim3((unsigned)((qrows + kRB - 1) / kRB)), dim3(256), 0, st,
                       a.part, a.nsplit, qrows, a.R, a.out);
  else if (a.d == 128)
    hipLaunchKernelGGL(combine_kernel<128>, rgrid, dim3(256), 0, st, a.part, a.nsplit, qrows, a.R, a.out);
  else
    hipLaunchKernelGGL(combine_kernel<256>, rgrid, dim3(256), 0, st, a.part, a.nsplit, qrows, a.R, a.out);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, const DecodeMfmaExtra& x, hipStream_t st) {
  const int64_t qrows = (int64_t)a.B * a.Hq * a.Tq;
  const dim3 rgrid((unsigned)qrows);
  DecodeMfmaParams p{};
  p.q = a.q;
  p.qdt = a.q_dtype;
  p.Rt = x.Rt;
  p.St = x.St;
  p.scales = x.scales;
  p.kidx = a.kidx;
  p.ksign = a.ksign;
  p.knorm = a.knorm;
  p.krnorm = a.krnorm;
  p.vidx = a.vidx;
  p.vnorm = a.vnorm;
  p.cb = a.cb;
  p.R = a.R;
  p.out = a.out;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Tq = a.Tq;
  p.N = a.N;
  p.cap = a.cap;
  p.causal = a.causal;
  p.keys_per_split = a.keys_per_split;
  p.part = a.part;
  p.scores = a.scores;
  p.rot_hi = x.rot_hi;
  p.rot_lo = x.rot_lo;
  p.proj_hi = x.proj_hi;
  p.proj_lo = x.proj_lo;
  p.kd0 = a.kd0;
  p.vd0 = a.vd0;
  hipError_t e;
  if (a.wide) {
    p.rgroups = (a.Hq / a.Hkv * a.Tq + kWideRowsPerGroup - 1) / kWideRowsPerGroup;
    p.first_wgs = 0;
    const dim3 grid((unsigned)((int64_t)a.B * a.Hkv * p.rgroups), (unsigned)a.nsplit);
    e = a.qjl ? launch_decode_wide<1>(p, a.kb, a.vb, grid, st) : launch_decode_wide<0>(p, a.kb, a.vb, grid, st);
    if (e != hipSuccess) return e;
    return launch_combine(a, qrows, rgrid, st);
  }
  const int rw = decode_rows_per_group(a.Hq / a.Hkv * a.Tq);
  p.rgroups = (a.Hq / a.Hkv * a.Tq + rw - 1) / rw;
  const dim3 grid((unsigned)((int64_t)a.B * a.Hkv * p.rgroups), (unsigned)a.nsplit);
  // Unequal splits when the grid is exactly two 4-wave workgroups per CU.
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const bool two_per_cu = a.waves == 4 && decode_simd_waves(a.d, a.qjl, rw) == 2 &&
                          (int64_t)grid.x * grid.y == 2 * (int64_t)cus;
  p.first_wgs = two_per_cu ? cus : 0;
  p.first_share = kFirstShare;
  const int w = a.waves;
  if (a.d == 128)
    e = a.qjl      ? launch_decode_split<128, kKeysQjl>(p, a.kb, a.vb, w, grid, st)
        : a.dither ? launch_decode_split<128, kKeysDither>(p, a.kb, a.vb, w, grid, st)
                   : launch_decode_split<128, kKeysMse>(p, a.kb, a.vb, w, grid, st);
  else
    e = a.qjl      ? launch_decode_split<256, kKeysQjl>(p, a.kb, a.vb, w, grid, st)
        : a.dither ? launch_decode_split<256, kKeysDither>(p, a.kb, a.vb, w, grid, st)
                   : launch_decode_split<256, kKeysMse>(p, a.kb, a.vb, w, grid, st);
  if (e != hipSuccess) return e;
  return launch_combine(a, qrows, rgrid, st);
}

}  // namespace tq
