// Straightforward fp32 VALU kernels of the whole path (any d, bit width, GQA
// ratio and query count within the checked limits).  They favour plain
// indexing over speed and serve the shapes the tuned kernels do not cover.
//
// Method steps and where the pages define them:
//   quantize  [cuTile] listing, key and value compression functions
//             (values without QJL); [Mobilint] "Two-Stage Approach" (stage 1 codes, stage 2
//             sign(S r) and ||r||).
//   decode    [cuTile] listing, asymmetric score estimator, attention
//             pipeline and fused attention with online softmax;
//             [Mobilint] "Two-Stage Approach" (<q, x~> = <Pi q, y~>).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxAcc = 64;  // accumulators per thread in the split kernel

__device__ __forceinline__ float load_in(const void* p, int dtype, int64_t i) {
  return dtype == TQ_F16 ? __half2float(static_cast<const __half*>(p)[i])
                         : static_cast<const float*>(p)[i];
}

// b-bit code at stream position `pos` (little-endian stream, LSB first).
__device__ __forceinline__ uint32_t stream_code(const uint8_t* s, int64_t pos, int bits) {
  const int64_t bit = pos * bits;
  const int64_t byte = bit >> 3;
  const int sh = (int)(bit & 7);
  uint32_t v = s[byte];
  if (sh + bits > 8) v |= (uint32_t)s[byte + 1] << 8;
  return (v >> sh) & ((1u << bits) - 1u);
}

// --------------------------------------------------------------- quantize --
// One block encodes one 8-token tile of one sequence.
template <typename T>
__global__ void __launch_bounds__(kThreads) quantize_tile_ref(
    const T* __restrict__ x, int64_t n, int64_t t0, int64_t cap, int d, int bits, int qjl,
    int value_layout, int64_t tile_first, const float* __restrict__ R,
    const float* __restrict__ SR, const float* __restrict__ cent, const float* __restrict__ bnd,
    uint8_t* __restrict__ idx, uint8_t* __restrict__ sign, float* __restrict__ norm,
    float* __restrict__ rnorm) {
  extern __shared__ float smem[];
  float* u = smem;                                      // [8][d] unit rows
  float* y = u + 8 * d;                                 // [8][d] rotated, then residual
  uint8_t* code = reinterpret_cast<uint8_t*>(y + 8 * d);  // [8][d]
  uint8_t* sg = code + 8 * d;                           // [8][d]
  __shared__ float nrm[8], rsum[8];

  const int64_t s = blockIdx.y;
  const int64_t tile = tile_first + blockIdx.x;
  const int tid = threadIdx.x;
  auto valid = [&](int64_t t) { return t >= t0 && t < t0 + n; };

  for (int e = tid; e < 8 * d; e += kThreads) {
    const int i = e / d, j = e % d;
    const int64_t t = tile * 8 + i;
    u[e] = valid(t) ? (float)x[(s * n + (t - t0)) * d + j] : 0.f;
  }
  __syncthreads();
  {
    const int i = tid / 32, l = tid % 32;
    float acc = 0.f;
    for (int j = l; j < d; j += 32) acc = fmaf(u[i * d + j], u[i * d + j], acc);
    for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 32);
    if (l == 0) nrm[i] = sqrtf(acc);
  }
  __syncthreads();
  for (int e = tid; e < 8 * d; e += kThreads) {
    const float nn = nrm[e / d];
    u[e] = nn > 0.f ? u[e] / nn : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < 8 * d; e += kThreads) {  // y = R u
    const int i = e / d, j = e % d;
    const float* Rj = R + (size_t)j * d;
    const float* ui = u + i * d;
    float acc = 0.f;
    for (int k = 0; k < d; ++k) acc = fmaf(Rj[k], ui[k], acc);
    y[e] = acc;
  }
  __syncthreads();
  const int levels = 1 << bits;
  for (int e = tid; e < 8 * d; e += kThreads) {  // code = #{beta_i < y}
    const float v = y[e];
    int c = 0;
    for (int b = 0; b < levels - 1; ++b) c += bnd[b] < v ? 1 : 0;
    code[e] = (uint8_t)c;
    y[e] = v - cent[c];  // residual, still rotated
  }
  __syncthreads();
  if (qjl) {
    {
      const int i = tid / 32, l = tid % 32;
      float acc = 0.f;
      for (int j = l; j < d; j += 32) acc = fmaf(y[i * d + j], y[i * d + j], acc);
      for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 32);
      if (l == 0) rsum[i] = acc;
    }
    for (int e = tid; e < 8 * d; e += kThreads) {  // sign((S R^T) r_rot) = sign(S r)
      const int i = e / d, o = e % d;
      const float* row = SR + (size_t)o * d;
      const float* ri = y + i * d;
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc = fmaf(row[k], ri[k], acc);
      sg[e] = acc >= 0.f ? 1 : 0;
    }
    __syncthreads();
  }
  if (tid < 8) {
    const int64_t t = tile * 8 + tid;
    if (valid(t)) {
      norm[s * cap + t] = nrm[tid];
      if (qjl) rnorm[s * cap + t] = sqrtf(rsum[tid]);
    }
  }
  if (!value_layout) {
    const int rb = d * bits / 8;
    for (int e = tid; e < 8 * rb; e += kThreads) {
      const int i = e / rb, k = e % rb;
      const int64_t t = tile * 8 + i;
      if (!valid(t)) continue;
      uint32_t byte = 0;
      for (int bit = 0; bit < 8; ++bit) {
        const int pos = k * 8 + bit;
        byte |= ((uint32_t)(code[i * d + pos / bits] >> (pos % bits)) & 1u) << bit;
      }
      idx[(s * cap + t) * rb + k] = (uint8_t)byte;
    }
  } else {
    const int tb = d * bits;  // bytes per 8-token tile
    for (int k = tid; k < tb; k += kThreads) {
      uint32_t byte = 0, keep = 0;
      for (int bit = 0; bit < 8; ++bit) {
        const int pos = k * 8 + bit;
        const int p = pos / bits, w = pos % bits;
        const int j = p / 8, i = p % 8;
        if (valid(tile * 8 + i))
          byte |= ((uint32_t)(code[i * d + j] >> w) & 1u) << bit;
        else
          keep |= 1u << bit;
      }
      uint8_t* dst = idx + (s * (cap / 8) + tile) * tb + k;
      if (keep) byte |= *dst & keep;
      *dst = (uint8_t)byte;
    }
  }
  if (qjl) {  // sign rows, one d/8-byte stream per token in both layouts
    const int sb = d / 8;
    for (int e = tid; e < 8 * sb; e += kThreads) {
      const int i = e / sb, k = e % sb;
      const int64_t t = tile * 8 + i;
      if (!valid(t)) continue;
      uint32_t byte = 0;
      for (int bit = 0; bit < 8; ++bit) byte |= (uint32_t)sg[i * d + k * 8 + bit] << bit;
      sign[(s * cap + t) * sb + k] = (uint8_t)byte;
    }
  }
}

// ----------------------------------------------------------------- decode --
__global__ void __launch_bounds__(kThreads) prerotate_ref(const void* __restrict__ q, int qdt,
                                                          int d, const float* __restrict__ R,
                                                          const float* __restrict__ S, int qjl,
                                                          float* __restrict__ q_rot,
                                                          float* __restrict__ q_proj) {
  __shared__ float qs[256];
  const int64_t row = blockIdx.x;
  const int j = threadIdx.x;
  if (j < d) qs[j] = load_in(q, qdt, row * d + j);
  __syncthreads();
  if (j >= d) return;
  float a = 0.f, b = 0.f;
  for (int k = 0; k < d; ++k) {
    a = fmaf(R[(size_t)j * d + k], qs[k], a);
    if (qjl) b = fmaf(S[(size_t)j * d + k], qs[k], b);
  }
  q_rot[row * d + j] = a;
  if (qjl) q_proj[row * d + j] = b;
}

__global__ void __launch_bounds__(kThreads) decode_split_ref(
    const float* __restrict__ q_rot, const float* __restrict__ q_proj, int Hq, int Hkv, int Tq,
    int64_t N, int64_t cap, int causal, int d, int kb, int vb, int qjl, int KC,
    int64_t keys_per_split, const uint8_t* __restrict__ kidx, const uint8_t* __restrict__ ksign,
    const float* __restrict__ knorm, const float* __restrict__ krnorm,
    const uint8_t* __restrict__ vidx, const float* __restrict__ vnorm,
    const float* __restrict__ cb, float* __restrict__ part, float* __restrict__ scores,
    int dither, uint64_t kd0, uint64_t vd0, const float* __restrict__ dwidth,
    int vqjl, const uint8_t* __restrict__ vsign, const float* __restrict__ vrnorm) {
  extern __shared__ float smem[];
  const int G = Hq / Hkv;
  const int rows = G * Tq;
  float* kc = smem;                 // [KC][d]
  float* ks = kc + KC * d;          // [KC][d]
  float* vv = ks + KC * d;          // [KC][d]
  // values with QJL: n_v gamma_v sigma_v, the value's QJL term before the
  // factor sqrt(pi/2)/d and S^T (applied once, in the combine)
  float* vs = vv + KC * d;          // [KC][d] (vqjl only)
  float* sc = vs + (vqjl ? KC * d : 0);  // [rows][KC]
  float* mrow = sc + rows * KC;     // [rows]
  float* lrow = mrow + rows;
  float* alpha = lrow + rows;
  float* kn = alpha + rows;         // [KC]
  float* kg = kn + KC;

  const int64_t seq = blockIdx.x;
  const int64_t b = seq / Hkv;
  const int g = (int)(seq % Hkv);
  const int split = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t k_begin = split * keys_per_split;
  const int64_t k_end = min(N, k_begin + keys_per_split);
  const float* ck = cb;
  const float* cv = cb + 2 * kMaxLevels;
  // dithered variant: offset widths of keys and values
  const float kw = dither ? dwidth[0] : 0.f, vw = dither ? dwidth[1] : 0.f;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  const float kappa = sqrtf(0.5f * (float)M_PI) / (float)d;
  const int64_t rows_total = (int64_t)gridDim.x / Hkv * Hq * Tq;
  auto qrow_of = [&](int r) { return (b * Hq + (int64_t)g * G + r / Tq) * Tq + r % Tq; };

  for (int r = tid; r < rows; r += kThreads) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.f;
  }
  // accumulator a of this thread: element tid + a kThreads of [rows][d] (the
  // values' MSE part), then, with vqjl, of [rows][d] again (their QJL part)
  const int nacc = (rows * d * (vqjl ? 2 : 1) + kThreads - 1) / kThreads;
  float acc[kMaxAcc];
#pragma unroll
  for (int a = 0; a < kMaxAcc; ++a) acc[a] = 0.f;
  const int krb = d * kb / 8;
  const int vtb = d * vb;

  for (int64_t k0 = k_begin; k0 < k_end; k0 += KC) {
    const int kcount = (int)min((int64_t)KC, k_end - k0);
    for (int e = tid; e < KC * d; e += kThreads) {
      const int kk = e / d, j = e % d;
      if (kk < kcount) {
        const int64_t t = k0 + kk;
        kc[e] = ck[stream_code(kidx + (seq * cap + t) * krb, j, kb)];
        if (qjl) ks[e] = stream_code(ksign + (seq * cap + t) * (d / 8), j, 1) ? 1.f : -1.f;
        const uint8_t* tile = vidx + (seq * (cap / 8) + t / 8) * vtb;
        vv[e] = vnorm[seq * cap + t] * cv[stream_code(tile, 8 * j + (t & 7), vb)];
        if (dither) {  // reconstruction c[idx] + delta
          kc[e] += dither_offset(kd0, seq, t, kw);
          vv[e] = fmaf(vnorm[seq * cap + t], dither_offset(vd0, seq, t, vw), vv[e]);
        }
        if (vqjl) {
          const float g = vnorm[seq * cap + t] * vrnorm[seq * cap + t];
          vs[e] = stream_code(vsign + (seq * cap + t) * (d / 8), j, 1) ? g : -g;
        }
      }
    }
    for (int kk = tid; kk < kcount; kk += kThreads) {
      kn[kk] = knorm[seq * cap + k0 + kk];
      kg[kk] = qjl ? krnorm[seq * cap + k0 + kk] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < rows * KC; e += kThreads) {
      const int r = e / KC, kk = e % KC;
      if (kk >= kcount) {
        sc[e] = -INFINITY;
        continue;
      }
      const int64_t qr = qrow_of(r);
      const float* qv = q_rot + qr * d;
      float t1 = 0.f;
      for (int j = 0; j < d; ++j) t1 = fmaf(qv[j], kc[kk * d + j], t1);
      float s = t1;
      if (qjl) {
        const float* qp = q_proj + qr * d;
        float t2 = 0.f;
        for (int j = 0; j < d; ++j) t2 = fmaf(qp[j], ks[kk * d + j], t2);
        s = fmaf(kg[kk] * kappa, t2, t1);
      }
      s = kn[kk] * s * inv_sqrt_d;
      const int64_t t = k0 + kk;
      if (causal && t > N - Tq + r % Tq) s = -INFINITY;
      sc[e] = s;
      if (scores) scores[qr * N + t] = s;
    }
    __syncthreads();
    for (int r = tid; r < rows; r += kThreads) {
      float cmax = -INFINITY;
      for (int kk = 0; kk < kcount; ++kk) cmax = fmaxf(cmax, sc[r * KC + kk]);
      const float mold = mrow[r];
      const float mnew = fmaxf(mold, cmax);
      const float a = mnew == -INFINITY ? 1.f : expf(mold - mnew);
      float sum = 0.f;
      for (int kk = 0; kk < KC; ++kk) {
        const float v = sc[r * KC + kk];
        const float p = v == -INFINITY ? 0.f : expf(v - mnew);
        sc[r * KC + kk] = p;
        sum += p;
      }
      lrow[r] = lrow[r] * a + sum;
      mrow[r] = mnew;
      alpha[r] = a;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < kMaxAcc; ++a) {
      if (a < nacc) {
        const int p0 = tid + a * kThreads;
        if (p0 < rows * d * (vqjl ? 2 : 1)) {
          const bool second = p0 >= rows * d;
          const int p = second ? p0 - rows * d : p0;
          const int r = p / d, j = p % d;
          const float* src = second ? vs : vv;
          float v = acc[a] * alpha[r];
          for (int kk = 0; kk < kcount; ++kk) v = fmaf(sc[r * KC + kk], src[kk * d + j], v);
          acc[a] = v;
        }
      }
    }
    __syncthreads();
  }
  // partial rows: [acc (d) | acc of the QJL terms (d, vqjl only) | max | sum | padding]
  const int dd = vqjl ? 2 * d : d;
#pragma unroll
  for (int a = 0; a < kMaxAcc; ++a) {
    if (a < nacc) {
      const int p0 = tid + a * kThreads;
      if (p0 < rows * d * (vqjl ? 2 : 1)) {
        const bool second = p0 >= rows * d;
        const int p = second ? p0 - rows * d : p0;
        const int r = p / d, j = p % d;
        part[((int64_t)split * rows_total + qrow_of(r)) * (dd + kPartPad) + (second ? d : 0) + j] = acc[a];
      }
    }
  }
  for (int r = tid; r < rows; r += kThreads) {
    float* dst = part + ((int64_t)split * rows_total + qrow_of(r)) * (dd + kPartPad) + dd;
    dst[0] = mrow[r];
    dst[1] = lrow[r];
  }
}

// Merge the per-split partial softmax sums and un-rotate once per query row.
// Partial rows are [acc (d) | max (natural log) | sum | padding], d + kPartPad
// floats; with values carrying QJL, [acc (d) | acc2 (d) | max | sum | padding]
// and the output adds sqrt(pi/2)/d S^T acc2 (S row-major).
__global__ void __launch_bounds__(kThreads) decode_combine_ref(const float* __restrict__ part,
                                                               int nsplit, int64_t rows_total,
                                                               int d, const float* __restrict__ R,
                                                               int vqjl, const float* __restrict__ S,
                                                               float* __restrict__ out) {
  __shared__ float o[2][256];
  __shared__ float wts[2][1024];  // per-split weight, and its contribution to the sum
  __shared__ float invL;
  const int dd = vqjl ? 2 * d : d, stride = dd + kPartPad;
  const int64_t row = blockIdx.x;
  const int j = threadIdx.x;
  // max over splits, then weights: one thread per split (looping if more splits than threads)
  __shared__ float red[kThreads];
  float M = -INFINITY;
  for (int s = j; s < nsplit; s += kThreads) M = fmaxf(M, part[((int64_t)s * rows_total + row) * stride + dd]);
  red[j] = M;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (j < off) red[j] = fmaxf(red[j], red[j + off]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  float lsum = 0.f;
  for (int s = j; s < nsplit; s += kThreads) {
    const float* p = part + ((int64_t)s * rows_total + row) * stride;
    const float w = p[dd] == -INFINITY ? 0.f : expf(p[dd] - M);
    if (s < 1024) wts[0][s] = w;
    lsum = fmaf(w, p[dd + 1], lsum);
  }
  red[j] = lsum;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (j < off) red[j] += red[j + off];
    __syncthreads();
  }
  if (j == 0) invL = 1.0f / red[0];
  __syncthreads();
  for (int h = 0; h < (vqjl ? 2 : 1); ++h) {
    if (j < d) {
      const int c = h * d + j;
      float a0 = 0.f, a1 = 0.f;
      int s = 0;
      for (; s + 1 < nsplit; s += 2) {
        const float w0 = s < 1024 ? wts[0][s] : 0.f, w1 = s + 1 < 1024 ? wts[0][s + 1] : 0.f;
        a0 = fmaf(w0, part[((int64_t)s * rows_total + row) * stride + c], a0);
        a1 = fmaf(w1, part[((int64_t)(s + 1) * rows_total + row) * stride + c], a1);
      }
      for (; s < nsplit; ++s) a0 = fmaf(s < 1024 ? wts[0][s] : 0.f, part[((int64_t)s * rows_total + row) * stride + c], a0);
      o[h][j] = (a0 + a1) * invL;
    }
  }
  __syncthreads();
  if (j >= d) return;
  float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
  for (int k = 0; k < d; k += 4) {  // (R^T o)_j
    v0 = fmaf(R[(size_t)k * d + j], o[0][k], v0);
    v1 = fmaf(R[(size_t)(k + 1) * d + j], o[0][k + 1], v1);
    v2 = fmaf(R[(size_t)(k + 2) * d + j], o[0][k + 2], v2);
    v3 = fmaf(R[(size_t)(k + 3) * d + j], o[0][k + 3], v3);
  }
  float y = (v0 + v1) + (v2 + v3);
  if (vqjl) {  // + sqrt(pi/2)/d (S^T o2)_j
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
    for (int k = 0; k < d; k += 4) {
      w0 = fmaf(S[(size_t)k * d + j], o[1][k], w0);
      w1 = fmaf(S[(size_t)(k + 1) * d + j], o[1][k + 1], w1);
      w2 = fmaf(S[(size_t)(k + 2) * d + j], o[1][k + 2], w2);
      w3 = fmaf(S[(size_t)(k + 3) * d + j], o[1][k + 3], w3);
    }
    y = fmaf(sqrtf(0.5f * (float)M_PI) / (float)d, (w0 + w1) + (w2 + w3), y);
  }
  out[row * d + j] = y;
}

}  // namespace

// ------------------------------------------------------------- launchers --

hipError_t launch_quantize_ref(const QuantizeArgs& a, hipStream_t st) {
  if (a.n == 0 || a.seqs == 0) return hipSuccess;
  const int64_t first = a.t0 / 8, last = (a.t0 + a.n - 1) / 8;
  const dim3 grid((unsigned)(last - first + 1), (unsigned)a.seqs);
  const size_t shm = (size_t)8 * a.d * (2 * sizeof(float) + 2);
  if (a.dtype == TQ_F16)
    hipLaunchKernelGGL(quantize_tile_ref<__half>, grid, dim3(kThreads), shm, st,
                       static_cast<const __half*>(a.x), a.n, a.t0, a.cap, a.d, a.bits, a.qjl,
                       a.value_layout, first, a.R, a.SR, a.cent, a.bnd, a.idx, a.sign, a.norm,
                       a.rnorm);
  else
    hipLaunchKernelGGL(quantize_tile_ref<float>, grid, dim3(kThreads), shm, st,
                       static_cast<const float*>(a.x), a.n, a.t0, a.cap, a.d, a.bits, a.qjl,
                       a.value_layout, first, a.R, a.SR, a.cent, a.bnd, a.idx, a.sign, a.norm,
                       a.rnorm);
  return hipGetLastError();
}

int ref_decode_kc(int d) { return d >= 256 ? 8 : 16; }

size_t ref_decode_smem(int d, int rows, bool vqjl) {
  const int KC = ref_decode_kc(d);
  return sizeof(float) * ((size_t)(vqjl ? 4 : 3) * KC * d + (size_t)rows * KC + 3 * rows + 2 * KC);
}

bool ref_decode_supports(int d, int rows, bool vqjl) {
  return rows <= kThreads && (int64_t)rows * d * (vqjl ? 2 : 1) <= (int64_t)kMaxAcc * kThreads &&
         ref_decode_smem(d, rows, vqjl) <= 64 * 1024;
}

hipError_t launch_decode_ref(const DecodeArgs& a, hipStream_t st) {
  const int rows = a.Hq / a.Hkv * a.Tq;
  const int64_t qrows = (int64_t)a.B * a.Hq * a.Tq;
  hipLaunchKernelGGL(prerotate_ref, dim3((unsigned)qrows), dim3(kThreads), 0, st, a.q, a.q_dtype,
                     a.d, a.R, a.S, a.qjl, a.q_rot, a.q_proj);
  const int KC = ref_decode_kc(a.d);
  hipLaunchKernelGGL(decode_split_ref, dim3((unsigned)(a.B * a.Hkv), (unsigned)a.nsplit),
                     dim3(kThreads), ref_decode_smem(a.d, rows, a.vqjl), st, a.q_rot, a.q_proj, a.Hq,
                     a.Hkv, a.Tq, a.N, a.cap, a.causal, a.d, a.kb, a.vb, a.qjl, KC,
                     a.keys_per_split, a.kidx, a.ksign, a.knorm, a.krnorm, a.vidx, a.vnorm,
                     a.cb, a.part, a.scores, a.dither, a.kd0, a.vd0, a.scales ? a.scales + 4 : nullptr,
                     a.vqjl, a.vsign, a.vrnorm);
  return launch_decode_combine(a, st);
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st) {
  const int64_t qrows = (int64_t)a.B * a.Hq * a.Tq;
  hipLaunchKernelGGL(decode_combine_ref, dim3((unsigned)qrows), dim3(kThreads), 0, st, a.part,
                     a.nsplit, qrows, a.d, a.R, a.vqjl, a.S, a.out);
  return hipGetLastError();
}

}  // namespace tq
