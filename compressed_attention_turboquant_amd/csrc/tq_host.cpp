// Host-side construction of a layer's tables, in float64.
//
// * Random stream: SplitMix64 (Steele, Lea, Flood, OOPSLA 2014) with its
//   published 64-bit finaliser.  Stream (seed, tag) starts from
//   seed ^ (tag * 0xD1B54A32D192ED03) and its k-th output (k >= 1) finalises
//   start + k * 0x9E3779B97F4A7C15.  Uniforms are ((z >> 11) + 0.5) / 2^53;
//   normals come from Box-Muller on consecutive uniform pairs (cos, then sin);
//   signs are +1 when the top bit is 0.  Tags: 0 rotation, 1 projection, 2 signs.
// * Haar rotation ([cuTile] listing, Haar rotation function): Householder QR of the row-major Gaussian G, Q formed
//   explicitly, columns signed so that diag(R) > 0 (the unique, Haar Q).
// * Randomized Hadamard ([Mobilint] "How JL Matrices Evolved"): R = H D with
//   H[i][j] = (-1)^popcount(i&j) / sqrt(d) (Sylvester order) and D the signs.
// * QJL projection S ([Mobilint] "Two-Stage Approach", stage 2): d x d i.i.d.
//   N(0,1), unnormalised.
// * Lloyd-Max codebook ([Mobilint] "Designing the Optimal Codebook Without
//   Data") for N(0, 1/d): solved on N(0,1) with exact conditional means
//   (pdf(a) - pdf(b)) / (P(a < X < b)), from linspace(-2, 2, 2^b), until no
//   centroid moves more than 1e-15; made symmetric, scaled by 1/sqrt(d) in
//   float64, rounded to float32; boundaries are the float64 midpoints rounded
//   to float32.
#include <cmath>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kTagMul = 0xD1B54A32D192ED03ull;

inline uint64_t finalise(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct Stream {
  uint64_t state;
  Stream(uint64_t seed, uint64_t tag) : state(seed ^ (tag * kTagMul)) {}
  uint64_t next() {
    state += kGamma;
    return finalise(state);
  }
  double uniform() { return ((double)(next() >> 11) + 0.5) * 0x1.0p-53; }
};

void householder_haar(int d, const std::vector<double>& G, double* Q_out) {
  // Work on A = G (row-major); reflect column k below the diagonal to alpha e_k.
  std::vector<double> A(G);
  std::vector<double> V((size_t)d * d, 0.0);  // reflector k stored in row k (entries k..d-1)
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += A[(size_t)i * d + k] * A[(size_t)i * d + k];
    const double norm = std::sqrt(norm2);
    const double x0 = A[(size_t)k * d + k];
    const double alpha = x0 > 0 ? -norm : norm;  // avoid cancellation in x0 - alpha
    double* v = &V[(size_t)k * d];
    for (int i = k; i < d; ++i) v[i] = A[(size_t)i * d + k];
    v[k] -= alpha;
    double vn2 = 0.0;
    for (int i = k; i < d; ++i) vn2 += v[i] * v[i];
    rdiag[k] = alpha;
    if (vn2 == 0.0) continue;  // column already reduced
    const double inv = 1.0 / std::sqrt(vn2);
    for (int i = k; i < d; ++i) v[i] *= inv;
    for (int j = k; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * A[(size_t)i * d + j];
      for (int i = k; i < d; ++i) A[(size_t)i * d + j] -= 2.0 * v[i] * dot;
    }
  }
  // Q = H_0 H_1 ... H_{d-1}, applied to the identity from the right-most reflector.
  std::vector<double> Q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) Q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &V[(size_t)k * d];
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * Q[(size_t)i * d + j];
      for (int i = k; i < d; ++i) Q[(size_t)i * d + j] -= 2.0 * v[i] * dot;
    }
  }
  // G = Q R with R_kk = rdiag[k]; flip columns where R_kk < 0.
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      Q_out[(size_t)i * d + j] = rdiag[j] < 0 ? -Q[(size_t)i * d + j] : Q[(size_t)i * d + j];
}

double normal_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) * 0.39894228040143267794;  // 1/sqrt(2 pi)
}

double normal_mass(double a, double b) {
  const double r2 = 0.70710678118654752440;  // 1/sqrt(2)
  if (a >= 0.0) return 0.5 * std::erfc(a * r2) - 0.5 * std::erfc(b * r2);
  return 0.5 * std::erfc(-b * r2) - 0.5 * std::erfc(-a * r2);
}

}  // namespace

void stream_normals(uint64_t seed, uint64_t tag, size_t count, double* out) {
  Stream s(seed, tag);
  for (size_t i = 0; i < count; i += 2) {
    const double u1 = s.uniform();
    const double u2 = s.uniform();
    const double rho = std::sqrt(-2.0 * std::log(u1));
    const double ang = 2.0 * M_PI * u2;
    out[i] = rho * std::cos(ang);
    if (i + 1 < count) out[i + 1] = rho * std::sin(ang);
  }
}

void stream_signs(uint64_t seed, uint64_t tag, size_t count, double* out) {
  Stream s(seed, tag);
  for (size_t i = 0; i < count; ++i) out[i] = (s.next() >> 63) == 0 ? 1.0 : -1.0;
}

void make_rotation_f64(int d, int rot, uint64_t seed, double* R) {
  if (rot == TQ_ROT_HAAR) {
    std::vector<double> G((size_t)d * d);
    stream_normals(seed, 0, G.size(), G.data());
    householder_haar(d, G, R);
    return;
  }
  std::vector<double> D(d);
  stream_signs(seed, 2, d, D.data());
  const double scale = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      R[(size_t)i * d + j] = ((__builtin_popcount(i & j) & 1) ? -scale : scale) * D[j];
}

void make_projection_f64(int d, uint64_t seed, double* S) { stream_normals(seed, 1, (size_t)d * d, S); }

void lloyd_max_codebook(int bits, int d, float* centroids, float* boundaries) {
  const int L = 1 << bits;
  std::vector<double> c(L), nc(L), edge(L + 1);
  for (int i = 0; i < L; ++i) c[i] = -2.0 + 4.0 * i / (L - 1);
  for (int it = 0; it < 200000; ++it) {
    edge[0] = -INFINITY;
    edge[L] = INFINITY;
    for (int i = 1; i < L; ++i) edge[i] = (c[i - 1] + c[i]) / 2.0;
    double moved = 0.0;
    for (int i = 0; i < L; ++i) {
      nc[i] = (normal_pdf(edge[i]) - normal_pdf(edge[i + 1])) / normal_mass(edge[i], edge[i + 1]);
      moved = std::fmax(moved, std::fabs(nc[i] - c[i]));
    }
    c.swap(nc);
    if (moved <= 1e-15) break;
  }
  std::vector<double> sym(L);
  for (int i = 0; i < L; ++i) sym[i] = -(c[L - 1 - i] - c[i]) / 2.0;
  const double sigma = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < L; ++i) centroids[i] = (float)(sym[i] * sigma);
  for (int i = 0; i + 1 < L; ++i) boundaries[i] = (float)((sym[i] * sigma + sym[i + 1] * sigma) / 2.0);
}

namespace {
// Nodes x and weights w of the n-point Gauss-Legendre rule on [-1, 1]: the
// roots of the Legendre polynomial P_n by Newton's method from the usual
// cosine start, with w_i = 2 / ((1 - x_i^2) P_n'(x_i)^2).
void gauss_legendre(int n, double* x, double* w) {
  for (int i = 0; i < n; ++i) {
    double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
    double dp = 1.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;  // P_0, P_1; recurrence (k+1) P_{k+1} = (2k+1) z P_k - k P_{k-1}
      for (int k = 1; k < n; ++k) {
        const double p2 = ((2.0 * k + 1.0) * z * p1 - k * p0) / (k + 1.0);
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);  // P_n'(z)
      const double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-16) break;
    }
    x[i] = z;
    w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

// Integral of (1 - t^2)^a over [lo, hi] (inside [-1, 1]) by composite 16-point
// Gauss-Legendre (nodes gx, weights gw) on panels no wider than spread / 4; the part beyond `cut`
// from the origin (where the integrand is below e^-72 of its peak) is left out.
double beta_kernel_integral(double a, double lo, double hi, double spread, double cut, const double* gx,
                            const double* gw) {
  lo = std::fmax(lo, -cut);
  hi = std::fmin(hi, cut);
  if (hi <= lo) return 0.0;
  const int panels = (int)std::ceil((hi - lo) / (spread / 4.0));
  const double h = (hi - lo) / panels;
  double total = 0.0;
  for (int pnl = 0; pnl < panels; ++pnl) {
    const double mid = lo + (pnl + 0.5) * h;
    double part = 0.0;
    for (int i = 0; i < 16; ++i) {
      const double t = mid + 0.5 * h * gx[i];
      part += gw[i] * std::pow(1.0 - t * t, a);
    }
    total += 0.5 * h * part;
  }
  return total;
}
}  // namespace

void lloyd_max_codebook_beta(int bits, int d, float* centroids, float* boundaries) {
  // Exact law of a coordinate of a rotated unit vector: density proportional
  // to (1 - t^2)^a on [-1, 1], a = (d - 3) / 2.  Lloyd-Max as for the Gaussian:
  // boundaries at midpoints, centroids the conditional means, here
  //   E[X | lo < X < hi] = ((1 - lo^2)^(a+1) - (1 - hi^2)^(a+1)) / (2 (a+1) M),
  //   M = integral of (1 - t^2)^a over [lo, hi] (quadrature).
  const int L = 1 << bits;
  const double a = (d - 3) / 2.0;
  const double spread = 1.0 / std::sqrt((double)d);
  const double cut = std::fmin(1.0, 12.0 * spread);
  const double top = std::fmin(2.0 * spread, 1.0 - 1.0 / L);
  double gx[16], gw[16];
  gauss_legendre(16, gx, gw);
  std::vector<double> c(L), nc(L), edge(L + 1);
  for (int i = 0; i < L; ++i) c[i] = -top + 2.0 * top * i / (L - 1);
  for (int it = 0; it < 200000; ++it) {
    edge[0] = -1.0;
    edge[L] = 1.0;
    for (int i = 1; i < L; ++i) edge[i] = (c[i - 1] + c[i]) / 2.0;
    double moved = 0.0;
    for (int i = 0; i < L; ++i) {
      const double lo = edge[i], hi = edge[i + 1];
      const double m1 = (std::pow(1.0 - lo * lo, a + 1.0) - std::pow(1.0 - hi * hi, a + 1.0)) / (2.0 * (a + 1.0));
      nc[i] = m1 / beta_kernel_integral(a, lo, hi, spread, cut, gx, gw);
      moved = std::fmax(moved, std::fabs(nc[i] - c[i]));
    }
    c.swap(nc);
    if (moved <= 1e-15) break;
  }
  std::vector<double> sym(L);
  for (int i = 0; i < L; ++i) sym[i] = -(c[L - 1 - i] - c[i]) / 2.0;
  for (int i = 0; i < L; ++i) centroids[i] = (float)sym[i];
  for (int i = 0; i + 1 < L; ++i) boundaries[i] = (float)((sym[i] + sym[i + 1]) / 2.0);
}

namespace {
// float -> IEEE half, round to nearest even (normal, subnormal and overflow cases).
uint16_t to_half(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  int32_t exp = (int32_t)((x >> 23) & 0xFF) - 127 + 15;
  uint32_t mant = x & 0x7FFFFFu;
  if (((x >> 23) & 0xFF) == 0xFF) return (uint16_t)(sign | 0x7C00u | (mant ? 0x200u : 0));
  if (exp >= 31) return (uint16_t)(sign | 0x7C00u);
  if (exp <= 0) {
    if (exp < -10) return (uint16_t)sign;
    mant |= 0x800000u;
    const int shift = 14 - exp;
    uint32_t h = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1))) ++h;
    return (uint16_t)(sign | h);
  }
  uint32_t h = ((uint32_t)exp << 10) | (mant >> 13);
  const uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1))) ++h;
  return (uint16_t)(sign | h);
}

float from_half(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t exp = (h >> 10) & 0x1F;
  const uint32_t mant = h & 0x3FF;
  float f;
  if (exp == 0) {
    f = std::ldexp((float)mant, -24);
    uint32_t x;
    std::memcpy(&x, &f, 4);
    x |= sign;
    std::memcpy(&f, &x, 4);
    return f;
  }
  uint32_t x = sign | ((exp == 31 ? 255u : exp - 15 + 127) << 23) | (mant << 13);
  std::memcpy(&f, &x, 4);
  return f;
}

void split_half(const double* M, size_t count, double scale, uint16_t* hi, uint16_t* lo) {
  for (size_t i = 0; i < count; ++i) {
    const double v = M[i] * scale;
    hi[i] = to_half((float)v);
    lo[i] = to_half((float)(v - (double)from_half(hi[i])));
  }
}
}  // namespace

float centroid_half_scale(const float* centroids, int levels, float* max_rel_err) {
  // The decode kernels multiply fp16 copies of the centroids on the matrix
  // cores.  Scaling the whole codebook by one factor s (undone on the query
  // side) does not change the result, so s is chosen to make every s*c_i land
  // as close as possible to an fp16 value.  Search s over [1, 2) * 2^k with
  // s * max|c| in [1, 2), 2^18 candidates (finer grids gain < 1%).
  double cmax = 0.0;
  for (int i = 0; i < levels; ++i) cmax = std::fmax(cmax, std::fabs((double)centroids[i]));
  const double base = std::ldexp(1.0, -(int)std::floor(std::log2(cmax)));
  const int steps = 1 << 18;
  double best_s = base, best_err = INFINITY;
  for (int k = 0; k < steps; ++k) {
    const double s = base * (1.0 + (double)k / steps);
    double err = 0.0;
    for (int i = levels / 2; i < levels && err < best_err; ++i) {  // codebooks are symmetric
      const double v = s * (double)centroids[i];
      const double h = (double)from_half(to_half((float)v));
      err = std::fmax(err, std::fabs(h / v - 1.0));
    }
    if (err < best_err) {
      best_err = err;
      best_s = s;
    }
  }
  // Report the error of the float32 scale actually stored.
  const float sf = (float)best_s;
  double err = 0.0;
  for (int i = 0; i < levels; ++i) {
    const double v = (double)sf * (double)centroids[i];
    if (v != 0.0) err = std::fmax(err, std::fabs((double)from_half(to_half((float)v)) / v - 1.0));
  }
  *max_rel_err = (float)err;
  return sf;
}

void build_blob_image(int d, int rot, uint64_t seed, int k_bits, int v_bits, int flags, unsigned char* image) {
  const BlobLayout L = blob_layout(d);
  std::memset(image, 0, L.total);
  const size_t dd = (size_t)d * d;
  std::vector<double> R(dd), S(dd), SR(dd, 0.0), D(d, 1.0);
  make_rotation_f64(d, rot, seed, R.data());
  make_projection_f64(d, seed, S.data());
  if (rot == TQ_ROT_HADAMARD) stream_signs(seed, 2, d, D.data());
  for (int i = 0; i < d; ++i)      // (S R^T)[i][j] = sum_k S[i][k] R[j][k]
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int k = 0; k < d; ++k) acc += S[(size_t)i * d + k] * R[(size_t)j * d + k];
      SR[(size_t)i * d + j] = acc;
    }
  float* rot_f = reinterpret_cast<float*>(image + L.rot);
  float* proj_f = reinterpret_cast<float*>(image + L.proj);
  float* projr_f = reinterpret_cast<float*>(image + L.projr);
  float* signs_f = reinterpret_cast<float*>(image + L.signs);
  for (size_t i = 0; i < dd; ++i) {
    rot_f[i] = (float)R[i];
    proj_f[i] = (float)S[i];
    projr_f[i] = (float)SR[i];
  }
  for (int i = 0; i < d; ++i) signs_f[i] = (float)D[i];
  float* rot_t = reinterpret_cast<float*>(image + L.rot_t);
  float* proj_t = reinterpret_cast<float*>(image + L.proj_t);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      rot_t[(size_t)j * d + i] = (float)R[(size_t)i * d + j];
      proj_t[(size_t)j * d + i] = (float)S[(size_t)i * d + j];
    }
  float* cb = reinterpret_cast<float*>(image + L.codebook);
  if (flags & TQ_LAYER_BETA_CODEBOOK) {
    lloyd_max_codebook_beta(k_bits, d, cb, cb + kMaxLevels);
    lloyd_max_codebook_beta(v_bits, d, cb + 2 * kMaxLevels, cb + 3 * kMaxLevels);
  } else {
    lloyd_max_codebook(k_bits, d, cb, cb + kMaxLevels);
    lloyd_max_codebook(v_bits, d, cb + 2 * kMaxLevels, cb + 3 * kMaxLevels);
  }
  float* sc = reinterpret_cast<float*>(image + L.scales);
  sc[0] = centroid_half_scale(cb, 1 << k_bits, &sc[2]);
  sc[1] = centroid_half_scale(cb + 2 * kMaxLevels, 1 << v_bits, &sc[3]);
  sc[4] = cb[(1 << k_bits) / 2] - cb[(1 << k_bits) / 2 - 1];
  sc[5] = cb[2 * kMaxLevels + (1 << v_bits) / 2] - cb[2 * kMaxLevels + (1 << v_bits) / 2 - 1];
  split_half(R.data(), dd, std::sqrt((double)d), reinterpret_cast<uint16_t*>(image + L.rot_hi),
             reinterpret_cast<uint16_t*>(image + L.rot_lo));
  split_half(SR.data(), dd, 1.0, reinterpret_cast<uint16_t*>(image + L.projr_hi),
             reinterpret_cast<uint16_t*>(image + L.projr_lo));
  split_half(S.data(), dd, 1.0, reinterpret_cast<uint16_t*>(image + L.proj_hi),
             reinterpret_cast<uint16_t*>(image + L.proj_lo));
}

}  // namespace tq
