// Internal definitions shared by the host set-up, the C ABI and the kernels.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxLevels = 16;  // 4-bit codes
// Decode split partials: one row of d + kPartPad floats per (split, query row):
// the rotated-domain accumulator (d), the running maximum (natural log), the
// sum of weights and padding to a 16-byte multiple.
constexpr int kPartPad = 4;

// Offsets (bytes) of the tables inside a layer blob.  All float32 unless noted.
struct BlobLayout {
  size_t rot;       // [d][d] R row-major (y = R u): Pi, or H*D for the Hadamard kind
  size_t proj;      // [d][d] S row-major (QJL projection)
  size_t projr;     // [d][d] S R^T, so that S r = (S R^T)(R r) for a residual kept rotated
  size_t signs;     // [d] D (all +1 for the Haar kind)
  size_t rot_t;     // [d][d] R^T row-major (coalesced reads of R by output index)
  size_t proj_t;    // [d][d] S^T row-major
  size_t codebook;  // [4][16]: key centroids, key boundaries, value centroids, value boundaries
  size_t scales;    // [8]: fp16 table scale for key and value centroids, their worst relative fp16
                    // rounding error (see centroid_half_scale), then the dither widths
                    // c[L/2] - c[L/2-1] of the key and value codebooks
  size_t rot_hi;    // half [d][d]: sqrt(d)*R split as hi + lo (MFMA operands)
  size_t rot_lo;
  size_t projr_hi;  // half [d][d]: S R^T split as hi + lo
  size_t projr_lo;
  size_t proj_hi;   // half [d][d]: S split as hi + lo (query projection on the matrix cores)
  size_t proj_lo;
  size_t total;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

inline BlobLayout blob_layout(int d) {
  BlobLayout L{};
  const size_t mat = (size_t)d * d * sizeof(float);
  const size_t hmat = (size_t)d * d * 2;
  size_t o = 0;
  L.rot = o;       o = align_up(o + mat, 256);
  L.proj = o;      o = align_up(o + mat, 256);
  L.projr = o;     o = align_up(o + mat, 256);
  L.signs = o;     o = align_up(o + d * sizeof(float), 256);
  L.rot_t = o;     o = align_up(o + mat, 256);
  L.proj_t = o;    o = align_up(o + mat, 256);
  L.codebook = o;  o = align_up(o + 4 * kMaxLevels * sizeof(float), 256);
  L.scales = o;    o = align_up(o + 8 * sizeof(float), 256);
  L.rot_hi = o;    o = align_up(o + hmat, 256);
  L.rot_lo = o;    o = align_up(o + hmat, 256);
  L.projr_hi = o;  o = align_up(o + hmat, 256);
  L.projr_lo = o;  o = align_up(o + hmat, 256);
  L.proj_hi = o;   o = align_up(o + hmat, 256);
  L.proj_lo = o;   o = align_up(o + hmat, 256);
  L.total = o;
  return L;
}

// ---- host set-up (tq_host.cpp) ----
void stream_normals(uint64_t seed, uint64_t tag, size_t count, double* out);
void stream_signs(uint64_t seed, uint64_t tag, size_t count, double* out);
void make_rotation_f64(int d, int rot, uint64_t seed, double* R);
void make_projection_f64(int d, uint64_t seed, double* S);
void lloyd_max_codebook(int bits, int d, float* centroids, float* boundaries);
// The same for the exact coordinate law (1 - t^2)^((d-3)/2) of a rotated unit vector.
void lloyd_max_codebook_beta(int bits, int d, float* centroids, float* boundaries);
// Common factor s for a codebook such that every s*c_i rounds to fp16 with the
// smallest worst-case relative error; returns s and writes that error.
float centroid_half_scale(const float* centroids, int levels, float* max_rel_err);
// Fills a host image of the whole blob (layout.total bytes).
void build_blob_image(int d, int rot, uint64_t seed, int k_bits, int v_bits, int flags, unsigned char* image);

// ---- error reporting (tq_api.hip) ----
tq_status fail(tq_status s, const std::string& msg);

}  // namespace tq
