// Kernel launch interfaces (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "tq_dither.h"
#include "tq_internal.h"

namespace tq {

struct QuantizeArgs {
  const void* x;
  int dtype;
  int64_t seqs, n, t0, cap;
  int d, bits, qjl, value_layout, rot;
  const float *R, *SR, *cent, *bnd;  // rotation, S R^T, codebook
  const float* dsign;                // [d] +-1 signs D of the Hadamard rotation
  const void *rot_hi, *rot_lo, *projr_hi, *projr_lo;  // half splits for MFMA
  uint8_t *idx, *sign;
  float *norm, *rnorm;
  // Dithered variant: offsets from the stream starting at dither_s0, width at
  // *dither_w (device, in the layer blob).
  int dither;
  uint64_t dither_s0;
  const float* dither_w;
};

struct DecodeArgs {
  const void* q;
  int q_dtype;
  int B, Hq, Hkv, Tq;
  int64_t N, cap;
  int causal, d, kb, vb, qjl;
  const float *R, *S, *cb;
  const uint8_t *kidx, *ksign, *vidx;
  const float *knorm, *krnorm, *vnorm;
  float *out, *scores;
  // workspace pieces
  float *q_rot, *q_proj, *part;
  int nsplit;
  int waves;  // waves per decode workgroup (matrix-core kernel)
  bool wide;  // the many-rows kernel (tq_decode_wide.hip)
  int64_t keys_per_split;
  // Values with QJL (reference kernels): their sign rows and residual norms.
  int vqjl;
  const uint8_t* vsign;
  const float* vrnorm;
  // Dithered variant: key / value offset streams; widths in the blob's scales[4], [5].
  int dither;
  uint64_t kd0, vd0;
  const float* scales;
};

struct DequantArgs {
  const uint8_t* idx;
  const float* norm;
  int64_t seqs, n, cap;
  int d, bits, value_layout;
  const float *R, *Rt, *cent;  // R and R^T row-major
  int rot;                      // TQ_ROT_*: the Hadamard rotation has its own kernel
  const float* dsign;           // [d] +-1 signs D of the Hadamard rotation
  void* out;
  int out_dtype;
  int dither;  // dithered variant: offsets from the stream at dither_s0, width *dither_w
  uint64_t dither_s0;
  const float* dither_w;
  const float* cscale;  // factor s of the codebook's fp16 copies (decode tables), for fp16 rows
  // Keys with QJL (Haar, d = 64 or 128): the two-stage reconstruction in the same
  // pass, adding n sqrt(pi/2)/d gamma S^T sigma to each row before it is stored.
  int qjl;
  const uint8_t* sign;  // the rows' sign bits
  const float* rnorm;   // the rows' residual norms gamma
  const float* St;      // S^T row-major
};

// Arguments of the kernel that adds the QJL term n sqrt(pi/2)/d gamma S^T sigma
// to dequantized key rows (tq_dequantize_mfma.hip).
struct DequantQjlArgs {
  const uint8_t* sign;
  const float *norm, *rnorm;
  int64_t seqs, n, cap;
  int d;
  const float* St;  // S^T row-major
  void* out;
  int out_dtype;
};

// Arguments of the matrix-core decode split kernel (tq_decode_mfma.hip).
struct DecodeMfmaParams {
  const void* q;                    // query rows [B][Hq][Tq][d]
  int qdt;                          // TQ_F16 or TQ_F32
  const float *Rt, *St;             // R^T and S^T (row-major) for the query rotation
  const uint8_t *kidx, *ksign, *vidx;
  const float *knorm, *krnorm, *vnorm, *cb;
  const float* scales;              // blob: fp16 table factors for key and value centroids
  const float* R;                   // rotation (row-major) for the final un-rotation
  const void *rot_hi, *rot_lo;      // sqrt(d) R split fp16 hi + lo (query rotation on the matrix cores)
  const void *proj_hi, *proj_lo;    // S split fp16 hi + lo
  float* out;
  int Hq, Hkv, Tq, causal;
  int rgroups;                      // groups of up to 4 query rows per KV head
  int64_t N, cap, keys_per_split;
  // Unequal splits (see split_blocks): workgroups with a linear index below
  // first_wgs get first_share / 1024 times the key blocks of the others; 0: all
  // splits of a row group have keys_per_split keys.
  int first_wgs, first_share;
  float *part, *scores;
  uint64_t kd0, vd0;  // dithered variant: key / value offset streams (widths in scales[4], [5])
};

// Blob and workspace pieces the matrix-core decode needs besides DecodeArgs.
struct DecodeMfmaExtra {
  const float *Rt, *St, *scales;
  const void *rot_hi, *rot_lo, *proj_hi, *proj_lo;
};

// Arguments of the matrix-core quantize kernel (tq_quantize_mfma.hip, d = 128, fp16 input).
struct QuantMfmaParams {
  const _Float16* x;
  int64_t seqs, n, t0, cap, tile_first, tile_last;
  const _Float16 *rot_hi, *rot_lo, *projr_hi, *projr_lo;
  const float *cent, *bnd;
  uint8_t *idx, *sign;
  float *norm, *rnorm;
};

hipError_t launch_quantize_ref(const QuantizeArgs& a, hipStream_t st);
bool mfma_quantize_supports(int d, int dtype);
hipError_t launch_quantize_mfma(const QuantizeArgs& a, hipStream_t st);
bool fwht_quantize_supports(int d, int rot, int qjl);
hipError_t launch_quantize_fwht(const QuantizeArgs& a, hipStream_t st);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st);
bool mfma_decode_supports(int d, int rows);
// Key kinds of the split kernel: MSE codes only, with QJL signs, or MSE codes of
// the dithered variant.
constexpr int kKeysMse = 0, kKeysQjl = 1, kKeysDither = 2;
// The split kernel for one head dimension and key kind; each (D, KIND) pair is
// instantiated by its own compilation of tq_decode_mfma_inst.hip.
template <int D, int KIND>
hipError_t launch_decode_split(const DecodeMfmaParams& p, int kb, int vb, int waves, dim3 grid, hipStream_t st);
// Query rows one decode workgroup serves (4, or 8 when a KV head has more than
// 4 query rows: the matrix-core rows then carry 8 query rows x {hi, lo}).
inline int decode_rows_per_group(int rows_per_head) { return rows_per_head > 4 ? 8 : 4; }

// KV heads with at least this many query rows (at d = 128) use the wide
// kernel (tq_decode_wide.hip): 4 waves x 16 rows per workgroup (two
// workgroups per CU), each decoded code serving 16 rows.  (32 rows per wave
// halve the decoding but need one wave per SIMD: 1037 vs 910 us at C4.)
constexpr int kWideMinRows = 64;
#ifndef TQ_WIDE_CT
#define TQ_WIDE_CT 1
#endif
constexpr int kWideCT = TQ_WIDE_CT;             // 16-row column tiles per wave
constexpr int kWideRowsPerGroup = 64 * kWideCT;  // 4 waves x 16 CT rows
// Workgroups of the wide kernel one CU holds at once.
constexpr int kWideGroupsPerCU = 3 - kWideCT;
inline bool decode_is_wide(int d, int rows_per_head) { return d == 128 && rows_per_head >= kWideMinRows; }
template <int QJL>
hipError_t launch_decode_wide(const DecodeMfmaParams& p, int kb, int vb, dim3 grid, hipStream_t st);

// Decode waves one SIMD runs at once: 2, except at d = 256 with QJL keys or row
// groups of 8, whose register use allows one.
constexpr int decode_simd_waves(int d, int qjl, int rows_per_group) {
  return d == 256 && (qjl || rows_per_group == 8) ? 1 : 2;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, const DecodeMfmaExtra& x, hipStream_t st);
hipError_t launch_decode_ref(const DecodeArgs& a, hipStream_t st);
hipError_t launch_dequant_mfma(const DequantArgs& a, hipStream_t st);
hipError_t launch_dequant_fwht(const DequantArgs& a, hipStream_t st);
// launch_dequant_fwht for the Hadamard rotation, launch_dequant_mfma otherwise.
hipError_t launch_dequant(const DequantArgs& a, hipStream_t st);
hipError_t launch_dequant_qjl(const DequantQjlArgs& a, hipStream_t st);
// vqjl: values with QJL (a second accumulator per query row and coordinate).
bool ref_decode_supports(int d, int rows, bool vqjl);

}  // namespace tq
