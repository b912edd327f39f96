// Kernel launch interfaces (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

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
  int64_t keys_per_split;
};

struct DequantArgs {
  const uint8_t* idx;
  const float* norm;
  int64_t seqs, n, cap;
  int d, bits, value_layout;
  const float *R, *Rt, *cent;  // R and R^T row-major
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
  float* out;
  int Hq, Hkv, Tq, causal;
  int rgroups;                      // groups of up to 4 query rows per KV head
  int64_t N, cap, keys_per_split;
  // Unequal splits (see split_blocks): workgroups with a linear index below
  // first_wgs get first_share / 1024 times the key blocks of the others; 0: all
  // splits of a row group have keys_per_split keys.
  int first_wgs, first_share;
  float *part, *scores;
};

// Blob and workspace pieces the matrix-core decode needs besides DecodeArgs.
struct DecodeMfmaExtra {
  const float *Rt, *St, *scales;
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
// The split kernel for one head dimension and key kind (tq_decode_mfma_d*.hip).
hipError_t launch_decode_split_d128_q0(const DecodeMfmaParams& p, int kb, int vb, int waves, dim3 grid,
                                       hipStream_t st);
hipError_t launch_decode_split_d128_q1(const DecodeMfmaParams& p, int kb, int vb, int waves, dim3 grid,
                                       hipStream_t st);
hipError_t launch_decode_split_d256_q0(const DecodeMfmaParams& p, int kb, int vb, int waves, dim3 grid,
                                       hipStream_t st);
hipError_t launch_decode_split_d256_q1(const DecodeMfmaParams& p, int kb, int vb, int waves, dim3 grid,
                                       hipStream_t st);
// Query rows one decode workgroup serves (4, or 8 when a KV head has more than
// 4 query rows: the matrix-core rows then carry 8 query rows x {hi, lo}).
inline int decode_rows_per_group(int rows_per_head) { return rows_per_head > 4 ? 8 : 4; }

// Decode waves one SIMD runs at once: 2, except at d = 256 with QJL keys or row
// groups of 8, whose register use allows one.
constexpr int decode_simd_waves(int d, int qjl, int rows_per_group) {
  return d == 256 && (qjl || rows_per_group == 8) ? 1 : 2;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, const DecodeMfmaExtra& x, hipStream_t st);
hipError_t launch_decode_ref(const DecodeArgs& a, hipStream_t st);
hipError_t launch_dequant_mfma(const DequantArgs& a, hipStream_t st);
bool ref_decode_supports(int d, int rows);

}  // namespace tq
