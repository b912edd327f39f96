// Decode split kernel instantiations for one head dimension and key kind:
// every (key bits, value bits, scores output, rows per group).  The build
// compiles this file once per (TQ_INST_D, TQ_INST_KIND) pair -- d = 128, 256 x
// kind kKeysMse, kKeysQjl, kKeysDither -- so that the six sets compile in
// parallel.
#include "tq_decode_mfma_impl.h"

#if !defined(TQ_INST_D) || !defined(TQ_INST_KIND)
#error "compile with -DTQ_INST_D=<128|256> -DTQ_INST_KIND=<0|1|2>"
#endif

namespace tq {
namespace {

constexpr int kQjl = TQ_INST_KIND == kKeysQjl, kDither = TQ_INST_KIND == kKeysDither;

template <int D, int KB, int QJL, int VB, int SCORES, int NR, int W>
hipError_t launch(const DecodeMfmaParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_mfma_kernel<D, KB, QJL, VB, SCORES, NR, W, kDither>), grid, dim3(64 * W), 0, st, p);
  return hipGetLastError();
}

// Where the plan asks for 8-wave workgroups (4-row groups with two waves per
// SIMD), calls without score output get them; calls that also write the scores,
// and the dithered variant, run 4-wave workgroups on the same grid.
template <int D, int KB, int QJL, int VB>
hipError_t launch_split(const DecodeMfmaParams& p, int waves, dim3 grid, hipStream_t st) {
  const bool r8 = decode_rows_per_group(p.Hq / p.Hkv * p.Tq) == 8;
  if (p.scores) return r8 ? launch<D, KB, QJL, VB, 1, 2, 4>(p, grid, st) : launch<D, KB, QJL, VB, 1, 1, 4>(p, grid, st);
  if (r8) return launch<D, KB, QJL, VB, 0, 2, 4>(p, grid, st);
  if constexpr (decode_simd_waves(D, QJL, 4) == 2 && !kDither) {
    if (waves == 8) return launch<D, KB, QJL, VB, 0, 1, 8>(p, grid, st);
  }
  return launch<D, KB, QJL, VB, 0, 1, 4>(p, grid, st);
}

template <int D, int KB, int QJL>
hipError_t dispatch_vb(const DecodeMfmaParams& p, int vb, int waves, dim3 grid, hipStream_t st) {
  switch (vb) {
    case 1: return launch_split<D, KB, QJL, 1>(p, waves, grid, st);
    case 2: return launch_split<D, KB, QJL, 2>(p, waves, grid, st);
    case 3: return launch_split<D, KB, QJL, 3>(p, waves, grid, st);
    default: return launch_split<D, KB, QJL, 4>(p, waves, grid, st);
  }
}

}  // namespace

template <>
hipError_t launch_decode_split<TQ_INST_D, TQ_INST_KIND>(const DecodeMfmaParams& p, int kb, int vb, int waves,
                                                        dim3 grid, hipStream_t st) {
  switch (kb) {
    case 1: return dispatch_vb<TQ_INST_D, 1, kQjl>(p, vb, waves, grid, st);
    case 2: return dispatch_vb<TQ_INST_D, 2, kQjl>(p, vb, waves, grid, st);
    case 3: return dispatch_vb<TQ_INST_D, 3, kQjl>(p, vb, waves, grid, st);
    default: return dispatch_vb<TQ_INST_D, 4, kQjl>(p, vb, waves, grid, st);
  }
}

}  // namespace tq
