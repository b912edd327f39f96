// Decode split kernel instantiations for head dimension 128, keys without QJL
// signs: every (key bits, value bits, scores output, rows per group).
#include "tq_decode_mfma_impl.h"

namespace tq {
namespace {

template <int D, int KB, int QJL, int VB>
hipError_t launch_split(const DecodeMfmaParams& p, dim3 grid, hipStream_t st) {
  const bool r8 = decode_rows_per_group(p.Hq / p.Hkv * p.Tq) == 8;
  if (p.scores) {
    if (r8)
      hipLaunchKernelGGL((decode_mfma_kernel<D, KB, QJL, VB, 1, 2>), grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<D, KB, QJL, VB, 1, 1>), grid, dim3(kThreads), 0, st, p);
  } else {
    if (r8)
      hipLaunchKernelGGL((decode_mfma_kernel<D, KB, QJL, VB, 0, 2>), grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<D, KB, QJL, VB, 0, 1>), grid, dim3(kThreads), 0, st, p);
  }
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

}  // namespace

hipError_t launch_decode_split_d128_q0(const DecodeMfmaParams& p, int kb, int vb, dim3 grid, hipStream_t st) {
  switch (kb) {
    case 1: return dispatch_vb<128, 1, 0>(p, vb, grid, st);
    case 2: return dispatch_vb<128, 2, 0>(p, vb, grid, st);
    case 3: return dispatch_vb<128, 3, 0>(p, vb, grid, st);
    default: return dispatch_vb<128, 4, 0>(p, vb, grid, st);
  }
}

}  // namespace tq
