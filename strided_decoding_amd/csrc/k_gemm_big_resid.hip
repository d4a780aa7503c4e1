// Tiled bf16 GEMM instances with the EPI_RESID epilogue (one translation unit per epilogue, so
// that the instances compile in parallel).
#include "gemm_tile.h"

namespace isd {

template <>
hipError_t launch_big_kernel<EPI_RESID>(const GemmArgs& a, dim3 grid, int WV, int n_mt, int units, int S, hipStream_t s) {
  return launch_big_impl<EPI_RESID>(a, grid, WV, n_mt, units, S, s);
}

}  // namespace isd
