// Tiled bf16 GEMM instances with the EPI_SWIGLU epilogue (one translation unit per epilogue, so
// that the instances compile in parallel).
#include "gemm_tile.h"

namespace isd {

template <>
hipError_t launch_big_kernel<EPI_SWIGLU>(const GemmArgs& a, dim3 grid, int WV, int n_mt, int units, int S, hipStream_t s) {
  return launch_big_impl<EPI_SWIGLU>(a, grid, WV, n_mt, units, S, s);
}

}  // namespace isd
