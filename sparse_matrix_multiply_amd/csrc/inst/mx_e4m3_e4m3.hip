// Block-scaled (MX) GEMM kernels (every tile shape) for A x B = OCP E4M3 x E4M3 with E8M0 block scales.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaMX<0, 0>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
