// Block-scaled (MX) GEMM kernels (every tile shape but 256 x 256) for A x B = OCP FP6 E2M3 x FP6 E2M3.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaMX6<2, 2>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
