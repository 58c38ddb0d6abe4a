// Block-scaled (MX) GEMM kernels (every tile shape but 256 x 256) for A x B = OCP FP4 E2M1 x FP4 E2M1.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaMX4>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
