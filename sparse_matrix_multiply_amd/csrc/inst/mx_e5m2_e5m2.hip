// Block-scaled (MX) GEMM kernels (every tile shape) for A x B = OCP E5M2 x E5M2 with E8M0 block scales.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaMX<1, 1>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
