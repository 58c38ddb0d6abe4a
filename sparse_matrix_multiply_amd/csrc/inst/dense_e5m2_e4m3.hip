// Dense GEMM kernels (every tile shape) for A x B = OCP bf8 E5M2 x fp8 E4M3.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaDenseF8<1, 0>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
