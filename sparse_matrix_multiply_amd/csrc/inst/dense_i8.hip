// Dense GEMM kernels (every tile shape) for A x B = int8 x int8.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaDenseI8>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
