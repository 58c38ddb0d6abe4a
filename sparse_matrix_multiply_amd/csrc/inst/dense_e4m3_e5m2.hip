// Dense GEMM kernels (every tile shape) for A x B = OCP fp8 E4M3 x bf8 E5M2.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaDenseF8<0, 1>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
