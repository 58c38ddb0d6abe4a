// Sparse GEMM kernels (every tile shape) for A x B = OCP bf8 E5M2 x bf8 E5M2.
#include "../tiles_sparse.h"

namespace mmac {
template hipError_t launch_sparse_op<MmaSparse8<DT_E5M2, DT_E5M2>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
