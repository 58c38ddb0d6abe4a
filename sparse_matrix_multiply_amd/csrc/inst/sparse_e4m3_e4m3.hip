// Sparse GEMM kernels (every tile shape) for A x B = OCP fp8 E4M3 x fp8 E4M3.
#include "../tiles_sparse.h"

namespace mmac {
template hipError_t launch_sparse_op<MmaSparse8<DT_E4M3, DT_E4M3>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
