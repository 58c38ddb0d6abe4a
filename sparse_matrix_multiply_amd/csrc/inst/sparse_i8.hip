// Sparse GEMM kernels (every tile shape) for A x B = int8 x int8.
#include "../tiles_sparse.h"

namespace mmac {
template hipError_t launch_sparse_op<MmaSparse8<DT_I8, DT_I8>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
