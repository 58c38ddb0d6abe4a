// Sparse GEMM kernels (every tile shape) for A x B = binary16 x binary16.
#include "../tiles_sparse.h"

namespace mmac {
template hipError_t launch_sparse_op<MmaSparse16<DT_F16>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
