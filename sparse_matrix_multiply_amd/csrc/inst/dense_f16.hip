// Dense GEMM kernels (every tile shape) for A x B = binary16 x binary16.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaDense16<DT_F16>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
