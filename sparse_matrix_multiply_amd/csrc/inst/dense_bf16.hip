// Dense GEMM kernels (every tile shape) for A x B = bfloat16 x bfloat16.
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<MmaDense16<DT_BF16>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
