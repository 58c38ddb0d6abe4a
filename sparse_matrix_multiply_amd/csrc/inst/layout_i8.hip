// Dense GEMM kernels (every tile shape) for int8 with A stored M-contiguous and / or B stored
// N-contiguous (fragments through transposed LDS reads).
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<Trans<MmaDenseI8, true, false>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDenseI8, false, true>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDenseI8, true, true>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
