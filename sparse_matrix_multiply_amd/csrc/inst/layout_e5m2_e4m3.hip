// Dense GEMM kernels (every tile shape) for A x B = OCP BF8 E5M2 x FP8 E4M3 with A stored M-contiguous
// and / or B stored N-contiguous (fragments through transposed LDS reads).
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<Trans<MmaDenseF8<1, 0>, true, false>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDenseF8<1, 0>, false, true>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDenseF8<1, 0>, true, true>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
