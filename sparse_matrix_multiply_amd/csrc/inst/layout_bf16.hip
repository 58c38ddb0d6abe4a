// Dense GEMM kernels (every tile shape) for bfloat16 with A stored M-contiguous and / or B stored
// N-contiguous (fragments through transposed LDS reads).
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<Trans<MmaDense16<DT_BF16>, true, false>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDense16<DT_BF16>, false, true>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDense16<DT_BF16>, true, true>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
