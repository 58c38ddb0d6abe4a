// Dense GEMM kernels (every tile shape) for binary16 with A stored M-contiguous and / or B stored
// N-contiguous (fragments through transposed LDS reads).
#include "../tiles_dense.h"

namespace mmac {
template hipError_t launch_dense_op<Trans<MmaDense16<DT_F16>, true, false>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDense16<DT_F16>, false, true>>(TileShape, const GemmParams &, hipStream_t);
template hipError_t launch_dense_op<Trans<MmaDense16<DT_F16>, true, true>>(TileShape, const GemmParams &, hipStream_t);
}  // namespace mmac
