// Sparse GEMM: dispatch on the element-type pair to the instantiations under inst/.
#include "device.h"
#include "launch.h"

namespace mmac {

// Defined in tiles_sparse.h, instantiated once per type pair under inst/.
template <class Op>
hipError_t launch_sparse_op(TileShape shape, const GemmParams &p, hipStream_t s);

hipError_t launch_gemm_sparse(int a, int b, TileShape shape, GemmParams p, hipStream_t s) {
    if (a == DT_F16 && b == DT_F16) return launch_sparse_op<MmaSparse16<DT_F16>>(shape, p, s);
    if (a == DT_BF16 && b == DT_BF16) return launch_sparse_op<MmaSparse16<DT_BF16>>(shape, p, s);
    if (a == DT_I8 && b == DT_I8) return launch_sparse_op<MmaSparse8<DT_I8, DT_I8>>(shape, p, s);
    if (a == DT_E4M3 && b == DT_E4M3) return launch_sparse_op<MmaSparse8<DT_E4M3, DT_E4M3>>(shape, p, s);
    if (a == DT_E4M3 && b == DT_E5M2) return launch_sparse_op<MmaSparse8<DT_E4M3, DT_E5M2>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E4M3) return launch_sparse_op<MmaSparse8<DT_E5M2, DT_E4M3>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E5M2) return launch_sparse_op<MmaSparse8<DT_E5M2, DT_E5M2>>(shape, p, s);
    return hipErrorInvalidValue;
}

}  // namespace mmac
