// Dense GEMM: dispatch on the element-type pair to the instantiations under inst/.
#include "device.h"
#include "launch.h"

namespace mmac {

// Defined in tiles_dense.h, instantiated once per type pair under inst/.
template <class Op>
hipError_t launch_dense_op(TileShape shape, const GemmParams &p, hipStream_t s);

hipError_t launch_gemm_dense(int a, int b, TileShape shape, GemmParams p, hipStream_t s) {
    if (a == DT_BF16 && b == DT_BF16) return launch_dense_op<MmaDense16<DT_BF16>>(shape, p, s);
    if (a == DT_F16 && b == DT_F16) return launch_dense_op<MmaDense16<DT_F16>>(shape, p, s);
    if (a == DT_I8 && b == DT_I8) return launch_dense_op<MmaDenseI8>(shape, p, s);
    // f8f6f4 format selectors: 0 = E4M3, 1 = E5M2
    if (a == DT_E4M3 && b == DT_E4M3) return launch_dense_op<MmaDenseF8<0, 0>>(shape, p, s);
    if (a == DT_E4M3 && b == DT_E5M2) return launch_dense_op<MmaDenseF8<0, 1>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E4M3) return launch_dense_op<MmaDenseF8<1, 0>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E5M2) return launch_dense_op<MmaDenseF8<1, 1>>(shape, p, s);
    return hipErrorInvalidValue;
}

template <class Op>
static hipError_t launch_trans(bool ta, bool tb, TileShape shape, const GemmParams &p, hipStream_t s) {
    if (ta && tb) return launch_dense_op<Trans<Op, true, true>>(shape, p, s);
    if (ta) return launch_dense_op<Trans<Op, true, false>>(shape, p, s);
    if (tb) return launch_dense_op<Trans<Op, false, true>>(shape, p, s);
    return launch_dense_op<Op>(shape, p, s);
}

hipError_t launch_gemm_layout(int a, int b, bool trans_a, bool trans_b, TileShape shape, GemmParams p, hipStream_t s) {
    if (a == DT_BF16 && b == DT_BF16) return launch_trans<MmaDense16<DT_BF16>>(trans_a, trans_b, shape, p, s);
    if (a == DT_F16 && b == DT_F16) return launch_trans<MmaDense16<DT_F16>>(trans_a, trans_b, shape, p, s);
    if (a == DT_I8 && b == DT_I8) return launch_trans<MmaDenseI8>(trans_a, trans_b, shape, p, s);
    if (a == DT_E4M3 && b == DT_E4M3) return launch_trans<MmaDenseF8<0, 0>>(trans_a, trans_b, shape, p, s);
    if (a == DT_E4M3 && b == DT_E5M2) return launch_trans<MmaDenseF8<0, 1>>(trans_a, trans_b, shape, p, s);
    if (a == DT_E5M2 && b == DT_E4M3) return launch_trans<MmaDenseF8<1, 0>>(trans_a, trans_b, shape, p, s);
    if (a == DT_E5M2 && b == DT_E5M2) return launch_trans<MmaDenseF8<1, 1>>(trans_a, trans_b, shape, p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_mx(int a, int b, TileShape shape, GemmParams p, hipStream_t s) {
    // f8f6f4 format selectors: 0 = E4M3, 1 = E5M2
    if (a == DT_E4M3 && b == DT_E4M3) return launch_dense_op<MmaMX<0, 0>>(shape, p, s);
    if (a == DT_E4M3 && b == DT_E5M2) return launch_dense_op<MmaMX<0, 1>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E4M3) return launch_dense_op<MmaMX<1, 0>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E5M2) return launch_dense_op<MmaMX<1, 1>>(shape, p, s);
    if (a == DT_FP4 && b == DT_FP4) return launch_dense_op<MmaMX4>(shape, p, s);
    // f8f6f4 format selectors: 2 = FP6 E2M3, 3 = BF6 E3M2
    if (a == DT_FP6 && b == DT_FP6) return launch_dense_op<MmaMX6<2, 2>>(shape, p, s);
    if (a == DT_FP6 && b == DT_BF6) return launch_dense_op<MmaMX6<2, 3>>(shape, p, s);
    if (a == DT_BF6 && b == DT_FP6) return launch_dense_op<MmaMX6<3, 2>>(shape, p, s);
    if (a == DT_BF6 && b == DT_BF6) return launch_dense_op<MmaMX6<3, 3>>(shape, p, s);
    return hipErrorInvalidValue;
}

}  // namespace mmac
