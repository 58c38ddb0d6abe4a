// Dense GEMM instantiations: bf16, fp16, int8 and the four OCP fp8/bf8 pairs.
// LDS stages of 128-byte rows: two for 256 x 256 tiles (64 KiB each; the next
// copy goes out right after the barrier that frees a stage), three for the
// 256 x 128 halves, four for the smaller tiles.
#include "gemm_tiled.h"

namespace mmac {

template <class Op>
static hipError_t launch_shape(TileShape shape, const GemmParams &p, hipStream_t s) {
    const dim3 grid(p.tiles_m * p.tiles_n), block(256);
    switch (shape) {
    case TILE_256: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 256, 256, 2, 4, 2>), grid, dim3(512), 0, s, p); break;
    case TILE_256x128: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 256, 128, 2, 2, 3>), grid, block, 0, s, p); break;
    case TILE_128x256: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 128, 256, 2, 2, 3>), grid, block, 0, s, p); break;
    case TILE_128: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 128, 128, 2, 2, 4>), grid, block, 0, s, p); break;
    case TILE_64: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 64, 64, 2, 2, 4>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_dense(int a, int b, TileShape shape, GemmParams p, hipStream_t s) {
    if (a == DT_BF16 && b == DT_BF16) return launch_shape<MmaDense16<DT_BF16>>(shape, p, s);
    if (a == DT_F16 && b == DT_F16) return launch_shape<MmaDense16<DT_F16>>(shape, p, s);
    if (a == DT_I8 && b == DT_I8) return launch_shape<MmaDenseI8>(shape, p, s);
    // f8f6f4 format selectors: 0 = E4M3, 1 = E5M2
    if (a == DT_E4M3 && b == DT_E4M3) return launch_shape<MmaDenseF8<0, 0>>(shape, p, s);
    if (a == DT_E4M3 && b == DT_E5M2) return launch_shape<MmaDenseF8<0, 1>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E4M3) return launch_shape<MmaDenseF8<1, 0>>(shape, p, s);
    if (a == DT_E5M2 && b == DT_E5M2) return launch_shape<MmaDenseF8<1, 1>>(shape, p, s);
    return hipErrorInvalidValue;
}

}  // namespace mmac
