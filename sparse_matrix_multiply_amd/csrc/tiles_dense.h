// Dense GEMM instantiations: bf16, fp16, int8, the four OCP fp8/bf8 pairs and
// their block-scaled (MX) forms.
// LDS stages of 128-byte rows: two for 256 x 256 tiles (64 KiB each; the next
// copy goes out right after the barrier that frees a stage), three for the
// 256 x 128 halves, four for the smaller tiles.
#pragma once

#include "gemm_tiled.h"

namespace mmac {

// Kernels of one instruction class Op for every tile shape; each element-type
// pair is instantiated in a source file of its own under inst/, so that the
// build compiles them in parallel.
template <class Op>
hipError_t launch_dense_op(TileShape shape, const GemmParams &p, hipStream_t s) {
    const dim3 grid(p.tiles_m * p.tiles_n * p.splits), block(256);   // one workgroup per tile and K range
    switch (shape) {
    case TILE_256:
        // block-scaled operands: the 8-wave tile has no registers left for the scale words
        if constexpr (Op::kScaled) return hipErrorInvalidValue;
        else hipLaunchKernelGGL((gemm_tiled_kernel<Op, 256, 256, 2, 4, 2>), grid, dim3(512), 0, s, p);
        break;
    // The halves of the 256 x 256 tile: eight waves of 64 x 64, two per SIMD to hide each other's
    // waits (measured against four waves of 64 x 128 on one GPU's 8192 x 1024 x 8192 share: bf16
    // 7 % and fp8 12 % faster; block-scaled fp8 11 % and FP4 6 % at 8192^3).
    case TILE_256x128: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 256, 128, 4, 2, 3>), grid, dim3(512), 0, s, p); break;
    case TILE_128x256: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 128, 256, 2, 4, 3>), grid, dim3(512), 0, s, p); break;
    case TILE_128: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 128, 128, 2, 2, 4>), grid, block, 0, s, p); break;
    case TILE_64: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 64, 64, 2, 2, 4>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mmac
