// Sparse (4:2 A) GEMM instantiations: fp16, bf16, int8 and the four fp8/bf8 pairs.
// Three LDS stages of 128-byte B rows: the sparse kernel moves 1.5x the bytes per
// unit of matrix work of the dense one, and whole 128-byte rows per copy
// request measured faster than more, narrower stages.
#pragma once

#include "gemm_tiled.h"

namespace mmac {

// Kernels of one instruction class Op for every tile shape; each element-type
// pair is instantiated in a source file of its own under inst/, so that the
// build compiles them in parallel.
template <class Op>
hipError_t launch_sparse_op(TileShape shape, const GemmParams &p, hipStream_t s) {
    const dim3 grid(p.tiles_m * p.tiles_n * p.splits), block(256);   // one workgroup per tile and K range
    switch (shape) {
    case TILE_256: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 256, 256, 2, 4, 3>), grid, dim3(512), 0, s, p); break;
    // the halves of the 256 x 256 tile: eight waves of 64 x 64, two per SIMD, as for the whole tile
    case TILE_256x128: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 256, 128, 4, 2, 4>), grid, dim3(512), 0, s, p); break;
    case TILE_128x256: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 128, 256, 2, 4, 3>), grid, dim3(512), 0, s, p); break;
    case TILE_128: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 128, 128, 2, 2, 3>), grid, block, 0, s, p); break;
    case TILE_64: hipLaunchKernelGGL((gemm_tiled_kernel<Op, 64, 64, 2, 2, 3>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mmac
