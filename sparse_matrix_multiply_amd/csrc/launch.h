// Host-side interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmac {

// One GEMM as the tiled kernels see it.  Pitches of A/Ac and B are in bytes,
// of idx in 32-bit words, of C and D in elements.
struct GemmParams {
    const uint8_t *A;
    int64_t a_pitch;
    const uint8_t *B;
    int64_t b_pitch;
    const uint32_t *idx;
    int64_t idx_pitch;
    const void *C;
    int64_t ldc;
    void *D;
    int64_t ldd;
    int M, N, K;     // K is the dense K
    float alpha, beta;
    int ialpha, ibeta;
    int use_c;       // beta != 0
    int tiles_m, tiles_n, group_m;
};

struct CompressParams {
    const uint8_t *A;
    int64_t a_pitch;  // bytes
    uint8_t *Ac;
    int64_t ac_pitch; // bytes
    uint32_t *idx;
    int64_t idx_pitch; // words
    uint32_t *bad;
    int M, K;
};

// Tile shapes the host can pick from.
enum TileShape : int { TILE_256 = 0, TILE_128 = 1, TILE_64 = 2, TILE_SKINNY = 3, TILE_256_W8 = 4 };

// Launchers (defined in the kernel files).  `dt_a`/`dt_b` use the public
// mmac_dtype_t codes.  They return hipSuccess or the launch error.
hipError_t launch_gemm_dense(int dt_a, int dt_b, TileShape shape, GemmParams p, hipStream_t s);
hipError_t launch_gemm_sparse(int dt_a, int dt_b, TileShape shape, GemmParams p, hipStream_t s);
hipError_t launch_gemm_skinny(int dt_a, int dt_b, GemmParams p, hipStream_t s);
hipError_t launch_compress(int dt, CompressParams p, hipStream_t s);

// Geometry of a tile shape.
inline int tile_rows(TileShape t) {
    return (t == TILE_256 || t == TILE_256_W8) ? 256 : t == TILE_128 ? 128 : t == TILE_64 ? 64 : 32;
}

}  // namespace mmac
