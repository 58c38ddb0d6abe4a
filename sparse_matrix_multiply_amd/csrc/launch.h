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
    // Block-scaled A and B (MX): E8M0 scale words, four 32-element blocks
    // along K per word; word t of row i of A at sa[t * ldsa + i] (t < scale_rows
    // = ceil(K / 128)), likewise sb for the columns of B.
    const uint32_t *sa, *sb;
    int64_t ldsa, ldsb;
    int scale_rows;
    const void *C;
    int64_t ldc;
    void *D;
    int64_t ldd;
    int M, N, K;     // K is the dense K
    float alpha, beta;
    int ialpha, ibeta;
    int use_c;       // beta != 0
    // fold_c: the accumulator starts as c_scale * C and the epilogue only
    // scales by alpha (float: c_scale = 1 when alpha == beta, c_scale = beta
    // when alpha == 1; int32: alpha == 1 and c_scale = beta, exact modulo
    // 2^32).  Other pairs read C in the epilogue.
    int fold_c;
    float c_scale;
    // vec_d: D starts on a 16-byte boundary and its row pitch is a multiple of
    // 16 bytes, so the epilogue may store 16 consecutive bytes of a row with
    // one access.
    int vec_d;
    // vec_c: the same for C (16- and 8-bit C is read four elements at a time
    // when it holds).
    int vec_c;
    // Epilogue variant (floating inputs only): d_type is OUT_ACC (C and D are
    // fp32) or one of the 16- / 8-bit types (C and D are of that type; C is
    // then never folded); bias is NULL or N fp32 values added per column;
    // act 1 applies ReLU.
    int d_type;
    int act;
    const float *bias;
    int tiles_m, tiles_n, group_m;
    // Split-K: K is cut into `splits` ranges of kt_per_split k-tiles (the last
    // range may be shorter) and each (output tile, range) pair is one
    // workgroup.  counters: one word per output tile, zero before and after
    // every call; partials: splits fp32 / int32 tiles of BM x BN per output
    // tile.  splits == 1: one range, counters and partials unused.
    int splits, kt_per_split;
    uint32_t *counters;
    uint8_t *partials;
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
// 256 x 256 tiles run 8 waves (2 per SIMD, 128 x 64 each); 256 x 128 and
// 128 x 256 tiles run 8 waves of 64 x 64 (2 per SIMD); 128 x 128 and 64 x 64
// tiles run 4 waves (one per SIMD, 64 x 64 and 32 x 32 each).
enum TileShape : int { TILE_256 = 0, TILE_128 = 1, TILE_64 = 2, TILE_SKINNY = 3, TILE_256x128 = 4, TILE_128x256 = 5 };

// Launchers (defined in the kernel files).  `dt_a`/`dt_b` use the public
// mmac_dtype_t codes.  They return hipSuccess or the launch error.
hipError_t launch_gemm_dense(int dt_a, int dt_b, TileShape shape, GemmParams p, hipStream_t s);
hipError_t launch_gemm_sparse(int dt_a, int dt_b, TileShape shape, GemmParams p, hipStream_t s);
hipError_t launch_gemm_skinny(int dt_a, int dt_b, GemmParams p, hipStream_t s);
hipError_t launch_gemm_mx(int dt_a, int dt_b, TileShape shape, GemmParams p, hipStream_t s);
hipError_t launch_gemm_layout(int dt_a, int dt_b, bool trans_a, bool trans_b, TileShape shape, GemmParams p,
                              hipStream_t s);
hipError_t launch_compress(int dt, CompressParams p, bool prune, hipStream_t s);

// Geometry of a tile shape.
inline int tile_rows(TileShape t) {
    return t == TILE_256 || t == TILE_256x128 ? 256 : t == TILE_128 || t == TILE_128x256 ? 128 : t == TILE_64 ? 64 : 32;
}
inline int tile_cols(TileShape t) {
    return t == TILE_256x128 ? 128 : t == TILE_128x256 ? 256 : tile_rows(t);
}

}  // namespace mmac
