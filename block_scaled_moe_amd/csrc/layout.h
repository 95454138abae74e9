// layout.h - byte layout of packed expert weights (codes and block scales), shared by
// the weight quantiser and the grouped GEMM kernels.
//
// Per expert, a weight matrix [N][K] (N % 32 == 0, K % 64 == 0) is cut into blocks of
// 32 rows x 64 columns, stored block-row-major ([N/32][K/64]). NVFP4: inside a block the
// 32 rows follow each other, each holding its 64 columns' codes in 32 bytes (E2M1,
// element 2i in the low nibble of byte i): 1 KiB. MXFP8 (E4M3, one byte per value): the
// block's four 16-column quarters are kept apart, [4][32 rows][16 bytes] (2 KiB), so
// that a wave's load of one quarter (or of two, one per half-wave) reads whole cache
// lines. The block scales follow the same block order, 4 bytes (four E4M3 scales of
// 16) or 2 bytes (two E8M0 scales of 32) per row.
//
// The GEMM kernels give each lane one weight row of a 32-row MFMA subtile, so a wave's
// codes for one 64-column chunk are a single contiguous run instead of 32 strided
// pieces, and its scales for the chunk one 128- or 64-byte run.
//
// MXFP4 keeps the two 32-column halves of a block apart: codes [2][32 rows][16 bytes],
// scales [2][32 rows]. The scaled FP4 MFMA takes one half-row (a whole 32-block with its
// scale) per lane, so lane l of a wave loads half l / 32 of row l % 32 and a wave's 64
// lanes read one contiguous 1 KiB of codes and 64 bytes of scales.
//
// In storage order, quantisation block r of an expert (16 values NVFP4, 32 MXFP8 and
// MXFP4) has its scale at byte r and, for NVFP4 and MXFP4, its codes at byte 8r / 16r
// (MXFP8: at code_offset of its row and first column, two 16-byte quarters); its source
// row and column follow from r below.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace layout {

__host__ __device__ constexpr int code_bytes_per_row(bool nv) { return nv ? 32 : 64; }
__host__ __device__ constexpr int scale_bytes_per_row(bool nv) { return nv ? 4 : 2; }
__host__ __device__ constexpr int code_block_bytes(bool nv) { return 32 * code_bytes_per_row(nv); }
__host__ __device__ constexpr int scale_block_bytes(bool nv) { return 32 * scale_bytes_per_row(nv); }

// index of the 32 x 64 block holding (n, k)
__host__ __device__ inline int64_t block_index(int64_t K, int64_t n, int64_t k) {
    return (n >> 5) * (K >> 6) + (k >> 6);
}

// byte offset inside one expert's codes of element (n, k); k even for NVFP4. MXFP8 keeps
// the four 16-column quarters of a block apart ([4][32 rows][16 bytes]).
__host__ __device__ inline int64_t code_offset(bool nv, int64_t K, int64_t n, int64_t k) {
    const int cb = code_bytes_per_row(nv);
    if (nv) return block_index(K, n, k) * (32 * cb) + (n & 31) * cb + ((k & 63) >> 1);
    return block_index(K, n, k) * (32 * cb) + ((k & 63) >> 4) * 512 + (n & 31) * 16 + (k & 15);
}

// byte offset inside one expert's scales of the block scale covering (n, k)
__host__ __device__ inline int64_t scale_offset(bool nv, int64_t K, int64_t n, int64_t k) {
    const int sb = scale_bytes_per_row(nv);
    return block_index(K, n, k) * (32 * sb) + (n & 31) * sb + ((k & 63) >> (nv ? 4 : 5));
}

// source row and first column of quantisation block r (storage order) of one expert
__host__ __device__ inline void block_source(bool nv, int64_t K, int64_t r, int64_t &n, int64_t &k) {
    const int per_row = nv ? 4 : 2;  // quantisation blocks per row of a 32 x 64 block
    const int64_t piece = r % per_row, row = (r / per_row) & 31, blk = r / (32 * per_row);
    const int64_t kb = K >> 6;
    n = 32 * (blk / kb) + row;
    k = 64 * (blk % kb) + (nv ? 16 : 32) * piece;
}

// bf16 weights (no quantisation) use the same 32 x 64 blocks (4 KiB), with the two
// 32-column halves kept apart like MXFP4: [2][32 rows][64 bytes], element k of a half at
// bytes 2k, 2k + 1. A lane's 32 values of a half are then one contiguous 64 bytes, and a
// wave load of 16 rows x 64 bytes covers whole cache lines. Storage piece r of an expert
// (16 bytes, 8 values) sits at byte 16r; its source row and first column:
__host__ __device__ inline void piece_source_bf16(int64_t K, int64_t r, int64_t &n, int64_t &k) {
    const int64_t piece = r & 3, row = (r >> 2) & 31, half = (r >> 7) & 1, blk = r >> 8;
    const int64_t kb = K >> 6;
    n = 32 * (blk / kb) + row;
    k = 64 * (blk % kb) + 32 * half + 8 * piece;
}
// byte offset inside one expert's bf16 codes of element (n, k)
__host__ __device__ inline int64_t code_offset_bf16(int64_t K, int64_t n, int64_t k) {
    return block_index(K, n, k) * 4096 + ((k & 63) >> 5) * 2048 + (n & 31) * 64 + 2 * (k & 31);
}

// MXFP4: source row and first column of quantisation block r (storage order)
__host__ __device__ inline void block_source_mx4(int64_t K, int64_t r, int64_t &n, int64_t &k) {
    const int64_t row = r & 31, half = (r >> 5) & 1, blk = r >> 6;
    const int64_t kb = K >> 6;
    n = 32 * (blk / kb) + row;
    k = 64 * (blk % kb) + 32 * half;
}

}  // namespace layout
}  // namespace moe
