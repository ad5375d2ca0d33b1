// Tiles of 64 rows x 256 columns (bf16) shared by the kernels for head dims
// in (128, 256]: the LDS swizzle, the direct global->LDS loads that fill a
// tile, the lane parts of the MFMA operand reads and the bf16 stores of a
// 32-column accumulator block.
#pragma once

#include "fa_common.h"

namespace fa {

constexpr int WD = 256;          // LDS tile row width (elements)
constexpr int WKK = WD / 16;     // 16-deep steps of a 256-deep contraction
constexpr int WDB = 4;           // 32-column blocks of 128 columns
constexpr int WBT = 64;          // rows per LDS tile
constexpr int WW = 4;            // waves per workgroup, one per SIMD
constexpr int WROWS = 32 * WW;   // query rows or keys per workgroup
static_assert(WROWS == kMaskBlock, "a workgroup covers one mask block");

// Tile layout: logical 16-byte chunk c of row r sits at chunk c ^ swz(r).
// swz is a bijection on any 16 consecutive rows (the 16 rows of one b128
// read cycle hit 16 distinct 4-bank groups) and swz / 4 differs across any 4
// aligned rows (a transpose read's 4 rows x 64 bytes cover all 64 banks);
// the bank of a byte depends on its address modulo 256, so 512-byte rows
// behave as the 256-byte rows this swizzle was laid out for.
__device__ __forceinline__ int wide_swz(int r)
{
    return 4 * (r % 4) + (r / 4) % 4;
}

// Direct global->LDS loads of rows row0 .. row0 + 63 of a [N][dh] bf16
// matrix into a 64 x 256 tile: 32 blocks of 1 KB (two 512-byte rows each),
// 8 per wave; lane l of block b writes physical chunk l % 32 of row
// 2 b + l / 32, which holds its logical chunk (l % 32) ^ swz(row). Rows past
// N read as zeros (the buffer resource ends at row N), so do the chunks
// past dh (an out-of-range offset; dh is a multiple of 8).
struct WideDma {
    uint32_t off[8];
    __device__ __forceinline__ WideDma(int wave, int lane, int dh)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 2 * (8 * wave + i) + lane / 32;
            const int c = (lane % 32) ^ wide_swz(r);
            off[i] = 8 * c < dh ? 2 * (r * dh + 8 * c) : kBufferOutOfRange;
        }
    }
    __device__ __forceinline__ static i32x4 rsrc(const uint16_t *src, int row0, int N, int dh)
    {
        return buffer_rsrc(src + (size_t)row0 * dh, (uint32_t)(N - row0) * (2 * dh));
    }
    // the i-th of this wave's 8 blocks (for spreading them over slots)
    __device__ __forceinline__ void issue_block(const i32x4 &rs, int i, uint32_t tile, int wave) const
    {
        lds_dma_buf_b128(rs, off[i], tile + (8 * wave + i) * 1024);
    }
    __device__ __forceinline__ void issue(const uint16_t *src, int row0, int N, int dh, uint32_t tile,
                                          int wave) const
    {
        const i32x4 rs = rsrc(src, row0, N, dh);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            issue_block(rs, i, tile, wave);
    }
};

// Lane parts of the LDS operand addresses on a 64 x 256 tile. The swizzle
// is an XOR on address bits 4..8 of a row's bytes, which a tile base (a
// multiple of 512) and the row offsets leave clear, so a read takes the
// tile base plus the lane part, XORs in a per-read constant and adds the
// row offset through the instruction's immediate:
//   b128 operand, rows rb + l32, depth 16 kk.. (logical chunk 2 kk + hi,
//     = (2 kk) ^ hi): ((base + b128) ^ (32 kk)) + 512 rb;
//   transpose operand of 16 rows r0.. (a multiple of 16) x 32 columns
//     32 db..: lane 4 t + u of 16-lane group g points at rows
//     rl = 4 (g / 2) + t and rl + 8, logical chunk 4 db + lc with
//     lc = 2 (g % 2) + u / 2 (= (4 db) ^ lc), element 4 (u % 2) in it:
//     ((base + tr0) ^ (64 db)) + 512 r0 and the same with tr1.
// (wide_swz depends on the row modulo 16, so row blocks at multiples of 16
// share the lane parts.)
struct WideLane {
    uint32_t b128, tr0, tr1;
    __device__ __forceinline__ explicit WideLane(int lane)
    {
        const int l32 = lane % 32, hi = lane / 32;
        b128 = l32 * (2 * WD) + 16 * (hi ^ wide_swz(l32));
        const int g = lane / 16, sl = lane % 16;
        const int rl = 4 * (g / 2) + sl / 4;
        const int lc = 2 * (g % 2) + (sl % 4) / 2;
        const int in = 4 * (sl % 2);
        tr0 = rl * (2 * WD) + 16 * (lc ^ wide_swz(rl)) + 2 * in;
        tr1 = (rl + 8) * (2 * WD) + 16 * (lc ^ wide_swz(rl + 8)) + 2 * in;
    }
    // base: tile address (a multiple of 512); off: byte offset of the row
    // block (and of the tile within a slot), a compile-time constant
    __device__ __forceinline__ bf16x8 rows(uint32_t base, uint32_t off, int kk) const
    {
        return lds_b128_at(((base + b128) ^ (32u * kk)) + off);
    }
    __device__ __forceinline__ bf16x8 trans(uint32_t base, uint32_t off, int db) const
    {
        return lds_tr_pair_at(((base + tr0) ^ (64u * db)) + off, ((base + tr1) ^ (64u * db)) + off);
    }
};

// Stores a 32-column accumulator block (lane = row, register r = column
// c0 + 8 (r / 4) + 4 hi + r % 4) as bf16 times `mul`, columns < dh only.
__device__ __forceinline__ void wide_store(uint16_t *row_ptr, const f32x16 &acc, int c0, int hi, float mul,
                                           int dh)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = c0 + 8 * j + 4 * hi;
        if (col >= dh)
            continue;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(acc[4 * j] * mul) | ((uint32_t)f32_to_bf16_bits(acc[4 * j + 1] * mul) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(acc[4 * j + 2] * mul) |
               ((uint32_t)f32_to_bf16_bits(acc[4 * j + 3] * mul) << 16);
        *reinterpret_cast<uint2 *>(row_ptr + col) = pk;
    }
}

// One workgroup per 128 query rows; each wave holds 32 query rows of Q and
// dO, the B operands of S^T and dP^T, in AGPRs beside its eight dQ^T
// accumulators, so that the VGPRs hold the scores, the softmax and the
// operands read ahead. Per 32 keys (a step):
//   A: S^T = K Q^T and dP^T = V dO^T (lane = query; 16 MFMA pairs, K and V
//      rows read from LDS);
//   B: P^T = 2^(c s - lse2), dS^T = P^T o (dP^T - D) (vector ALU);
//   C: dQ^T += K^T dS^T over all 256 columns (16 MFMAs, K^T by transpose
//      reads).
// Every step ends inside its tile (WidePlan), so two LDS slots suffice: the
// next tile streams into the other one, a load per slot of the first step.
}  // namespace fa
