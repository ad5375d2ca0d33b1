// Tiles of 64 rows x D columns (bf16; D = 256 for head dims in (128, 256],
// 128 or 64 below that) shared by the slot-scheduled kernels: the LDS
// swizzle, the direct global->LDS loads that fill a tile, the lane parts of
// the MFMA operand reads and the bf16 stores of a 32-column accumulator
// block.
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
// For rows of 256 bytes or more, swz is a bijection on any 16 consecutive
// rows (the 16 rows of one b128 read cycle hit 16 distinct 4-bank groups)
// and swz / 4 differs across any 4 aligned rows (a transpose read's 4 rows
// x 64 bytes cover all 64 banks); the bank of a byte depends on its address
// modulo 256, so 512-byte rows behave as 256-byte rows. 128-byte rows
// (D = 64) put two rows in one 256-byte bank window, and the row parity
// takes the place of one bit. swz depends on the row modulo 16 only.
template <int D>
__device__ __forceinline__ int wide_swz(int r)
{
    return D >= 128 ? 4 * (r % 4) + (r / 4) % 4 : 4 * ((r / 2) % 2) + (r / 4) % 4;
}

// Direct global->LDS loads of rows row0 .. row0 + 63 of a [N][dh] bf16
// matrix into a 64 x D tile: 1 KB blocks of 512 / D rows, LPW per wave;
// lane l of block b writes physical chunk l % CPR of row
// (512 / D) b + l / CPR (CPR = D / 8 chunks per row), which holds its
// logical chunk (l % CPR) ^ swz(row). Rows past N read as zeros (the buffer
// resource ends at row N), so do the chunks past dh (an out-of-range offset;
// dh is a multiple of 8).
template <int D>
struct WideDmaT {
    static constexpr int CPR = D / 8;
    static constexpr int LPW = 64 * D * 2 / 1024 / WW;  // blocks per wave
    uint32_t off[LPW];
    __device__ __forceinline__ WideDmaT(int wave, int lane, int dh)
    {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int r = (512 / D) * (LPW * wave + i) + lane / CPR;
            const int c = (lane % CPR) ^ wide_swz<D>(r);
            off[i] = 8 * c < dh ? 2 * (r * dh + 8 * c) : kBufferOutOfRange;
        }
    }
    __device__ __forceinline__ static i32x4 rsrc(const uint16_t *src, int row0, int N, int dh)
    {
        return buffer_rsrc(src + (size_t)row0 * dh, (uint32_t)(N - row0) * (2 * dh));
    }
    // the i-th of this wave's LPW blocks (for spreading them over slots)
    __device__ __forceinline__ void issue_block(const i32x4 &rs, int i, uint32_t tile, int wave) const
    {
        lds_dma_buf_b128(rs, off[i], tile + (LPW * wave + i) * 1024);
    }
    __device__ __forceinline__ void issue(const uint16_t *src, int row0, int N, int dh, uint32_t tile,
                                          int wave) const
    {
        const i32x4 rs = rsrc(src, row0, N, dh);
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            issue_block(rs, i, tile, wave);
    }
};
using WideDma = WideDmaT<WD>;

// Lane parts of the LDS operand addresses on a 64 x D tile (rows of 2 D
// bytes). The swizzle is an XOR on the address bits 4..8 of a row's bytes
// (4..7 for 256-byte rows, 4..6 for 128-byte rows), which a tile base (a
// multiple of 512) and the
// row offsets leave clear, so a read takes the tile base plus the lane
// part, XORs in a per-read constant and adds the row offset through the
// instruction's immediate:
//   b128 operand, rows rb + l32, depth 16 kk.. (logical chunk 2 kk + hi,
//     = (2 kk) ^ hi): ((base + b128) ^ (32 kk)) + 2 D rb;
//   transpose operand of 16 rows r0.. (a multiple of 16) x 32 columns
//     32 db..: lane 4 t + u of 16-lane group g points at rows
//     rl = 4 (g / 2) + t and rl + 8, logical chunk 4 db + lc with
//     lc = 2 (g % 2) + u / 2 (= (4 db) ^ lc), element 4 (u % 2) in it:
//     ((base + tr0) ^ (64 db)) + 2 D r0 and the same with tr1.
// (Row blocks at multiples of 16 share the lane parts.)
template <int D>
struct WideLaneT {
    uint32_t b128, tr0, tr1;
    __device__ __forceinline__ explicit WideLaneT(int lane)
    {
        const int l32 = lane % 32, hi = lane / 32;
        b128 = l32 * (2 * D) + 16 * (hi ^ wide_swz<D>(l32));
        const int g = lane / 16, sl = lane % 16;
        const int rl = 4 * (g / 2) + sl / 4;
        const int lc = 2 * (g % 2) + (sl % 4) / 2;
        const int in = 4 * (sl % 2);
        tr0 = rl * (2 * D) + 16 * (lc ^ wide_swz<D>(rl)) + 2 * in;
        tr1 = (rl + 8) * (2 * D) + 16 * (lc ^ wide_swz<D>(rl + 8)) + 2 * in;
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
using WideLane = WideLaneT<WD>;

// The lane parts with each read's XOR constant already applied (computed
// once, D / 8 registers): a tile base that is a multiple of 512 adds to them
// without touching the XORed bits ((base + x) ^ c = base + (x ^ c) for
// c < 512), so a read whose tile base and row offset are compile-time
// constants takes no address arithmetic at all, the sum going into the
// instruction's offset field.
template <int D>
struct WideLaneXT {
    uint32_t rx[D / 16], tx0[D / 32], tx1[D / 32];
    __device__ __forceinline__ explicit WideLaneXT(int lane)
    {
        const WideLaneT<D> w(lane);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            rx[kk] = w.b128 ^ (32u * kk);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            tx0[db] = w.tr0 ^ (64u * db);
            tx1[db] = w.tr1 ^ (64u * db);
        }
    }
    // at: tile base (a multiple of 512) plus the row block's byte offset
    __device__ __forceinline__ bf16x8 rows(uint32_t at, int kk) const
    {
        return lds_b128_at(rx[kk] + at);
    }
    __device__ __forceinline__ bf16x8 trans(uint32_t at, int db) const
    {
        return lds_tr_pair_at(tx0[db] + at, tx1[db] + at);
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

}  // namespace fa
