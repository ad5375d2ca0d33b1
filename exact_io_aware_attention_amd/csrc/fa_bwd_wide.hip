// Backward of exact attention for head dims in (128, 256] on the matrix
// cores, by recomputation as in the 64/128-wide kernels
// (lukebest.github.io FlashAttention, "反向：重算而非存储"; mstx.cn/posts/485
// §三.3): P = 2^(c s - lse2), dP = dO V^T, dS = P o (dP - D), dQ = scale dS K,
// dK = scale dS^T Q, dV = P^T dO.
//
// At d = 256 a wave holds 32 rows of two 256-wide operands (128 VGPRs) and
// the accumulators of one 256-column gradient (128 AGPRs, asm MFMAs), but
// not those of two:
//   - bwd_wide_dq_kernel: one workgroup per 128 query rows; each wave holds
//     32 query rows of Q and dO as MFMA B operands; key/value tiles of 64
//     rows stream through LDS; S^T = K Q^T and dP^T = V dO^T (lane =
//     query), dS^T by the vector ALU, dQ^T += K^T dS^T over all 256 columns
//     with K^T from LDS transpose reads;
//   - bwd_wide_dkdv_kernel: one workgroup per 128 keys; each wave holds 32
//     keys of K (and V); query tiles of 64 rows (Q, dO, lse2, -D) stream
//     through LDS; S = Q K^T (lane = key). dV and dK take a pass each (dV^T
//     += dO^T P; then dP = dO V^T, dK^T += Q^T dS), so S is built twice:
//     8 contractions of work against the method's 5 (splitting each
//     gradient into column halves whose workgroups both rebuild S and dP
//     would take 11).
// The D and lse2 rows come from the 256-wide instance of the backward's
// preprocessing kernel. LDS tiles (512-byte rows, 16-byte chunks
// XOR-swizzled) are double-buffered: the next tile streams in by direct
// global->LDS loads while the current one is computed, one barrier per tile.
// A plain schedule, far from the pipelined 128-wide kernels. Work items
// (128-row blocks) are dealt so that each XCD takes one contiguous range of
// them: a head's blocks then share that XCD's L2, which reads their K/V (or
// Q/dO) tiles once for all of them.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int WD = 256;          // LDS tile row width (elements)
constexpr int WKK = WD / 16;     // 16-deep steps of a 256-deep contraction
constexpr int WDB = 4;           // 32-column blocks of 128 columns
constexpr int WBT = 64;          // rows per LDS tile
constexpr int WW = 4;            // waves per workgroup, one per SIMD
constexpr int WROWS = 32 * WW;   // query rows or keys per workgroup
static_assert(WROWS == kMaskBlock, "a workgroup covers one mask block");

struct WideParams {
    const uint16_t *Q, *K, *V, *dO;
    uint16_t *dQ, *dK, *dV;
    const float *ndelta, *lse2;
    const uint8_t *mask;
    int N, dh;
    int nblk;   // 128-row blocks per head
    int ntile;  // 64-row tiles per head
    int nmb;    // mask blocks per mask row
    int items;    // B * H * nblk
    int per_xcd;  // items per XCD (xcd_work_item)
    float c, scale;
};

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
    __device__ __forceinline__ void issue(const uint16_t *src, int row0, int N, int dh, uint32_t tile,
                                          int wave) const
    {
        const i32x4 rs = buffer_rsrc(src + (size_t)row0 * dh, (uint32_t)(N - row0) * (2 * dh));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            lds_dma_buf_b128(rs, off[i], tile + (8 * wave + i) * 1024);
    }
};

// MFMA A operand: rows rb .. rb + 31 of a tile (rb a multiple of 16), depth
// 16 kk .. 16 kk + 15 (logical chunk 2 kk + hi).
__device__ __forceinline__ bf16x8 wide_rows(const uint16_t *tile, int rb, int kk, int l32, int hi)
{
    return *reinterpret_cast<const bf16x8 *>(tile + (rb + l32) * WD + 8 * ((2 * kk + hi) ^ wide_swz(l32)));
}

// Lane part of a transpose read: 16 tile rows starting at r0, 32 columns
// starting at c0 (the A operand whose depth runs over rows, in the row order
// that matches a C tile's registers 8 s .. 8 s + 7 used as B operand).
struct WideTr {
    // lane offsets: rows 4 (g / 2) + sl / 4 and 8 further, logical chunk lc
    // (plus the block's), element in within it
    int row, lc, in;
    __device__ __forceinline__ explicit WideTr(int lane)
    {
        const int g = lane / 16, sl = lane % 16;
        row = 4 * (g / 2) + sl / 4;
        lc = 2 * (g % 2) + (sl % 4) / 2;
        in = 4 * (sl % 2);
    }
    // r0 a multiple of 16, c0 a multiple of 32
    __device__ __forceinline__ bf16x8 read(const uint16_t *tile, int r0, int c0) const
    {
        const int c = c0 / 8 + lc;
        return lds_read_tr_pair(tile + (r0 + row) * WD + 8 * (c ^ wide_swz(row)) + in,
                                tile + (r0 + row + 8) * WD + 8 * (c ^ wide_swz(row + 8)) + in);
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

template <bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(WW * kWave, 1) bwd_wide_dq_kernel(WideParams p)
{
    // one workgroup per block computes all 256 dQ columns (its 8
    // accumulators in AGPRs), so S^T and dP^T are built once
    constexpr int NC = 2 * WDB;  // 32-column blocks of dQ
    // two buffers of [K tile | V tile]
    constexpr uint32_t TB = WBT * WD * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TB];
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item0 = xcd_work_item(p.per_xcd);
    if (item0 >= p.items)
        return;
    const int item = item0;
    const int bh = item / p.nblk;
    const int bi = item - bh * p.nblk;
    const int qb = CAUSAL ? p.nblk - 1 - bi : bi;  // causal: heaviest first
    const int q0 = qb * WROWS;
    const int N = p.N, dh = p.dh;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave, l32 = lane % 32, hi = lane / 32;
    const int row = q0 + 32 * wave + l32;  // this lane's query
    const size_t head = (size_t)bh * N * dh;
    const WideTr tr(lane);

    bf16x8 qf[WKK], gf[WKK];
#pragma unroll
    for (int kk = 0; kk < WKK; ++kk) {
        const bool in = row < N && 16 * kk + 8 * hi < dh;
        qf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.Q + head + (size_t)row * dh + 16 * kk + 8 * hi)
                    : bf16x8{};
        gf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.dO + head + (size_t)row * dh + 16 * kk + 8 * hi)
                    : bf16x8{};
    }
    const float lse2 = row < N ? p.lse2[(size_t)bh * N + row] : INFINITY;
    const float nDi = row < N ? p.ndelta[(size_t)bh * N + row] : 0.f;
    f32x16 ndv;  // dP^T accumulates from -D (this lane's row)
#pragma unroll
    for (int r = 0; r < 16; ++r)
        ndv[r] = nDi;

    f32x16 dq[NC];
#pragma unroll
    for (int db = 0; db < NC; ++db)
        dq[db] = f32x16{};

    const int t_end = CAUSAL ? min(p.ntile, (q0 + WROWS - 1) / WBT + 1) : p.ntile;
    // key tiles the workgroup needs (one mask row, so uniform over it)
    MaskCursor mc;
    if (SPARSE)
        mc.init(p.mask + (size_t)qb * p.nmb, 1, p.nmb);
    auto next_tile = [&](int t) -> int {
        return SPARSE ? next_kept_tile(mc, t + 1, t_end, kMaskBlock / WBT) : t + 1;
    };
    const WideDma dma(wave, lane, dh);
    auto issue = [&](int t, int buf) {
        dma.issue(p.K + head, t * WBT, N, dh, lds0 + (2 * buf) * TB, wave);
        dma.issue(p.V + head, t * WBT, N, dh, lds0 + (2 * buf + 1) * TB, wave);
    };
    int t = next_tile(-1);
    if (t < t_end)
        issue(t, 0);
    lds_dma_wait<0>();
    __syncthreads();
    // Tile t computes from buffer `buf` while tile t+1 loads into the other,
    // whose last reads ended before the previous barrier.
    for (int buf = 0; t < t_end; buf ^= 1) {
        const int tn = next_tile(t);
        if (tn < t_end)
            issue(tn, buf ^ 1);
        const uint16_t *ks = reinterpret_cast<const uint16_t *>(smem + (2 * buf) * TB);
        const uint16_t *vs = reinterpret_cast<const uint16_t *>(smem + (2 * buf + 1) * TB);
        // The tile's two steps of 32 keys (tile rows kr..): S^T and dP^T
        // (MFMA), dS^T (vector ALU), dQ^T += K^T dS^T (MFMA). The second
        // step's S^T and dP^T are issued before the first step's dS^T, so
        // that the vector work runs beside independent MFMAs.
        auto scores = [&](int kr, f32x16 &s, f32x16 &dp) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < WKK; ++kk) {
                s = mfma32x32x16(wide_rows(ks, kr, kk, l32, hi), qf[kk], kk == 0 ? f32x16{} : s);
                dp = mfma32x32x16(wide_rows(vs, kr, kk, l32, hi), gf[kk], kk == 0 ? ndv : dp);
            }
        };
        // register r: key t * 64 + kr + 8 (r / 4) + 4 hi + r % 4
        auto dscores = [&](int kr, const f32x16 &s, const f32x16 &dp) __attribute__((always_inline)) {
            f32x16 ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = t * WBT + kr + 8 * (r / 4) + 4 * hi + (r % 4);
                float pe = exp2_fast(fmaf(s[r], p.c, -lse2));
                if (key >= N || (CAUSAL && key > row))
                    pe = 0.f;
                ds[r] = pe * dp[r];
            }
            return ds;
        };
        auto update = [&](int kr, const f32x16 &ds) __attribute__((always_inline)) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const bf16x8 sb = pack_bf16x8(ds, hh);
#pragma unroll
                for (int db = 0; db < NC; ++db)
                    mfma_acc_agpr(dq[db], tr.read(ks, kr + 16 * hh, 32 * db), sb);
            }
        };
        f32x16 s0, dp0, s1, dp1;
        scores(0, s0, dp0);
        scores(32, s1, dp1);
        update(0, dscores(0, s0, dp0));
        update(32, dscores(32, s1, dp1));
        mfma_drain();  // before the loop edge, where accumulators may be moved
        lds_dma_wait<0>();
        __syncthreads();
        t = tn;
    }
    mfma_drain();
#pragma unroll
    for (int db = 0; db < NC; ++db)
        mfma_settle(dq[db]);
    if (row < N) {
        uint16_t *out = p.dQ + head + (size_t)row * dh;
#pragma unroll
        for (int db = 0; db < NC; ++db)
            wide_store(out, dq[db], 32 * db, hi, p.scale, dh);
    }
}

// One workgroup per 128 keys. DV: all 256 columns of dV (S only); else all
// 256 columns of dK (S and dP): the accumulators of both gradients do not
// fit beside the K and V rows, so they take a pass each (5 contractions of
// work, against 6 for both gradients in column halves that each rebuild S
// and dP).
template <bool CAUSAL, bool SPARSE, bool DV>
__global__ void __launch_bounds__(WW * kWave, 1) bwd_wide_dkdv_kernel(WideParams p)
{
    constexpr bool DO_DV = DV, DO_DK = !DV;
    constexpr int NC = 2 * WDB;  // 32-column blocks of the gradient
    // two buffers of [Q tile | dO tile], then lse2 and -D rows per buffer
    constexpr uint32_t TB = WBT * WD * 2;
    constexpr uint32_t VEC = 4 * TB;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TB + 4 * WBT * 4];
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item0 = xcd_work_item(p.per_xcd);
    if (item0 >= p.items)
        return;
    const int item = item0;
    const int bh = item / p.nblk;
    const int kb = item - bh * p.nblk;  // causal: low key blocks see the most queries
    const int k0 = kb * WROWS;
    const int N = p.N, dh = p.dh;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave, l32 = lane % 32, hi = lane / 32;
    const int key = k0 + 32 * wave + l32;  // this lane's key
    const size_t head = (size_t)bh * N * dh;
    const WideTr tr(lane);

    bf16x8 kf[WKK], vf[WKK];
#pragma unroll
    for (int kk = 0; kk < WKK; ++kk) {
        const bool in = key < N && 16 * kk + 8 * hi < dh;
        kf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.K + head + (size_t)key * dh + 16 * kk + 8 * hi)
                    : bf16x8{};
        vf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.V + head + (size_t)key * dh + 16 * kk + 8 * hi)
                    : bf16x8{};
    }

    f32x16 dk[DO_DK ? NC : 1], dv[DO_DV ? NC : 1];
#pragma unroll
    for (int db = 0; db < NC; ++db) {
        if (DO_DK)
            dk[db] = f32x16{};
        if (DO_DV)
            dv[db] = f32x16{};
    }

    const int t_begin = CAUSAL ? k0 / WBT : 0;
    // query tiles the workgroup needs (one mask column, so uniform over it)
    MaskCursor mc;
    if (SPARSE)
        mc.init(p.mask + kb, p.nmb, p.nmb);
    auto next_tile = [&](int t) -> int {
        return SPARSE ? next_kept_tile(mc, t + 1, p.ntile, kMaskBlock / WBT) : t + 1;
    };
    const WideDma dma(wave, lane, dh);
    // rows past N read as zeros: their queries are masked below
    auto issue = [&](int t, int buf) {
        dma.issue(p.Q + head, t * WBT, N, dh, lds0 + (2 * buf) * TB, wave);
        dma.issue(p.dO + head, t * WBT, N, dh, lds0 + (2 * buf + 1) * TB, wave);
        if (wave < 2) {
            const float *v = (wave == 0 ? p.lse2 : p.ndelta) + (size_t)bh * N + t * WBT;
            const i32x4 rs = buffer_rsrc(v, (uint32_t)(N - t * WBT) * 4);
            lds_dma_buf_b32(rs, 4 * lane, lds0 + VEC + (2 * buf + wave) * WBT * 4);
        }
    };
    int t = next_tile(t_begin - 1);
    if (t < p.ntile)
        issue(t, 0);
    lds_dma_wait<0>();
    __syncthreads();
    // Tile t computes from buffer `buf` while tile t+1 loads into the other,
    // whose last reads ended before the previous barrier.
    for (int buf = 0; t < p.ntile; buf ^= 1) {
        const int tn = next_tile(t);
        if (tn < p.ntile)
            issue(tn, buf ^ 1);
        const uint16_t *qs = reinterpret_cast<const uint16_t *>(smem + (2 * buf) * TB);
        const uint16_t *gs = reinterpret_cast<const uint16_t *>(smem + (2 * buf + 1) * TB);
        const float *ls = reinterpret_cast<const float *>(smem + VEC + (2 * buf) * WBT * 4);
        const float *ns = reinterpret_cast<const float *>(smem + VEC + (2 * buf + 1) * WBT * 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int qr = 32 * h;  // tile rows (queries) of this step
            // register r: query t * 64 + qr + 8 (r / 4) + 4 hi + r % 4, so
            // registers 4 j .. 4 j + 3 are 4 consecutive queries
            f32x16 s = f32x16{}, dp, lq;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 nv = *reinterpret_cast<const f32x4 *>(ns + qr + 8 * j + 4 * hi);
                const f32x4 lv = *reinterpret_cast<const f32x4 *>(ls + qr + 8 * j + 4 * hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dp[4 * j + e] = nv[e];
                    lq[4 * j + e] = lv[e];
                }
            }
#pragma unroll
            for (int kk = 0; kk < WKK; ++kk) {
                s = mfma32x32x16(wide_rows(qs, qr, kk, l32, hi), kf[kk], s);
                if constexpr (DO_DK)
                    dp = mfma32x32x16(wide_rows(gs, qr, kk, l32, hi), vf[kk], dp);
            }
            f32x16 pm, ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qi = qr + 8 * (r / 4) + 4 * hi + (r % 4);
                const int q = t * WBT + qi;
                float pe = exp2_fast(fmaf(s[r], p.c, -lq[r]));
                if (q >= N || (CAUSAL && key > q))
                    pe = 0.f;
                pm[r] = pe;
                if constexpr (DO_DK)
                    ds[r] = pe * dp[r];
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const bf16x8 pb = pack_bf16x8(pm, hh);
                const bf16x8 sb = DO_DK ? pack_bf16x8(ds, hh) : bf16x8{};
#pragma unroll
                for (int db = 0; db < NC; ++db) {
                    if constexpr (DO_DV)
                        mfma_acc_agpr(dv[db], tr.read(gs, qr + 16 * hh, 32 * db), pb);
                    if constexpr (DO_DK)
                        mfma_acc_agpr(dk[db], tr.read(qs, qr + 16 * hh, 32 * db), sb);
                }
            }
        }
        mfma_drain();  // before the loop edge, where accumulators may be moved
        lds_dma_wait<0>();
        __syncthreads();
        t = tn;
    }
    mfma_drain();
#pragma unroll
    for (int db = 0; db < NC; ++db) {
        if constexpr (DO_DK)
            mfma_settle(dk[db]);
        if constexpr (DO_DV)
            mfma_settle(dv[db]);
    }
    if (key < N) {
        uint16_t *ok = p.dK + head + (size_t)key * dh;
        uint16_t *ov = p.dV + head + (size_t)key * dh;
#pragma unroll
        for (int db = 0; db < NC; ++db) {
            if constexpr (DO_DK)
                wide_store(ok, dk[db], 32 * db, hi, p.scale, dh);
            if constexpr (DO_DV)
                wide_store(ov, dv[db], 32 * db, hi, 1.f, dh);
        }
    }
}

template <bool CAUSAL, bool SPARSE>
hipError_t launch_wide(const WideParams &wp, hipStream_t stream)
{
    const dim3 grid(wp.per_xcd * kXcds), block(WW * kWave);
    hipLaunchKernelGGL((bwd_wide_dq_kernel<CAUSAL, SPARSE>), grid, block, 0, stream, wp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((bwd_wide_dkdv_kernel<CAUSAL, SPARSE, true>), grid, block, 0, stream, wp);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((bwd_wide_dkdv_kernel<CAUSAL, SPARSE, false>), grid, block, 0, stream, wp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16_wide(const Problem &pr, const uint16_t *dO, const uint16_t *Q,
                                const uint16_t *K, const uint16_t *V, const uint16_t *O,
                                const float *LSE, uint16_t *dQ, uint16_t *dK, uint16_t *dV,
                                void *workspace)
{
    hipError_t e = launch_bwd_prep_bf16(pr, dO, O, LSE, workspace);
    if (e != hipSuccess)
        return e;
    const BwdWorkspace L = bwd_workspace_layout(pr.B, pr.H, pr.N, pr.d);
    WideParams wp{};
    wp.Q = Q;
    wp.K = K;
    wp.V = V;
    wp.dO = dO;
    wp.dQ = dQ;
    wp.dK = dK;
    wp.dV = dV;
    wp.ndelta = reinterpret_cast<const float *>(static_cast<const char *>(workspace) + L.delta_off);
    wp.lse2 = reinterpret_cast<const float *>(static_cast<const char *>(workspace) + L.lse2_off);
    wp.mask = pr.mask;
    wp.N = pr.N;
    wp.dh = pr.d;
    wp.nblk = (pr.N + WROWS - 1) / WROWS;
    wp.ntile = (pr.N + WBT - 1) / WBT;
    wp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    wp.items = pr.B * pr.H * wp.nblk;
    wp.per_xcd = (wp.items + kXcds - 1) / kXcds;
    wp.c = pr.scale * kLog2e;
    wp.scale = pr.scale;
    const bool sparse = pr.mask != nullptr;
    if (pr.causal)
        return sparse ? launch_wide<true, true>(wp, pr.stream) : launch_wide<true, false>(wp, pr.stream);
    return sparse ? launch_wide<false, true>(wp, pr.stream) : launch_wide<false, false>(wp, pr.stream);
}

}  // namespace fa
