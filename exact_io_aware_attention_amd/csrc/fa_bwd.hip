// Backward of exact attention on gfx950 by recomputation: P is rebuilt
// tile by tile from Q, K and the saved LSE instead of being stored
// (lukebest.github.io FlashAttention, "反向：重算而非存储"; mstx.cn/posts/485
// §三.3 "重计算"; nanhubrain.csdn.net §二 "反向传播的代价").
//
// Gradient rule (the softmax Jacobian written out; the formula printed in
// cloud.baidu.com §工作原理 "梯度计算优化" is garbled):
//   P = exp(scale Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,
//   dS = P o (dP - D),  D_i = sum_k dO_ik O_ik,
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Kernels, all on the caller's stream:
//   1. bwd_pre:  -D and LSE * log2(e) per row (bandwidth-bound, one pass
//      over dO and O);
//   2. bwd_dq:   one workgroup per 128 (d = 128) or 256 (d = 64) query
//      rows, key/value tiles streamed through LDS; recomputes S^T and dP^T,
//      forms dS^T and accumulates dQ^T = K^T dS^T (lane = query, as in the
//      forward);
//   3. bwd_dkdv: one workgroup per 128 or 256 keys (K and V rows in
//      registers), query tiles streamed through LDS; recomputes S and dP,
//      accumulates dV^T = dO^T P and dK^T = Q^T dS (lane = key).
// Splitting dQ from dK/dV recomputes S and dP once more (7 contractions
// instead of 5) but needs no atomics and is deterministic. (Accumulating dQ
// across key blocks with fp32 global atomics instead was measured at about
// 1.4 TB/s of atomic traffic on MI355X, which at 128 keys per block costs
// more time than the two extra contractions.)
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

// ---------------------------------------------------------------- pre ----

template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const uint16_t *dO, const uint16_t *O,
                                                      const float *LSE, float *ndelta,
                                                      float *lse2, long rows)
{
    constexpr int LPR = D / 8;  // lanes per row, 8 bf16 each
    const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const uint4 a = *reinterpret_cast<const uint4 *>(dO + row * D + 8 * part);
        const uint4 b = *reinterpret_cast<const uint4 *>(O + row * D + 8 * part);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), acc);
            acc = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(bv[i] & 0xffff0000u), acc);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off /= 2)
        acc += __shfl_xor(acc, off, kWave);
    if (row < rows && part == 0) {
        ndelta[row] = -acc;
        const float L = LSE[row];
        lse2[row] = (L == -INFINITY) ? INFINITY : L * kLog2e;
    }
}

// ------------------------------------------------------- shared pieces ---
//
// Both main kernels run 4 waves per workgroup, one per SIMD (up to 512
// registers each), with 32 rows per wave for d = 128 and 64 for d = 64 (so
// each operand fragment read from LDS feeds two MFMAs). The long-lived
// accumulators (dQ^T, or dK^T and dV^T) stay in AGPRs; operands, S, dP and
// the softmax temporaries use the VGPRs.
//
// Tiles of 64 rows stream through LDS by direct global->LDS loads (rows past
// the end of the sequence are loaded from the last row and masked). The
// row-major tiles are read two ways: b128 operand reads (16 consecutive rows
// per LDS cycle) and transpose reads (4 consecutive rows x 32 bytes per 16
// lanes). The swizzle f(r) below stores logical 16-byte chunk c of row r at
// chunk c ^ f(r); f is a bijection on any 16 consecutive rows (b128 reads
// conflict-free) and f(r) / 2 differs across any 4 aligned rows (transpose
// reads conflict-free).
template <int D>
__device__ __forceinline__ int tile_swz(int r)
{
    if (D == 128)  // 16 chunks per 256-byte row
        return 2 * (r % 4) + 8 * ((r / 4) % 2) + ((r / 8) % 2);
    return 2 * ((r / 2) % 4) + ((r / 8) % 2);  // 8 chunks per 128-byte row
}

// Issues the direct loads of one 64-row tile (row-major, d contiguous) into
// LDS: 1 KB blocks spread over the workgroup's waves.
template <int D, int W>
__device__ __forceinline__ void issue_rows_tile(const uint16_t *src, uint16_t *dst, int row0, int N,
                                                int wave, int lane)
{
    constexpr int CPR = D / 8;
    constexpr int BLOCKS = 64 * D * 2 / 1024;
    static_assert(BLOCKS % W == 0, "tile blocks per wave");
#pragma unroll
    for (int i = 0; i < BLOCKS / W; ++i) {
        const int b = wave * (BLOCKS / W) + i;
        const int r = b * (64 / CPR) + lane / CPR;
        const int lc = (lane % CPR) ^ tile_swz<D>(r);
        const int row = min(row0 + r, N - 1);
        lds_dma_b128(src + (size_t)row * D + 8 * lc, lds_byte_addr(dst) + b * 1024);
    }
}

// Direct load of 64 consecutive floats (one wave): row-vector statistics.
__device__ __forceinline__ void issue_vec64(const float *src, float *dst, int row0, int N, int lane)
{
    const int row = min(row0 + lane, N - 1);
    lds_dma_b32(src + row, lds_byte_addr(dst));
}

// b128 operand read: row r, logical chunk c of a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 tile_b128(const uint16_t *t, int r, int c)
{
    return lds_read_b128(t + r * D + 8 * (c ^ tile_swz<D>(r)));
}

// Transpose-read operand (32 columns x 16 rows, as the A operand whose k
// index runs over rows): lane 4t+u of 16-lane group g points at row
// r0 + 4*(g/2) + t (and r0 + 8 + ... for slots 4..7), columns
// col0 + 16*(g%2) + 4u.
template <int D>
__device__ __forceinline__ bf16x8 tile_tr(const uint16_t *t, int r0, int col0, int lane)
{
    const int g = lane / 16, sl = lane % 16;
    const int r = r0 + 4 * (g / 2) + sl / 4;
    const int col = col0 + 16 * (g % 2) + 4 * (sl % 4);
    const int c = col / 8, e = col % 8;
    return lds_read_tr_pair(t + r * D + 8 * (c ^ tile_swz<D>(r)) + e,
                            t + (r + 8) * D + 8 * (c ^ tile_swz<D>(r + 8)) + e);
}

// Stores a 32-row accumulator block (lane = row, registers = 32 columns in
// runs of 4) as bf16, times a factor.
__device__ __forceinline__ void store_rows_bf16(uint16_t *dst_row, const f32x16 &acc, int col0, int hi,
                                                float mul)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(acc[4 * j + 0] * mul) |
               ((uint32_t)f32_to_bf16_bits(acc[4 * j + 1] * mul) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(acc[4 * j + 2] * mul) |
               ((uint32_t)f32_to_bf16_bits(acc[4 * j + 3] * mul) << 16);
        *reinterpret_cast<uint2 *>(dst_row + col0 + 8 * j + 4 * hi) = pk;
    }
}

// ----------------------------------------------------------------- dQ ----

struct DqParams {
    const uint16_t *dO, *Q, *K, *V;
    const float *ndelta, *lse2;  // -D and LSE * log2(e) per row
    uint16_t *dQ;
    const uint8_t *mask;
    int N, nqb, nkt, nmb, items, per_xcd;
    float c, scale;
};

// One workgroup owns 256 query rows of one (b, h) (64 per wave, Q and dO
// rows held as MFMA B operands); key/value tiles of 64 stream through LDS.
// Per 32 keys: S^T = K Q^T and dP^T = V dO^T (lane = query), then
// dS^T = P^T o (dP^T - D) with P^T = 2^(c s - lse2), then
// dQ^T += K^T dS^T with K^T from transpose reads of the K tile.
// Waves per workgroup and 32-row MFMA blocks per wave. The dK/dV kernel
// holds K and V operands, two accumulators per block and two pipelined steps
// of S, dP, P and dS, which only fit the register file with one block per
// wave; its workgroup then covers 128 keys, one block-mask column.
template <int D, bool DKDV>
struct BwdShape {
    static constexpr int W = 4;
    static constexpr int NB = (D == 128 || DKDV) ? 1 : 2;
    static constexpr int ROWS = 32 * NB * W;  // rows per workgroup
};

template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256, 1) bwd_dq_kernel(DqParams p)
{
    static_assert(BwdShape<D, false>::W * 64 == 256, "launch bounds");
    constexpr int W = BwdShape<D, false>::W;
    constexpr int NB = BwdShape<D, false>::NB;
    constexpr int QW = 32 * NB;     // query rows per wave
    constexpr int BR = W * QW;      // query rows per workgroup
    constexpr int BC = 64;          // keys per LDS tile
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = BC * D;

    __shared__ __attribute__((aligned(1024))) uint16_t Ks[2][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs[2][TILE];

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nqb;
    const int qi = item - bh * p.nqb;
    const int qblk = CAUSAL ? (p.nqb - 1 - qi) : qi;
    const int q0 = qblk * BR;
    const int N = p.N;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int wr0 = q0 + wave * QW;

    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t *Qh = p.Q + head, *dOh = p.dO + head;
    const uint16_t *Kh = p.K + head, *Vh = p.V + head;

    bf16x8 qf[NB][KK], gf[NB][KK];
    float lse2[NB], nDi[NB];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
        const int row = wr0 + 32 * qb + l32;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qf[qb][kk] = row < N ? *reinterpret_cast<const bf16x8 *>(Qh + (size_t)row * D + 16 * kk + 8 * hi)
                                 : bf16x8{};
            gf[qb][kk] = row < N ? *reinterpret_cast<const bf16x8 *>(dOh + (size_t)row * D + 16 * kk + 8 * hi)
                                 : bf16x8{};
        }
        lse2[qb] = row < N ? p.lse2[(size_t)bh * N + row] : INFINITY;
        nDi[qb] = row < N ? p.ndelta[(size_t)bh * N + row] : 0.f;
    }

    int t_end = p.nkt;
    if (CAUSAL)
        t_end = min(p.nkt, (q0 + BR - 1) / BC + 1);
    const int mr_lo = q0 / kMaskBlock;
    const int mr_hi = min(q0 + BR - 1, N - 1) / kMaskBlock;
    const int wmr = min(wr0, N - 1) / kMaskBlock;  // <= 64 rows: one mask row per wave
    auto tile_needed = [&](int t) -> bool {
        if (!SPARSE)
            return true;
        bool keep = false;
        for (int mr = mr_lo; mr <= mr_hi; ++mr)
            keep |= p.mask[(size_t)mr * p.nmb + (t * BC) / kMaskBlock] != 0;
        return keep;
    };
    auto next_tile = [&](int t) -> int {
        ++t;
        if (SPARSE)
            while (t < t_end && !tile_needed(t))
                ++t;
        return t;
    };

    f32x16 dq[NB][DB];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            dq[qb][db] = f32x16{};

    int t = next_tile(-1);
    if (t < t_end) {
        issue_rows_tile<D, W>(Kh, Ks[0], t * BC, N, wave, lane);
        issue_rows_tile<D, W>(Vh, Vs[0], t * BC, N, wave, lane);
    }
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            wait_loaded(qf[qb][kk]);
            wait_loaded(gf[qb][kk]);
        }
        wait_loaded(lse2[qb]);
        wait_loaded(nDi[qb]);
    }
    lds_dma_wait<0>();
    __syncthreads();
    int buf = 0;
    while (t < t_end) {
        const int tn = next_tile(t);
        if (tn < t_end) {
            issue_rows_tile<D, W>(Kh, Ks[buf ^ 1], tn * BC, N, wave, lane);
            issue_rows_tile<D, W>(Vh, Vs[buf ^ 1], tn * BC, N, wave, lane);
        }
        const int kbase = t * BC;
        const bool drop = SPARSE && p.mask[(size_t)wmr * p.nmb + kbase / kMaskBlock] == 0;
        {
            const uint16_t *ks = Ks[buf];
            const uint16_t *vs = Vs[buf];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                f32x16 s[NB], dp[NB];
#pragma unroll
                for (int qb = 0; qb < NB; ++qb)
                    s[qb] = dp[qb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const bf16x8 ka = tile_b128<D>(ks, 32 * kh + l32, 2 * kk + hi);
                    const bf16x8 va = tile_b128<D>(vs, 32 * kh + l32, 2 * kk + hi);
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb) {
                        s[qb] = mfma32x32x16(ka, qf[qb][kk], s[qb]);
                        dp[qb] = mfma32x32x16(va, gf[qb][kk], dp[qb]);
                    }
                }
                const int k0 = kbase + 32 * kh;
                const bool need_mask = drop || (k0 + 32 > N) || (CAUSAL && k0 + 31 > wr0);
                bf16x8 sb[NB][2];
#pragma unroll
                for (int qb = 0; qb < NB; ++qb) {
                    const int row = wr0 + 32 * qb + l32;
                    f32x16 ds;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float pr = exp2_fast(fmaf(s[qb][r], p.c, -lse2[qb]));
                        if (need_mask) {
                            const int key = k0 + 8 * (r / 4) + 4 * hi + (r % 4);
                            if (drop || key >= N || (CAUSAL && key > row))
                                pr = 0.f;
                        }
                        ds[r] = pr * (dp[qb][r] + nDi[qb]);
                    }
                    sb[qb][0] = pack_bf16x8(ds, 0);
                    sb[qb][1] = pack_bf16x8(ds, 1);
                }
                // dQ^T += K^T dS^T: K^T (32 d x 16 keys) by transpose reads,
                // one read per NB MFMAs.
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 kt = tile_tr<D>(ks, 32 * kh + 16 * hh, 32 * db, lane);
#pragma unroll
                        for (int qb = 0; qb < NB; ++qb)
                            mfma_acc_agpr(dq[qb][db], kt, sb[qb][hh]);
                    }
            }
        }
        // before the loop edges, where the compiler may move accumulators
        mfma_drain();
        lds_dma_wait<0>();  // the next tile has landed (all waves: barrier)
        __syncthreads();
        buf ^= 1;
        t = tn;
    }

    mfma_drain();
#pragma unroll
    for (int qb = 0; qb < NB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            mfma_settle(dq[qb][db]);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
        const int row = wr0 + 32 * qb + l32;
        if (row < N) {
            uint16_t *dst = p.dQ + head + (size_t)row * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                store_rows_bf16(dst, dq[qb][db], 32 * db, hi, p.scale);
        }
    }
}

// -------------------------------------------------------------- dK dV ----

struct DkvParams {
    const uint16_t *dO, *Q, *K, *V;
    const float *ndelta, *lse2;  // -D and LSE * log2(e) per row
    uint16_t *dK, *dV;
    const uint8_t *mask;
    int N, nkb, nqt, nmb, items, per_xcd;
    float c, scale;
};

// One workgroup owns 128 keys of one (b, h), K and V rows held as MFMA B
// operands; query tiles of 64 (Q, dO, LSE, -D) stream
// through LDS. Per 32 queries (a step):
//   A: S = Q K^T and dP - D = dO V^T - D (lane = key, MFMA; the dP
//      accumulator starts from -D);
//   B: P = 2^(c s - lse2), dS = P o (dP - D) (vector ALU);
//   C: dV^T += dO^T P and dK^T += Q^T dS (MFMA, dO^T and Q^T by transpose
//      reads; accumulators in AGPRs).
// With one wave per SIMD nothing hides a wave's own latencies, so the steps
// are software-pipelined and the order is fixed by hand: step i runs A(i),
// then C(i-1) with B(i) spread over its MFMA slots, every LDS operand read
// issued a few MFMAs ahead of its use. Scheduling fences keep the compiler
// from regrouping the slots (it cannot see the asm MFMAs' latencies).
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(DkvParams p)
{
    static_assert(BwdShape<D, true>::W * 64 == 256, "launch bounds");
    constexpr int W = BwdShape<D, true>::W;
    constexpr int NB = BwdShape<D, true>::NB;
    constexpr int KW = 32 * NB;     // keys per wave
    constexpr int BK = W * KW;      // keys per workgroup
    constexpr int BQ = 64;          // queries per LDS tile
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = BQ * D;
    constexpr int NPR = 2 * DB;          // transpose-operand pairs (dO^T, Q^T) per step
    constexpr int EPP = 16 * NB / NPR;   // softmax elements per pair slot
    constexpr int PA = D == 128 ? 3 : 2; // A operand reads issued this many slots ahead
    constexpr int PD = D == 128 ? 3 : 2; // C operand pairs issued this many slots ahead
    static_assert(2 * NB * NPR == KK * NB * 2, "as many MFMAs in A as in C");
    static_assert(PA <= KK && PD <= KK && EPP * NPR == 16 * NB && 8 % EPP == 0, "slot plan");
    // One mask column per workgroup: a tile it visits is kept for all waves.
    static_assert(BK == kMaskBlock, "workgroup keys = one mask block");

    __shared__ __attribute__((aligned(1024))) uint16_t Qs[3][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Gs[3][TILE];
    __shared__ __attribute__((aligned(256))) float Ls[3][BQ];
    __shared__ __attribute__((aligned(256))) float Ds[3][BQ];

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nkb;
    const int kblk = item - bh * p.nkb;  // causal: low key blocks see the most queries
    const int k0 = kblk * BK;
    const int N = p.N;
    const float c = p.c;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int wk0 = k0 + wave * KW;

    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t *Qh = p.Q + head, *dOh = p.dO + head;
    const uint16_t *Kh = p.K + head, *Vh = p.V + head;
    const float *lse2h = p.lse2 + (size_t)bh * N;
    const float *ndh = p.ndelta + (size_t)bh * N;

    bf16x8 kf[NB][KK], vf[NB][KK];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
        const int key = wk0 + 32 * kb + l32;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            kf[kb][kk] = key < N ? *reinterpret_cast<const bf16x8 *>(Kh + (size_t)key * D + 16 * kk + 8 * hi)
                                 : bf16x8{};
            vf[kb][kk] = key < N ? *reinterpret_cast<const bf16x8 *>(Vh + (size_t)key * D + 16 * kk + 8 * hi)
                                 : bf16x8{};
        }
    }

    const int t_begin = CAUSAL ? k0 / BQ : 0;
    auto tile_needed = [&](int t) __attribute__((always_inline)) -> bool {
        return !SPARSE || p.mask[(size_t)((t * BQ) / kMaskBlock) * p.nmb + kblk] != 0;
    };
    auto next_tile = [&](int t) __attribute__((always_inline)) -> int {
        ++t;
        if (SPARSE)
            while (t < p.nqt && !tile_needed(t))
                ++t;
        return t;
    };
    auto issue_tile = [&](int t, int b) __attribute__((always_inline)) {
        issue_rows_tile<D, W>(Qh, Qs[b], t * BQ, N, wave, lane);
        issue_rows_tile<D, W>(dOh, Gs[b], t * BQ, N, wave, lane);
        if (wave == 0)
            issue_vec64(lse2h, Ls[b], t * BQ, N, lane);
        else if (wave == 1)
            issue_vec64(ndh, Ds[b], t * BQ, N, lane);
    };

    f32x16 dk[NB][DB], dv[NB][DB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            dk[kb][db] = f32x16{};
            dv[kb][db] = f32x16{};
        }

    // P and dS of the previous step (bf16, the B operands of C), and where
    // its Q and dO rows are.
    bf16x8 pb[NB][2], sb[NB][2];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
        pb[kb][0] = pb[kb][1] = sb[kb][0] = sb[kb][1] = bf16x8{};
    int pbuf = 0, pqh = 0;

    // Transpose-read operands of pair pr = (hh, db) of a step: dO^T and Q^T,
    // 32 columns x 16 queries starting at query 32 qh + 16 hh.
    auto read_pair = [&](int b, int qh, int pr, bf16x8 &g, bf16x8 &q) __attribute__((always_inline)) {
        const int hh = pr / DB, db = pr % DB;
        g = tile_tr<D>(Gs[b], 32 * qh + 16 * hh, 32 * db, lane);
        q = tile_tr<D>(Qs[b], 32 * qh + 16 * hh, 32 * db, lane);
    };
    auto c_mfmas = [&](int pr, const bf16x8 &g, const bf16x8 &q) __attribute__((always_inline)) {
        const int hh = pr / DB, db = pr % DB;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            mfma_acc_agpr_ordered(dv[kb][db], g, pb[kb][hh]);
            mfma_acc_agpr_ordered(dk[kb][db], q, sb[kb][hh]);
        }
    };

    // One step: 32 queries (rows 32 qh.. of tile buffer b, first query
    // qrow0). MASKED applies the element mask: query past the end or key
    // above the query (causal).
    auto step = [&](auto mtag, int b, int qh, int qrow0) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        const uint16_t *qs = Qs[b];
        const uint16_t *gs = Gs[b];
        // lse2 and -D of the 16 queries a lane's S/dP registers cover:
        // register r <-> query 8 (r / 4) + 4 hi + r % 4 of the step.
        float lq[16];
        f32x16 nd;
        {
            const float *ls = Ls[b] + 32 * qh + 4 * hi;
            const float *ds = Ds[b] + 32 * qh + 4 * hi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 dv4 = *reinterpret_cast<const float4 *>(ds + 8 * j);
                nd[4 * j + 0] = dv4.x; nd[4 * j + 1] = dv4.y;
                nd[4 * j + 2] = dv4.z; nd[4 * j + 3] = dv4.w;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 lv = *reinterpret_cast<const float4 *>(ls + 8 * j);
                lq[4 * j + 0] = lv.x; lq[4 * j + 1] = lv.y;
                lq[4 * j + 2] = lv.z; lq[4 * j + 3] = lv.w;
            }
        }
        bf16x8 qa[KK], ga[KK];
#pragma unroll
        for (int kk = 0; kk < PA; ++kk) {
            qa[kk] = tile_b128<D>(qs, 32 * qh + l32, 2 * kk + hi);
            ga[kk] = tile_b128<D>(gs, 32 * qh + l32, 2 * kk + hi);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- A(i), with the first C(i-1) operand pairs issued behind it
        f32x16 s[NB], dp[NB];
        bf16x8 gt[NPR], qt[NPR];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int kb = 0; kb < NB; ++kb) {
                s[kb] = mfma32x32x16(qa[kk], kf[kb][kk], kk == 0 ? f32x16{} : s[kb]);
                dp[kb] = mfma32x32x16(ga[kk], vf[kb][kk], kk == 0 ? nd : dp[kb]);
            }
            if (kk + PA < KK) {
                qa[kk + PA] = tile_b128<D>(qs, 32 * qh + l32, 2 * (kk + PA) + hi);
                ga[kk + PA] = tile_b128<D>(gs, 32 * qh + l32, 2 * (kk + PA) + hi);
            }
            if (kk >= KK - PD)
                read_pair(pbuf, pqh, kk - (KK - PD), gt[kk - (KK - PD)], qt[kk - (KK - PD)]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- C(i-1) beside B(i)
        bf16x8 pb2[NB][2], sb2[NB][2];
        float pm[NB][16], dsm[NB][16];
#pragma unroll
        for (int pr = 0; pr < NPR; ++pr) {
            c_mfmas(pr, gt[pr], qt[pr]);
            __builtin_amdgcn_sched_barrier(0);
            if (pr + PD < NPR)
                read_pair(pbuf, pqh, pr + PD, gt[pr + PD], qt[pr + PD]);
#pragma unroll
            for (int e = pr * EPP; e < (pr + 1) * EPP; ++e) {
                const int kb = e / 16, r = e % 16;
                float pe = exp2_fast(fmaf(s[kb][r], c, -lq[r]));
                if (MASKED) {
                    const int key = wk0 + 32 * kb + l32;
                    const int q = qrow0 + 8 * (r / 4) + 4 * hi + (r % 4);
                    if (q >= N || (CAUSAL && key > q))
                        pe = 0.f;
                }
                pm[kb][r] = pe;
                dsm[kb][r] = pe * dp[kb][r];
                if (r % 8 == 7) {
                    const int h = r / 8;
                    bf16x8 pk, sk;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        pk[i] = (__bf16)pm[kb][8 * h + i];
                        sk[i] = (__bf16)dsm[kb][8 * h + i];
                    }
                    pb2[kb][h] = pk;
                    sb2[kb][h] = sk;
                    slot_done(pk);
                    slot_done(sk);
                } else {
                    slot_done(pe);
                    slot_done(dsm[kb][r]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                pb[kb][h] = pb2[kb][h];
                sb[kb][h] = sb2[kb][h];
            }
        pbuf = b;
        pqh = qh;
    };

    int t = t_begin;
    if (SPARSE && t < p.nqt && !tile_needed(t))
        t = next_tile(t);
    if (t < p.nqt) {
        issue_tile(t, 0);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                wait_loaded(kf[kb][kk]);
                wait_loaded(vf[kb][kk]);
            }
        lds_dma_wait<0>();
        __syncthreads();
        int j = 0;
        // Whether this wave's elements of tile t need the element mask.
        auto tile_masked = [&](int t) __attribute__((always_inline)) -> bool {
            const int qbase = t * BQ;
            return (qbase + BQ > N) || (CAUSAL && qbase < wk0 + KW - 1);
        };
        // One tile: its two steps, then the barrier after which tile t+1
        // has landed and buffer (j+2)%3 is free.
        auto tile = [&](auto mtag) __attribute__((always_inline)) {
            const int tn = next_tile(t);
            const int bc = j % 3;
            if (tn < p.nqt)
                issue_tile(tn, (j + 1) % 3);
            const int qbase = t * BQ;
            step(mtag, bc, 0, qbase);
            step(mtag, bc, 1, qbase + 32);
            mfma_drain();  // before the loop edges, where accumulators may be moved
            lds_dma_wait<0>();
            __syncthreads();
            t = tn;
            ++j;
        };
        // Runs of masked and unmasked tiles each get a loop of their own, so
        // the hot loop has no join at which the compiler could reassign the
        // accumulators (causal: the masked tiles are the first ones, on the
        // diagonal, and the ragged last one).
        while (t < p.nqt) {
            while (t < p.nqt && tile_masked(t))
                tile(std::true_type{});
            while (t < p.nqt && !tile_masked(t))
                tile(std::false_type{});
        }
        // C of the last step
#pragma unroll
        for (int pr = 0; pr < NPR; ++pr) {
            bf16x8 g, q;
            read_pair(pbuf, pqh, pr, g, q);
            c_mfmas(pr, g, q);
        }
        mfma_drain();
    }

#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            mfma_settle(dk[kb][db]);
            mfma_settle(dv[kb][db]);
        }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
        const int key = wk0 + 32 * kb + l32;
        if (key < N) {
            uint16_t *dKr = p.dK + head + (size_t)key * D;
            uint16_t *dVr = p.dV + head + (size_t)key * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                store_rows_bf16(dKr, dk[kb][db], 32 * db, hi, p.scale);
                store_rows_bf16(dVr, dv[kb][db], 32 * db, hi, 1.f);
            }
        }
    }
}

struct BwdPtrs {
    const uint16_t *dO, *Q, *K, *V, *O;
    const float *LSE;
    uint16_t *dQ, *dK, *dV;
    float *ndelta, *lse2;
};

BwdPtrs bwd_ptrs(const Problem &pr, const uint16_t *dO, const uint16_t *Q, const uint16_t *K,
                 const uint16_t *V, const uint16_t *O, const float *LSE, uint16_t *dQ,
                 uint16_t *dK, uint16_t *dV, void *ws)
{
    const BwdWorkspace L = bwd_workspace_layout(pr.B, pr.H, pr.N, pr.d);
    BwdPtrs b;
    b.dO = dO; b.Q = Q; b.K = K; b.V = V; b.O = O; b.LSE = LSE;
    b.dQ = dQ; b.dK = dK; b.dV = dV;
    b.ndelta = reinterpret_cast<float *>(static_cast<char *>(ws) + L.delta_off);
    b.lse2 = reinterpret_cast<float *>(static_cast<char *>(ws) + L.lse2_off);
    return b;
}

template <int D>
hipError_t prep_d(const Problem &pr, const BwdPtrs &b)
{
    const long rows = (long)pr.B * pr.H * pr.N;
    const long threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       pr.stream, b.dO, b.O, b.LSE, b.ndelta, b.lse2, rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t dq_t(const Problem &pr, const BwdPtrs &b)
{
    DqParams qp{};
    qp.dO = b.dO; qp.Q = b.Q; qp.K = b.K; qp.V = b.V;
    qp.ndelta = b.ndelta; qp.lse2 = b.lse2; qp.dQ = b.dQ; qp.mask = pr.mask;
    qp.N = pr.N;
    qp.nqb = (pr.N + BwdShape<D, false>::ROWS - 1) / BwdShape<D, false>::ROWS;
    qp.nkt = (pr.N + 63) / 64;
    qp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    qp.items = pr.B * pr.H * qp.nqb;
    qp.per_xcd = (qp.items + kXcds - 1) / kXcds;
    qp.c = pr.scale * kLog2e;
    qp.scale = pr.scale;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, SPARSE>), dim3(qp.per_xcd * kXcds), dim3(256), 0,
                       pr.stream, qp);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t dkdv_t(const Problem &pr, const BwdPtrs &b)
{
    DkvParams kp{};
    kp.dO = b.dO; kp.Q = b.Q; kp.K = b.K; kp.V = b.V;
    kp.ndelta = b.ndelta; kp.lse2 = b.lse2; kp.dK = b.dK; kp.dV = b.dV; kp.mask = pr.mask;
    kp.N = pr.N;
    kp.nkb = (pr.N + BwdShape<D, true>::ROWS - 1) / BwdShape<D, true>::ROWS;
    kp.nqt = (pr.N + 63) / 64;
    kp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    kp.items = pr.B * pr.H * kp.nkb;
    kp.per_xcd = (kp.items + kXcds - 1) / kXcds;
    kp.c = pr.scale * kLog2e;
    kp.scale = pr.scale;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, SPARSE>), dim3(kp.per_xcd * kXcds), dim3(256), 0,
                       pr.stream, kp);
    return hipGetLastError();
}

// Dispatch on (d, causal, sparse) for a kernel template taking <D, CAUSAL, SPARSE>.
#define FA_DISPATCH(FN, pr, b)                                                              \
    ((pr).d == 64 ? ((pr).causal ? ((pr).mask ? FN<64, true, true>(pr, b)                  \
                                              : FN<64, true, false>(pr, b))                \
                                 : ((pr).mask ? FN<64, false, true>(pr, b)                 \
                                              : FN<64, false, false>(pr, b)))              \
                  : ((pr).causal ? ((pr).mask ? FN<128, true, true>(pr, b)                 \
                                              : FN<128, true, false>(pr, b))               \
                                 : ((pr).mask ? FN<128, false, true>(pr, b)                \
                                              : FN<128, false, false>(pr, b))))

}  // namespace

BwdWorkspace bwd_workspace_layout(int B, int H, int N, int d)
{
    (void)d;
    const size_t rows = (size_t)B * (size_t)H * (size_t)N;
    const size_t vec = ((rows * sizeof(float)) + 255) / 256 * 256;
    BwdWorkspace w;
    w.delta_off = 0;
    w.lse2_off = vec;
    w.bytes = 2 * vec;
    return w;
}

hipError_t launch_bwd_prep_bf16(const Problem &pr, const uint16_t *dO, const uint16_t *O,
                                const float *LSE, void *workspace)
{
    const BwdPtrs b = bwd_ptrs(pr, dO, nullptr, nullptr, nullptr, O, LSE, nullptr, nullptr,
                               nullptr, workspace);
    return pr.d == 64 ? prep_d<64>(pr, b) : prep_d<128>(pr, b);
}

hipError_t launch_bwd_dq_bf16(const Problem &pr, const uint16_t *dO, const uint16_t *Q,
                              const uint16_t *K, const uint16_t *V, uint16_t *dQ,
                              const void *workspace)
{
    const BwdPtrs b = bwd_ptrs(pr, dO, Q, K, V, nullptr, nullptr, dQ, nullptr, nullptr,
                               const_cast<void *>(workspace));
    return FA_DISPATCH(dq_t, pr, b);
}

hipError_t launch_bwd_dkdv_bf16(const Problem &pr, const uint16_t *dO, const uint16_t *Q,
                                const uint16_t *K, const uint16_t *V, uint16_t *dK,
                                uint16_t *dV, const void *workspace)
{
    const BwdPtrs b = bwd_ptrs(pr, dO, Q, K, V, nullptr, nullptr, nullptr, dK, dV,
                               const_cast<void *>(workspace));
    return FA_DISPATCH(dkdv_t, pr, b);
}

hipError_t launch_bwd_bf16(const Problem &pr, const uint16_t *dO, const uint16_t *Q,
                           const uint16_t *K, const uint16_t *V, const uint16_t *O,
                           const float *LSE, uint16_t *dQ, uint16_t *dK, uint16_t *dV,
                           void *workspace)
{
    hipError_t e = launch_bwd_prep_bf16(pr, dO, O, LSE, workspace);
    if (e != hipSuccess)
        return e;
    e = launch_bwd_dq_bf16(pr, dO, Q, K, V, dQ, workspace);
    if (e != hipSuccess)
        return e;
    return launch_bwd_dkdv_bf16(pr, dO, Q, K, V, dK, dV, workspace);
}

}  // namespace fa
