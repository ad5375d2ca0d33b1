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
//   2. bwd_dq:   one workgroup per 128 query rows, key/value tiles
//      streamed through LDS; recomputes S^T and dP^T,
//      forms dS^T and accumulates dQ^T = K^T dS^T (lane = query, as in the
//      forward);
//   3. bwd_dkdv: one workgroup per 128 keys (K and V rows in
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
                                                      float *lse2, long rows, int dh)
{
    constexpr int LPR = D / 8;  // lanes per row, 8 bf16 each (rows are dh <= D wide)
    const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows && 8 * part < dh) {
        const uint4 a = *reinterpret_cast<const uint4 *>(dO + row * dh + 8 * part);
        const uint4 b = *reinterpret_cast<const uint4 *>(O + row * dh + 8 * part);
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
// registers each), with 32 rows per wave. The long-lived
// accumulators (dQ^T, or dK^T and dV^T) stay in AGPRs; operands, S, dP and
// the softmax temporaries use the VGPRs.
//
// Tiles of 64 rows stream through LDS by direct loads (rows past the end of
// the sequence read as zeros and are masked). The row-major tiles are read
// two ways: b128 operand reads (16 consecutive rows per LDS cycle) and
// transpose reads (4 consecutive rows x 64 bytes per 32 lanes). The swizzle
// f(r) below stores logical 16-byte chunk c of row r at chunk c ^ f(r). For
// d = 128, f is a bijection on any 16 consecutive rows (b128 reads hit 16
// distinct 4-bank groups) and f(r) / 4 differs across any 4 aligned rows (the
// aligned 4-chunk blocks a transpose read touches land in distinct banks);
// for d = 64 (two rows per 256-byte bank cycle) the same holds with the row
// parity taking the place of one bit.
template <int D>
__device__ __forceinline__ int tile_swz(int r)
{
    if (D == 128)  // 16 chunks per 256-byte row
        return 4 * (r % 4) + (r / 4) % 4;
    return 4 * ((r / 2) % 2) + (r / 4) % 4;  // 8 chunks per 128-byte row
}

// Lane-dependent parts of the addresses a wave uses on swizzled 64-row tiles,
// computed once per kernel.
template <int D, int W>
struct TileLane {
    static constexpr int KK = D / 16, DB = D / 32, CPR = D / 8;
    static constexpr int LPW = 64 * D * 2 / 1024 / W;  // direct-load blocks per wave
    static_assert(LPW * W * 1024 == 64 * D * 2, "tile blocks per wave");
    uint32_t b128[KK];    // b128 operand read: row l32, logical chunk 2 kk + hi
    uint32_t tr[DB][2];   // transpose reads: rows rl and rl + 8, columns 32 db..
    uint32_t dma[LPW];    // direct-load source offset of block wave * LPW + i
    int dh;               // global row width (<= D; the rest reads as zeros)

    __device__ __forceinline__ TileLane(int wave, int lane, int dh_) : dh(dh_)
    {
        const int l32 = lane % 32, hi = lane / 32;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            b128[kk] = 2 * (l32 * D + 8 * ((2 * kk + hi) ^ tile_swz<D>(l32)));
        // Transpose read of 16 rows x 32 columns (the A operand whose k index
        // runs over rows): lane 4t+u of 16-lane group g points at row
        // 4 (g / 2) + t (and 8 rows further for operand slots 4..7),
        // columns 32 db + 16 (g % 2) + 4u.
        const int g = lane / 16, sl = lane % 16;
        const int rl = 4 * (g / 2) + sl / 4;
        const int cl = 2 * (g % 2) + (sl % 4) / 2, e = 4 * (sl % 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            tr[db][0] = 2 * (rl * D + 8 * ((4 * db + cl) ^ tile_swz<D>(rl)) + e);
            tr[db][1] = 2 * ((rl + 8) * D + 8 * ((4 * db + cl) ^ tile_swz<D>(rl + 8)) + e);
        }
        // Direct loads: 1 KB blocks, lane l of block b writes physical chunk
        // l % CPR of row b * (64 / CPR) + l / CPR, i.e. its logical chunk
        // (l % CPR) ^ swz(row); global rows are dh wide and chunks past dh
        // read as zeros.
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int b = wave * LPW + i;
            const int r = b * (64 / CPR) + lane / CPR;
            const int c = (lane % CPR) ^ tile_swz<D>(r);
            dma[i] = 8 * c < dh ? 2 * (r * dh + 8 * c) : kBufferOutOfRange;
        }
    }
    // Issues this wave's direct loads of rows row0.. of a row-major [N, D]
    // matrix into the tile at LDS address `tile`; rows past the end read as
    // zeros (the resource ends at row N).
    __device__ __forceinline__ void load(const uint16_t *src, uint32_t tile, int row0, int N, int wave) const
    {
        const i32x4 rs = rsrc(src, row0, N, dh);
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            load_block(rs, tile, wave, i);
    }
    __device__ __forceinline__ static i32x4 rsrc(const uint16_t *src, int row0, int N, int dh)
    {
        return buffer_rsrc(src + (size_t)row0 * dh, (uint32_t)(N - row0) * (2 * dh));
    }
    // The i-th of this wave's LPW loads of a tile (for spreading them out).
    __device__ __forceinline__ void load_block(const i32x4 &rs, uint32_t tile, int wave, int i) const
    {
        lds_dma_buf_b128(rs, dma[i], tile + (wave * LPW + i) * 1024);
    }
};

// Operand addresses of one tile slot: the slot's LDS base plus the lane
// offsets, one register per pattern; reads add compile-time row and tensor
// offsets through the instruction's offset field.
template <int D>
struct SlotAddr {
    uint32_t b128[D / 16];
    uint32_t tr[D / 32][2];
    template <int W>
    __device__ __forceinline__ void set(const TileLane<D, W> &tl, uint32_t slot)
    {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            b128[kk] = opaque_addr(slot + tl.b128[kk]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            tr[db][0] = opaque_addr(slot + tl.tr[db][0]);
            tr[db][1] = opaque_addr(slot + tl.tr[db][1]);
        }
    }
    // b128 operand of row 32 rb + l32 of the tile at byte offset `off` in the slot
    __device__ __forceinline__ bf16x8 b128_at(uint32_t off, int rb, int kk) const
    {
        return lds_b128_at(b128[kk] + off + 2 * 32 * rb * D);
    }
    // transpose operand of rows r0.. (a multiple of 16), columns 32 db..
    __device__ __forceinline__ bf16x8 tr_at(uint32_t off, int r0, int db) const
    {
        return lds_tr_pair_at(tr[db][0] + off + 2 * r0 * D, tr[db][1] + off + 2 * r0 * D);
    }
};

// Direct load of 64 consecutive floats (one wave): row-vector statistics;
// entries past the end read as zeros.
__device__ __forceinline__ void load_vec64(const float *src, uint32_t dst, int row0, int N, int lane)
{
    const i32x4 rs = buffer_rsrc(src + row0, (uint32_t)(N - row0) * 4);
    lds_dma_buf_b32(rs, 4 * lane, dst);
}

// Stores a 32-row accumulator block (lane = row, registers = 32 columns in
// runs of 4) as bf16, times a factor; columns from dh on are padding and are
// not stored.
__device__ __forceinline__ void store_rows_bf16(uint16_t *dst_row, const f32x16 &acc, int col0, int hi,
                                                float mul, int dh)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (col0 + 8 * j + 4 * hi >= dh)
            continue;
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
    int N, dh, nqb, nkt, nmb, items, per_xcd;
    float c, scale;
    DropParams drop;  // used by the DROP instances
};

// Rows per wave and per workgroup of both main kernels: 4 waves (one per
// SIMD) of 32 rows. Each kernel holds its row operands in registers, a
// long-lived accumulator pair or single in AGPRs and two pipelined steps of
// S, dP and dS, which only fit the register file at 32 rows per wave; the
// workgroup then covers 128 rows, one block-mask row or column, so a tile it
// visits is kept for all of its waves.
struct BwdShape {
    static constexpr int W = 4;
    static constexpr int ROWS = 32 * W;  // rows per workgroup
    static_assert(ROWS == kMaskBlock, "one mask block per workgroup");
};

// One workgroup owns 128 query rows of one (b, h) (32 per wave, Q and dO
// rows held as MFMA B operands); key/value tiles of 64 stream through LDS.
// Per 32 keys (a step):
//   A: S^T = K Q^T and dP^T = V dO^T (lane = query, MFMA);
//   B: P^T = 2^(c s - lse2), dS^T = P^T o (dP^T - D) (vector ALU);
//   C: dQ^T += K^T dS^T (MFMA, K^T by transpose reads; accumulator in
//      AGPRs).
// The steps are software-pipelined by hand: step i runs A(i) with B(i-1)
// spread over its MFMA slots, then C(i-1) (C has half as many MFMAs as A,
// too few to hide B). C reads the previous step's K tile, so K tiles are
// triple-buffered.
template <int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ void __launch_bounds__(256, 1) bwd_dq_kernel(DqParams p)
{
    static_assert(BwdShape::W * 64 == 256, "launch bounds");
    constexpr int W = BwdShape::W;
    constexpr int BR = BwdShape::ROWS;  // query rows per workgroup
    constexpr int BC = 64;              // keys per LDS tile
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = BC * D;
    constexpr int NPR = 2 * DB;          // K^T transpose operands per step
    constexpr int PA = D == 128 ? 3 : 2; // A operand reads issued this many slots ahead
    constexpr int PD = D == 128 ? 3 : 2; // C operands issued this many slots ahead
    static_assert(PA <= KK && PD <= KK, "slot plan");

    // LDS: three slots of [K tile | V tile].
    constexpr uint32_t TB = TILE * 2;  // bytes per tile
    constexpr uint32_t SLOT = 2 * TB, K_OFF = 0, V_OFF = TB;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[3 * SLOT];
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nqb;
    const int qi = item - bh * p.nqb;
    const int qblk = CAUSAL ? (p.nqb - 1 - qi) : qi;  // causal: heaviest blocks first
    const int q0 = qblk * BR;
    const int N = p.N;
    const float c = p.c;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int wr0 = q0 + wave * 32;
    const int row = wr0 + l32;  // this lane's query row
    const int dh = p.dh;
    const TileLane<D, W> tl(wave, lane, dh);

    const size_t head = (size_t)bh * (size_t)N * dh;
    const uint16_t *Qh = p.Q + head, *dOh = p.dO + head;
    const uint16_t *Kh = p.K + head, *Vh = p.V + head;

    bf16x8 qf[KK], gf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const bool in = row < N && 16 * kk + 8 * hi < dh;
        qf[kk] = in ? *reinterpret_cast<const bf16x8 *>(Qh + (size_t)row * dh + 16 * kk + 8 * hi) : bf16x8{};
        gf[kk] = in ? *reinterpret_cast<const bf16x8 *>(dOh + (size_t)row * dh + 16 * kk + 8 * hi) : bf16x8{};
    }
    const float lse2 = row < N ? p.lse2[(size_t)bh * N + row] : INFINITY;
    const float nDi = row < N ? p.ndelta[(size_t)bh * N + row] : 0.f;
    // dP^T accumulates from -D (this lane's row), so that dS^T = P^T o dP^T
    // takes one multiply; with dropout dP^T needs its own scaling first and
    // starts from zero
    f32x16 ndv;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        ndv[r] = DROP ? 0.f : nDi;

    int t_end = p.nkt;
    if (CAUSAL)
        t_end = min(p.nkt, (q0 + BR - 1) / BC + 1);
    // block-sparse: the kept key tiles of this workgroup's mask row
    MaskCursor mc;
    if (SPARSE)
        mc.init(p.mask + (size_t)(q0 / kMaskBlock) * p.nmb, 1, p.nmb);
    auto next_tile = [&](int t) __attribute__((always_inline)) -> int {
        return SPARSE ? next_kept_tile(mc, t + 1, t_end, kMaskBlock / BC) : t + 1;
    };

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        dq[db] = f32x16{};

    // S^T and dP^T of the previous step (fp32), its first key and where its
    // K rows are. Before the first step: S = -inf, so that its P, dS and
    // dQ^T update are zero (on valid K data).
    f32x16 s_prev, dp_prev = f32x16{};
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s_prev[r] = -INFINITY;
    int key0_prev = 0;
    uint32_t z_prev = 0;  // dropout keep bits of the previous step's elements
    // Operand addresses of the current tile's slot and of the previous
    // step's slot (C reads). The previous step of step kh is step 1 - kh
    // (before the first step its weights are zero and it reads valid rows
    // of slot 0).
    SlotAddr<D> cur, prev;
    prev.set(tl, lds0);

    // K^T operand pr = (hh, db) of a step: 32 columns x 16 keys starting at
    // key 32 kh + 16 hh of the tile.
    auto read_kt = [&](const SlotAddr<D> &sa, int kh, int pr) __attribute__((always_inline)) -> bf16x8 {
        const int hh = pr / DB, db = pr % DB;
        return sa.tr_at(K_OFF, 32 * kh + 16 * hh, db);
    };

    // Softmax element r of the previous step: dS^T = P^T o (dP^T - D), with
    // dropout P^T o (Z o dP^T / (1 - p) - D). MASKED applies the element
    // mask: key past the end or above the query (causal). Packs each 8
    // finished elements into an MFMA operand.
    bf16x8 sb[2];
    float dsm[16];
    auto softmax_elem = [&](auto mtag, int r) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        float pe = exp2_fast(fmaf(s_prev[r], c, -lse2));
        if (MASKED) {
            const int key = key0_prev + 8 * (r / 4) + 4 * hi + (r % 4);
            if (key >= N || (CAUSAL && key > row))
                pe = 0.f;
        }
        if constexpr (DROP)
            dsm[r] = pe * ((((z_prev >> r) & 1u) ? dp_prev[r] * p.drop.inv_keep : 0.f) + nDi);
        else
            dsm[r] = pe * dp_prev[r];
        if (r % 8 == 7) {
            bf16x8 sk;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sk[i] = (__bf16)dsm[8 * (r / 8) + i];
            sb[r / 8] = sk;
            slot_done(sk);
        } else {
            slot_done(dsm[r]);
        }
    };

    // One step: keys 32 kh.. of the tile in the current slot, first key
    // key0; `ps` holds the previous step's slot addresses. Runs A of this
    // step with B of the previous step spread
    // over its MFMA slots, then C of the previous step. B uses the mask
    // variant of this tile: masked tiles only ever follow masked ones (the
    // masked tiles, diagonal and ragged end, are the last of the sequence),
    // and masking an unmasked step changes nothing.
    auto step = [&](auto mtag, int kh, int key0, const SlotAddr<D> &ps) __attribute__((always_inline)) {
        constexpr int EPS = 16 / (2 * KK);  // B elements per A slot
        static_assert(EPS * 2 * KK == 16, "elements per slot");
        // dropout keep bits of this step's elements (keys key0 + 8 g + 4 hi
        // + 0..3, query `row`), used by B of the next step
        uint32_t z_cur = 0;
        if constexpr (DROP) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                z_cur |= drop_keep4(p.drop, (uint32_t)(key0 + 8 * g + 4 * hi), (uint32_t)row,
                                    (uint32_t)bh) << (4 * g);
        }
        bf16x8 ka[KK], va[KK];
#pragma unroll
        for (int kk = 0; kk < PA; ++kk) {
            ka[kk] = cur.b128_at(K_OFF, kh, kk);
            va[kk] = cur.b128_at(V_OFF, kh, kk);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- A(i) beside B(i-1), the first C(i-1) operands issued behind
        f32x16 s, dp;
        bf16x8 kt[NPR];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            s = mfma32x32x16(ka[kk], qf[kk], kk == 0 ? f32x16{} : s);
            if (kk + PA < KK)
                ka[kk + PA] = cur.b128_at(K_OFF, kh, kk + PA);
#pragma unroll
            for (int e = 0; e < EPS; ++e)
                softmax_elem(mtag, (2 * kk) * EPS + e);
            __builtin_amdgcn_sched_barrier(0);
            dp = mfma32x32x16(va[kk], gf[kk], kk == 0 ? ndv : dp);
            if (kk + PA < KK)
                va[kk + PA] = cur.b128_at(V_OFF, kh, kk + PA);
            if (kk >= KK - PD)
                kt[kk - (KK - PD)] = read_kt(ps, 1 - kh, kk - (KK - PD));
#pragma unroll
            for (int e = 0; e < EPS; ++e)
                softmax_elem(mtag, (2 * kk + 1) * EPS + e);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- C(i-1)
#pragma unroll
        for (int pr = 0; pr < NPR; ++pr) {
            mfma_acc_agpr_ordered(dq[pr % DB], kt[pr], sb[pr / DB]);
            if (pr + PD < NPR)
                kt[pr + PD] = read_kt(ps, 1 - kh, pr + PD);
            __builtin_amdgcn_sched_barrier(0);
        }
        s_prev = s;
        dp_prev = dp;
        key0_prev = key0;
        z_prev = z_cur;
    };

    int t = next_tile(-1);
    if (t < t_end) {
        tl.load(Kh, lds0 + K_OFF, t * BC, N, wave);
        tl.load(Vh, lds0 + V_OFF, t * BC, N, wave);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            wait_loaded(qf[kk]);
            wait_loaded(gf[kk]);
        }
        wait_loaded(lse2);
        wait_loaded(nDi);
        lds_dma_wait<0>();
        __syncthreads();
        int j = 0;
        // Whether this wave's elements of tile t need the element mask.
        auto tile_masked = [&](int t) __attribute__((always_inline)) -> bool {
            const int kbase = t * BC;
            return (kbase + BC > N) || (CAUSAL && kbase + BC - 1 > wr0);
        };
        // One tile: its two steps, then the barrier after which tile t+1 has
        // landed; K buffer (j+2)%3 and V buffer j%2 are then free.
        auto tile = [&](auto mtag) __attribute__((always_inline)) {
            const int tn = next_tile(t);
            if (tn < t_end) {
                tl.load(Kh, lds0 + ((j + 1) % 3) * SLOT + K_OFF, tn * BC, N, wave);
                tl.load(Vh, lds0 + ((j + 1) % 3) * SLOT + V_OFF, tn * BC, N, wave);
            }
            const int kbase = t * BC;
            cur.set(tl, lds0 + (j % 3) * SLOT);
            step(mtag, 0, kbase, prev);
            step(mtag, 1, kbase + 32, cur);
            prev = cur;
            mfma_drain();  // before the loop edges, where accumulators may be moved
            lds_dma_wait<0>();
            __syncthreads();
            t = tn;
            ++j;
        };
        // Runs of masked and unmasked tiles each get a loop of their own, so
        // the hot loop has no join (causal: the masked tiles are the last
        // ones, on the diagonal).
        while (t < t_end) {
            while (t < t_end && !tile_masked(t))
                tile(std::false_type{});
            while (t < t_end && tile_masked(t))
                tile(std::true_type{});
        }
        // B and C of the last step
#pragma unroll
        for (int r = 0; r < 16; ++r)
            softmax_elem(std::true_type{}, r);
#pragma unroll
        for (int pr = 0; pr < NPR; ++pr)
            mfma_acc_agpr_ordered(dq[pr % DB], read_kt(prev, 1, pr), sb[pr / DB]);
        mfma_drain();
    }

#pragma unroll
    for (int db = 0; db < DB; ++db)
        mfma_settle(dq[db]);
    if (row < N) {
        uint16_t *dst = p.dQ + head + (size_t)row * dh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            store_rows_bf16(dst, dq[db], 32 * db, hi, p.scale, dh);
    }
}

// -------------------------------------------------------------- dK dV ----

struct DkvParams {
    const uint16_t *dO, *Q, *K, *V;
    const float *ndelta, *lse2;  // -D and LSE * log2(e) per row
    uint16_t *dK, *dV;
    const uint8_t *mask;
    int N, dh, nkb, nqt, nmb, items, per_xcd;
    float c, scale;
    DropParams drop;  // used by the DROP instances
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
template <int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(DkvParams p)
{
    static_assert(BwdShape::W * 64 == 256, "launch bounds");
    constexpr int W = BwdShape::W;
    constexpr int NB = 1;
    constexpr int KW = 32 * NB;     // keys per wave
    constexpr int BK = W * KW;      // keys per workgroup
    constexpr int BQ = 64;          // queries per LDS tile
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = BQ * D;
    constexpr int NPR = 2 * DB;          // transpose-operand pairs (dO^T, Q^T) per step
    constexpr int PA = D == 128 ? 3 : 2; // A operand reads issued this many MFMA pairs ahead
    constexpr int PD = D == 128 ? 3 : 2; // C operand pairs issued this many pairs ahead
    static_assert(2 * NB * NPR == KK * NB * 2, "as many MFMAs in A as in C");
    static_assert(PA <= KK && PD <= KK, "slot plan");
    // One mask column per workgroup: a tile it visits is kept for all waves.
    static_assert(BK == kMaskBlock, "workgroup keys = one mask block");

    // LDS: three slots of [Q tile | dO tile], then lse2 and -D rows per slot.
    constexpr uint32_t TB = TILE * 2;  // bytes per tile
    constexpr uint32_t SLOT = 2 * TB, Q_OFF = 0, G_OFF = TB;
    constexpr uint32_t L_OFF = 3 * SLOT, D_OFF = L_OFF + 3 * BQ * 4;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[D_OFF + 3 * BQ * 4];
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nkb;
    const int kblk = item - bh * p.nkb;  // causal: low key blocks see the most queries
    const int k0 = kblk * BK;
    const int N = p.N;
    const float c = p.c;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int wk0 = k0 + wave * KW;
    const int dh = p.dh;
    const TileLane<D, W> tl(wave, lane, dh);

    const size_t head = (size_t)bh * (size_t)N * dh;
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
            const bool in = key < N && 16 * kk + 8 * hi < dh;
            kf[kb][kk] = in ? *reinterpret_cast<const bf16x8 *>(Kh + (size_t)key * dh + 16 * kk + 8 * hi)
                            : bf16x8{};
            vf[kb][kk] = in ? *reinterpret_cast<const bf16x8 *>(Vh + (size_t)key * dh + 16 * kk + 8 * hi)
                            : bf16x8{};
        }
    }

    const int t_begin = CAUSAL ? k0 / BQ : 0;
    // block-sparse: the kept query tiles of this workgroup's mask column
    MaskCursor mc;
    if (SPARSE)
        mc.init(p.mask + kblk, p.nmb, p.nmb);
    auto next_tile = [&](int t) __attribute__((always_inline)) -> int {
        return SPARSE ? next_kept_tile(mc, t + 1, p.nqt, kMaskBlock / BQ) : t + 1;
    };
    auto issue_tile = [&](int t, int b) __attribute__((always_inline)) {
        tl.load(Qh, lds0 + b * SLOT + Q_OFF, t * BQ, N, wave);
        tl.load(dOh, lds0 + b * SLOT + G_OFF, t * BQ, N, wave);
        if (wave == 0)
            load_vec64(lse2h, lds0 + L_OFF + b * BQ * 4, t * BQ, N, lane);
        else if (wave == 1)
            load_vec64(ndh, lds0 + D_OFF + b * BQ * 4, t * BQ, N, lane);
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
    // Operand addresses of the current tile's slot (A reads, C of its first
    // step) and of the previous step's slot (C reads). The previous step of
    // step qh is step 1 - qh: the second step of the previous tile, or the
    // first of this one (before the first step its weights are zero, and it
    // reads valid rows of slot 0).
    SlotAddr<D> cur, prev;
    prev.set(tl, lds0);

    // Transpose-read operands of pair pr = (hh, db) of a step: dO^T and Q^T,
    // 32 columns x 16 queries starting at query 32 qh + 16 hh.
    auto read_pair = [&](const SlotAddr<D> &sa, int qh, int pr, bf16x8 &g, bf16x8 &q) __attribute__((always_inline)) {
        const int hh = pr / DB, db = pr % DB;
        g = sa.tr_at(G_OFF, 32 * qh + 16 * hh, db);
        q = sa.tr_at(Q_OFF, 32 * qh + 16 * hh, db);
    };
    auto c_mfmas = [&](int pr, const bf16x8 &g, const bf16x8 &q) __attribute__((always_inline)) {
        const int hh = pr / DB, db = pr % DB;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            mfma_acc_agpr_ordered(dv[kb][db], g, pb[kb][hh]);
            mfma_acc_agpr_ordered(dk[kb][db], q, sb[kb][hh]);
        }
    };

    // One step: 32 queries (rows 32 qh.. of the tile in slot b, first query
    // qrow0); `ps` holds the operand addresses of the previous step's slot.
    // MASKED applies the element mask: query past the end or key above the
    // query (causal).
    auto step = [&](auto mtag, int b, int qh, int qrow0, const SlotAddr<D> &ps, auto &&hook) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        // lse2 and -D of the 16 queries a lane's S/dP registers cover:
        // register r <-> query 8 (r / 4) + 4 hi + r % 4 of the step.
        float lq[16];
        f32x16 nd;
        {
            const uint32_t st = lds0 + b * BQ * 4 + 4 * (32 * qh + 4 * hi);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 dv4 = lds_f32x4_at(st + D_OFF + 32 * j);
                nd[4 * j + 0] = dv4.x; nd[4 * j + 1] = dv4.y;
                nd[4 * j + 2] = dv4.z; nd[4 * j + 3] = dv4.w;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 lv = lds_f32x4_at(st + L_OFF + 32 * j);
                lq[4 * j + 0] = lv.x; lq[4 * j + 1] = lv.y;
                lq[4 * j + 2] = lv.z; lq[4 * j + 3] = lv.w;
            }
        }
        // dropout keep bits of this step's elements (key of this lane,
        // query qrow0 + 8 (r / 4) + 4 hi + r % 4 for bit r). The four lanes
        // of a quad hold four consecutive keys, which share one draw per
        // query: lane u of the quad draws for the queries r = 4 a + u
        // (bits 4 a + w of its mask: key 4 (key / 4) + w), the quad's masks
        // are broadcast to every lane, and lane v takes bit 4 a + v of lane
        // b's mask as its bit 4 a + b.
        uint32_t zb[NB];
        if constexpr (DROP) {
            const uint32_t u = (uint32_t)(l32 & 3);
#pragma unroll
            for (int kb = 0; kb < NB; ++kb) {
                const uint32_t key = (uint32_t)(wk0 + 32 * kb + l32);
                uint32_t mine = 0;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint32_t q = (uint32_t)(qrow0 + 8 * a + 4 * hi) + u;
                    mine |= drop_keep4(p.drop, key & ~3u, q, (uint32_t)bh) << (4 * a);
                }
                // quad_perm broadcasts of lanes 0..3 of the quad
                const uint32_t x0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x00, 0xF, 0xF, false);
                const uint32_t x1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x55, 0xF, 0xF, false);
                const uint32_t x2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xAA, 0xF, 0xF, false);
                const uint32_t x3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xFF, 0xF, 0xF, false);
                zb[kb] = ((x0 >> u) & 0x1111u) | (((x1 >> u) & 0x1111u) << 1) |
                         (((x2 >> u) & 0x1111u) << 2) | (((x3 >> u) & 0x1111u) << 3);
            }
        }
        bf16x8 qa[KK], ga[KK];
#pragma unroll
        for (int kk = 0; kk < PA; ++kk) {
            qa[kk] = cur.b128_at(Q_OFF, qh, kk);
            ga[kk] = cur.b128_at(G_OFF, qh, kk);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- A(i), with the first C(i-1) operand pairs issued behind it.
        // One MFMA per slot: a second MFMA issued right behind the first
        // would hold up everything after it until the matrix pipe frees.
        f32x16 s[NB], dp[NB];
        bf16x8 gt[NPR], qt[NPR];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int kb = 0; kb < NB; ++kb) {
                s[kb] = mfma32x32x16(qa[kk], kf[kb][kk], kk == 0 ? f32x16{} : s[kb]);
                if (kb == 0 && kk + PA < KK)
                    qa[kk + PA] = cur.b128_at(Q_OFF, qh, kk + PA);
                hook(2 * (kk * NB + kb));
                __builtin_amdgcn_sched_barrier(0);
                dp[kb] = mfma32x32x16(ga[kk], vf[kb][kk], kk == 0 ? nd : dp[kb]);
                if (kb == 0 && kk + PA < KK)
                    ga[kk + PA] = cur.b128_at(G_OFF, qh, kk + PA);
                if (kb == 0 && kk >= KK - PD)
                    read_pair(ps, 1 - qh, kk - (KK - PD), gt[kk - (KK - PD)], qt[kk - (KK - PD)]);
                hook(2 * (kk * NB + kb) + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- C(i-1) beside B(i): one MFMA per slot, each followed by the
        // next operand reads and its share of the softmax. The softmax of an
        // element is itself pipelined over three slots (exponent argument,
        // exponential, product and packing), so no slot waits on a result
        // it produced itself.
        bf16x8 pb2[NB][2], sb2[NB][2];
        float tx[NB][16], pm[NB][16], dsm[NB][16], pt[NB][16];
        auto stage_f = [&](int e) __attribute__((always_inline)) {
            const int kb = e / 16, r = e % 16;
            tx[kb][r] = fmaf(s[kb][r], c, -lq[r]);
            slot_done(tx[kb][r]);
        };
        auto stage_e = [&](int e) __attribute__((always_inline)) {
            const int kb = e / 16, r = e % 16;
            float pe = exp2_fast(tx[kb][r]);
            if (MASKED) {
                const int key = wk0 + 32 * kb + l32;
                const int q = qrow0 + 8 * (r / 4) + 4 * hi + (r % 4);
                if (q >= N || (CAUSAL && key > q))
                    pe = 0.f;
            }
            pm[kb][r] = pe;
            slot_done(pe);
        };
        auto stage_m = [&](int e) __attribute__((always_inline)) {
            const int kb = e / 16, r = e % 16;
            // dp holds dP - D (its accumulator started from -D); with
            // dropout dS = P o (Z o dP / (1 - p) - D) and dV takes
            // P o Z / (1 - p)
            if constexpr (DROP) {
                const bool z = (zb[kb] >> r) & 1u;
                const float ik = p.drop.inv_keep;
                dsm[kb][r] = pm[kb][r] * (z ? (dp[kb][r] - nd[r]) * ik + nd[r] : nd[r]);
                pt[kb][r] = z ? pm[kb][r] * ik : 0.f;
            } else {
                dsm[kb][r] = pm[kb][r] * dp[kb][r];
                pt[kb][r] = pm[kb][r];
            }
            if (r % 8 == 7) {
                const int h = r / 8;
                bf16x8 pk, sk;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    pk[i] = (__bf16)pt[kb][8 * h + i];
                    sk[i] = (__bf16)dsm[kb][8 * h + i];
                }
                pb2[kb][h] = pk;
                sb2[kb][h] = sk;
                slot_done(pk);
                slot_done(sk);
            } else {
                slot_done(dsm[kb][r]);
            }
        };
        constexpr int NSLOT = 2 * NB * NPR;   // C MFMAs per step
        constexpr int EPS = 16 * NB / NSLOT;  // softmax elements per slot
        static_assert(EPS * NSLOT == 16 * NB, "elements per slot");
#pragma unroll
        for (int m = 0; m < NSLOT + 2; ++m) {
            if (m < NSLOT) {
                const int pr = m / (2 * NB), kb = (m / 2) % NB, hh = pr / DB, db = pr % DB;
                if (m % 2 == 0)
                    mfma_acc_agpr_ordered(dv[kb][db], gt[pr], pb[kb][hh]);
                else
                    mfma_acc_agpr_ordered(dk[kb][db], qt[pr], sb[kb][hh]);
                if (m % (2 * NB) == 0 && pr + PD < NPR)
                    read_pair(ps, 1 - qh, pr + PD, gt[pr + PD], qt[pr + PD]);
#pragma unroll
                for (int e = m * EPS; e < (m + 1) * EPS; ++e)
                    stage_f(e);
            }
            if (m >= 1 && m - 1 < NSLOT) {
#pragma unroll
                for (int e = (m - 1) * EPS; e < m * EPS; ++e)
                    stage_e(e);
            }
            if (m >= 2) {
#pragma unroll
                for (int e = (m - 2) * EPS; e < (m - 1) * EPS; ++e)
                    stage_m(e);
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
    };

    int t = next_tile(t_begin - 1);
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
            // Loads of the next tile into the free slot, one per A slot of
            // the first step rather than in a burst (without a next tile the
            // current one is loaded again, into the free slot: no branch).
            const int tl_next = tn < p.nqt ? tn : t;
            const uint32_t nslot = lds0 + ((j + 1) % 3) * SLOT;
            const i32x4 rq = TileLane<D, W>::rsrc(Qh, tl_next * BQ, N, dh);
            const i32x4 rg = TileLane<D, W>::rsrc(dOh, tl_next * BQ, N, dh);
            auto dma_hook = [&](int sl) __attribute__((always_inline)) {
                constexpr int LPW = TileLane<D, W>::LPW;
                if (sl < LPW)
                    tl.load_block(rq, nslot + Q_OFF, wave, sl);
                else if (sl < 2 * LPW)
                    tl.load_block(rg, nslot + G_OFF, wave, sl - LPW);
                else if (sl == 2 * LPW)  // lse2 (even waves) or -D (odd waves): same bytes twice
                    load_vec64((wave & 1) ? ndh : lse2h,
                               lds0 + ((wave & 1) ? D_OFF : L_OFF) + ((j + 1) % 3) * BQ * 4,
                               tl_next * BQ, N, lane);
            };
            auto no_hook = [](int) {};
            const int qbase = t * BQ;
            cur.set(tl, lds0 + bc * SLOT);
            step(mtag, bc, 0, qbase, prev, dma_hook);
            step(mtag, bc, 1, qbase + 32, cur, no_hook);
            prev = cur;
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
            read_pair(prev, 1, pr, g, q);
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
            uint16_t *dKr = p.dK + head + (size_t)key * dh;
            uint16_t *dVr = p.dV + head + (size_t)key * dh;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                store_rows_bf16(dKr, dk[kb][db], 32 * db, hi, p.scale, dh);
                store_rows_bf16(dVr, dv[kb][db], 32 * db, hi, 1.f, dh);
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
                       pr.stream, b.dO, b.O, b.LSE, b.ndelta, b.lse2, rows, pr.d);
    return hipGetLastError();
}

DropParams drop_params(const Problem &pr)
{
    DropParams d;
    d.threshold = pr.drop_threshold;
    d.seed_lo = (uint32_t)pr.drop_seed;
    d.seed_hi = (uint32_t)(pr.drop_seed >> 32);
    d.inv_keep = pr.drop_inv_keep;
    return d;
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t dq_t(const Problem &pr, const BwdPtrs &b)
{
    // without dropout: the slot-scheduled kernel
    if (!pr.dropout)
        return launch_bwd_dq_bf16_slot(pr, b.dO, b.Q, b.K, b.V, b.dQ, b.ndelta, b.lse2);
    DqParams qp{};
    qp.dO = b.dO; qp.Q = b.Q; qp.K = b.K; qp.V = b.V;
    qp.ndelta = b.ndelta; qp.lse2 = b.lse2; qp.dQ = b.dQ; qp.mask = pr.mask;
    qp.N = pr.N;
    qp.dh = pr.d;
    qp.nqb = (pr.N + BwdShape::ROWS - 1) / BwdShape::ROWS;
    qp.nkt = (pr.N + 63) / 64;
    qp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    qp.items = pr.B * pr.H * qp.nqb;
    qp.per_xcd = (qp.items + kXcds - 1) / kXcds;
    qp.c = pr.scale * kLog2e;
    qp.scale = pr.scale;
    qp.drop = drop_params(pr);
    if (pr.dropout)
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, SPARSE, true>), dim3(qp.per_xcd * kXcds),
                           dim3(256), 0, pr.stream, qp);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, SPARSE, false>), dim3(qp.per_xcd * kXcds),
                           dim3(256), 0, pr.stream, qp);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t dkdv_t(const Problem &pr, const BwdPtrs &b)
{
    // 64 < d <= 128 without dropout: the slot-scheduled kernel (at d = 64,
    // where the softmax work per MFMA doubles, this kernel is faster)
    if constexpr (D == 128) {
        if (!pr.dropout)
            return launch_bwd_dkdv_bf16_slot(pr, b.dO, b.Q, b.K, b.V, b.dK, b.dV, b.ndelta, b.lse2);
    }
    DkvParams kp{};
    kp.dO = b.dO; kp.Q = b.Q; kp.K = b.K; kp.V = b.V;
    kp.ndelta = b.ndelta; kp.lse2 = b.lse2; kp.dK = b.dK; kp.dV = b.dV; kp.mask = pr.mask;
    kp.N = pr.N;
    kp.dh = pr.d;
    kp.nkb = (pr.N + BwdShape::ROWS - 1) / BwdShape::ROWS;
    kp.nqt = (pr.N + 63) / 64;
    kp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    kp.items = pr.B * pr.H * kp.nkb;
    kp.per_xcd = (kp.items + kXcds - 1) / kXcds;
    kp.c = pr.scale * kLog2e;
    kp.scale = pr.scale;
    kp.drop = drop_params(pr);
    if (pr.dropout)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, SPARSE, true>), dim3(kp.per_xcd * kXcds),
                           dim3(256), 0, pr.stream, kp);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, SPARSE, false>), dim3(kp.per_xcd * kXcds),
                           dim3(256), 0, pr.stream, kp);
    return hipGetLastError();
}

// Dispatch on (d, causal, sparse) for a kernel template taking <D, CAUSAL, SPARSE>;
// head dims up to 64 run in the 64-wide kernels, the others in the 128-wide ones.
#define FA_DISPATCH(FN, pr, b)                                                              \
    ((pr).d <= 64 ? ((pr).causal ? ((pr).mask ? FN<64, true, true>(pr, b)                  \
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
    if (pr.d <= 64)
        return prep_d<64>(pr, b);
    return pr.d <= 128 ? prep_d<128>(pr, b) : prep_d<256>(pr, b);  // 256: the wide backward
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
    if (pr.d > 128)
        return launch_bwd_bf16_wide(pr, dO, Q, K, V, O, LSE, dQ, dK, dV, workspace);
    hipError_t e = launch_bwd_prep_bf16(pr, dO, O, LSE, workspace);
    if (e != hipSuccess)
        return e;
    e = launch_bwd_dq_bf16(pr, dO, Q, K, V, dQ, workspace);
    if (e != hipSuccess)
        return e;
    return launch_bwd_dkdv_bf16(pr, dO, Q, K, V, dK, dV, workspace);
}

}  // namespace fa
