// Slot-scheduled backward kernels of exact attention on the matrix cores,
// by recomputation (lukebest.github.io FlashAttention, "反向：重算而非存储";
// mstx.cn/posts/485 §三.3): P = 2^(c s - lse2), dP = dO V^T,
// dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO. They
// run the backward at every head dim without dropout, except dK/dV at
// d <= 64: dQ at row widths 64, 128 and 256; dK and dV in one pass at 128
// (both accumulators fit beside the K and V rows) and in a pass each at 256.
// The description below is written for d = 256; the 128- and 64-wide
// instances differ only in sizes (8 or 4 depth steps, 4 or 2 column blocks,
// tiles of 256- or 128-byte rows).
//
// At d = 256 a wave holds 32 rows of two 256-wide MFMA B operands and the
// accumulators of one 256-column gradient (128 + 128 AGPRs), but not those
// of two:
//   - bwd_wide_dq_kernel: one workgroup per 128 query rows; each wave holds
//     32 query rows of Q and dO; key/value tiles of 64 rows stream through
//     LDS; S^T = K Q^T and dP^T = V dO^T (lane = query), dS^T by the vector
//     ALU, dQ^T += K^T dS^T over all 256 columns with K^T from LDS
//     transpose reads;
//   - bwd_wide_dkdv_kernel: one workgroup per 128 keys; each wave holds 32
//     keys of K (and V); query tiles of 64 rows (Q, dO, lse2, -D) stream
//     through LDS; S = Q K^T (lane = key). dV and dK take a pass each (dV^T
//     += dO^T P; then dP = dO V^T, dK^T += Q^T dS), so S is built twice:
//     8 contractions of work against the method's 5 (splitting each
//     gradient into column halves whose workgroups both rebuild S and dP
//     would take 11).
// The D and lse2 rows come from the backward's preprocessing kernel. LDS
// tiles (512-byte rows, 16-byte chunks XOR-swizzled) are double-buffered:
// the next tile streams in by direct global->LDS loads while the current
// one is computed, one barrier per tile; the tile loop is unrolled by
// buffer, so every operand read is a per-lane register (the swizzle's XOR
// already applied) plus an immediate. With one wave per SIMD nothing hides
// a wave's own latencies, and the wave issues every instruction of its tile
// itself, so a tile's work is laid out by hand in MFMA slots (WidePlan):
// every LDS operand is read a few slots ahead of its MFMA and the softmax of
// one step runs beside the MFMAs of the next phase; the B operands sit in
// AGPRs, which leaves the VGPRs room for the reads in flight. Only tiles on
// the diagonal or at the
// ragged end apply the element mask. Work items (128-row blocks) are dealt
// so that each XCD takes one contiguous range of them: a head's blocks then
// share that XCD's L2, which reads their K/V (or Q/dO) tiles once for all of
// them.
#include "fa_common.h"
#include "fa_internal.h"
#include "fa_wide.h"

namespace fa {

namespace {

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

// Slot plan of a tile's two steps (32 rows each) shared by the kernels
// below: A(0), A(1) with B(0) spread over its MFMAs, C(0) with B(1), C(1),
// one MFMA per slot. A step's softmax elements pass three stages (F: the
// exponent argument, E: the exponential and the mask, M: the product and
// the packing into MFMA operands) in consecutive slots; element e of B(0)
// starts at slot NA + e NA / 16, of B(1) at slot 2 NA + e NCS / 16 (up to
// four elements a slot when a phase has fewer than 16 MFMAs), so that no
// slot waits on a value it produced itself. The last stages run into the
// next phase, whose MFMAs take the operand half of elements 8..15 only from
// their second half on (checked below).
template <int NA, int NCS>
struct WidePlan {
    static constexpr int NSLOT = 2 * NA + 2 * NCS;
    static constexpr int PF = 5;  // operand reads issued this many slots ahead
    // most elements of one step in one slot's stage
    static constexpr int MAXE = (NA >= 16 && NCS >= 16) ? 1 : (NA >= 8 && NCS >= 8) ? 2 : 4;
    // slot of stage k (0 F, 1 E, 2 M) of element e of step st
    __device__ static constexpr int slot(int st, int k, int e)
    {
        return (st == 0 ? NA + e * NA / 16 : 2 * NA + e * NCS / 16) + k;
    }
    // the elements of step st whose stage k falls into slot m: the j-th
    // (j < MAXE) of them, or 16 when there are fewer
    __device__ static constexpr int elem(int m, int st, int k, int j)
    {
        const int S = st == 0 ? NA : NCS;
        const int d = m - k - (st == 0 ? NA : 2 * NA);
        if (d < 0)
            return 16;
        const int lo = (16 * d + S - 1) / S, hi = (16 * (d + 1) + S - 1) / S;
        return (lo + j < hi && lo + j < 16) ? lo + j : 16;
    }
    // each step's two operand halves (elements 0..7, 8..15) are packed
    // before the first C MFMA that takes them
    static constexpr bool ordered()
    {
        return NA % 8 == 0 && NCS % 4 == 0 && 16 / NA <= MAXE && 16 / NCS <= MAXE &&
               slot(0, 0, 0) >= NA && slot(0, 2, 7) < 2 * NA && slot(0, 2, 15) < 2 * NA + NCS / 2 &&
               slot(1, 0, 0) >= 2 * NA && slot(1, 2, 7) < 2 * NA + NCS &&
               slot(1, 2, 15) < 2 * NA + NCS + NCS / 2;
    }
    static_assert(ordered(), "slot plan");
};

// One workgroup per 128 query rows; each wave holds 32 query rows of Q and
// dO (D columns), the B operands of S^T and dP^T, in AGPRs beside its D / 32
// dQ^T accumulators, so that the VGPRs hold the scores, the softmax and the
// operands read ahead. Per 32 keys (a step):
//   A: S^T = K Q^T and dP^T = V dO^T (lane = query; D / 16 MFMA pairs, K
//      and V rows read from LDS);
//   B: P^T = 2^(c s - lse2), dS^T = P^T o (dP^T - D) (vector ALU);
//   C: dQ^T += K^T dS^T over all D columns (D / 16 MFMAs, K^T by transpose
//      reads).
// Every step ends inside its tile (WidePlan), so two LDS slots suffice: the
// next tile streams into the other one, a load per slot of the first step.
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(WW * kWave, 1) bwd_wide_dq_kernel(WideParams p)
{
    constexpr int KK = D / 16;             // 16-deep steps of S^T and dP^T
    constexpr int NC = D / 32;             // 32-column blocks of dQ
    constexpr uint32_t ROW = 2 * D;        // bytes per tile row
    constexpr uint32_t TB = WBT * ROW;     // bytes per tile
    constexpr uint32_t SLOT = 2 * TB;      // [K tile | V tile]
    using Plan = WidePlan<2 * KK, 2 * NC>;
    using Lane = WideLaneXT<D>;
    using Dma = WideDmaT<D>;
    constexpr int NA = 2 * KK, NSLOT = Plan::NSLOT, PF = Plan::PF, LPW = Dma::LPW;
    static_assert(4 * LPW <= NSLOT, "a tile's loads, one every second slot, fit its slots");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * SLOT];
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
    const float c = p.c;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave, l32 = lane % 32, hi = lane / 32;
    const int wr0 = q0 + 32 * wave;  // this wave's first query
    const int row = wr0 + l32;       // this lane's query
    const size_t head = (size_t)bh * N * dh;
    const Lane wl(lane);

    bf16x8 qf[KK], gf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const bool in = row < N && 16 * kk + 8 * hi < dh;
        qf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.Q + head + (size_t)row * dh + 16 * kk + 8 * hi)
                    : bf16x8{};
        gf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.dO + head + (size_t)row * dh + 16 * kk + 8 * hi)
                    : bf16x8{};
        keep_in_agpr(qf[kk]);
        keep_in_agpr(gf[kk]);
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
    const Dma dma(wave, lane, dh);

    // One tile (keys t * 64..) in slot b (a compile-time constant, so that
    // every operand read is a lane register plus an immediate); the loads
    // of tile tl go into slot 1 - b. MASKED applies the element mask: key
    // past the end or above the query (causal).
    auto tile = [&](auto mtag, auto btag, int t, int tl) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        constexpr int b = decltype(btag)::value;
        const uint32_t base = lds0 + b * SLOT, nbase = lds0 + (1 - b) * SLOT;
        const int kbase = t * WBT;
        const i32x4 rk = Dma::rsrc(p.K + head, tl * WBT, N, dh);
        const i32x4 rv = Dma::rsrc(p.V + head, tl * WBT, N, dh);
        // operand of slot m: A slots alternate K rows (S^T) and V rows
        // (dP^T); C slot pr = (hh, db) takes K^T of keys 16 hh.. of its step
        bf16x8 op[NSLOT];
        auto read_op = [&](int m) __attribute__((always_inline)) {
            if (m < 2 * NA) {
                const int st = m / NA, kk = (m % NA) / 2;
                op[m] = wl.rows(base + (m % 2) * TB + 32 * st * ROW, kk);
            } else {
                const int st = (m - 2 * NA) / (2 * NC), pr = (m - 2 * NA) % (2 * NC);
                op[m] = wl.trans(base + (32 * st + 16 * (pr / NC)) * ROW, pr % NC);
            }
        };
        f32x16 s[2], dp[2];
        float tx[2][16], pe[2][16], dsm[2][16];
        bf16x8 sb[2][2];
        auto stage = [&](int st, int k, int e) __attribute__((always_inline)) {
            if (k == 0) {
                tx[st][e] = fmaf(s[st][e], c, -lse2);
                slot_done(tx[st][e]);
            } else if (k == 1) {
                float v = exp2_fast(tx[st][e]);
                if (MASKED) {
                    const int key = kbase + 32 * st + 8 * (e / 4) + 4 * hi + (e % 4);
                    if (key >= N || (CAUSAL && key > row))
                        v = 0.f;
                }
                pe[st][e] = v;
                slot_done(v);
            } else {
                dsm[st][e] = pe[st][e] * dp[st][e];
                if (e % 8 == 7) {
                    bf16x8 sk;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        sk[i] = (__bf16)dsm[st][e - 7 + i];
                    sb[st][e / 8] = sk;
                    slot_done(sk);
                } else {
                    slot_done(dsm[st][e]);
                }
            }
        };
        static_for<PF>([&](auto mc) __attribute__((always_inline)) { read_op(decltype(mc)::value); });
        __builtin_amdgcn_sched_barrier(0);
        static_for<NSLOT>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            if constexpr (m < 2 * NA) {
                constexpr int st = m / NA, kk = (m % NA) / 2;
                if constexpr (m % 2 == 0)
                    s[st] = mfma32x32x16(op[m], qf[kk], kk == 0 ? f32x16{} : s[st]);
                else
                    dp[st] = mfma32x32x16(op[m], gf[kk], kk == 0 ? ndv : dp[st]);
            } else {
                constexpr int st = (m - 2 * NA) / (2 * NC), pr = (m - 2 * NA) % (2 * NC);
                // (at D = 64 the plan packs an operand just before its MFMA)
                if constexpr (D == 64)
                    mfma_acc_agpr_ordered(dq[pr % NC], op[m], sb[st][pr / NC]);
                else
                    mfma_acc_agpr_nowait(dq[pr % NC], op[m], sb[st][pr / NC]);
            }
            if constexpr (m + PF < NSLOT)
                read_op(m + PF);
            // the next tile's loads, one every second slot (spread over more
            // slots, their writes into LDS compete less with the operand reads)
            if constexpr (m % 2 == 0 && m / 2 < LPW)
                dma.issue_block(rk, m / 2, nbase, wave);
            else if constexpr (m % 2 == 0 && m / 2 < 2 * LPW)
                dma.issue_block(rv, m / 2 - LPW, nbase + TB, wave);
            static_for<6 * Plan::MAXE>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                constexpr int st = i / (3 * Plan::MAXE), k = 2 - i / Plan::MAXE % 3;
                constexpr int e = Plan::elem(m, st, k, i % Plan::MAXE);
                if constexpr (e < 16)
                    stage(st, k, e);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    int t = next_tile(-1);
    if (t < t_end) {
        dma.issue(p.K + head, t * WBT, N, dh, lds0, wave);
        dma.issue(p.V + head, t * WBT, N, dh, lds0 + TB, wave);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        wait_loaded(qf[kk]);
        wait_loaded(gf[kk]);
    }
    wait_loaded(lse2);
    wait_loaded(nDi);
    lds_dma_wait<0>();
    __syncthreads();
    // Whether this wave's elements of tile t need the element mask.
    auto tile_masked = [&](int t) __attribute__((always_inline)) -> bool {
        const int kbase = t * WBT;
        return (kbase + WBT > N) || (CAUSAL && kbase + WBT - 1 > wr0);
    };
    // One tile and the barrier after which the next one has landed (without
    // a next tile the current one is loaded again, into the free slot).
    auto step_tile = [&](auto mtag, auto btag) __attribute__((always_inline)) {
        const int tn = next_tile(t);
        tile(mtag, btag, t, tn < t_end ? tn : t);
        // Before the loop edges, where the compiler may copy accumulators, the
        // MFMAs must have written them; the 128- and 256-wide instances need
        // no drain there: their generated code moves no accumulator that soon
        // (the ISA hazard test checks every access to an AGPR an MFMA is still
        // writing, on every path), while the 64-wide dQ kernel's block-sparse
        // instances do copy one at a loop edge.
        if constexpr (D == 64)
            mfma_drain();
        lds_dma_wait<0>();
        __syncthreads();
        t = tn;
    };
    // Runs of masked and unmasked tiles each get a loop of their own
    // (causal: the masked tiles are the last ones, on the diagonal),
    // unrolled twice so that each copy knows its slot.
    int phase = 0;  // the slot of tile t
    auto run = [&](auto mtag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        for (;;) {
            if (phase == 0) {
                if (t >= t_end || tile_masked(t) != MASKED)
                    return;
                step_tile(mtag, std::integral_constant<int, 0>{});
                phase = 1;
            }
            if (t >= t_end || tile_masked(t) != MASKED)
                return;
            step_tile(mtag, std::integral_constant<int, 1>{});
            phase = 0;
        }
    };
    while (t < t_end) {
        run(std::false_type{});
        run(std::true_type{});
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

// Which gradients a dK/dV pass accumulates.
enum WidePass { kPassDV = 0, kPassDK = 1, kPassBoth = 2 };

// One workgroup per 128 keys; each wave holds 32 keys of K (and of V when
// dP is built), the B operands of S (and dP), in AGPRs beside the
// accumulators of its gradients. At D = 256 the accumulators of both
// gradients do not fit beside the K and V rows, so dV and dK take a pass
// each (5 contractions of work; 6 for both gradients in column halves that
// each rebuild S and dP); at D = 128 one pass accumulates both (the
// method's 4 contractions of this side). Per 32 queries (a step), lane =
// key:
//   A: S = Q K^T (and dP - D = dO V^T - D for dK, the accumulator starting
//      from -D); Q and dO rows read from LDS;
//   B: P = 2^(c s - lse2) (and dS = P o (dP - D)) (vector ALU);
//   C: dV^T += dO^T P and / or dK^T += Q^T dS (transpose reads; with both,
//      the two alternate slot by slot).
// The slots follow WidePlan, as in the dQ kernel.
template <int D, int PASS, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(WW * kWave, 1) bwd_wide_dkdv_kernel(WideParams p)
{
    constexpr bool DO_DV = PASS != kPassDK, DO_DK = PASS != kPassDV;
    constexpr int KK = D / 16;             // 16-deep steps of S and dP
    constexpr int NC = D / 32;             // 32-column blocks of a gradient
    constexpr uint32_t ROW = 2 * D;        // bytes per tile row
    constexpr uint32_t TB = WBT * ROW;     // bytes per tile
    constexpr uint32_t SLOT = 2 * TB;      // [Q tile | dO tile]
    constexpr uint32_t VEC = 2 * SLOT;     // then lse2 and -D rows per slot
    constexpr int NA = DO_DK ? 2 * KK : KK;                  // A MFMAs per step
    constexpr int NCS = (DO_DV && DO_DK ? 2 : 1) * 2 * NC;   // C MFMAs per step
    using Plan = WidePlan<NA, NCS>;
    using Lane = WideLaneXT<D>;
    using Dma = WideDmaT<D>;
    constexpr int NSLOT = Plan::NSLOT, PF = Plan::PF, LPW = Dma::LPW;
    static_assert(4 * LPW < NSLOT, "a tile's loads, one every second slot, fit its slots");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[VEC + 4 * WBT * 4];
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item0 = xcd_work_item(p.per_xcd);
    if (item0 >= p.items)
        return;
    const int item = item0;
    const int bh = item / p.nblk;
    const int kb = item - bh * p.nblk;  // causal: low key blocks see the most queries
    const int k0 = kb * WROWS;
    const int N = p.N, dh = p.dh;
    const float c = p.c;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave, l32 = lane % 32, hi = lane / 32;
    const int wk0 = k0 + 32 * wave;  // this wave's first key
    const int key = wk0 + l32;       // this lane's key
    const size_t head = (size_t)bh * N * dh;
    const Lane wl(lane);

    bf16x8 kf[KK], vf[DO_DK ? KK : 1];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const bool in = key < N && 16 * kk + 8 * hi < dh;
        kf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.K + head + (size_t)key * dh + 16 * kk + 8 * hi)
                    : bf16x8{};
        keep_in_agpr(kf[kk]);
        if constexpr (DO_DK) {
            vf[kk] = in ? *reinterpret_cast<const bf16x8 *>(p.V + head + (size_t)key * dh + 16 * kk + 8 * hi)
                        : bf16x8{};
            keep_in_agpr(vf[kk]);
        }
    }

    f32x16 acc_v[DO_DV ? NC : 1], acc_k[DO_DK ? NC : 1];  // dV^T, dK^T
#pragma unroll
    for (int db = 0; db < NC; ++db) {
        if constexpr (DO_DV)
            acc_v[db] = f32x16{};
        if constexpr (DO_DK)
            acc_k[db] = f32x16{};
    }

    const int t_begin = CAUSAL ? k0 / WBT : 0;
    // query tiles the workgroup needs (one mask column, so uniform over it)
    MaskCursor mc;
    if (SPARSE)
        mc.init(p.mask + kb, p.nmb, p.nmb);
    auto next_tile = [&](int t) -> int {
        return SPARSE ? next_kept_tile(mc, t + 1, p.ntile, kMaskBlock / WBT) : t + 1;
    };
    const Dma dma(wave, lane, dh);
    // the statistics rows of tile t into slot b: lse2 by the even waves, -D
    // by the odd ones (the same bytes twice, no branch in the slot plan;
    // rows past N read as zeros: their queries are masked)
    auto issue_vec = [&](int t, int b) __attribute__((always_inline)) {
        const float *v = ((wave & 1) ? p.ndelta : p.lse2) + (size_t)bh * N + t * WBT;
        const i32x4 rs = buffer_rsrc(v, (uint32_t)(N - t * WBT) * 4);
        lds_dma_buf_b32(rs, 4 * lane, lds0 + VEC + (2 * b + (wave & 1)) * WBT * 4);
    };

    // One tile (queries t * 64..) in slot b (a compile-time constant, so
    // that every operand read is a lane register plus an immediate); the
    // loads of tile tl go into slot 1 - b. MASKED applies the element mask:
    // query past the end or key above the query (causal).
    auto tile = [&](auto mtag, auto btag, int t, int tl) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        constexpr int b = decltype(btag)::value;
        const uint32_t base = lds0 + b * SLOT, nbase = lds0 + (1 - b) * SLOT;
        const int qbase = t * WBT;
        const i32x4 rq = Dma::rsrc(p.Q + head, tl * WBT, N, dh);
        const i32x4 rg = Dma::rsrc(p.dO + head, tl * WBT, N, dh);
        // lse2 and -D of the 16 queries a lane's S / dP registers cover in
        // step st: register r <-> query 32 st + 8 (r / 4) + 4 hi + r % 4
        float lq[2][16];
        f32x16 nd[2];
        auto read_vec = [&](int st) __attribute__((always_inline)) {
            const uint32_t a = lds0 + VEC + 2 * b * WBT * 4 + 4 * (32 * st + 4 * hi);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x4 lv = lds_f32x4_at(a + 32 * jj);
                lq[st][4 * jj + 0] = lv.x; lq[st][4 * jj + 1] = lv.y;
                lq[st][4 * jj + 2] = lv.z; lq[st][4 * jj + 3] = lv.w;
                if constexpr (DO_DK) {
                    const f32x4 dv4 = lds_f32x4_at(a + WBT * 4 + 32 * jj);
                    nd[st][4 * jj + 0] = dv4.x; nd[st][4 * jj + 1] = dv4.y;
                    nd[st][4 * jj + 2] = dv4.z; nd[st][4 * jj + 3] = dv4.w;
                }
            }
        };
        // C slot ci of a step: pair pr = ci / 2 (both gradients) or ci, the
        // gradient of the slot, and the operand half hh = pr / NC
        auto c_slot = [](int ci, int &pr, bool &is_v) __attribute__((always_inline)) {
            if (DO_DV && DO_DK) {
                pr = ci / 2;
                is_v = ci % 2 == 0;
            } else {
                pr = ci;
                is_v = DO_DV;
            }
        };
        // operand of slot m: A slots take Q rows (S), alternating with dO
        // rows (dP) when dP is built; C slots take dO^T (dV) or Q^T (dK)
        // of queries 16 hh.. of their step
        bf16x8 op[NSLOT];
        auto read_op = [&](int m) __attribute__((always_inline)) {
            if (m < 2 * NA) {
                const int st = m / NA, i = m % NA;
                const int kk = DO_DK ? i / 2 : i;
                const uint32_t mat = (DO_DK && i % 2 == 1) ? TB : 0;
                op[m] = wl.rows(base + mat + 32 * st * ROW, kk);
            } else {
                const int st = (m - 2 * NA) / NCS;
                int pr;
                bool is_v;
                c_slot((m - 2 * NA) % NCS, pr, is_v);
                op[m] = wl.trans(base + (is_v ? TB : 0) + (32 * st + 16 * (pr / NC)) * ROW, pr % NC);
            }
        };
        f32x16 s[2], dp[2];
        float tx[2][16], pe[2][16], gs[2][16];
        bf16x8 ob_v[2][2], ob_k[2][2];  // the B operands of C: P (dV), dS (dK)
        auto stage = [&](int st, int k, int e) __attribute__((always_inline)) {
            if (k == 0) {
                tx[st][e] = fmaf(s[st][e], c, -lq[st][e]);
                slot_done(tx[st][e]);
            } else if (k == 1) {
                float v = exp2_fast(tx[st][e]);
                if (MASKED) {
                    const int q = qbase + 32 * st + 8 * (e / 4) + 4 * hi + (e % 4);
                    if (q >= N || (CAUSAL && key > q))
                        v = 0.f;
                }
                pe[st][e] = v;
                slot_done(v);
            } else {
                if constexpr (DO_DK)
                    gs[st][e] = pe[st][e] * dp[st][e];
                if (e % 8 == 7) {
                    if constexpr (DO_DV) {
                        bf16x8 pk;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            pk[i] = (__bf16)pe[st][e - 7 + i];
                        ob_v[st][e / 8] = pk;
                        slot_done(pk);
                    }
                    if constexpr (DO_DK) {
                        bf16x8 sk;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            sk[i] = (__bf16)gs[st][e - 7 + i];
                        ob_k[st][e / 8] = sk;
                        slot_done(sk);
                    }
                } else if constexpr (DO_DK) {
                    slot_done(gs[st][e]);
                }
            }
        };
        read_vec(0);
        static_for<PF>([&](auto mc) __attribute__((always_inline)) { read_op(decltype(mc)::value); });
        __builtin_amdgcn_sched_barrier(0);
        static_for<NSLOT>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            if constexpr (m < 2 * NA) {
                constexpr int st = m / NA, i = m % NA;
                constexpr int kk = DO_DK ? i / 2 : i;
                if constexpr (DO_DK && i % 2 == 1)
                    dp[st] = mfma32x32x16(op[m], vf[DO_DK ? kk : 0], kk == 0 ? nd[st] : dp[st]);
                else
                    s[st] = mfma32x32x16(op[m], kf[kk], kk == 0 ? f32x16{} : s[st]);
            } else {
                constexpr int st = (m - 2 * NA) / NCS, ci = (m - 2 * NA) % NCS;
                constexpr int pr = (DO_DV && DO_DK) ? ci / 2 : ci;
                constexpr bool is_v = (DO_DV && DO_DK) ? ci % 2 == 0 : DO_DV;
                if constexpr (is_v)
                    mfma_acc_agpr_nowait(acc_v[pr % NC], op[m], ob_v[st][pr / NC]);
                else
                    mfma_acc_agpr_nowait(acc_k[pr % NC], op[m], ob_k[st][pr / NC]);
            }
            if constexpr (m + PF < NSLOT)
                read_op(m + PF);
            if constexpr (m == 4)
                read_vec(1);
            // the next tile's loads, one every second slot
            if constexpr (m % 2 == 0 && m / 2 < LPW)
                dma.issue_block(rq, m / 2, nbase, wave);
            else if constexpr (m % 2 == 0 && m / 2 < 2 * LPW)
                dma.issue_block(rg, m / 2 - LPW, nbase + TB, wave);
            else if constexpr (m == 4 * LPW)
                issue_vec(tl, 1 - b);
            static_for<6 * Plan::MAXE>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                constexpr int st = i / (3 * Plan::MAXE), k = 2 - i / Plan::MAXE % 3;
                constexpr int e = Plan::elem(m, st, k, i % Plan::MAXE);
                if constexpr (e < 16)
                    stage(st, k, e);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    int t = next_tile(t_begin - 1);
    if (t < p.ntile) {
        dma.issue(p.Q + head, t * WBT, N, dh, lds0, wave);
        dma.issue(p.dO + head, t * WBT, N, dh, lds0 + TB, wave);
        issue_vec(t, 0);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        wait_loaded(kf[kk]);
        if constexpr (DO_DK)
            wait_loaded(vf[kk]);
    }
    lds_dma_wait<0>();
    __syncthreads();
    // Whether this wave's elements of tile t need the element mask.
    auto tile_masked = [&](int t) __attribute__((always_inline)) -> bool {
        const int qbase = t * WBT;
        return (qbase + WBT > N) || (CAUSAL && qbase < wk0 + 31);
    };
    // One tile and the barrier after which the next one has landed (without
    // a next tile the current one is loaded again, into the free slot).
    auto step_tile = [&](auto mtag, auto btag) __attribute__((always_inline)) {
        const int tn = next_tile(t);
        tile(mtag, btag, t, tn < p.ntile ? tn : t);
        // Before the loop edges, where the compiler may copy accumulators, the
        // MFMAs must have written them; the 128- and 256-wide instances need
        // no drain there: their generated code moves no accumulator that soon
        // (the ISA hazard test checks every access to an AGPR an MFMA is still
        // writing, on every path), while the 64-wide dQ kernel's block-sparse
        // instances do copy one at a loop edge.
        if constexpr (D == 64)
            mfma_drain();
        lds_dma_wait<0>();
        __syncthreads();
        t = tn;
    };
    // Runs of masked and unmasked tiles each get a loop of their own
    // (causal: the masked tiles are the first ones, on the diagonal, and
    // the ragged last one), unrolled twice so that each copy knows its slot.
    int phase = 0;  // the slot of tile t
    auto run = [&](auto mtag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        for (;;) {
            if (phase == 0) {
                if (t >= p.ntile || tile_masked(t) != MASKED)
                    return;
                step_tile(mtag, std::integral_constant<int, 0>{});
                phase = 1;
            }
            if (t >= p.ntile || tile_masked(t) != MASKED)
                return;
            step_tile(mtag, std::integral_constant<int, 1>{});
            phase = 0;
        }
    };
    while (t < p.ntile) {
        run(std::true_type{});
        run(std::false_type{});
    }
    mfma_drain();
#pragma unroll
    for (int db = 0; db < NC; ++db) {
        if constexpr (DO_DV)
            mfma_settle(acc_v[db]);
        if constexpr (DO_DK)
            mfma_settle(acc_k[db]);
    }
    if (key < N) {
#pragma unroll
        for (int db = 0; db < NC; ++db) {
            if constexpr (DO_DV)
                wide_store(p.dV + head + (size_t)key * dh, acc_v[db], 32 * db, hi, 1.f, dh);
            if constexpr (DO_DK)
                wide_store(p.dK + head + (size_t)key * dh, acc_k[db], 32 * db, hi, p.scale, dh);
        }
    }
}

template <bool CAUSAL, bool SPARSE>
hipError_t launch_wide(const WideParams &wp, hipStream_t stream)
{
    const dim3 grid(wp.per_xcd * kXcds), block(WW * kWave);
    hipLaunchKernelGGL((bwd_wide_dq_kernel<WD, CAUSAL, SPARSE>), grid, block, 0, stream, wp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((bwd_wide_dkdv_kernel<WD, kPassDV, CAUSAL, SPARSE>), grid, block, 0, stream, wp);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((bwd_wide_dkdv_kernel<WD, kPassDK, CAUSAL, SPARSE>), grid, block, 0, stream, wp);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_dkdv_slot(const WideParams &wp, hipStream_t stream)
{
    hipLaunchKernelGGL((bwd_wide_dkdv_kernel<D, kPassBoth, CAUSAL, SPARSE>), dim3(wp.per_xcd * kXcds),
                       dim3(WW * kWave), 0, stream, wp);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_dq_slot(const WideParams &wp, hipStream_t stream)
{
    hipLaunchKernelGGL((bwd_wide_dq_kernel<D, CAUSAL, SPARSE>), dim3(wp.per_xcd * kXcds), dim3(WW * kWave), 0,
                       stream, wp);
    return hipGetLastError();
}

// Dispatch on (d <= 64, causal, sparse) for the launchers above.
#define FA_SLOT_DISPATCH(FN, pr, wp)                                                               \
    ((pr).d <= 64 ? ((pr).causal ? ((pr).mask ? FN<64, true, true>(wp, (pr).stream)              \
                                              : FN<64, true, false>(wp, (pr).stream))             \
                                 : ((pr).mask ? FN<64, false, true>(wp, (pr).stream)              \
                                              : FN<64, false, false>(wp, (pr).stream)))           \
                  : ((pr).causal ? ((pr).mask ? FN<128, true, true>(wp, (pr).stream)              \
                                              : FN<128, true, false>(wp, (pr).stream))            \
                                 : ((pr).mask ? FN<128, false, true>(wp, (pr).stream)             \
                                              : FN<128, false, false>(wp, (pr).stream))))

// The parameters of the slot-scheduled kernels at d <= 128.
WideParams slot_params(const Problem &pr, const uint16_t *dO, const uint16_t *Q, const uint16_t *K,
                       const uint16_t *V, const float *ndelta, const float *lse2)
{
    WideParams wp{};
    wp.Q = Q;
    wp.K = K;
    wp.V = V;
    wp.dO = dO;
    wp.ndelta = ndelta;
    wp.lse2 = lse2;
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
    return wp;
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16_slot(const Problem &pr, const uint16_t *dO, const uint16_t *Q,
                                     const uint16_t *K, const uint16_t *V, uint16_t *dK, uint16_t *dV,
                                     const float *ndelta, const float *lse2)
{
    WideParams wp = slot_params(pr, dO, Q, K, V, ndelta, lse2);
    wp.dK = dK;
    wp.dV = dV;
    if (pr.causal)
        return pr.mask ? launch_dkdv_slot<128, true, true>(wp, pr.stream)
                       : launch_dkdv_slot<128, true, false>(wp, pr.stream);
    return pr.mask ? launch_dkdv_slot<128, false, true>(wp, pr.stream)
                   : launch_dkdv_slot<128, false, false>(wp, pr.stream);
}

hipError_t launch_bwd_dq_bf16_slot(const Problem &pr, const uint16_t *dO, const uint16_t *Q,
                                   const uint16_t *K, const uint16_t *V, uint16_t *dQ, const float *ndelta,
                                   const float *lse2)
{
    WideParams wp = slot_params(pr, dO, Q, K, V, ndelta, lse2);
    wp.dQ = dQ;
    return FA_SLOT_DISPATCH(launch_dq_slot, pr, wp);
}

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
