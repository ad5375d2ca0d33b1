// Forward of exact attention for head dims in (128, 256] on the matrix
// cores: bf16 storage, bf16 MFMA contractions, fp32 online softmax, the
// N x N S and P held only as register tiles (lukebest.github.io
// FlashAttention, "Kernel fusion"; mstx.cn/posts/485 §三.1 "Tiling", §三.2
// "Online Softmax"). The method and its readings are those of the 64- and
// 128-wide forward kernel (lazy rescale with a slack of 2^8, exponentials in
// base 2, O divided by the sum of its own rounded weights, LSE from the fp32
// weights); this kernel differs in how the work is laid out:
//   - a workgroup of 4 waves (one per SIMD) owns 128 query rows of one
//     (b, h), a wave 32 of them; a wave's Q rows (the B operands of
//     S^T = K Q^T) and its 256 columns of O^T (8 accumulators) sit in AGPRs,
//     which leaves the VGPRs to the scores, the softmax and the operands
//     read ahead;
//   - K tiles of 64 keys are triple-buffered and V tiles double-buffered in
//     LDS (5 x 32 KB), filled by direct global->LDS loads: at the top of tile
//     j the wave issues tile j+1's V and tile j+2's K, which land by the
//     barrier that ends tile j;
//   - a half-step covers 32 keys and is laid out by hand in 32 MFMA slots:
//     the 16 MFMAs of the next 32 keys' scores, then the 16 P V MFMAs of the
//     current ones; the current keys' softmax runs beside the score MFMAs
//     (each weight's argument, exponential and sums in consecutive slots),
//     the next keys' row max beside the P V MFMAs; every LDS operand is read
//     five slots ahead of its MFMA (across half-steps too), so no MFMA waits
//     on LDS; the rescale test stands between half-steps, and the rescale
//     itself (rare with the slack) runs outside the slot plan.
// LDS tiles have 512-byte rows whose 16-byte chunks are XOR-swizzled
// (fa_wide.h): K is read by b128 operand reads (16 rows per LDS cycle), V
// by transpose reads (4 rows x 64 bytes per 32 lanes), both free of bank
// conflicts. Causal (key j visible to query i iff j <= i,
// nanhubrain.csdn.net §三.1): key tiles past the workgroup's diagonal are
// never loaded and only tiles on the diagonal or at the ragged end run the
// element mask, in a loop of their own. Block-sparse
// (lukebest.github.io "Block-Sparse FlashAttention"): the workgroup's 128
// rows are one row of the 128 x 128 block mask, whose dropped tiles are
// never loaded.
#include "fa_common.h"
#include "fa_internal.h"
#include "fa_wide.h"

namespace fa {

namespace {

struct WideFwdParams {
    const uint16_t *Q, *K, *V;
    uint16_t *O;
    float *LSE;
    const uint8_t *mask;
    int N, dh;
    int nqb;      // 128-row query blocks per head
    int nkt;      // 64-key tiles per head
    int nmb;      // mask blocks per mask row
    int items;    // B * H * nqb
    int per_xcd;  // work items per XCD
    float c;      // scale * log2(e)
};

constexpr float kWideSlack = 8.f;  // log2 growth of the row max tolerated without rescale

// acc + the sum of the 8 bf16 values in p (dot products with (1, 1)).
__device__ __forceinline__ float bf16x8_sum(bf16x8 p, float acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}

template <bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(WW * kWave, 1) fwd_wide_kernel(WideFwdParams p)
{
    constexpr int NC = 2 * WDB;            // 32-column blocks of O
    constexpr uint32_t TB = WBT * WD * 2;  // bytes per tile
    constexpr uint32_t V_OFF = 3 * TB;     // three K tiles, then two V tiles
    constexpr uint32_t ROW = 2 * WD;       // bytes per tile row
    constexpr int NSL = 2 * WKK;           // MFMA slots per half-step
    constexpr int PF = 5;                  // operand reads issued this many slots ahead
    __shared__ __attribute__((aligned(1024))) unsigned char smem[V_OFF + 2 * TB];
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nqb;
    const int qi = item - bh * p.nqb;
    const int qblk = CAUSAL ? (p.nqb - 1 - qi) : qi;  // causal: longest rows first
    const int q0 = qblk * WROWS;
    const int N = p.N, dh = p.dh;
    const float c = p.c;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave, l32 = lane % 32, hi = lane / 32;
    const int wr0 = q0 + 32 * wave;  // this wave's first query
    const int row = wr0 + l32;       // this lane's query
    const size_t head = (size_t)bh * N * dh;
    const WideLane wl(lane);

    bf16x8 qf[WKK];
#pragma unroll
    for (int kk = 0; kk < WKK; ++kk) {
        qf[kk] = row < N && 16 * kk + 8 * hi < dh
                     ? *reinterpret_cast<const bf16x8 *>(p.Q + head + (size_t)row * dh + 16 * kk + 8 * hi)
                     : bf16x8{};
        keep_in_agpr(qf[kk]);
    }

    const int t_end = CAUSAL ? min(p.nkt, (q0 + WROWS - 1) / WBT + 1) : p.nkt;
    MaskCursor mc;
    if (SPARSE)
        mc.init(p.mask + (size_t)(q0 / kMaskBlock) * p.nmb, 1, p.nmb);
    auto next_tile = [&](int t) -> int {
        return SPARSE ? next_kept_tile(mc, t + 1, t_end, kMaskBlock / WBT) : t + 1;
    };
    const WideDma dma(wave, lane, dh);

    const int t0 = next_tile(-1);
    if (t0 >= t_end) {
        // no visible key tile (fully masked rows): O = 0, LSE = -inf
        if (row < N) {
            uint16_t *Oh = p.O + head + (size_t)row * dh;
            const f32x16 z = f32x16{};
#pragma unroll
            for (int db = 0; db < NC; ++db)
                wide_store(Oh, z, 32 * db, hi, 1.f, dh);
            if (hi == 0)
                p.LSE[(size_t)bh * N + row] = -INFINITY;
        }
        return;
    }

    f32x16 o[NC];
#pragma unroll
    for (int db = 0; db < NC; ++db)
        o[db] = f32x16{};
    // Row sums against the reference max m: l of the fp32 weights (the
    // LSE), lb of the bf16 weights P V multiplies (O's divisor).
    float m = -INFINITY, l = 0.f, lb = 0.f;
    float thr = -INFINITY, nmref = 0.f;  // (m + slack) / c on raw scores; -m (0 while m = -inf)
    const float inv_c = 1.f / c;

    // Element mask of 32 keys starting at kbase (keys past the end, keys
    // above the query).
    auto half_masked = [&](int kbase) __attribute__((always_inline)) -> bool {
        return (kbase + 32 > N) || (CAUSAL && kbase + 31 > wr0);
    };
    auto mask_half = [&](int kbase, f32x16 &s) __attribute__((always_inline)) {
        if (half_masked(kbase)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kbase + 8 * (r / 4) + 4 * hi + (r % 4);
                if (key >= N || (CAUSAL && key > row))
                    s[r] = -INFINITY;
            }
        }
    };
    // Row max of a 32-key score block (lane-local over 16 registers, then
    // across the two 32-lane halves); its two asm chains start at registers
    // 0 and 3, which pass through mfma_result_touch first.
    auto row_max = [&](f32x16 &sv) __attribute__((always_inline)) -> float {
        mfma_result_touch(sv, 0);
        mfma_result_touch(sv, 3);
        float ma = vmax3(sv[0], sv[1], sv[2]);
        float mb = vmax3(sv[3], sv[4], sv[5]);
        ma = vmax3(ma, sv[6], sv[7]);
        mb = vmax3(mb, sv[8], sv[9]);
        ma = vmax3(ma, sv[10], sv[11]);
        mb = vmax3(mb, sv[12], sv[13]);
        ma = vmax3(ma, sv[14], sv[15]);
        return halves_max(vmax2(ma, mb));
    };

    // Tile loads: K of tile t into K buffer kb, V of tile t into V buffer vb.
    auto load_k = [&](int t, int kb) __attribute__((always_inline)) {
        dma.issue(p.K + head, t * WBT, N, dh, lds0 + kb * TB, wave);
    };
    auto load_v = [&](int t, int vb) __attribute__((always_inline)) {
        dma.issue(p.V + head, t * WBT, N, dh, lds0 + V_OFF + vb * TB, wave);
    };

    int t = t0;
    int t1 = next_tile(t0);
    load_k(t0, 0);
    load_v(t0, 0);
    if (t1 < t_end)
        load_k(t1, 1);
#pragma unroll
    for (int kk = 0; kk < WKK; ++kk)
        wait_loaded(qf[kk]);
    lds_dma_wait<0>();
    __syncthreads();

    // Scores of the first 32 keys; the operands of the first half-step's
    // first slots (K rows of tile t0's second 32 keys) are carried in op.
    f32x16 s_cur = f32x16{};
#pragma unroll
    for (int kk = 0; kk < WKK; ++kk)
        s_cur = mfma32x32x16(wl.rows(lds0, 0, kk), qf[kk], s_cur);
    mask_half(t0 * WBT, s_cur);
    float mx_cur = row_max(s_cur);
    bf16x8 carry[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i)
        carry[i] = wl.rows(lds0, 32 * ROW, i);

    // One half-step h of tile t (keys t * 64 + 32 h..): the scores of the
    // next 32 keys (K buffer kn, row block rn), the softmax and P V of the
    // current ones (V buffer vb, rows 32 h..). kn2 / rn2: where the next
    // half-step's scores read, for the operands carried into it.
    auto half = [&](auto mtag, auto htag, int kbase_next, bool next_valid, uint32_t kn, uint32_t kn2,
                    uint32_t vb, auto &&dma_hook) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        constexpr int h = decltype(htag)::value;
        constexpr uint32_t rn = h == 0 ? 32 * ROW : 0;   // next keys' rows in their K tile
        constexpr uint32_t rn2 = h == 0 ? 0 : 32 * ROW;  // the half-step after
        // Rescale (outside the slot plan): the reference max moves to the
        // row max when it grew past the slack.
        if (__any(mx_cur > thr)) {
            const float mnew = fmaxf(m, mx_cur * c);
            const float alpha = (m == -INFINITY) ? 0.f : exp2_fast(m - mnew);
            m = mnew;
            thr = (m + kWideSlack) * inv_c;
            nmref = (m == -INFINITY) ? 0.f : -m;
            l *= alpha;
            lb *= alpha;
            mfma_drain();
#pragma unroll
            for (int db = 0; db < NC; ++db) {
                mfma_settle(o[db]);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o[db][r] *= alpha;
            }
        }
        // operand of slot i: K rows of the next keys (i < 16), V^T of the
        // current keys (pr = i - 16: keys 16 (pr / 8).., columns 32 (pr % 8)..)
        bf16x8 op[NSL + PF];
#pragma unroll
        for (int i = 0; i < PF; ++i)
            op[i] = carry[i];
        auto read_op = [&](int i) __attribute__((always_inline)) {
            if (i < WKK) {
                op[i] = wl.rows(kn, rn, i);
            } else if (i < NSL) {
                const int pr = i - WKK;
                op[i] = wl.trans(vb, (32 * h + 16 * (pr / NC)) * ROW, pr % NC);
            } else {
                op[i] = wl.rows(kn2, rn2, i - NSL);  // carried into the next half-step
            }
        };
        f32x16 s_nxt;
        float tx[16], ex[16];
        float ls0 = 0.f, ls1 = 0.f;
        bf16x8 pb[2];
        float mx_nxt = 0.f;
        // softmax stages of element e of the current keys: F (argument) in
        // slot e, E (exponential) in slot e + 1, M (sums, packing) in slot
        // e + 2; P V of keys 16 hh.. starts in slot 16 + 8 hh
        auto stage = [&](int k, int e) __attribute__((always_inline)) {
            if (k == 0) {
                tx[e] = fmaf(s_cur[e], c, nmref);
                slot_done(tx[e]);
            } else if (k == 1) {
                ex[e] = exp2_fast(tx[e]);
                slot_done(ex[e]);
            } else {
                if (e % 2 == 0)
                    ls0 += ex[e];
                else
                    ls1 += ex[e];
                if (e % 8 == 7) {
                    bf16x8 pk;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        pk[i] = (__bf16)ex[e - 7 + i];
                    pb[e / 8] = pk;
                    lb = bf16x8_sum(pk, lb);
                    slot_done(pk);
                } else {
                    slot_done(e % 2 == 0 ? ls0 : ls1);
                }
            }
        };
        __builtin_amdgcn_sched_barrier(0);
        static_for<NSL>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i < WKK) {
                s_nxt = mfma32x32x16(op[i], qf[i], i == 0 ? f32x16{} : s_nxt);
            } else {
                constexpr int pr = i - WKK;
                mfma_acc_agpr_nowait(o[pr % NC], op[i], pb[pr / NC]);
            }
            read_op(i + PF);
            dma_hook(i);
            static_for<3>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = 2 - decltype(kc)::value;
                constexpr int e = i - k;
                if constexpr (e >= 0 && e < 16)
                    stage(k, e);
            });
            if constexpr (i == WKK + 2) {
                // the next keys' scores are complete: element mask, row max
                if (MASKED && next_valid)
                    mask_half(kbase_next, s_nxt);
                mx_nxt = row_max(s_nxt);
                l += ls0 + ls1;
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int i = 0; i < PF; ++i)
            carry[i] = op[NSL + i];
        s_cur = s_nxt;
        mx_cur = mx_nxt;
    };

    // Whether the keys of tile t's iteration need the element mask: its
    // second 32 keys and the first 32 of the next tile (their scores are
    // built in it).
    auto tile_masked = [&]() __attribute__((always_inline)) -> bool {
        return half_masked(t * WBT + 32) || (t1 < t_end && half_masked(t1 * WBT));
    };
    int j = 0;  // tile t sits in K buffer j % 3 and V buffer j % 2
    auto tile = [&](auto mtag) __attribute__((always_inline)) {
        const int tn = t1;                                   // tile j+1
        const int tnn = tn < t_end ? next_tile(tn) : t_end;  // tile j+2
        const uint32_t kc = lds0 + (j % 3) * TB, kn = lds0 + ((j + 1) % 3) * TB;
        const uint32_t vc = lds0 + V_OFF + (j % 2) * TB;
        // tile j+1's V replaces tile j-1's, tile j+2's K tile j-1's K, both
        // last read before the previous barrier; one load per slot
        const i32x4 rv = WideDma::rsrc(p.V + head, (tn < t_end ? tn : t) * WBT, N, dh);
        const i32x4 rk = WideDma::rsrc(p.K + head, (tnn < t_end ? tnn : t) * WBT, N, dh);
        // (without a next tile the current one is loaded again, into a free
        // buffer: no branch in the slot plan)
        const uint32_t vnext = lds0 + V_OFF + ((j + 1) % 2) * TB;
        const uint32_t knn = lds0 + ((j + 2) % 3) * TB;
        auto dma_first = [&](int i) __attribute__((always_inline)) {
            if (i < 8)
                dma.issue_block(rv, i, vnext, wave);
            else if (i < 16)
                dma.issue_block(rk, i - 8, knn, wave);
        };
        auto no_dma = [](int) {};
        half(mtag, std::integral_constant<int, 0>{}, t * WBT + 32, true, kc, kn, vc, dma_first);
        half(mtag, std::integral_constant<int, 1>{}, tn * WBT, tn < t_end, kn, kn, vc, no_dma);
        // (no MFMA drain before the loop edges: the generated code moves no
        // accumulator there, which the ISA hazard test checks)
        lds_dma_wait<0>();
        barrier_reads_in_flight();  // the carried K reads (tile j+1's) stay in flight
        t = tn;
        t1 = tnn;
        ++j;
    };
    // Tiles whose keys need no element mask run in a loop of their own
    // (causal: the masked ones are the last, on the diagonal).
    while (t < t_end) {
        while (t < t_end && !tile_masked())
            tile(std::false_type{});
        while (t < t_end && tile_masked())
            tile(std::true_type{});
    }

    // Epilogue: O = O^T / lb, LSE from l in natural log.
    mfma_drain();
#pragma unroll
    for (int db = 0; db < NC; ++db)
        mfma_settle(o[db]);
    const float lt = halves_sum(l);
    const float lbt = halves_sum(lb);
    if (row < N) {
        const float inv = lbt > 0.f ? 1.f / lbt : 0.f;
        uint16_t *Oh = p.O + head + (size_t)row * dh;
#pragma unroll
        for (int db = 0; db < NC; ++db)
            wide_store(Oh, o[db], 32 * db, hi, inv, dh);
        if (hi == 0)
            p.LSE[(size_t)bh * N + row] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    }
}

template <bool CAUSAL, bool SPARSE>
hipError_t launch_fwd_wide_t(const Problem &pr, const WideFwdParams &wp)
{
    hipLaunchKernelGGL((fwd_wide_kernel<CAUSAL, SPARSE>), dim3(wp.per_xcd * kXcds), dim3(WW * kWave), 0,
                       pr.stream, wp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_wide(const Problem &pr, const uint16_t *Q, const uint16_t *K,
                                const uint16_t *V, uint16_t *O, float *LSE)
{
    WideFwdParams wp{};
    wp.Q = Q;
    wp.K = K;
    wp.V = V;
    wp.O = O;
    wp.LSE = LSE;
    wp.mask = pr.mask;
    wp.N = pr.N;
    wp.dh = pr.d;
    wp.nqb = (pr.N + WROWS - 1) / WROWS;
    wp.nkt = (pr.N + WBT - 1) / WBT;
    wp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    wp.items = pr.B * pr.H * wp.nqb;
    wp.per_xcd = (wp.items + kXcds - 1) / kXcds;
    wp.c = pr.scale * kLog2e;
    const bool sparse = pr.mask != nullptr;
    if (pr.causal)
        return sparse ? launch_fwd_wide_t<true, true>(pr, wp) : launch_fwd_wide_t<true, false>(pr, wp);
    return sparse ? launch_fwd_wide_t<false, true>(pr, wp) : launch_fwd_wide_t<false, false>(pr, wp);
}

}  // namespace fa
