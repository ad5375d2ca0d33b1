// Forward of exact attention on gfx950: bf16 storage, bf16 MFMA contractions,
// fp32 online softmax. One fused kernel: S = scale Q K^T -> mask -> online
// softmax -> O += P V, with the N x N S and P held only as register tiles
// (lukebest.github.io FlashAttention, "Kernel fusion"; mstx.cn/posts/485
// §三.1 "Tiling", §三.2 "Online Softmax").
//
// Work decomposition (a re-derivation for CDNA4, not the pages' A100 tiles):
//   - a workgroup of 8 waves (two per SIMD) owns 256 consecutive query rows
//     of one (b, h); each wave owns 32 rows and keeps its Q rows in
//     registers for the whole key loop, so O, m and l never leave registers
//     (the key loop is the inner loop, the order of the pages'
//     sequence-parallel successor, lukebest.github.io "谱系");
//   - K and V stream through LDS in 64-key tiles (three buffers each) by
//     direct global->LDS loads, which need no staging
//     registers; the loads of later tiles are in flight while one is
//     computed, and one barrier per tile orders the buffers;
//   - scores are computed transposed, S^T = K Q^T, so that each lane owns one
//     query and row max / row sum are lane-local plus one exchange between
//     the two 32-lane halves;
//   - software pipeline at 32-key granularity: the MFMAs of S^T for the next
//     32 keys are issued in the same basic blocks as the softmax and the
//     P V MFMAs of the current 32 keys, so the matrix cores and the vector
//     ALU work at the same time; the second wave of each SIMD covers what
//     one wave's dependencies leave idle;
//   - P^T goes back into the MFMA as the B operand of O^T = V^T P^T, the V^T
//     operand coming from the row-major V tile by LDS transpose reads.
//
// LDS layouts (no padding; XOR swizzles of the 16-byte chunks of each row
// keep the reads free of bank conflicts on the 64-bank LDS, which serves 16
// lanes of a b128 read per cycle): K row r, chunk c is stored at chunk
// c ^ (r % 16) for 256-byte rows (d = 128) or c ^ ((r / 2) % 8) for 128-byte
// rows (d = 64), so the 16 rows of one b128 read cycle land in 16 different
// bank groups; V row r, chunk c at c ^ (4 (r % 4) + (r / 4) % 4) (d = 128) --
// the four rows x 64 bytes of one 32-lane transpose read cover all 64 banks.
//
// Online softmax (mstx.cn/posts/485 §三.2 update rule) in base 2, c = scale
// * log2(e). Each row keeps a reference max m (the exponent offset of its
// partial sums). For the next 32 keys with row max t = c * max_j s_j:
//   - if t > m + 8 (or m = -inf): m' = t, O and l are multiplied by 2^(m - m')
//     (the pages' rescaling step, taken only when the max grows enough);
//   - else m' = m and the new weights 2^(c s - m) stay <= 2^8;
//   - p = 2^(c s - m'),  l' = l + sum p,  O' = O + p V.
// Both branches keep O = sum_j 2^(c s_j - m) V_j and l = sum_j 2^(c s_j - m)
// for the current m, so O / l and LSE = (m + log2 l) ln 2 are exact; skipping
// the rescale while the max moves by less than 2^8 saves the O multiply on
// almost every step. (The slack trades speed for the rounding of the largest
// weights: with m at the row max the largest weight is 1, exact in bf16. On
// the long causal workload the largest O error is 1.55e-2 at slack 0,
// 1.81e-2 at 8 and 2.56e-2 at 16; slack 0 costs 7% of the forward's time.)
// A row that has seen no visible key keeps m = -inf and takes exponents
// against 0, so no (-inf) - (-inf) arises; it ends with O = 0, LSE = -inf.
//
// Head dims below the kernel width (64 or 128) are zero-padded: the tile
// loads read zeros for the columns past dh and only dh columns are stored.
// Head dims past 128 run in the 256-wide kernel of fa_fwd_wide.hip.
//
// Masking: causal (key j visible to query i iff j <= i, nanhubrain.csdn.net
// §三.1 tile set) -- key tiles wholly above the diagonal of the workgroup are
// never loaded, and the per-element mask runs only on 32-key steps that
// straddle the diagonal or the end of the sequence; block-sparse
// (lukebest.github.io "Block-Sparse FlashAttention") -- a block-sparse
// workgroup's 128 rows are one row of the 128 x 128 block mask, and key tiles
// whose block that row drops are skipped without being loaded (the kept ones
// come from a ballot over 64 mask entries at a time, not a walk tile by tile). Rows past the end of the sequence read as zeros
// (the tile loads go through buffer resources that end at row N, so no load
// leaves the tensor) and are always masked. Iterations that need no element
// mask run in a loop of their own, without any mask arithmetic.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

struct FwdParams {
    const uint16_t *Q, *K, *V;
    uint16_t *O;
    float *LSE;
    const uint8_t *mask;
    int N;
    int dh;       // head dimension (<= DK; columns dh..DK-1 are zero padding)
    int nqb;      // query blocks per head
    int nkt;      // 64-key tiles per head
    int nmb;      // mask blocks per mask row
    int items;    // B * H * nqb
    int per_xcd;  // work items per XCD
    float c;      // scale * log2(e)
    DropParams drop;  // used by the DROP instances
};

constexpr float kRescaleSlack = 8.f;  // log2 growth of the row max tolerated without rescale

// acc + the sum of the 8 bf16 values in p, by dot products with (1, 1): the
// row sum of the rounded weights that P V multiplies.
__device__ __forceinline__ float bf16x8_sum_acc(bf16x8 p, float acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}

// DK: width of the Q and K rows the kernel reads (the depth of Q K^T); DV:
// width of the V and O rows (equal to DK; head dims past 128 run in
// fa_fwd_wide.hip). W: waves per workgroup (32 query rows each). 8 (two
// per SIMD) by default; 4 (one per SIMD) for block-sparse masks (so that a
// workgroup's 128 rows are one mask row and it loads exactly the key tiles
// that row keeps; 256 rows would load the union of two rows' tiles and mask
// out, wave by wave, what each row drops), and for problems too small to
// give every CU two 256-row workgroups (twice as many workgroups, and at
// d = 64 three fit a CU at once).
template <int DK, int DV, bool CAUSAL, bool SPARSE, bool DROP, int W>
__global__ void __launch_bounds__((64 * W), 1) fwd_bf16_kernel(FwdParams p)
{
    constexpr int RW = 32;          // query rows per wave
    constexpr int BR = RW * W;      // query rows per workgroup
    constexpr int BC = 64;          // keys per LDS tile
    constexpr int KK = DK / 16;     // depth steps of Q K^T
    constexpr int DB = DV / 32;     // 32-row blocks of O^T
    static_assert(DV == DK && DV >= 64 && DV <= 128, "64- or 128-wide rows");
    constexpr int CPRK = DK / 8;    // 16-byte chunks per K row
    constexpr int CPRV = DV / 8;    // 16-byte chunks per V tile row
    constexpr int LPWK = BC * DK * 2 / 1024 / W;  // 1 KB direct loads per wave per K tile
    constexpr int LPWV = BC * DV * 2 / 1024 / W;  // ... per V tile
    static_assert(LPWV >= 1, "tile too small for the direct-load layout");
    constexpr int U = 3;  // buffer phases (tile j in buffers j % 3)

    // LDS: three K tiles, then three V tiles.
    constexpr uint32_t TBK = BC * DK * 2;  // bytes per K tile
    constexpr uint32_t TBV = BC * DV * 2;  // bytes per V tile
    constexpr uint32_t V_OFF = 3 * TBK;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[V_OFF + 3 * TBV];
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nqb;
    const int qi = item - bh * p.nqb;
    const int qblk = CAUSAL ? (p.nqb - 1 - qi) : qi;  // causal: longest rows first
    const int q0 = qblk * BR;
    const int N = p.N;
    const int dh = p.dh;
    const float c = p.c;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int wr0 = q0 + wave * RW;
    const int row = wr0 + l32;

    const size_t head = (size_t)bh * (size_t)N * dh;
    const uint16_t *Qh = p.Q + head;
    const uint16_t *Kh = p.K + head;
    const uint16_t *Vh = p.V + head;

    // This wave's query rows as MFMA B operands (d-slices of 16).
    bf16x8 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = row < N && 16 * kk + 8 * hi < dh
                     ? *reinterpret_cast<const bf16x8 *>(Qh + (size_t)row * dh + 16 * kk + 8 * hi)
                     : bf16x8{};

    int t_end = p.nkt;
    if (CAUSAL)
        t_end = min(p.nkt, (q0 + BR - 1) / BC + 1);

    // Block-sparse: the workgroup's rows are one mask row, so a key tile is
    // loaded exactly when that row keeps its block, and then for every wave;
    // the kept tiles come from a cursor over the row.
    static_assert(!SPARSE || BR == kMaskBlock, "one mask row per block-sparse workgroup");
    static_assert(kMaskBlock % BC == 0, "tiles per mask block");
    MaskCursor mc;
    if (SPARSE)
        mc.init(p.mask + (size_t)(q0 / kMaskBlock) * p.nmb, 1, p.nmb);
    auto next_tile = [&](int t) -> int {
        return SPARSE ? next_kept_tile(mc, t + 1, t_end, kMaskBlock / BC) : t + 1;
    };

    // Lane-dependent byte offsets, computed once. Direct loads: lane `lane`
    // of 1 KB block b writes chunk `lane` of the block, i.e. row
    // r = b * (64 / CPR) + lane / CPR, physical chunk lane % CPR, which holds
    // logical chunk (lane % CPR) ^ swz(r), CPR the chunks per row. K rows of
    // 256 bytes: r % 16 (16 consecutive rows, one logical chunk, 16
    // distinct bank groups).
    auto k_swz = [](int r) -> int { return CPRK >= 16 ? (r % 16) : ((r / 2) % 8); };
    // V rows are only read by transpose reads: the aligned 4-chunk blocks of
    // any 4 aligned rows land on distinct banks (f(r) / 4 distinct), for
    // d = 64 with the row parity taking one bit's place.
    auto v_swz = [](int r) -> int {
        return CPRV >= 16 ? 4 * (r % 4) + (r / 4) % 4 : 4 * ((r / 2) % 2) + (r / 4) % 4;
    };
    // Global rows are dh wide; chunks past dh read as zeros.
    uint32_t kdma[LPWK], vdma[LPWV];
#pragma unroll
    for (int i = 0; i < LPWK; ++i) {
        const int r = (wave * LPWK + i) * (64 / CPRK) + lane / CPRK;
        const int kc = (lane % CPRK) ^ k_swz(r);
        kdma[i] = 8 * kc < dh ? 2 * (r * dh + 8 * kc) : kBufferOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < LPWV; ++i) {
        const int r = (wave * LPWV + i) * (64 / CPRV) + lane / CPRV;
        const int vc = (lane % CPRV) ^ v_swz(r);
        vdma[i] = 8 * vc < dh ? 2 * (r * dh + 8 * vc) : kBufferOutOfRange;
    }
    // Rows past the end of the sequence read as zeros (the buffer resource
    // ends at row N) and are masked.
    auto issue = [&](const uint16_t *src, auto const &off, uint32_t tile, int t)
                     __attribute__((always_inline)) {
        constexpr int L = sizeof(off) / sizeof(off[0]);
        const i32x4 rs = buffer_rsrc(src + (size_t)t * BC * dh, (uint32_t)(N - t * BC) * (2 * dh));
#pragma unroll
        for (int i = 0; i < L; ++i)
            lds_dma_buf_b128(rs, off[i], tile + (wave * L + i) * 1024);
    };
    auto issue_k = [&](int t, int buf) __attribute__((always_inline)) { issue(Kh, kdma, lds0 + buf * TBK, t); };
    auto issue_v = [&](int t, int buf) __attribute__((always_inline)) { issue(Vh, vdma, lds0 + V_OFF + buf * TBV, t); };

    // Operand read addresses are this lane's byte address in buffer 0; the
    // buffer, which each unrolled iteration fixes, and the row block go into
    // the read instruction's immediate offset.
    // K operand reads: row 32*h + l32 of the tile, logical chunk 2*kk + hi
    // (k_swz of row 32 h + l32 equals k_swz of l32).
    uint32_t kaddr[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        kaddr[kk] = lds0 + 2 * (l32 * DK + 8 * ((2 * kk + hi) ^ k_swz(l32)));
    auto qk_half = [&](uint32_t kofs, f32x16 &s) __attribute__((always_inline)) {
        s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            s = mfma32x32x16(lds_b128_at(kaddr[kk] + kofs), qf[kk], s);
    };
    // V^T operand (transpose reads): lane 4t+u of 16-lane group g points at
    // key row 4*(g/2)+t (and 8 rows further for operand slots 4..7),
    // columns 32*db + 16*(g%2) + 4u, i.e. logical chunk 4*db + 2*(g%2) + u/2,
    // element offset 4*(u%2) within it (v_swz depends on the row modulo 16,
    // so the rows 16 and 32 further take the same offsets).
    uint32_t vaddr[DB][2];
    {
        const int g = lane / 16, sl = lane % 16;
        const int v_row = 4 * (g / 2) + sl / 4;
        const int v_lc = 2 * (g % 2) + (sl % 4) / 2;
        const int v_in = 4 * (sl % 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            // opaque: the V base stays in the register, so that the buffer
            // and row offsets (< 64 KB) fit the immediate
            vaddr[db][0] = opaque_addr(lds0 + V_OFF + 2 * (v_row * DV + 8 * ((4 * db + v_lc) ^ v_swz(v_row)) + v_in));
            vaddr[db][1] = opaque_addr(lds0 + V_OFF + 2 * ((v_row + 8) * DV + 8 * ((4 * db + v_lc) ^ v_swz(v_row + 8)) + v_in));
        }
    }

    // Element mask of 32 keys starting at kbase: keys past the end of the
    // sequence and keys above the diagonal (causal). (A visited tile of a
    // block-sparse workgroup is kept for all of its rows.)
    auto mask_half = [&](int kbase, f32x16 &s) {
        const bool edge = (kbase + 32 > N) || (CAUSAL && kbase + 31 > wr0);
        if (edge) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kbase + 8 * (r / 4) + 4 * hi + (r % 4);
                if (key >= N || (CAUSAL && key > row))
                    s[r] = -INFINITY;
            }
        }
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        o[db] = f32x16{};
    // Row sums against the reference max m: l of the fp32 weights (gives the
    // LSE), lb of the bf16-rounded weights P V multiplies (divides O, so that
    // a row dominated by one key gets that key's value row without the
    // weight's rounding error). O is divided by l with dropout, and in the
    // 64-deep instances, whose vector work bounds them: there the 8 extra
    // dot products per 32 keys cost about 10%.
    constexpr bool RSUM = DK >= 128 && !DROP;
    float m = -INFINITY, l = 0.f, lb = 0.f;

    const int t0 = next_tile(-1);
    if (t0 >= t_end) {
        // no visible key tile at all (fully masked rows): O = 0, LSE = -inf
        if (row < N) {
            uint16_t *Oh = p.O + head + (size_t)row * dh;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (32 * db + 8 * j + 4 * hi < dh)
                        *reinterpret_cast<uint2 *>(Oh + 32 * db + 8 * j + 4 * hi) = uint2{0, 0};
            if (hi == 0)
                p.LSE[(size_t)bh * N + row] = -INFINITY;
        }
        return;
    }
    int t1 = next_tile(t0);
    issue_k(t0, 0);
    issue_v(t0, 0);
    if (t1 < t_end) {
        issue_k(t1, 1);
        issue_v(t1, 1);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        wait_loaded(qf[kk]);
    lds_dma_wait<0>();
    __syncthreads();

    // Row max of a 32-key score block (unscaled scores): lane-local over the
    // 16 registers, then across the two 32-lane halves (both hold the row).
    // Its two asm chains start at registers 0 and 3, which the caller passes
    // through mfma_result_touch first.
    auto row_max = [&](const f32x16 &sv) __attribute__((always_inline)) -> float {
        // two interleaved chains, so that no max waits on the one before
        float ma = vmax3(sv[0], sv[1], sv[2]);
        float mb = vmax3(sv[3], sv[4], sv[5]);
#pragma unroll
        for (int r = 6; r < 14; r += 4) {
            ma = vmax3(ma, sv[r], sv[r + 1]);
            mb = vmax3(mb, sv[r + 2], sv[r + 3]);
        }
        ma = vmax3(ma, sv[14], sv[15]);
        return halves_max(vmax2(ma, mb));
    };

    f32x16 s_cur;
    qk_half(0, s_cur);
    mask_half(t0 * BC, s_cur);
    mfma_result_touch(s_cur, 0);
    mfma_result_touch(s_cur, 3);
    float mx_cur = row_max(s_cur);
    // Quantities of the reference max m that change only when it does: the
    // rescale threshold (m + slack) / c on unscaled scores, and the exponent
    // offset -m (0 while m = -inf).
    const float inv_c = 1.f / c;
    float thr = -INFINITY, nmref = 0.f;
    // The first K^T fragments of each half-step are read one half-step
    // early, so that its first MFMAs wait for no LDS read: here those of the
    // first half-step (tile t0's second 32 keys, buffer 0). Half the depth
    // steps.
    constexpr int NPRE = KK / 2 < 4 ? KK / 2 : 4;
    bf16x8 kpre[NPRE];
#pragma unroll
    for (int kk = 0; kk < NPRE; ++kk)
        kpre[kk] = lds_b128_at(kaddr[kk] + 2 * 32 * DK);

    // Tile j's K and V sit in buffer j % 3; the loop below is unrolled three
    // times so that each copy knows its buffers.
    int t = t0;
    // Whether the keys the iteration of tile t masks (the second half of t,
    // the first half of the next tile) need the element mask.
    auto half_masked = [&](int kbase) __attribute__((always_inline)) -> bool {
        return (kbase + 32 > N) || (CAUSAL && kbase + 31 > wr0);
    };
    auto tile_masked = [&]() __attribute__((always_inline)) -> bool {
        return half_masked(t * BC + 32) || (t1 < t_end && half_masked(t1 * BC));
    };
    auto tile = [&](auto mtag, auto ptag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        constexpr int P = decltype(ptag)::value;           // j % U
        constexpr uint32_t KB_CUR = (P % 3) * TBK;         // tile j's K buffer
        constexpr uint32_t KB_NXT = (P + 1) % 3 * TBK;     // tile j+1's
        constexpr uint32_t VB_CUR = (P % 3) * TBV;         // tile j's V buffer
        constexpr int KB_NN = (P + 2) % 3;                 // tile j+2's
        const int tn = t1;                                   // tile j+1
        const int tnn = tn < t_end ? next_tile(tn) : t_end;  // tile j+2
        // K and V of tile j+2 replace tile j-1's, last read before the
        // previous barrier; tile j+1's were issued one iteration ago (its K
        // has landed, its V may still be in flight).
        // (without a tile j+2 tile j is loaded again, into the free buffer:
        // no branch, so the tile's code stays one block for the scheduler;
        // the last iteration's second half-step reads that buffer for scores
        // it does not use)
        const bool more = tnn < t_end;
        issue_k(more ? tnn : t, KB_NN);
        issue_v(more ? tnn : t, KB_NN);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // S^T of the next 32 keys: the second half of this tile, then the
            // first half of tile j+1 (on the last tile a stale buffer is read
            // and the result unused). Its first half-depth runs beside the
            // row max, its second beside the exponentials.
            const uint32_t kofs = (h == 0 ? KB_CUR : KB_NXT) + 2 * 32 * (h ^ 1) * DK;
            // Rescale first, so that the rest of the half-step (the next
            // scores' MFMAs beside this block's exponentials, then P V) is one
            // straight-line block the scheduler can interleave.
            if (__any(mx_cur > thr)) {
                const float mnew = fmaxf(m, mx_cur * c);
                const float alpha = (m == -INFINITY) ? 0.f : exp2_fast(m - mnew);
                m = mnew;
                thr = (m + kRescaleSlack) * inv_c;
                nmref = (m == -INFINITY) ? 0.f : -m;
                l *= alpha;
                lb *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o[db][r] *= alpha;
            }
            f32x16 s_nxt = f32x16{};
            bf16x8 kf[KK];
#pragma unroll
            for (int kk = 0; kk < NPRE; ++kk)
                kf[kk] = kpre[kk];
#pragma unroll
            for (int kk = NPRE; kk < KK / 2; ++kk)
                kf[kk] = lds_b128_at(kaddr[kk] + kofs);
#pragma unroll
            for (int kk = 0; kk < KK / 2; ++kk)
                s_nxt = mfma32x32x16(kf[kk], qf[kk], s_nxt);
#pragma unroll
            for (int kk = KK / 2; kk < KK; ++kk)
                kf[kk] = lds_b128_at(kaddr[kk] + kofs);
            bf16x8 vf[2][DB];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint32_t vofs = VB_CUR + 2 * (32 * h + 16 * hh) * DV;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    vf[hh][db] = lds_tr_pair_at(vaddr[db][0] + vofs, vaddr[db][1] + vofs);
            }
            // dropout: keep bits of this block's 16 elements (keys
            // kb + 8 g + 4 hi + 0..3 for g = 0..3, query `row`); the row sum
            // takes the weights before dropout, P V the kept ones scaled
            uint32_t zb = 0;
            if constexpr (DROP) {
                const uint32_t kb = (uint32_t)(t * BC + 32 * h + 4 * hi);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    zb |= drop_keep4(p.drop, kb + 8 * g, (uint32_t)row, (uint32_t)bh) << (4 * g);
            }
            auto dropped = [&](float e, int r) __attribute__((always_inline)) -> float {
                if constexpr (DROP)
                    return ((zb >> r) & 1u) ? e * p.drop.inv_keep : 0.f;
                return e;
            };
            float ls0, ls1;
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                const float e0 = exp2_fast(fmaf(s_cur[r], c, nmref));
                const float e1 = exp2_fast(fmaf(s_cur[r + 1], c, nmref));
                s_cur[r] = dropped(e0, r);
                s_cur[r + 1] = dropped(e1, r + 1);
                ls0 = r == 0 ? e0 : ls0 + e0;
                ls1 = r == 0 ? e1 : ls1 + e1;
            }
#pragma unroll
            for (int kk = KK / 2; kk < KK; ++kk)
                s_nxt = mfma32x32x16(kf[kk], qf[kk], s_nxt);
            // O^T += V^T P^T over these 32 keys, 16 keys per MFMA.
            const bf16x8 p0 = pack_bf16x8(s_cur, 0);
#pragma unroll
            for (int r = 8; r < 16; r += 2) {
                const float e0 = exp2_fast(fmaf(s_cur[r], c, nmref));
                const float e1 = exp2_fast(fmaf(s_cur[r + 1], c, nmref));
                s_cur[r] = dropped(e0, r);
                s_cur[r + 1] = dropped(e1, r + 1);
                ls0 += e0;
                ls1 += e1;
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = mfma32x32x16(vf[0][db], p0, o[db]);
            l += ls0 + ls1;
            const bf16x8 p1 = pack_bf16x8(s_cur, 1);
            if constexpr (RSUM)
                lb = bf16x8_sum_acc(p1, bf16x8_sum_acc(p0, lb));
            // the row sums are needed here: otherwise the compiler sinks the
            // second half-step's sums past the tile's load wait, behind the
            // last MFMA, instead of interleaving them with the MFMAs
            // (causal d = 64: 425-433 -> 392-401 us, B=2 H=16 N=8192)
            slot_done(l);
            if constexpr (RSUM)
                slot_done(lb);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = mfma32x32x16(vf[1][db], p1, o[db]);
            // the next half-step's first K^T fragments: tile j+1's first 32
            // keys, then its second 32 (visible since the last barrier). The
            // latter stay in flight across the barrier below, which then must
            // find no other read pending: another wave's loads of tile j+3
            // overwrite tile j's buffer once past it.
            {
                if (h == 1)
                    lds_reads_wait_all();
                const uint32_t nofs = h == 0 ? KB_NXT : KB_NXT + 2 * 32 * DK;
#pragma unroll
                for (int kk = 0; kk < NPRE; ++kk)
                    kpre[kk] = lds_b128_at(kaddr[kk] + nofs);
            }
            sched_interleave<KK / 2 + 2 * DB, 2, 4>();
            __builtin_amdgcn_sched_group_barrier(0x100, NPRE, 0);

            if (MASKED) {
                if (h == 0)
                    mask_half(t * BC + 32, s_nxt);
                else if (tn < t_end)
                    mask_half(tn * BC, s_nxt);
            }
            mfma_result_touch(s_nxt, 0);  // heads of row_max's two asm chains
            mfma_result_touch(s_nxt, 3);
            mx_cur = row_max(s_nxt);  // beside the P V MFMAs still in flight
            s_cur = s_nxt;
        }
        // Tile j+1's V and tile j+2's K have landed (tile j+2's V, issued
        // last, may still be in flight); the barrier extends that to all
        // waves. The next iteration reads tile j+2's K from its second
        // half-step on and its V one iteration later.
        lds_dma_wait<LPWV>();
        barrier_reads_in_flight();
        t = tn;
        t1 = tnn;
    };
    // Iterations whose keys need no element mask run in a loop of their own
    // (causal: the masked ones are the last, on the diagonal; block-sparse:
    // a wave whose mask row drops a tile another wave keeps).
    int phase = 0;  // j % U
    auto run = [&](auto mtag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
#define FA_FWD_PHASE(k)                                                     \
        if constexpr (k < U) {                                              \
            if (phase == k) {                                               \
                if (t >= t_end || tile_masked() != MASKED)                  \
                    return;                                                 \
                tile(mtag, std::integral_constant<int, k>{});               \
                phase = (k + 1) % U;                                        \
            }                                                               \
        }
        for (;;) {
            FA_FWD_PHASE(0) FA_FWD_PHASE(1) FA_FWD_PHASE(2)
        }
#undef FA_FWD_PHASE
    };
    while (t < t_end) {
        run(std::false_type{});
        run(std::true_type{});
    }

    // Epilogue: O = O^T / lb (transposed back per lane), LSE from l in
    // natural log.
    lds_dma_wait<0>();  // the last (repeated) tile load has landed: none outlives the workgroup
    const float lt = halves_sum(l);
    const float lbt = RSUM ? halves_sum(lb) : lt;
    if (row < N) {
        const float inv = lbt > 0.f ? 1.f / lbt : 0.f;
        uint16_t *Oh = p.O + head + (size_t)row * dh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if (32 * db + 8 * jj + 4 * hi >= dh)
                    continue;
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16_bits(o[db][4 * jj + 0] * inv) |
                       ((uint32_t)f32_to_bf16_bits(o[db][4 * jj + 1] * inv) << 16);
                pk.y = (uint32_t)f32_to_bf16_bits(o[db][4 * jj + 2] * inv) |
                       ((uint32_t)f32_to_bf16_bits(o[db][4 * jj + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(Oh + 32 * db + 8 * jj + 4 * hi) = pk;
            }
        if (hi == 0)
            p.LSE[(size_t)bh * N + row] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    }
}

template <int DK, int DV, bool CAUSAL, bool SPARSE, bool DROP, int W>
static hipError_t launch_fwd_w(const Problem &pr, const FwdParams &fp0)
{
    FwdParams fp = fp0;
    constexpr int BR = 32 * W;  // query rows per workgroup
    fp.nqb = (pr.N + BR - 1) / BR;
    fp.items = pr.B * pr.H * fp.nqb;
    fp.per_xcd = (fp.items + kXcds - 1) / kXcds;
    const int grid = fp.per_xcd * kXcds;
    hipLaunchKernelGGL((fwd_bf16_kernel<DK, DV, CAUSAL, SPARSE, DROP, W>), dim3(grid), dim3(64 * W), 0,
                       pr.stream, fp);
    return hipGetLastError();
}

constexpr int kCus = 256;  // MI355X compute units

template <int DK, int DV, bool CAUSAL, bool SPARSE, bool DROP>
static hipError_t launch_fwd_t(const Problem &pr, const FwdParams &fp)
{
    if constexpr (SPARSE) {
        return launch_fwd_w<DK, DV, CAUSAL, SPARSE, DROP, 4>(pr, fp);
    } else if constexpr (DROP) {
        return launch_fwd_w<DK, DV, CAUSAL, SPARSE, DROP, 8>(pr, fp);
    } else {
        // fewer 256-row blocks than two per CU: 128-row workgroups
        const long blocks256 = (long)pr.B * pr.H * ((pr.N + 255) / 256);
        if (blocks256 < 2 * kCus)
            return launch_fwd_w<DK, DV, CAUSAL, SPARSE, DROP, 4>(pr, fp);
        return launch_fwd_w<DK, DV, CAUSAL, SPARSE, DROP, 8>(pr, fp);
    }
}

template <int DK, int DV, bool DROP>
static hipError_t launch_fwd_dd(const Problem &pr, const FwdParams &fp)
{
    const bool sparse = pr.mask != nullptr;
    if (pr.causal)
        return sparse ? launch_fwd_t<DK, DV, true, true, DROP>(pr, fp)
                      : launch_fwd_t<DK, DV, true, false, DROP>(pr, fp);
    return sparse ? launch_fwd_t<DK, DV, false, true, DROP>(pr, fp)
                  : launch_fwd_t<DK, DV, false, false, DROP>(pr, fp);
}

template <int D>
static hipError_t launch_fwd_d(const Problem &pr, const FwdParams &fp)
{
    return pr.dropout ? launch_fwd_dd<D, D, true>(pr, fp) : launch_fwd_dd<D, D, false>(pr, fp);
}

hipError_t launch_fwd_bf16(const Problem &pr, const uint16_t *Q, const uint16_t *K,
                           const uint16_t *V, uint16_t *O, float *LSE)
{
    FwdParams fp{};
    fp.Q = Q;
    fp.K = K;
    fp.V = V;
    fp.O = O;
    fp.LSE = LSE;
    fp.mask = pr.mask;
    fp.N = pr.N;
    fp.dh = pr.d;
    fp.nkt = (pr.N + 63) / 64;
    fp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    fp.c = pr.scale * kLog2e;
    fp.drop.threshold = pr.drop_threshold;
    fp.drop.seed_lo = (uint32_t)pr.drop_seed;
    fp.drop.seed_hi = (uint32_t)(pr.drop_seed >> 32);
    fp.drop.inv_keep = pr.drop_inv_keep;
    // head dims up to 64 run in the 64-wide kernel, up to 128 in the
    // 128-wide one, up to 256 in the 256-wide kernel (no dropout there),
    // zero-padded
    if (pr.d <= 64)
        return launch_fwd_d<64>(pr, fp);
    if (pr.d <= 128)
        return launch_fwd_d<128>(pr, fp);
    if (pr.dropout)
        return hipErrorInvalidValue;
    return launch_fwd_bf16_wide(pr, Q, K, V, O, LSE);
}

}  // namespace fa
