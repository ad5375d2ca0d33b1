// Decode-shaped forward on gfx950: Nq queries (a few: the newest positions)
// against Nk keys of the same head, with the key axis split into chunks whose
// partial results are merged afterwards (the FlashDecoding line of
// lukebest.github.io's lineage table, "谱系": few queries leave one query
// block per head, far too little parallel work, so the keys are split too).
//
// What each chunk computes is the forward of the square kernel restricted to
// its keys: S = scale Q K^T, online softmax (mstx.cn/posts/485 §三.2), O = P V,
// normalised, with LSE = m + ln l. The merge is the same rule applied across
// chunks: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
//
// Causal: the queries are the last Nq positions of the sequence whose first
// Nk positions are the keys, so query i sees keys j <= Nk - Nq + i (for
// Nq = Nk this is the square kernel's rule).
//
// Kernel 1, decode_partial_kernel: every wave is an independent work item
// (head, 32-query block, key chunk). It keeps its 32 queries' Q^T fragments in
// registers and streams its chunk in 32-key tiles through its own two LDS
// buffers by direct global->LDS loads (no other wave reads them, so there is
// no workgroup barrier: the wave's own load counter orders them), computes
// S^T = K Q^T (lane = query) on MFMA, the online softmax in fp32 registers and
// O^T += V^T P^T on MFMA (V^T by LDS transpose reads), and writes its chunk's
// normalised O and LSE (fp32) to the workspace. The path is bound by reading
// K and V from HBM once; the MFMA work per byte is small.
//
// Kernel 2, decode_merge_kernel: merges the chunk results of each (head,
// query) and writes O (bf16) and LSE.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDecRows = 32;   // queries per wave
constexpr int kDecTile = 32;   // keys per LDS tile

// Waves per workgroup: four, each with two 32-key K+V buffers in LDS (32 KB
// per wave, 128 KB per workgroup at d = 128); at d = 256 the buffers are
// twice as large and two waves fill the same 128 KB.
template <int D>
constexpr int dec_waves()
{
    return D > 128 ? 2 : 4;
}

struct DecodeParams {
    const uint16_t *Q, *K, *V;
    float *Opart, *Lpart;
    int Nq, Nk, dh;
    int nqb;      // 32-query blocks per head
    int nsplit;   // key chunks per head
    int chunk;    // keys per chunk (multiple of kDecTile)
    long items;   // B*H*nqb*nsplit
    float c;      // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(dec_waves<D>() * kWave, 1) decode_partial_kernel(DecodeParams p)
{
    constexpr int kDecWaves = dec_waves<D>();
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int CPR = D / 8;
    constexpr uint32_t TB = kDecTile * D * 2;  // bytes of one K or V tile
    constexpr uint32_t BUF = 2 * TB;           // K tile then V tile
    constexpr int LPT = TB / 1024;             // 1 KB direct loads per K (or V) tile
    static_assert(LPT >= 1, "tile too small for the direct-load layout");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kDecWaves * 2 * BUF];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int l32 = lane % 32, hi = lane / 32;
    const long item = (long)blockIdx.x * kDecWaves + wave;
    if (item >= p.items)
        return;  // no barrier anywhere: a wave may leave on its own
    const int s = (int)(item % p.nsplit);
    const long rest = item / p.nsplit;
    const int qb = (int)(rest % p.nqb);
    const long bh = rest / p.nqb;
    const int Nq = p.Nq, Nk = p.Nk, dh = p.dh;
    const int q = qb * kDecRows + l32;  // this lane's query
    const int k0 = s * p.chunk;
    const int k1 = min(Nk, k0 + p.chunk);
    const uint32_t lds0 = lds_byte_addr(smem) + wave * 2 * BUF;

    const uint16_t *Qh = p.Q + (size_t)bh * Nq * dh;
    const uint16_t *Kh = p.K + (size_t)bh * Nk * dh;
    const uint16_t *Vh = p.V + (size_t)bh * Nk * dh;

    bf16x8 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = q < Nq && 16 * kk + 8 * hi < dh
                     ? *reinterpret_cast<const bf16x8 *>(Qh + (size_t)q * dh + 16 * kk + 8 * hi)
                     : bf16x8{};

    // LDS layouts as in the square forward: K rows swizzled for b128 reads
    // (chunk c at c ^ (r % 16), or c ^ ((r / 2) % 8) for 128-byte rows), V
    // rows for transpose reads (c ^ (4 (r % 4) + (r / 4) % 4), or with the
    // row parity in one bit's place).
    // (rows of 256 or 512 bytes take the same swizzles: the bank of a byte
    // depends on its address modulo 256)
    auto k_swz = [](int r) -> int { return CPR >= 16 ? (r % 16) : ((r / 2) % 8); };
    auto v_swz = [](int r) -> int {
        return CPR >= 16 ? 4 * (r % 4) + (r / 4) % 4 : 4 * ((r / 2) % 2) + (r / 4) % 4;
    };
    // Direct loads: lane `lane` of 1 KB block b writes physical chunk
    // lane % CPR of row b * (64 / CPR) + lane / CPR; global rows are dh wide
    // and chunks past dh (or rows past the chunk's keys) read as zeros.
    uint32_t kdma[LPT], vdma[LPT];
#pragma unroll
    for (int b = 0; b < LPT; ++b) {
        const int r = b * (64 / CPR) + lane / CPR;
        const int kc = (lane % CPR) ^ k_swz(r), vc = (lane % CPR) ^ v_swz(r);
        kdma[b] = 8 * kc < dh ? 2 * (r * dh + 8 * kc) : kBufferOutOfRange;
        vdma[b] = 8 * vc < dh ? 2 * (r * dh + 8 * vc) : kBufferOutOfRange;
    }
    auto issue = [&](int kb, uint32_t buf) __attribute__((always_inline)) {
        const uint32_t bytes = (uint32_t)(k1 - kb) * (2 * dh);
        const i32x4 rk = buffer_rsrc(Kh + (size_t)kb * dh, bytes);
        const i32x4 rv = buffer_rsrc(Vh + (size_t)kb * dh, bytes);
#pragma unroll
        for (int b = 0; b < LPT; ++b)
            lds_dma_buf_b128(rk, kdma[b], buf + b * 1024);
#pragma unroll
        for (int b = 0; b < LPT; ++b)
            lds_dma_buf_b128(rv, vdma[b], buf + TB + b * 1024);
    };

    uint32_t kaddr[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        kaddr[kk] = 2 * (l32 * D + 8 * ((2 * kk + hi) ^ k_swz(l32)));
    uint32_t vaddr[DB][2];
    {
        const int g = lane / 16, sl = lane % 16;
        const int v_row = 4 * (g / 2) + sl / 4;
        const int v_lc = 2 * (g % 2) + (sl % 4) / 2;
        const int v_in = 4 * (sl % 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            vaddr[db][0] = TB + 2 * (v_row * D + 8 * ((4 * db + v_lc) ^ v_swz(v_row)) + v_in);
            vaddr[db][1] = TB + 2 * ((v_row + 8) * D + 8 * ((4 * db + v_lc) ^ v_swz(v_row + 8)) + v_in);
        }
    }

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        o[db] = f32x16{};
    float m = -INFINITY, l = 0.f;
    const float c = p.c;
    // last key this lane's query may see
    const int kvis = CAUSAL ? Nk - Nq + q : Nk - 1;

    const int ntiles = k1 > k0 ? (k1 - k0 + kDecTile - 1) / kDecTile : 0;
    if (ntiles > 0)
        issue(k0, lds0);
    for (int i = 0; i < ntiles; ++i) {
        const int kb = k0 + i * kDecTile;
        const uint32_t buf = lds0 + (i & 1) * BUF;
        if (i + 1 < ntiles) {
            // the other buffer was last read in the previous iteration
            lds_reads_wait_all();
            issue(kb + kDecTile, lds0 + ((i + 1) & 1) * BUF);
            lds_dma_wait<2 * LPT>();
        } else {
            lds_dma_wait<0>();
        }

        f32x16 sv = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            sv = mfma32x32x16(lds_b128_at(buf + kaddr[kk]), qf[kk], sv);
        // element r of the block is key kb + 8 (r / 4) + 4 hi + r % 4
        if (kb + kDecTile > k1 || (CAUSAL && kb + kDecTile - 1 > Nk - Nq + qb * kDecRows)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb + 8 * (r / 4) + 4 * hi + (r % 4);
                if (key >= k1 || key > kvis)
                    sv[r] = -INFINITY;
            }
        }
        mfma_result_touch(sv, 0);  // head of the asm max chain
        float mx = vmax3(sv[0], sv[1], sv[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2)
            mx = vmax3(mx, sv[r], sv[r + 1]);
        mx = halves_max(vmax2(mx, sv[15])) * c;
        const float mnew = fmaxf(m, mx);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = m == -INFINITY ? 0.f : exp2_fast(m - mref);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o[db][r] *= alpha;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sv[r] = exp2_fast(fmaf(sv[r], c, -mref));
            ls += sv[r];
        }
        l += ls;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x8 pp = pack_bf16x8(sv, hh);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint32_t vo = buf + 2 * 16 * hh * D;
                o[db] = mfma32x32x16(lds_tr_pair_at(vaddr[db][0] + vo, vaddr[db][1] + vo), pp, o[db]);
            }
        }
    }

    // this chunk's normalised O (rows of O^T per lane) and LSE
    const float lt = halves_sum(l);
    if (q < Nq) {
        const size_t prow = ((size_t)(bh * p.nsplit + s) * Nq + q);
        float *Op = p.Opart + prow * dh;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = 32 * db + 8 * j + 4 * hi;
                if (col < dh)
                    *reinterpret_cast<float4 *>(Op + col) =
                        float4{o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                               o[db][4 * j + 3] * inv};
            }
        if (hi == 0)
            p.Lpart[prow] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    }
}

// Merge of the chunk results: LSE = M + ln sum_s exp(LSE_s - M) with
// M = max_s LSE_s, O = sum_s exp(LSE_s - LSE) O_s; no visible key at all gives
// O = 0, LSE = -inf. A workgroup covers 32 columns of one (head, query) row;
// its 8 groups of 32 threads take every 8th chunk (coalesced 128-byte reads
// of the chunks' rows, independent of one another) and add up through LDS.
constexpr int kMergeCols = 32;
constexpr int kMergeGroups = 8;

__global__ void __launch_bounds__(kMergeCols * kMergeGroups)
    decode_merge_kernel(const float *Opart, const float *Lpart, uint16_t *O, float *LSE, int Nq,
                        int dh, int nsplit)
{
    __shared__ float red[kMergeGroups][kMergeCols];
    __shared__ float stat[2][kMergeGroups];
    const long row = blockIdx.x;  // bh * Nq + q
    const long bh = row / Nq;
    const int q = (int)(row % Nq);
    const int t = threadIdx.x;
    const int g = t / kMergeCols;               // group (one wave holds two)
    const int col = blockIdx.y * kMergeCols + t % kMergeCols;
    const float *L = Lpart + (size_t)bh * nsplit * Nq + q;  // stride Nq over chunks

    // M and W over all chunks: per thread, then per wave, then per workgroup
    float M = -INFINITY;
    for (int sp = t; sp < nsplit; sp += kMergeCols * kMergeGroups)
        M = fmaxf(M, L[(size_t)sp * Nq]);
#pragma unroll
    for (int off = kWave / 2; off > 0; off /= 2)
        M = fmaxf(M, __shfl_xor(M, off, kWave));
    if (t % kWave == 0)
        stat[0][t / kWave] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kMergeCols * kMergeGroups / kWave; ++w)
        M = fmaxf(M, stat[0][w]);
    float W = 0.f;
    if (M != -INFINITY)
        for (int sp = t; sp < nsplit; sp += kMergeCols * kMergeGroups) {
            const float ls = L[(size_t)sp * Nq];
            W += ls == -INFINITY ? 0.f : __expf(ls - M);
        }
#pragma unroll
    for (int off = kWave / 2; off > 0; off /= 2)
        W += __shfl_xor(W, off, kWave);
    if (t % kWave == 0)
        stat[1][t / kWave] = W;
    __syncthreads();
    W = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeCols * kMergeGroups / kWave; ++w)
        W += stat[1][w];
    const float lse = M == -INFINITY ? -INFINITY : M + __logf(W);

    float acc = 0.f;
    if (col < dh && M != -INFINITY) {
#pragma unroll 4
        for (int sp = g; sp < nsplit; sp += kMergeGroups) {
            const float ls = L[(size_t)sp * Nq];
            const float v = Opart[((size_t)(bh * nsplit + sp) * Nq + q) * dh + col];
            acc = fmaf(ls == -INFINITY ? 0.f : __expf(ls - lse), v, acc);
        }
    }
    red[g][t % kMergeCols] = acc;
    __syncthreads();
    if (g == 0 && col < dh) {
        float o = 0.f;
#pragma unroll
        for (int k = 0; k < kMergeGroups; ++k)
            o += red[k][t];
        O[(size_t)row * dh + col] = f32_to_bf16_bits(o);
    }
    if (blockIdx.y == 0 && t == 0)
        LSE[row] = lse;
}

template <int D>
hipError_t decode_d(const DecodeProblem &pr, const DecodeSplit &sp, const uint16_t *Q,
                    const uint16_t *K, const uint16_t *V, uint16_t *O, float *LSE, void *ws)
{
    DecodeParams dp{};
    dp.Q = Q;
    dp.K = K;
    dp.V = V;
    dp.Opart = reinterpret_cast<float *>(ws);
    dp.Lpart = reinterpret_cast<float *>(static_cast<char *>(ws) + sp.lpart_off);
    dp.Nq = pr.Nq;
    dp.Nk = pr.Nk;
    dp.dh = pr.d;
    dp.nqb = (pr.Nq + kDecRows - 1) / kDecRows;
    dp.nsplit = sp.nsplit;
    dp.chunk = sp.chunk;
    dp.items = (long)pr.B * pr.H * dp.nqb * sp.nsplit;
    dp.c = pr.scale * kLog2e;
    constexpr int kDecWaves = dec_waves<D>();
    const unsigned grid = (unsigned)((dp.items + kDecWaves - 1) / kDecWaves);
    if (pr.causal)
        hipLaunchKernelGGL((decode_partial_kernel<D, true>), dim3(grid), dim3(kDecWaves * kWave), 0,
                           pr.stream, dp);
    else
        hipLaunchKernelGGL((decode_partial_kernel<D, false>), dim3(grid), dim3(kDecWaves * kWave), 0,
                           pr.stream, dp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const long rows = (long)pr.B * pr.H * pr.Nq;
    const unsigned colblocks = (unsigned)((pr.d + kMergeCols - 1) / kMergeCols);
    hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)rows, colblocks),
                       dim3(kMergeCols * kMergeGroups), 0, pr.stream, dp.Opart, dp.Lpart, O, LSE,
                       pr.Nq, pr.d, sp.nsplit);
    return hipGetLastError();
}

}  // namespace

DecodeSplit decode_split(int B, int H, int Nq, int Nk, int d)
{
    DecodeSplit sp{};
    if (B <= 0 || H <= 0 || Nq <= 0)
        return sp;
    // Enough independent waves to fill the chip a few times over (1024 run
    // at once: one 4-wave workgroup per CU at d = 128), chunks of at least
    // 256 keys so that each wave streams a while.
    const long blocks = (long)B * H * ((Nq + kDecRows - 1) / kDecRows);
    const long want = (4096 + blocks - 1) / blocks;
    const long most = Nk > 0 ? (Nk + 255) / 256 : 1;
    const long ns = want < 1 ? 1 : (want > most ? most : want);
    int chunk = Nk > 0 ? (int)((Nk + ns - 1) / ns) : kDecTile;
    chunk = (chunk + kDecTile - 1) / kDecTile * kDecTile;
    sp.chunk = chunk;
    sp.nsplit = Nk > 0 ? (Nk + chunk - 1) / chunk : 1;
    const size_t rows = (size_t)B * H * sp.nsplit * Nq;
    sp.lpart_off = (rows * d * sizeof(float) + 255) / 256 * 256;
    sp.bytes = sp.lpart_off + (rows * sizeof(float) + 255) / 256 * 256;
    return sp;
}

hipError_t launch_decode_bf16(const DecodeProblem &pr, const uint16_t *Q, const uint16_t *K,
                              const uint16_t *V, uint16_t *O, float *LSE, void *workspace)
{
    const DecodeSplit sp = decode_split(pr.B, pr.H, pr.Nq, pr.Nk, pr.d);
    if (pr.d <= 64)
        return decode_d<64>(pr, sp, Q, K, V, O, LSE, workspace);
    if (pr.d <= 128)
        return decode_d<128>(pr, sp, Q, K, V, O, LSE, workspace);
    return decode_d<256>(pr, sp, Q, K, V, O, LSE, workspace);
}

}  // namespace fa
