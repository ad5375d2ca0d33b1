// Forward of exact attention on gfx950: bf16 storage, bf16 MFMA contractions,
// fp32 online softmax. One fused kernel: S = scale Q K^T -> mask -> online
// softmax -> O += P V, with the N x N S and P held only as register tiles
// (lukebest.github.io FlashAttention, "Kernel fusion"; mstx.cn/posts/485
// §三.1 "Tiling", §三.2 "Online Softmax").
//
// Work decomposition (a re-derivation for CDNA4, not the pages' A100 tiles):
//   - one workgroup = 4 waves (one per SIMD) owns BR = 128*QB consecutive
//     query rows of one (b, h); each wave owns 32*QB rows and keeps its Q
//     rows in registers for the whole key loop, so O, m and l never leave
//     registers (the key loop is the inner loop, the order the pages'
//     sequence-parallel successor uses, lukebest.github.io "谱系");
//   - K and V stream through LDS in 64-key tiles, double-buffered: the global
//     loads of tile j+1 are in flight while tile j is computed;
//   - scores are computed transposed, S^T = K Q^T, so that each lane owns one
//     query and row max / row sum are lane-local plus one exchange between
//     the two 32-lane halves;
//   - P^T goes back into the MFMA as the B operand of O^T = V^T P^T, the V^T
//     operand coming from the row-major V tile by LDS transpose reads.
//
// Online softmax (mstx.cn/posts/485 §三.2 update rule), in base 2 with
// c = scale * log2(e):
//   m' = max(m, c * rowmax(S_tile)),  alpha = 2^(m - m'),
//   p = 2^(c * s - m'),  l' = alpha * l + sum p,  O' = alpha * O + p V,
// and O = O / l, LSE = (m + log2 l) * ln 2 at the end. A row that has seen
// no visible key keeps m = -inf; exponents are then taken against 0 so that
// no (-inf) - (-inf) arises, and such a row ends with O = 0, LSE = -inf.
//
// Masking: causal (key j visible to query i iff j <= i, nanhubrain.csdn.net
// §三.1 tile set) -- key tiles wholly above the diagonal of the workgroup are
// never loaded, and the per-element mask runs only on tiles that straddle the
// diagonal or the end of the sequence; block-sparse (lukebest.github.io
// "Block-Sparse FlashAttention") -- key tiles whose 128 x 128 mask block is
// zero for every wave of the workgroup are skipped without being loaded.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

struct FwdParams {
    const uint16_t *Q, *K, *V;
    uint16_t *O;
    float *LSE;
    const uint8_t *mask;
    int N;
    int nqb;      // query blocks per head
    int nkt;      // 64-key tiles per head
    int nmb;      // mask blocks per mask row
    int items;    // B * H * nqb
    int per_xcd;  // work items per XCD
    float c;      // scale * log2(e)
};

template <int D, int QB, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256, 1) fwd_bf16_kernel(FwdParams p)
{
    constexpr int BR = 128 * QB;    // query rows per workgroup
    constexpr int RW = 32 * QB;     // query rows per wave
    constexpr int BC = 64;          // keys per LDS tile
    constexpr int KSTR = D + 8;     // K tile row stride in elements (conflict-free b128 reads)
    constexpr int VSTR = D + 16;    // V tile row stride in elements (conflict-free transpose reads)
    constexpr int KK = D / 16;      // depth steps of Q K^T
    constexpr int DB = D / 32;      // 32-row blocks of O^T
    constexpr int CPR = D / 8;      // 16-byte chunks per row
    constexpr int RPI = 256 / CPR;  // rows per staging pass
    constexpr int NI = BC / RPI;    // staging passes per tile

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BC * VSTR];

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nqb;
    const int qi = item - bh * p.nqb;
    const int qblk = CAUSAL ? (p.nqb - 1 - qi) : qi;  // causal: longest rows first
    const int q0 = qblk * BR;
    const int N = p.N;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int wr0 = q0 + wave * RW;

    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t *Qh = p.Q + head;
    const uint16_t *Kh = p.K + head;
    const uint16_t *Vh = p.V + head;

    // This wave's query rows as MFMA B operands (d-slices of 16).
    bf16x8 qf[QB][KK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wr0 + 32 * qb + l32;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (row < N)
                qf[qb][kk] = *reinterpret_cast<const bf16x8 *>(Qh + (size_t)row * D + 16 * kk + 8 * hi);
            else
                qf[qb][kk] = bf16x8{};
        }
    }

    int t_end = p.nkt;
    if (CAUSAL)
        t_end = min(p.nkt, (q0 + BR - 1) / BC + 1);

    // Block-sparse: the mask rows this workgroup and this wave fall in.
    const int mr_lo = q0 / kMaskBlock;
    const int mr_hi = min(q0 + BR - 1, N - 1) / kMaskBlock;
    const int wmr = wr0 / kMaskBlock;
    auto tile_needed = [&](int t) -> bool {
        if (!SPARSE)
            return true;
        const int kbk = (t * BC) / kMaskBlock;
        bool keep = false;
        for (int mr = mr_lo; mr <= mr_hi; ++mr)
            keep |= p.mask[(size_t)mr * p.nmb + kbk] != 0;
        return keep;
    };
    auto next_tile = [&](int t) -> int {
        ++t;
        if (SPARSE)
            while (t < t_end && !tile_needed(t))
                ++t;
        return t;
    };

    uint4 kst[NI], vst[NI];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = tid / CPR + i * RPI;
            const int c = tid % CPR;
            const int key = t * BC + r;
            if (key < N) {
                kst[i] = *reinterpret_cast<const uint4 *>(Kh + (size_t)key * D + 8 * c);
                vst[i] = *reinterpret_cast<const uint4 *>(Vh + (size_t)key * D + 8 * c);
            } else {
                kst[i] = uint4{0, 0, 0, 0};
                vst[i] = uint4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = tid / CPR + i * RPI;
            const int c = tid % CPR;
            *reinterpret_cast<uint4 *>(&Ks[buf][r * KSTR + 8 * c]) = kst[i];
            *reinterpret_cast<uint4 *>(&Vs[buf][r * VSTR + 8 * c]) = vst[i];
        }
    };

    f32x16 o[QB][DB];
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            o[qb][db] = f32x16{};
    }

    // Transpose-read addressing of the V^T operand: lane 4t+u of each
    // 16-lane group g points at key row 4*(g/2)+t, columns 16*(g%2)+4u.
    const int g = lane / 16;
    const int sl = lane % 16;
    const int v_key = 4 * (g / 2) + sl / 4;
    const int v_col = 16 * (g % 2) + 4 * (sl % 4);

    int t = next_tile(-1);
    if (t < t_end) {
        load_tile(t);
        store_tile(0);
    }
    __syncthreads();
    int buf = 0;
    while (t < t_end) {
        const int tn = next_tile(t);
        if (tn < t_end)
            load_tile(tn);

        const int kbase = t * BC;
        bool active = wr0 < N;
        if (SPARSE)
            active = active && p.mask[(size_t)wmr * p.nmb + kbase / kMaskBlock] != 0;
        if (CAUSAL)
            active = active && kbase <= wr0 + RW - 1;
        if (active) {
            const uint16_t *ks = Ks[buf];
            const uint16_t *vs = Vs[buf];
            f32x16 s[QB][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                s[qb][0] = f32x16{};
                s[qb][1] = f32x16{};
            }
            // S^T = K Q^T for two 32-key halves of the tile.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const bf16x8 kf = lds_read_b128(ks + (32 * kb + l32) * KSTR + 16 * kk + 8 * hi);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        s[qb][kb] = mfma32x32x16(kf, qf[qb][kk], s[qb][kb]);
                }
            }
            // Element mask: keys past the end of the sequence, and (causal)
            // keys above the diagonal.
            const bool need_mask = (kbase + BC > N) || (CAUSAL && kbase + BC - 1 > wr0);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int row = wr0 + 32 * qb + l32;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kbase + 32 * kb + 8 * (r / 4) + 4 * hi + (r % 4);
                            if (key >= N || (CAUSAL && key > row))
                                s[qb][kb][r] = -INFINITY;
                        }
                }
            }
            // Online softmax update (base 2).
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        mx = fmaxf(mx, s[qb][kb][r]);
                mx = fmaxf(mx, lane_swap32(mx));
                const float mnew = fmaxf(m[qb], mx * p.c);
                const float mref = (mnew == -INFINITY) ? 0.f : mnew;
                const float alpha = exp2_fast(m[qb] - mref);
                m[qb] = mnew;
                float lsum = l[qb] * alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o[qb][db][r] *= alpha;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = exp2_fast(fmaf(s[qb][kb][r], p.c, -mref));
                        s[qb][kb][r] = e;
                        lsum += e;
                    }
                l[qb] = lsum;
            }
            // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    bf16x8 pf[QB];
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        pf[qb] = pack_bf16x8(s[qb][kb], hh);
                    const uint16_t *vrow = vs + (32 * kb + 16 * hh + v_key) * VSTR + v_col;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 vf = lds_read_tr_pair(vrow + 32 * db, vrow + 8 * VSTR + 32 * db);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb)
                            o[qb][db] = mfma32x32x16(vf, pf[qb], o[qb][db]);
                    }
                }
            }
        }

        if (tn < t_end)
            store_tile(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        t = tn;
    }

    // Epilogue: O = O^T / l (transposed back per lane), LSE in natural log.
    uint16_t *Oh = p.O + head;
    float *Lh = p.LSE + (size_t)bh * N;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = l[qb] + lane_swap32(l[qb]);
        const int row = wr0 + 32 * qb + l32;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (row < N) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int dcol = 32 * db + 8 * j + 4 * hi;
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16_bits(o[qb][db][4 * j + 0] * inv) |
                           ((uint32_t)f32_to_bf16_bits(o[qb][db][4 * j + 1] * inv) << 16);
                    pk.y = (uint32_t)f32_to_bf16_bits(o[qb][db][4 * j + 2] * inv) |
                           ((uint32_t)f32_to_bf16_bits(o[qb][db][4 * j + 3] * inv) << 16);
                    *reinterpret_cast<uint2 *>(Oh + (size_t)row * D + dcol) = pk;
                }
            if (hi == 0)
                Lh[row] = lt > 0.f ? (m[qb] + log2f(lt)) * kLn2 : -INFINITY;
        }
    }
}

template <int D, int QB, bool CAUSAL, bool SPARSE>
static hipError_t launch_fwd_t(const Problem &pr, const FwdParams &fp0)
{
    FwdParams fp = fp0;
    constexpr int BR = 128 * QB;
    fp.nqb = (pr.N + BR - 1) / BR;
    fp.items = pr.B * pr.H * fp.nqb;
    fp.per_xcd = (fp.items + kXcds - 1) / kXcds;
    const int grid = fp.per_xcd * kXcds;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, CAUSAL, SPARSE>), dim3(grid), dim3(256), 0,
                       pr.stream, fp);
    return hipGetLastError();
}

template <int D, int QB>
static hipError_t launch_fwd_d(const Problem &pr, const FwdParams &fp)
{
    const bool sparse = pr.mask != nullptr;
    if (pr.causal)
        return sparse ? launch_fwd_t<D, QB, true, true>(pr, fp) : launch_fwd_t<D, QB, true, false>(pr, fp);
    return sparse ? launch_fwd_t<D, QB, false, true>(pr, fp) : launch_fwd_t<D, QB, false, false>(pr, fp);
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
    fp.nkt = (pr.N + 63) / 64;
    fp.nmb = (pr.N + kMaskBlock - 1) / kMaskBlock;
    fp.c = pr.scale * kLog2e;
    if (pr.d == 64)
        return launch_fwd_d<64, 2>(pr, fp);
    return launch_fwd_d<128, 2>(pr, fp);
}

}  // namespace fa
