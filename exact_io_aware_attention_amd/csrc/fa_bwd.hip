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
//   1. bwd_pre:  D and LSE * log2(e) per row (bandwidth-bound, one pass
//      over dO and O);
//   2. bwd_dq:   one workgroup per query block, key tiles streamed through
//      LDS; recomputes S^T and dP^T, forms dS^T and accumulates
//      dQ^T = K^T dS^T in registers (lane = query, as in the forward);
//   3. bwd_dkdv: one workgroup per key block (32 keys per wave, K and V in
//      registers), query tiles streamed through LDS; recomputes S and dP,
//      accumulates dV^T = dO^T P and dK^T = Q^T dS in registers
//      (lane = key).
// Splitting dQ from dK/dV recomputes S and dP once more (7 contractions
// instead of 5) but needs no atomics and is deterministic.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

// ---------------------------------------------------------------- pre ----

template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const uint16_t *dO, const uint16_t *O,
                                                      const float *LSE, float *delta,
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
        delta[row] = acc;
        const float L = LSE[row];
        lse2[row] = (L == -INFINITY) ? INFINITY : L * kLog2e;
    }
}

// ----------------------------------------------------------------- dQ ----

struct DqParams {
    const uint16_t *dO, *Q, *K, *V;
    const float *delta, *lse2;
    uint16_t *dQ;
    const uint8_t *mask;
    int N, nqb, nkt, nmb, items, per_xcd;
    float c, scale;
};

template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256, 1) bwd_dq_kernel(DqParams p)
{
    constexpr int RW = 32;         // query rows per wave
    constexpr int BR = 4 * RW;     // query rows per workgroup
    constexpr int BC = 64;         // keys per LDS tile
    constexpr int KSTR = D + 16;   // K tile: row reads and transpose reads
    constexpr int VSTR = D + 8;    // V tile: row reads
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int CPR = D / 8;
    constexpr int RPI = 256 / CPR;
    constexpr int NI = BC / RPI;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BC * VSTR];

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
    const int wr0 = q0 + wave * RW;
    const int row = wr0 + l32;

    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t *Qh = p.Q + head, *dOh = p.dO + head;
    const uint16_t *Kh = p.K + head, *Vh = p.V + head;

    bf16x8 qf[KK], gf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (row < N) {
            qf[kk] = *reinterpret_cast<const bf16x8 *>(Qh + (size_t)row * D + 16 * kk + 8 * hi);
            gf[kk] = *reinterpret_cast<const bf16x8 *>(dOh + (size_t)row * D + 16 * kk + 8 * hi);
        } else {
            qf[kk] = bf16x8{};
            gf[kk] = bf16x8{};
        }
    }
    const float lse2 = row < N ? p.lse2[(size_t)bh * N + row] : INFINITY;
    const float Di = row < N ? p.delta[(size_t)bh * N + row] : 0.f;

    int t_end = p.nkt;
    if (CAUSAL)
        t_end = min(p.nkt, (q0 + BR - 1) / BC + 1);
    const int mrow = q0 / kMaskBlock;  // BR = 128: one mask row per workgroup
    auto tile_needed = [&](int t) -> bool {
        return !SPARSE || p.mask[(size_t)mrow * p.nmb + (t * BC) / kMaskBlock] != 0;
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

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        dq[db] = f32x16{};

    const int g = lane / 16;
    const int sl = lane % 16;
    const int t_key = 4 * (g / 2) + sl / 4;
    const int t_col = 16 * (g % 2) + 4 * (sl % 4);

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
        if (CAUSAL)
            active = active && kbase <= wr0 + RW - 1;
        if (active) {
            const uint16_t *ks = Ks[buf];
            const uint16_t *vs = Vs[buf];
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16{};
                dp[kb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const bf16x8 kf = lds_read_b128(ks + (32 * kb + l32) * KSTR + 16 * kk + 8 * hi);
                    const bf16x8 vf = lds_read_b128(vs + (32 * kb + l32) * VSTR + 16 * kk + 8 * hi);
                    s[kb] = mfma32x32x16(kf, qf[kk], s[kb]);
                    dp[kb] = mfma32x32x16(vf, gf[kk], dp[kb]);
                }
            }
            const bool need_mask = (kbase + BC > N) || (CAUSAL && kbase + BC - 1 > wr0);
            // dS^T = P^T o (dP^T - D), P^T = 2^(c s - lse2); masked entries 0.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr = exp2_fast(fmaf(s[kb][r], p.c, -lse2));
                    if (need_mask) {
                        const int key = kbase + 32 * kb + 8 * (r / 4) + 4 * hi + (r % 4);
                        if (key >= N || (CAUSAL && key > row))
                            pr = 0.f;
                    }
                    s[kb][r] = pr * (dp[kb][r] - Di);
                }
            // dQ^T += K^T dS^T (transpose reads of the K tile).
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const bf16x8 sf = pack_bf16x8(s[kb], hh);
                    const uint16_t *krow = ks + (32 * kb + 16 * hh + t_key) * KSTR + t_col;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 kt = lds_read_tr_pair(krow + 32 * db, krow + 8 * KSTR + 32 * db);
                        dq[db] = mfma32x32x16(kt, sf, dq[db]);
                    }
                }
        }
        if (tn < t_end)
            store_tile(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        t = tn;
    }

    if (row < N) {
        uint16_t *dQh = p.dQ + head;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dcol = 32 * db + 8 * j + 4 * hi;
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16_bits(dq[db][4 * j + 0] * p.scale) |
                       ((uint32_t)f32_to_bf16_bits(dq[db][4 * j + 1] * p.scale) << 16);
                pk.y = (uint32_t)f32_to_bf16_bits(dq[db][4 * j + 2] * p.scale) |
                       ((uint32_t)f32_to_bf16_bits(dq[db][4 * j + 3] * p.scale) << 16);
                *reinterpret_cast<uint2 *>(dQh + (size_t)row * D + dcol) = pk;
            }
    }
}

// -------------------------------------------------------------- dK dV ----

struct DkvParams {
    const uint16_t *dO, *Q, *K, *V;
    const float *delta, *lse2;
    uint16_t *dK, *dV;
    const uint8_t *mask;
    int N, nkb, nqt, nmb, items, per_xcd;
    float c, scale;
};

template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(DkvParams p)
{
    constexpr int KW = 32;         // keys per wave
    constexpr int BK = 4 * KW;     // keys per workgroup
    constexpr int BQ = 64;         // queries per LDS tile
    constexpr int STR = D + 16;    // Q / dO tiles: row reads and transpose reads
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int CPR = D / 8;
    constexpr int RPI = 256 / CPR;
    constexpr int NI = BQ / RPI;

    __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BQ * STR];
    __shared__ __attribute__((aligned(16))) uint16_t Gs[2][BQ * STR];
    __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
    __shared__ __attribute__((aligned(16))) float Ds[2][BQ];

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nkb;
    const int kblk = item - bh * p.nkb;  // causal: later key blocks see fewer queries
    const int k0 = kblk * BK;
    const int N = p.N;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int wk0 = k0 + wave * KW;
    const int key = wk0 + l32;

    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t *Qh = p.Q + head, *dOh = p.dO + head;
    const uint16_t *Kh = p.K + head, *Vh = p.V + head;
    const float *lse2h = p.lse2 + (size_t)bh * N;
    const float *deltah = p.delta + (size_t)bh * N;

    // This wave's keys as MFMA B operands (lane = key, 8 d-values each).
    bf16x8 kf[KK], vf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (key < N) {
            kf[kk] = *reinterpret_cast<const bf16x8 *>(Kh + (size_t)key * D + 16 * kk + 8 * hi);
            vf[kk] = *reinterpret_cast<const bf16x8 *>(Vh + (size_t)key * D + 16 * kk + 8 * hi);
        } else {
            kf[kk] = bf16x8{};
            vf[kk] = bf16x8{};
        }
    }

    const int t_begin = CAUSAL ? k0 / BQ : 0;
    const int kmb = k0 / kMaskBlock;  // BK = 128: one mask column per workgroup
    auto tile_needed = [&](int t) -> bool {
        return !SPARSE || p.mask[(size_t)((t * BQ) / kMaskBlock) * p.nmb + kmb] != 0;
    };
    auto next_tile = [&](int t) -> int {
        ++t;
        if (SPARSE)
            while (t < p.nqt && !tile_needed(t))
                ++t;
        return t;
    };

    uint4 qst[NI], gst[NI];
    float lst = 0.f, dst = 0.f;
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = tid / CPR + i * RPI;
            const int c = tid % CPR;
            const int q = t * BQ + r;
            if (q < N) {
                qst[i] = *reinterpret_cast<const uint4 *>(Qh + (size_t)q * D + 8 * c);
                gst[i] = *reinterpret_cast<const uint4 *>(dOh + (size_t)q * D + 8 * c);
            } else {
                qst[i] = uint4{0, 0, 0, 0};
                gst[i] = uint4{0, 0, 0, 0};
            }
        }
        if (tid < BQ) {
            const int q = t * BQ + tid;
            lst = q < N ? lse2h[q] : INFINITY;
            dst = q < N ? deltah[q] : 0.f;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = tid / CPR + i * RPI;
            const int c = tid % CPR;
            *reinterpret_cast<uint4 *>(&Qs[buf][r * STR + 8 * c]) = qst[i];
            *reinterpret_cast<uint4 *>(&Gs[buf][r * STR + 8 * c]) = gst[i];
        }
        if (tid < BQ) {
            Ls[buf][tid] = lst;
            Ds[buf][tid] = dst;
        }
    };

    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    const int g = lane / 16;
    const int sl = lane % 16;
    const int t_row = 4 * (g / 2) + sl / 4;
    const int t_col = 16 * (g % 2) + 4 * (sl % 4);

    int t = t_begin;
    if (SPARSE && t < p.nqt && !tile_needed(t))
        t = next_tile(t);
    if (t < p.nqt) {
        load_tile(t);
        store_tile(0);
    }
    __syncthreads();
    int buf = 0;
    while (t < p.nqt) {
        const int tn = next_tile(t);
        if (tn < p.nqt)
            load_tile(tn);
        const int qbase = t * BQ;
        bool active = wk0 < N;
        if (CAUSAL)
            active = active && qbase + BQ - 1 >= wk0;
        if (active) {
            const uint16_t *qs = Qs[buf];
            const uint16_t *gs = Gs[buf];
            const float *ls = Ls[buf];
            const float *ds = Ds[buf];
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) {
                // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
                // (lane = key, register r = query 8(r/4) + 4 hi + r%4).
                f32x16 s = f32x16{}, dpv = f32x16{};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const bf16x8 qa = lds_read_b128(qs + (32 * qh + l32) * STR + 16 * kk + 8 * hi);
                    const bf16x8 ga = lds_read_b128(gs + (32 * qh + l32) * STR + 16 * kk + 8 * hi);
                    s = mfma32x32x16(qa, kf[kk], s);
                    dpv = mfma32x32x16(ga, vf[kk], dpv);
                }
                const int qrow0 = qbase + 32 * qh;
                const bool need_mask = (qrow0 + 32 > N) || (CAUSAL && qrow0 < wk0 + KW - 1);
                f32x16 pm, dsm;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 lv = *reinterpret_cast<const float4 *>(ls + 32 * qh + 8 * j + 4 * hi);
                    const float4 dv4 = *reinterpret_cast<const float4 *>(ds + 32 * qh + 8 * j + 4 * hi);
                    const float lq[4] = {lv.x, lv.y, lv.z, lv.w};
                    const float dq[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 4 * j + u;
                        float pr = exp2_fast(fmaf(s[r], p.c, -lq[u]));
                        if (need_mask) {
                            const int q = qrow0 + 8 * j + 4 * hi + u;
                            if (q >= N || (CAUSAL && key > q))
                                pr = 0.f;
                        }
                        pm[r] = pr;
                        dsm[r] = pr * (dpv[r] - dq[u]);
                    }
                }
                // dV^T += dO^T P and dK^T += Q^T dS (transpose reads of the
                // query tiles; P and dS enter as B operands, k = queries).
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const bf16x8 pf = pack_bf16x8(pm, hh);
                    const bf16x8 sf = pack_bf16x8(dsm, hh);
                    const int trow = 32 * qh + 16 * hh + t_row;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const uint16_t *gp = gs + trow * STR + t_col + 32 * db;
                        const uint16_t *qp = qs + trow * STR + t_col + 32 * db;
                        const bf16x8 gt = lds_read_tr_pair(gp, gp + 8 * STR);
                        const bf16x8 qt = lds_read_tr_pair(qp, qp + 8 * STR);
                        dv[db] = mfma32x32x16(gt, pf, dv[db]);
                        dk[db] = mfma32x32x16(qt, sf, dk[db]);
                    }
                }
            }
        }
        if (tn < p.nqt)
            store_tile(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        t = tn;
    }

    if (key < N) {
        uint16_t *dKh = p.dK + head, *dVh = p.dV + head;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dcol = 32 * db + 8 * j + 4 * hi;
                uint2 pk, pv;
                pk.x = (uint32_t)f32_to_bf16_bits(dk[db][4 * j + 0] * p.scale) |
                       ((uint32_t)f32_to_bf16_bits(dk[db][4 * j + 1] * p.scale) << 16);
                pk.y = (uint32_t)f32_to_bf16_bits(dk[db][4 * j + 2] * p.scale) |
                       ((uint32_t)f32_to_bf16_bits(dk[db][4 * j + 3] * p.scale) << 16);
                pv.x = (uint32_t)f32_to_bf16_bits(dv[db][4 * j + 0]) |
                       ((uint32_t)f32_to_bf16_bits(dv[db][4 * j + 1]) << 16);
                pv.y = (uint32_t)f32_to_bf16_bits(dv[db][4 * j + 2]) |
                       ((uint32_t)f32_to_bf16_bits(dv[db][4 * j + 3]) << 16);
                *reinterpret_cast<uint2 *>(dKh + (size_t)key * D + dcol) = pk;
                *reinterpret_cast<uint2 *>(dVh + (size_t)key * D + dcol) = pv;
            }
    }
}

struct BwdPtrs {
    const uint16_t *dO, *Q, *K, *V, *O;
    const float *LSE;
    uint16_t *dQ, *dK, *dV;
    float *delta, *lse2;
};

BwdPtrs bwd_ptrs(const Problem &pr, const uint16_t *dO, const uint16_t *Q, const uint16_t *K,
                 const uint16_t *V, const uint16_t *O, const float *LSE, uint16_t *dQ,
                 uint16_t *dK, uint16_t *dV, void *ws)
{
    const BwdWorkspace L = bwd_workspace_layout(pr.B, pr.H, pr.N, pr.d);
    BwdPtrs b;
    b.dO = dO; b.Q = Q; b.K = K; b.V = V; b.O = O; b.LSE = LSE;
    b.dQ = dQ; b.dK = dK; b.dV = dV;
    b.delta = reinterpret_cast<float *>(static_cast<char *>(ws) + L.delta_off);
    b.lse2 = reinterpret_cast<float *>(static_cast<char *>(ws) + L.lse2_off);
    return b;
}

template <int D>
hipError_t prep_d(const Problem &pr, const BwdPtrs &b)
{
    const long rows = (long)pr.B * pr.H * pr.N;
    const long threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       pr.stream, b.dO, b.O, b.LSE, b.delta, b.lse2, rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t dq_t(const Problem &pr, const BwdPtrs &b)
{
    DqParams qp{};
    qp.dO = b.dO; qp.Q = b.Q; qp.K = b.K; qp.V = b.V;
    qp.delta = b.delta; qp.lse2 = b.lse2; qp.dQ = b.dQ; qp.mask = pr.mask;
    qp.N = pr.N;
    qp.nqb = (pr.N + 127) / 128;
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
    kp.delta = b.delta; kp.lse2 = b.lse2; kp.dK = b.dK; kp.dV = b.dV; kp.mask = pr.mask;
    kp.N = pr.N;
    kp.nkb = (pr.N + 127) / 128;
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
