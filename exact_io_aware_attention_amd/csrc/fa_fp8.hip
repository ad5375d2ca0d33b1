// FP8 forward of exact attention on gfx950 (lukebest.github.io FlashAttention,
// lineage table "谱系": the third generation adds an FP8 forward). Q, K, V
// are OCP E4M3 codes with one fp32 descale each (value = code * descale); the
// result is the forward of those values: S = scale (Q K^T) computed from the
// exact fp8 products in fp32, online softmax in fp32 (mstx.cn/posts/485
// §三.2) whose reference follows the row max exactly, P rounded to E4M3 for
// the P V contraction (weights <= 1; the one that sets a new max is exactly 1,
// so rows dominated by few keys keep them exact -- a reference lagging below
// the max, as the bf16 kernel's lazy rescale allows, would round them with up
// to 6% error); O = (P V) * v_descale / l in fp32, stored as bf16; LSE as in
// fa_fwd.
//
// Contractions on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales): one
// MFMA covers 64 of the contraction index, so S^T = K Q^T of a 32-key block
// takes D / 64 MFMAs and O^T += V^T P^T takes one MFMA per 32 output columns
// for 64 keys. In both operands a lane holds 32 bytes, and lane-half h of A
// pairs byte for byte with lane-half h of B.
//
// S^T per 32-key block has the bf16 kernel's layout: lane = query, register r
// = key 8 (r / 4) + 4 hi + r % 4. A lane's 32 P values of a 64-key tile (16 of
// each block) are packed as bytes 0..31 of its B operand, so byte b of
// lane-half h stands for key k(h, b) = 32 (b / 16) + 8 ((b % 16) / 4) + 4 h +
// b % 4. V^T therefore needs the keys of a tile in that order: a pre-pass
// writes V^T per 64-key tile as D rows of 64 bytes, key j at position
// 32 ((j / 4) % 2) + 16 (j / 32) + 4 ((j % 32) / 8) + j % 4, so that each
// lane's V^T operand is 32 contiguous bytes. Tiles stream into LDS by direct
// loads (three buffers, two tiles ahead; the next tile's S^T MFMAs are issued
// beside the current softmax); 16-byte chunks are XOR-swizzled so that the
// b128 operand reads of 16 lanes hit 16 different bank groups.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c)
{
    // formats 0/0: E4M3 for both operands; block scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// V [bh][N][D] -> V^T tiles [bh][tile][D][64] in the P byte order; keys past
// N are zero. One workgroup per (tile, bh): the 64 x D tile is read row-major
// into LDS with 16-byte loads, then every thread writes 16 consecutive bytes of
// a V^T row.
template <int D>
__global__ void __launch_bounds__(256) fp8_vt_kernel(const uint8_t *V, uint8_t *Vt, int N)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[64 * D];
    const int t = blockIdx.x;
    const long bh = blockIdx.y;
    const int nkt = gridDim.x;
    const uint8_t *Vh = V + (size_t)bh * N * D;
    for (int c = threadIdx.x; c < 64 * D / 16; c += 256) {
        const int j = c / (D / 16), col = 16 * (c % (D / 16));
        const int key = t * 64 + j;
        uint4 x = {0, 0, 0, 0};
        if (key < N)
            x = *reinterpret_cast<const uint4 *>(Vh + (size_t)key * D + col);
        *reinterpret_cast<uint4 *>(tile + j * D + col) = x;
    }
    __syncthreads();
    uint8_t *out = Vt + ((size_t)bh * nkt + t) * (size_t)(D * 64);
    for (int c = threadIdx.x; c < D * 4; c += 256) {
        const int row = c / 4, seg = c % 4;  // output bytes 16 seg .. 16 seg + 15 of row `row`
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // output position p = 16 seg + 4 q + e -> key
                const int p = 16 * seg + 4 * q + e;
                const int h = p / 32, b = p % 32;
                const int j = 32 * (b / 16) + 8 * ((b % 16) / 4) + 4 * h + b % 4;
                v |= (uint32_t)tile[j * D + row] << (8 * e);
            }
            w[q] = v;
        }
        *reinterpret_cast<uint4 *>(out + row * 64 + 16 * seg) = uint4{w[0], w[1], w[2], w[3]};
    }
}

struct Fp8Params {
    const uint8_t *Q, *K, *Vt;
    uint16_t *O;
    float *LSE;
    int N, nqb, nkt, items, per_xcd;
    float c;      // scale * q_descale * k_descale * log2(e)
    float o_mul;  // v_descale
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_fp8_kernel(Fp8Params p)
{
    constexpr int W = 8, RW = 32, BR = RW * W, BC = 64;
    constexpr int KK = D / 64;   // MFMAs per 32-key S block
    constexpr int DB = D / 32;   // 32-column blocks of O^T
    constexpr int KCH = D / 16;  // 16-byte chunks per K row
    constexpr uint32_t TB = 64 * D;   // bytes of a K tile, and of a V^T tile
    constexpr int NBLK = TB / 1024;   // 1 KB direct loads per tile
    __shared__ __attribute__((aligned(1024))) unsigned char smem[6 * TB];  // K0 K1 K2 V0 V1 V2
    const uint32_t lds0 = lds_byte_addr(smem);

    const int item = xcd_work_item(p.per_xcd);
    if (item >= p.items)
        return;
    const int bh = item / p.nqb;
    const int qi = item - bh * p.nqb;
    const int qblk = CAUSAL ? (p.nqb - 1 - qi) : qi;
    const int q0 = qblk * BR;
    const int N = p.N;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane % 32, hi = lane / 32;
    const int wr0 = q0 + wave * RW;
    const int row = wr0 + l32;

    const uint8_t *Qh = p.Q + (size_t)bh * N * D;
    const uint8_t *Kh = p.K + (size_t)bh * N * D;
    const uint8_t *Vth = p.Vt + (size_t)bh * p.nkt * TB;

    // Q^T operands: bytes 64 kk + 32 hi .. +31 of this lane's query row
    i32x8 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        uint4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
        if (row < N) {
            const uint8_t *src = Qh + (size_t)row * D + 64 * kk + 32 * hi;
            a = *reinterpret_cast<const uint4 *>(src);
            b = *reinterpret_cast<const uint4 *>(src + 16);
        }
        qf[kk] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }

    // swizzles: K rows (D bytes) and V^T rows (64 bytes)
    auto k_swz = [](int r) -> int { return KCH == 8 ? (r / 2) % 8 : (r / 4) % 4; };
    auto v_swz = [](int r) -> int { return (r / 4) % 4; };
    auto k_read = [&](uint32_t buf, int r, int c) __attribute__((always_inline)) -> uint4 {
        const uint32_t a = buf + r * D + 16 * (c ^ k_swz(r));
        const bf16x8 x = lds_b128_at(a);
        return __builtin_bit_cast(uint4, x);
    };
    auto v_read = [&](uint32_t buf, int r, int c) __attribute__((always_inline)) -> uint4 {
        const uint32_t a = buf + r * 64 + 16 * (c ^ v_swz(r));
        const bf16x8 x = lds_b128_at(a);
        return __builtin_bit_cast(uint4, x);
    };
    // Tile t's K and V^T go to buffers t % 3; per wave the K loads are
    // issued before the V^T loads, so that waiting for all but the last
    // LPV loads leaves only V^T in flight.
    auto issue = [&](int t, int slot) __attribute__((always_inline)) {
        const uint32_t kbuf = lds0 + slot * TB, vbuf = lds0 + (3 + slot) * TB;
        const i32x4 rk = buffer_rsrc(Kh + (size_t)t * BC * D, (uint32_t)(N - t * BC) * D);
        const i32x4 rv = buffer_rsrc(Vth + (size_t)t * TB, TB);
        for (int b = wave; b < NBLK; b += W) {
            const int kr = b * (1024 / D) + lane / KCH, kc = (lane % KCH) ^ k_swz(kr);
            lds_dma_buf_b128(rk, kr * D + 16 * kc, kbuf + b * 1024);
        }
        for (int b = wave; b < NBLK; b += W) {
            const int vr = b * 16 + lane / 4, vc = (lane % 4) ^ v_swz(vr);
            lds_dma_buf_b128(rv, vr * 64 + 16 * vc, vbuf + b * 1024);
        }
    };
    static_assert(NBLK <= W, "one K and one V^T load per wave and tile at most");
    // S^T of tile t's two 32-key blocks (K in buffer `slot`)
    auto qk = [&](int slot, f32x16 (&sv)[2]) __attribute__((always_inline)) {
        const uint32_t kbuf = lds0 + slot * TB;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sv[blk] = f32x16{};
            const int r = 32 * blk + l32;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint4 a = k_read(kbuf, r, 4 * kk + 2 * hi);
                const uint4 b = k_read(kbuf, r, 4 * kk + 2 * hi + 1);
                const i32x8 ka = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
                sv[blk] = mfma_fp8(ka, qf[kk], sv[blk]);
            }
        }
    };

    int t_end = p.nkt;
    if (CAUSAL)
        t_end = min(p.nkt, (q0 + BR - 1) / BC + 1);

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        o[db] = f32x16{};
    float m = -INFINITY, l = 0.f, nmref = 0.f;
    const float c = p.c;

    // Software pipeline: iteration t issues the loads of tile t+2, the S^T
    // MFMAs of tile t+1 (their results are used one iteration later, so the
    // matrix pipe works beside this tile's softmax), then tile t's softmax
    // and P V.
    issue(0, 0);
    if (t_end > 1)
        issue(1, 1);
    lds_dma_wait<0>();
    __syncthreads();
    f32x16 s[2], s_nxt[2];
    qk(0, s);
    for (int t = 0; t < t_end; ++t) {
        const int slot = t % 3;
        // tile t+2 into the buffers of tile t-1, free since the last barrier
        // (without a tile t+2 tile t is loaded again: no branch, so that the
        // MFMAs below stay in the block of the softmax)
        issue(t + 2 < t_end ? t + 2 : t, (t + 2) % 3);
        const uint32_t vbuf = lds0 + (3 + slot) * TB;
        // keys past the end, above the diagonal (causal)
        const int kb = t * BC;
        if (kb + BC > N || (CAUSAL && kb + BC - 1 > wr0)) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 32 * blk + 8 * (r / 4) + 4 * hi + (r % 4);
                    if (key >= N || (CAUSAL && key > row))
                        s[blk][r] = -INFINITY;
                }
        }
        // row max: one asm max chain per 32-key block, starting at s[0][0]
        // and s[1][0] (two MFMA accumulators), which pass through a
        // compiler-visible add first
        mfma_result_touch(s[0], 0);
        mfma_result_touch(s[1], 0);
        float ma = vmax3(s[0][0], s[0][1], s[0][2]);
        float mb = vmax3(s[1][0], s[1][1], s[1][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
            ma = vmax3(ma, s[0][r], s[0][r + 1]);
            mb = vmax3(mb, s[1][r], s[1][r + 1]);
        }
        ma = vmax2(ma, s[0][15]);
        mb = vmax2(mb, s[1][15]);
        const float mx = halves_max(vmax2(ma, mb)) * c;
        // The reference follows the row max exactly (no slack): every weight
        // is <= 1 and the one that sets a new max is exactly 1 in E4M3.
        if (__any(mx > m)) {
            const float mnew = fmaxf(m, mx);
            const float alpha = (m == -INFINITY) ? 0.f : exp2_fast(m - mnew);
            m = mnew;
            nmref = (m == -INFINITY) ? 0.f : -m;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o[db][r] *= alpha;
        }
        // The next tile's S^T MFMAs (on the last tile a stale buffer is read
        // and the result unused) in the same block as this tile's softmax,
        // so that the scheduler interleaves them.
        qk((t + 1) % 3, s_nxt);
        // P = 2^(c s - m) <= 1 in fp32 for the row sum, E4M3 for P V
        i32x8 pp;
        float ls = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[i] = exp2_fast(fmaf(s[blk][4 * w + i], c, nmref));
                    ls += e[i];
                }
                int v = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
                v = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], v, true);
                pp[4 * blk + w] = v;
            }
        l += ls;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int r = 32 * db + l32;
            const uint4 a = v_read(vbuf, r, 2 * hi);
            const uint4 b = v_read(vbuf, r, 2 * hi + 1);
            const i32x8 va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
            o[db] = mfma_fp8(va, pp, o[db]);
        }
        slot_done(l);  // the row sum in this block, not sunk past the wait below
        // Tile t+1's V^T and tile t+2's K have landed (the next iteration
        // computes tile t+2's S^T), tile t+2's V^T may still be in flight;
        // the barrier extends that to all waves and frees tile t's buffers.
        lds_dma_wait<1>();
        __syncthreads();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
            s[blk] = s_nxt[blk];
    }

    lds_dma_wait<0>();  // the last (repeated) tile load has landed: none outlives the workgroup
    const float lt = halves_sum(l);
    if (row < N) {
        const float inv = lt > 0.f ? p.o_mul / lt : 0.f;
        uint16_t *Oh = p.O + ((size_t)bh * N + row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
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

template <int D>
hipError_t fp8_d(const Fp8Problem &pr, const uint8_t *Q, const uint8_t *K, const uint8_t *V,
                 uint16_t *O, float *LSE, void *ws)
{
    const int nkt = (pr.N + 63) / 64;
    uint8_t *Vt = static_cast<uint8_t *>(ws);
    hipLaunchKernelGGL((fp8_vt_kernel<D>), dim3((unsigned)nkt, (unsigned)(pr.B * pr.H)), dim3(256), 0,
                       pr.stream, V, Vt, pr.N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    Fp8Params fp{};
    fp.Q = Q;
    fp.K = K;
    fp.Vt = Vt;
    fp.O = O;
    fp.LSE = LSE;
    fp.N = pr.N;
    fp.nqb = (pr.N + 255) / 256;
    fp.nkt = nkt;
    fp.items = pr.B * pr.H * fp.nqb;
    fp.per_xcd = (fp.items + kXcds - 1) / kXcds;
    fp.c = pr.scale * pr.q_descale * pr.k_descale * kLog2e;
    fp.o_mul = pr.v_descale;
    const unsigned grid = (unsigned)(fp.per_xcd * kXcds);
    if (pr.causal)
        hipLaunchKernelGGL((fwd_fp8_kernel<D, true>), dim3(grid), dim3(512), 0, pr.stream, fp);
    else
        hipLaunchKernelGGL((fwd_fp8_kernel<D, false>), dim3(grid), dim3(512), 0, pr.stream, fp);
    return hipGetLastError();
}

}  // namespace

size_t fp8_workspace_bytes(int B, int H, int N, int d)
{
    const size_t nkt = ((size_t)N + 63) / 64;
    return ((size_t)B * H * nkt * 64 * (size_t)d + 255) / 256 * 256;
}

hipError_t launch_fwd_fp8(const Fp8Problem &pr, const uint8_t *Q, const uint8_t *K,
                          const uint8_t *V, uint16_t *O, float *LSE, void *workspace)
{
    if (pr.d == 64)
        return fp8_d<64>(pr, Q, K, V, O, LSE, workspace);
    return fp8_d<128>(pr, Q, K, V, O, LSE, workspace);
}

}  // namespace fa
