// fp32 debug path: the same tiled online-softmax forward and recompute
// backward as the bf16 path, in plain fp32 vector arithmetic (no MFMA, no
// bf16 rounding anywhere), so that a disagreement with the reference can be
// told apart from bf16 rounding. One thread owns one query row (forward,
// dQ) or one key row (dK, dV); key/query tiles are staged in LDS and read by
// broadcast. (The element type of the backward kernels is a template
// parameter; only fp32 storage is instantiated.) Head dims below the compiled width (64, 128 or 256) are
// zero-padded on load and not stored. (At 256 a thread's row vectors exceed
// the register file and live partly in scratch memory: slow, still exact
// fp32.)
//
// Forward: mstx.cn/posts/485 §三.2 "Online Softmax" update rule (base 2,
// c = scale * log2 e), O divided by l once at the end.
// Backward: P rebuilt from the saved LSE (lukebest.github.io FlashAttention,
// "反向：重算而非存储"), then dV = P^T dO, dP = dO V^T,
// dS = P o (dP - D) with D_i = rowsum(dO o O), dQ = scale dS K,
// dK = scale dS^T Q. (The gradient formula printed in cloud.baidu.com
// §工作原理 "梯度计算优化" is garbled; this is the softmax Jacobian rule.)
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kT = 64;  // rows per LDS tile and threads per workgroup

// Element access of the backward kernels, which also serve bf16 tensors
// (uint16 bit patterns: widened exactly to fp32 on load, rounded to nearest
// even on store).
__device__ __forceinline__ float ldf(const float *p) { return *p; }
__device__ __forceinline__ float ldf(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void stf(float *p, float x) { *p = x; }
__device__ __forceinline__ void stf(uint16_t *p, float x) { *p = f32_to_bf16_bits(x); }

__device__ __forceinline__ bool visible(int i, int j, bool causal, const uint8_t *mask, int nmb)
{
    if (causal && j > i)
        return false;
    if (mask && mask[(size_t)(i / kMaskBlock) * nmb + (j / kMaskBlock)] == 0)
        return false;
    return true;
}

template <int D>
__global__ void __launch_bounds__(kT) fwd_f32_kernel(const float *Q, const float *K, const float *V,
                                                     float *O, float *LSE, int N, int dh, float c,
                                                     int causal, const uint8_t *mask, int nmb)
{
    __shared__ float Ks[kT][D];
    __shared__ float Vs[kT][D];
    const int bh = blockIdx.y;
    const int row = blockIdx.x * kT + threadIdx.x;
    const size_t head = (size_t)bh * N * dh;
    float q[D], o[D];
    for (int x = 0; x < D; ++x) {
        q[x] = row < N && x < dh ? Q[head + (size_t)row * dh + x] : 0.f;
        o[x] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int kend = causal ? min(N, (int)(blockIdx.x + 1) * kT) : N;
    for (int k0 = 0; k0 < kend; k0 += kT) {
        __syncthreads();
        for (int e = threadIdx.x; e < kT * D; e += kT) {
            const int r = e / D, x = e % D;
            const bool in = k0 + r < N && x < dh;
            Ks[r][x] = in ? K[head + (size_t)(k0 + r) * dh + x] : 0.f;
            Vs[r][x] = in ? V[head + (size_t)(k0 + r) * dh + x] : 0.f;
        }
        __syncthreads();
        if (row >= N)
            continue;
        float s[kT];
        float mx = -INFINITY;
        for (int j = 0; j < kT; ++j) {
            const int key = k0 + j;
            float acc = 0.f;
            for (int x = 0; x < D; ++x)
                acc = fmaf(q[x], Ks[j][x], acc);
            s[j] = (key < N && visible(row, key, causal, mask, nmb)) ? acc * c : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        const float mnew = fmaxf(m, mx);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = exp2f(m - mref);
        m = mnew;
        l *= alpha;
        for (int x = 0; x < D; ++x)
            o[x] *= alpha;
        for (int j = 0; j < kT; ++j) {
            const float e = exp2f(s[j] - mref);
            l += e;
            for (int x = 0; x < D; ++x)
                o[x] = fmaf(e, Vs[j][x], o[x]);
        }
    }
    if (row < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        for (int x = 0; x < dh; ++x)
            O[head + (size_t)row * dh + x] = o[x] * inv;
        LSE[(size_t)bh * N + row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    }
}

// D_i = rowsum(dO o O) and LSE in base 2 (+inf for a row without visible
// keys, so that 2^(c s - lse2) = 0 there).
template <typename T, int D>
__global__ void __launch_bounds__(kT) bwd_pre_f32_kernel(const T *dO, const T *O,
                                                         const float *LSE, float *delta,
                                                         float *lse2, int N, int dh)
{
    const int bh = blockIdx.y;
    const int row = blockIdx.x * kT + threadIdx.x;
    if (row >= N)
        return;
    const size_t base = ((size_t)bh * N + row) * dh;
    float acc = 0.f;
    for (int x = 0; x < dh; ++x)
        acc = fmaf(ldf(dO + base + x), ldf(O + base + x), acc);
    const size_t r = (size_t)bh * N + row;
    delta[r] = acc;
    const float L = LSE[r];
    lse2[r] = L == -INFINITY ? INFINITY : L * kLog2e;
}

// dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j, one thread per query row.
template <typename T, int D>
__global__ void __launch_bounds__(kT) bwd_dq_f32_kernel(const T *dO, const T *Q,
                                                        const T *K, const T *V,
                                                        const float *delta, const float *lse2,
                                                        T *dQ, int N, int dh, float scale, float c,
                                                        int causal, const uint8_t *mask, int nmb)
{
    __shared__ float Ks[kT][D];
    __shared__ float Vs[kT][D];
    const int bh = blockIdx.y;
    const int row = blockIdx.x * kT + threadIdx.x;
    const size_t head = (size_t)bh * N * dh;
    float q[D], go[D], dq[D];
    for (int x = 0; x < D; ++x) {
        q[x] = row < N && x < dh ? ldf(Q + head + (size_t)row * dh + x) : 0.f;
        go[x] = row < N && x < dh ? ldf(dO + head + (size_t)row * dh + x) : 0.f;
        dq[x] = 0.f;
    }
    const float Di = row < N ? delta[(size_t)bh * N + row] : 0.f;
    const float Li = row < N ? lse2[(size_t)bh * N + row] : INFINITY;
    const int kend = causal ? min(N, (int)(blockIdx.x + 1) * kT) : N;
    for (int k0 = 0; k0 < kend; k0 += kT) {
        __syncthreads();
        for (int e = threadIdx.x; e < kT * D; e += kT) {
            const int r = e / D, x = e % D;
            const bool in = k0 + r < N && x < dh;
            Ks[r][x] = in ? ldf(K + head + (size_t)(k0 + r) * dh + x) : 0.f;
            Vs[r][x] = in ? ldf(V + head + (size_t)(k0 + r) * dh + x) : 0.f;
        }
        __syncthreads();
        if (row >= N)
            continue;
        for (int j = 0; j < kT; ++j) {
            const int key = k0 + j;
            if (key >= N || !visible(row, key, causal, mask, nmb))
                continue;
            float s = 0.f, dp = 0.f;
            for (int x = 0; x < D; ++x) {
                s = fmaf(q[x], Ks[j][x], s);
                dp = fmaf(go[x], Vs[j][x], dp);
            }
            const float pij = exp2f(s * c - Li);
            const float ds = pij * (dp - Di);
            for (int x = 0; x < D; ++x)
                dq[x] = fmaf(ds, Ks[j][x], dq[x]);
        }
    }
    if (row < N)
        for (int x = 0; x < dh; ++x)
            stf(dQ + head + (size_t)row * dh + x, dq[x] * scale);
}

// One thread per key row. WANT_DK: dK_j = scale * sum_i dS_ij Q_i;
// otherwise dV_j = sum_i P_ij dO_i.
template <typename T, int D, bool WANT_DK>
__global__ void __launch_bounds__(kT) bwd_dkv_f32_kernel(const T *dO, const T *Q,
                                                         const T *K, const T *V,
                                                         const float *delta, const float *lse2,
                                                         T *dOut, int N, int dh, float scale, float c,
                                                         int causal, const uint8_t *mask, int nmb)
{
    __shared__ float Qs[kT][D];
    __shared__ float Gs[kT][D];
    __shared__ float Ls[kT], Ds[kT];
    const int bh = blockIdx.y;
    const int key = blockIdx.x * kT + threadIdx.x;
    const size_t head = (size_t)bh * N * dh;
    float k[D], v[D], acc[D];
    for (int x = 0; x < D; ++x) {
        k[x] = key < N && x < dh ? ldf(K + head + (size_t)key * dh + x) : 0.f;
        v[x] = (WANT_DK && key < N && x < dh) ? ldf(V + head + (size_t)key * dh + x) : 0.f;
        acc[x] = 0.f;
    }
    const int qstart = causal ? (int)blockIdx.x * kT : 0;
    for (int q0 = qstart; q0 < N; q0 += kT) {
        __syncthreads();
        for (int e = threadIdx.x; e < kT * D; e += kT) {
            const int r = e / D, x = e % D;
            const bool in = q0 + r < N && x < dh;
            Qs[r][x] = in ? ldf(Q + head + (size_t)(q0 + r) * dh + x) : 0.f;
            Gs[r][x] = in ? ldf(dO + head + (size_t)(q0 + r) * dh + x) : 0.f;
        }
        {
            const int r = threadIdx.x;
            const bool in = q0 + r < N;
            Ls[r] = in ? lse2[(size_t)bh * N + q0 + r] : INFINITY;
            Ds[r] = in ? delta[(size_t)bh * N + q0 + r] : 0.f;
        }
        __syncthreads();
        if (key >= N)
            continue;
        for (int i = 0; i < kT; ++i) {
            const int row = q0 + i;
            if (row >= N || !visible(row, key, causal, mask, nmb))
                continue;
            float s = 0.f;
            for (int x = 0; x < D; ++x)
                s = fmaf(Qs[i][x], k[x], s);
            const float pij = exp2f(s * c - Ls[i]);
            if (WANT_DK) {
                float dp = 0.f;
                for (int x = 0; x < D; ++x)
                    dp = fmaf(Gs[i][x], v[x], dp);
                const float ds = pij * (dp - Ds[i]);
                for (int x = 0; x < D; ++x)
                    acc[x] = fmaf(ds, Qs[i][x], acc[x]);
            } else {
                for (int x = 0; x < D; ++x)
                    acc[x] = fmaf(pij, Gs[i][x], acc[x]);
            }
        }
    }
    if (key < N)
        for (int x = 0; x < dh; ++x)
            stf(dOut + head + (size_t)key * dh + x, WANT_DK ? acc[x] * scale : acc[x]);
}

template <int D>
hipError_t fwd_f32_d(const Problem &p, const float *Q, const float *K, const float *V, float *O,
                     float *LSE)
{
    const dim3 grid((p.N + kT - 1) / kT, p.B * p.H);
    const int nmb = (p.N + kMaskBlock - 1) / kMaskBlock;
    hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, dim3(kT), 0, p.stream, Q, K, V, O, LSE, p.N,
                       p.d, p.scale * kLog2e, p.causal, p.mask, nmb);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_f32_d(const Problem &p, const T *dO, const T *Q, const T *K, const T *V,
                     const T *O, const float *LSE, T *dQ, T *dK, T *dV, void *ws)
{
    const BwdWorkspace L = bwd_workspace_layout(p.B, p.H, p.N, p.d);
    float *delta = reinterpret_cast<float *>(static_cast<char *>(ws) + L.delta_off);
    float *lse2 = reinterpret_cast<float *>(static_cast<char *>(ws) + L.lse2_off);
    const dim3 grid((p.N + kT - 1) / kT, p.B * p.H);
    const int nmb = (p.N + kMaskBlock - 1) / kMaskBlock;
    const float c = p.scale * kLog2e;
    hipLaunchKernelGGL((bwd_pre_f32_kernel<T, D>), grid, dim3(kT), 0, p.stream, dO, O, LSE, delta,
                       lse2, p.N, p.d);
    hipLaunchKernelGGL((bwd_dq_f32_kernel<T, D>), grid, dim3(kT), 0, p.stream, dO, Q, K, V, delta,
                       lse2, dQ, p.N, p.d, p.scale, c, p.causal, p.mask, nmb);
    hipLaunchKernelGGL((bwd_dkv_f32_kernel<T, D, true>), grid, dim3(kT), 0, p.stream, dO, Q, K, V,
                       delta, lse2, dK, p.N, p.d, p.scale, c, p.causal, p.mask, nmb);
    hipLaunchKernelGGL((bwd_dkv_f32_kernel<T, D, false>), grid, dim3(kT), 0, p.stream, dO, Q, K, V,
                       delta, lse2, dV, p.N, p.d, p.scale, c, p.causal, p.mask, nmb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const Problem &p, const float *Q, const float *K, const float *V,
                          float *O, float *LSE)
{
    if (p.d <= 64)
        return fwd_f32_d<64>(p, Q, K, V, O, LSE);
    if (p.d <= 128)
        return fwd_f32_d<128>(p, Q, K, V, O, LSE);
    return fwd_f32_d<256>(p, Q, K, V, O, LSE);
}

hipError_t launch_bwd_f32(const Problem &p, const float *dO, const float *Q, const float *K,
                          const float *V, const float *O, const float *LSE, float *dQ,
                          float *dK, float *dV, void *ws)
{
    if (p.d <= 64)
        return bwd_f32_d<float, 64>(p, dO, Q, K, V, O, LSE, dQ, dK, dV, ws);
    if (p.d <= 128)
        return bwd_f32_d<float, 128>(p, dO, Q, K, V, O, LSE, dQ, dK, dV, ws);
    return bwd_f32_d<float, 256>(p, dO, Q, K, V, O, LSE, dQ, dK, dV, ws);
}


}  // namespace fa
