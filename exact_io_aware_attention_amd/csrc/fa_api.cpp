// C ABI of the attention library: argument validation, dispatch to the
// kernel launchers, status codes. No exception crosses this boundary and no
// device memory is allocated here.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

thread_local char g_last_hip_error[256] = "";

fa_status hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return FA_OK;
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s (%d): %s",
                  hipGetErrorName(e), (int)e, hipGetErrorString(e));
    return FA_ERR_HIP;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Head dims: multiples of 8 up to 128 everywhere, up to 256 in the plain
// forward and backward, the decode path and the fp32 path.
constexpr int kMaxD = 128;
constexpr int kMaxDWide = 256;

// Checks common to every entry point, in a fixed order. *empty is set when
// the problem has no elements (then nothing is launched).
fa_status check_common(int B, int H, int N, int d, float scale, int causal, bool *empty,
                       int max_d = kMaxD)
{
    if (B < 0 || H < 0 || N < 0)
        return FA_ERR_SHAPE;
    if (d < 8 || d > max_d || d % 8 != 0)
        return FA_ERR_HEADDIM;
    if (!std::isfinite(scale) || !(scale > 0.f) || (causal != 0 && causal != 1))
        return FA_ERR_SCALE;
    // every element index of a [B][H][N][d] tensor must fit in 63 bits and a
    // per-head slab in 30 bits of elements (2^31 bytes of bf16: buffer
    // offsets from 2^31 on are then out of range for every tile load)
    const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
    const unsigned long long head = (unsigned long long)N * (unsigned long long)d;
    if (head >= (1ull << 30))
        return FA_ERR_SHAPE;
    if (bh > 0 && head > 0 && bh > (unsigned long long)std::numeric_limits<long long>::max() / head)
        return FA_ERR_SHAPE;
    // work items per launch (B*H*ceil(N/64)) must fit in an int
    if (bh * (((unsigned long long)N + 63) / 64) > (unsigned long long)std::numeric_limits<int>::max() / 2)
        return FA_ERR_SHAPE;
    *empty = (B == 0 || H == 0 || N == 0);
    return FA_OK;
}

fa_status check_ptrs(std::initializer_list<const void *> ptrs)
{
    for (const void *p : ptrs)
        if (p == nullptr)
            return FA_ERR_NULL;
    for (const void *p : ptrs)
        if (!aligned16(p))
            return FA_ERR_ALIGN;
    return FA_OK;
}

fa::Problem make_problem(int B, int H, int N, int d, float scale, int causal,
                         const uint8_t *mask, void *stream)
{
    fa::Problem p;
    p.B = B;
    p.H = H;
    p.N = N;
    p.d = d;
    p.scale = scale;
    p.causal = causal;
    p.mask = mask;
    p.stream = static_cast<hipStream_t>(stream);
    return p;
}

// Dropout probability: finite, in [0, 1). Sets the problem's dropout fields
// (threshold floor(p 2^32), seed, 1 / (1 - p)).
fa_status set_dropout(fa::Problem &p, float p_drop, unsigned long long seed)
{
    if (!std::isfinite(p_drop) || p_drop < 0.f || p_drop >= 1.f)
        return FA_ERR_SCALE;
    if (p_drop > 0.f) {
        const double t = std::floor((double)p_drop * 4294967296.0);
        p.dropout = 1;
        p.drop_threshold = t >= 4294967295.0 ? 4294967295u : (uint32_t)t;
        p.drop_seed = seed;
        p.drop_inv_keep = (float)(1.0 / (1.0 - (double)p_drop));
    }
    return FA_OK;
}

template <typename T>
fa_status fwd_common(const T *Q, const T *K, const T *V, T *O, float *LSE, int B, int H, int N,
                     int d, float scale, int causal, const uint8_t *blockmask, void *stream,
                     bool f32, int max_d, float p_drop = 0.f, unsigned long long seed = 0)
{
    bool empty = false;
    fa_status st = check_common(B, H, N, d, scale, causal, &empty, max_d);
    if (st != FA_OK)
        return st;
    fa::Problem p = make_problem(B, H, N, d, scale, causal, blockmask, stream);
    st = set_dropout(p, p_drop, seed);
    if (st != FA_OK)
        return st;
    if (empty)
        return FA_OK;
    st = check_ptrs({Q, K, V, O, LSE});
    if (st != FA_OK)
        return st;
    if (f32)
        return hip_status(fa::launch_fwd_f32(p, reinterpret_cast<const float *>(Q),
                                             reinterpret_cast<const float *>(K),
                                             reinterpret_cast<const float *>(V),
                                             reinterpret_cast<float *>(O), LSE));
    return hip_status(fa::launch_fwd_bf16(p, reinterpret_cast<const uint16_t *>(Q),
                                          reinterpret_cast<const uint16_t *>(K),
                                          reinterpret_cast<const uint16_t *>(V),
                                          reinterpret_cast<uint16_t *>(O), LSE));
}

fa_status check_workspace(int B, int H, int N, int d, const void *workspace, size_t bytes);

template <typename T>
fa_status bwd_common(const T *dO, const T *Q, const T *K, const T *V, const T *O,
                     const float *LSE, T *dQ, T *dK, T *dV, int B, int H, int N, int d,
                     float scale, int causal, const uint8_t *blockmask, void *workspace,
                     size_t workspace_bytes, void *stream, bool f32, int max_d, float p_drop = 0.f,
                     unsigned long long seed = 0)
{
    bool empty = false;
    fa_status st = check_common(B, H, N, d, scale, causal, &empty, max_d);
    if (st != FA_OK)
        return st;
    fa::Problem p = make_problem(B, H, N, d, scale, causal, blockmask, stream);
    st = set_dropout(p, p_drop, seed);
    if (st != FA_OK)
        return st;
    if (empty)
        return FA_OK;
    st = check_ptrs({dO, Q, K, V, O, LSE, dQ, dK, dV});
    if (st != FA_OK)
        return st;
    st = check_workspace(B, H, N, d, workspace, workspace_bytes);
    if (st != FA_OK)
        return st;
    if (f32)
        return hip_status(fa::launch_bwd_f32(
            p, reinterpret_cast<const float *>(dO), reinterpret_cast<const float *>(Q),
            reinterpret_cast<const float *>(K), reinterpret_cast<const float *>(V),
            reinterpret_cast<const float *>(O), LSE, reinterpret_cast<float *>(dQ),
            reinterpret_cast<float *>(dK), reinterpret_cast<float *>(dV), workspace));
    return hip_status(fa::launch_bwd_bf16(
        p, reinterpret_cast<const uint16_t *>(dO), reinterpret_cast<const uint16_t *>(Q),
        reinterpret_cast<const uint16_t *>(K), reinterpret_cast<const uint16_t *>(V),
        reinterpret_cast<const uint16_t *>(O), LSE, reinterpret_cast<uint16_t *>(dQ),
        reinterpret_cast<uint16_t *>(dK), reinterpret_cast<uint16_t *>(dV), workspace));
}

fa_status check_workspace(int B, int H, int N, int d, const void *workspace, size_t bytes)
{
    const fa::BwdWorkspace L = fa::bwd_workspace_layout(B, H, N, d);
    if (workspace == nullptr || bytes < L.bytes ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return FA_ERR_WORKSPACE;
    return FA_OK;
}

// Validation shared by the backward phase entry points; *empty as above.
fa_status bwd_phase_checks(int B, int H, int N, int d, float scale, int causal,
                           std::initializer_list<const void *> ptrs, const void *workspace,
                           size_t workspace_bytes, bool *empty)
{
    fa_status st = check_common(B, H, N, d, scale, causal, empty);
    if (st != FA_OK || *empty)
        return st;
    st = check_ptrs(ptrs);
    if (st != FA_OK)
        return st;
    return check_workspace(B, H, N, d, workspace, workspace_bytes);
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H,
                 int N, int d, float scale, int causal, const uint8_t *blockmask, void *stream)
{
    return fwd_common<uint16_t>(static_cast<const uint16_t *>(Q), static_cast<const uint16_t *>(K),
                                static_cast<const uint16_t *>(V), static_cast<uint16_t *>(O), LSE,
                                B, H, N, d, scale, causal, blockmask, stream, false, kMaxDWide);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d)
{
    if (B <= 0 || H <= 0 || N <= 0)
        return 0;
    return fa::bwd_workspace_layout(B, H, N, d).bytes;
}

fa_status fa_bwd(const void *dO, const void *Q, const void *K, const void *V, const void *O,
                 const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int N, int d,
                 float scale, int causal, const uint8_t *blockmask, void *workspace,
                 size_t workspace_bytes, void *stream)
{
    return bwd_common<uint16_t>(
        static_cast<const uint16_t *>(dO), static_cast<const uint16_t *>(Q),
        static_cast<const uint16_t *>(K), static_cast<const uint16_t *>(V),
        static_cast<const uint16_t *>(O), LSE, static_cast<uint16_t *>(dQ),
        static_cast<uint16_t *>(dK), static_cast<uint16_t *>(dV), B, H, N, d, scale, causal,
        blockmask, workspace, workspace_bytes, stream, false, kMaxDWide);
}

fa_status fa_bwd_noalloc(const void *dO, const void *Q, const void *K, const void *V,
                         const void *O, const float *LSE, void *dQ, void *dK, void *dV, int B,
                         int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                         void *stream)
{
    bool empty = false;
    fa_status st = check_common(B, H, N, d, scale, causal, &empty, kMaxDWide);
    if (st != FA_OK || empty)
        return st;
    st = check_ptrs({dO, Q, K, V, O, LSE, dQ, dK, dV});
    if (st != FA_OK)
        return st;
    const size_t need = fa::bwd_workspace_layout(B, H, N, d).bytes;
    if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_SCRATCH;
    void *scratch = nullptr;
    st = hip_status(fa::noalloc_scratch(need, &scratch));
    if (st != FA_OK)
        return st;
    const fa::Problem p = make_problem(B, H, N, d, scale, causal, blockmask, stream);
    return hip_status(fa::launch_bwd_bf16(
        p, static_cast<const uint16_t *>(dO), static_cast<const uint16_t *>(Q),
        static_cast<const uint16_t *>(K), static_cast<const uint16_t *>(V),
        static_cast<const uint16_t *>(O), LSE, static_cast<uint16_t *>(dQ),
        static_cast<uint16_t *>(dK), static_cast<uint16_t *>(dV), scratch));
}

fa_status fa_bwd_prep(const void *dO, const void *O, const float *LSE, int B, int H, int N, int d,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    bool empty = false;
    fa_status st = bwd_phase_checks(B, H, N, d, 1.f, 0, {dO, O, LSE}, workspace, workspace_bytes,
                                    &empty);
    if (st != FA_OK || empty)
        return st;
    const fa::Problem p = make_problem(B, H, N, d, 1.f, 0, nullptr, stream);
    return hip_status(fa::launch_bwd_prep_bf16(p, static_cast<const uint16_t *>(dO),
                                               static_cast<const uint16_t *>(O), LSE, workspace));
}

fa_status fa_bwd_dq(const void *dO, const void *Q, const void *K, const void *V, void *dQ, int B,
                    int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                    const void *workspace, size_t workspace_bytes, void *stream)
{
    bool empty = false;
    fa_status st = bwd_phase_checks(B, H, N, d, scale, causal, {dO, Q, K, V, dQ}, workspace,
                                    workspace_bytes, &empty);
    if (st != FA_OK || empty)
        return st;
    const fa::Problem p = make_problem(B, H, N, d, scale, causal, blockmask, stream);
    return hip_status(fa::launch_bwd_dq_bf16(
        p, static_cast<const uint16_t *>(dO), static_cast<const uint16_t *>(Q),
        static_cast<const uint16_t *>(K), static_cast<const uint16_t *>(V),
        static_cast<uint16_t *>(dQ), workspace));
}

fa_status fa_bwd_dkdv(const void *dO, const void *Q, const void *K, const void *V, void *dK,
                      void *dV, int B, int H, int N, int d, float scale, int causal,
                      const uint8_t *blockmask, const void *workspace, size_t workspace_bytes,
                      void *stream)
{
    bool empty = false;
    fa_status st = bwd_phase_checks(B, H, N, d, scale, causal, {dO, Q, K, V, dK, dV}, workspace,
                                    workspace_bytes, &empty);
    if (st != FA_OK || empty)
        return st;
    const fa::Problem p = make_problem(B, H, N, d, scale, causal, blockmask, stream);
    return hip_status(fa::launch_bwd_dkdv_bf16(
        p, static_cast<const uint16_t *>(dO), static_cast<const uint16_t *>(Q),
        static_cast<const uint16_t *>(K), static_cast<const uint16_t *>(V),
        static_cast<uint16_t *>(dK), static_cast<uint16_t *>(dV), workspace));
}

fa_status fa_fwd_dropout(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                         int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                         float p_drop, unsigned long long seed, void *stream)
{
    return fwd_common<uint16_t>(static_cast<const uint16_t *>(Q), static_cast<const uint16_t *>(K),
                                static_cast<const uint16_t *>(V), static_cast<uint16_t *>(O), LSE,
                                B, H, N, d, scale, causal, blockmask, stream, false, kMaxD, p_drop,
                                seed);
}

fa_status fa_bwd_dropout(const void *dO, const void *Q, const void *K, const void *V,
                         const void *O, const float *LSE, void *dQ, void *dK, void *dV, int B,
                         int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                         float p_drop, unsigned long long seed, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    return bwd_common<uint16_t>(
        static_cast<const uint16_t *>(dO), static_cast<const uint16_t *>(Q),
        static_cast<const uint16_t *>(K), static_cast<const uint16_t *>(V),
        static_cast<const uint16_t *>(O), LSE, static_cast<uint16_t *>(dQ),
        static_cast<uint16_t *>(dK), static_cast<uint16_t *>(dV), B, H, N, d, scale, causal,
        blockmask, workspace, workspace_bytes, stream, false, kMaxD, p_drop, seed);
}

size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N, int d)
{
    if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128))
        return 0;
    return fa::fp8_workspace_bytes(B, H, N, d);
}

fa_status fa_fwd_fp8(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                     int H, int N, int d, float scale, float q_descale, float k_descale,
                     float v_descale, int causal, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    bool empty = false;
    fa_status st = check_common(B, H, N, d, scale, causal, &empty);
    if (st != FA_OK)
        return st;
    if (d != 64 && d != 128)
        return FA_ERR_HEADDIM;
    for (float s : {q_descale, k_descale, v_descale})
        if (!std::isfinite(s) || !(s > 0.f))
            return FA_ERR_SCALE;
    if (empty)
        return FA_OK;
    st = check_ptrs({Q, K, V, O, LSE});
    if (st != FA_OK)
        return st;
    if (workspace == nullptr || workspace_bytes < fa::fp8_workspace_bytes(B, H, N, d) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return FA_ERR_WORKSPACE;
    fa::Fp8Problem p;
    p.B = B;
    p.H = H;
    p.N = N;
    p.d = d;
    p.scale = scale;
    p.q_descale = q_descale;
    p.k_descale = k_descale;
    p.v_descale = v_descale;
    p.causal = causal;
    p.stream = static_cast<hipStream_t>(stream);
    return hip_status(fa::launch_fwd_fp8(p, static_cast<const uint8_t *>(Q),
                                         static_cast<const uint8_t *>(K),
                                         static_cast<const uint8_t *>(V),
                                         static_cast<uint16_t *>(O), LSE, workspace));
}

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d)
{
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk < 0 || d <= 0)
        return 0;
    return fa::decode_split(B, H, Nq, Nk, d).bytes;
}

fa_status fa_decode(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                    int H, int Nq, int Nk, int d, float scale, int causal, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    bool empty = false;
    // the key side and the query side each pass the checks of a [B][H][N][d]
    // tensor (Nk may be 0: every query then sees no key)
    fa_status st = check_common(B, H, Nq, d, scale, causal, &empty, kMaxDWide);
    if (st != FA_OK)
        return st;
    bool no_keys = false;
    st = check_common(B, H, Nk, d, scale, causal, &no_keys, kMaxDWide);
    if (st != FA_OK)
        return st;
    if (empty)
        return FA_OK;
    st = check_ptrs({Q, O, LSE});
    if (st == FA_OK && !no_keys)
        st = check_ptrs({K, V});
    if (st != FA_OK)
        return st;
    const fa::DecodeSplit sp = fa::decode_split(B, H, Nq, Nk, d);
    if (workspace == nullptr || workspace_bytes < sp.bytes ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return FA_ERR_WORKSPACE;
    fa::DecodeProblem p;
    p.B = B;
    p.H = H;
    p.Nq = Nq;
    p.Nk = Nk;
    p.d = d;
    p.scale = scale;
    p.causal = causal;
    p.stream = static_cast<hipStream_t>(stream);
    return hip_status(fa::launch_decode_bf16(p, static_cast<const uint16_t *>(Q),
                                             static_cast<const uint16_t *>(K),
                                             static_cast<const uint16_t *>(V),
                                             static_cast<uint16_t *>(O), LSE, workspace));
}

fa_status fa_fwd_f32(const float *Q, const float *K, const float *V, float *O, float *LSE, int B,
                     int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                     void *stream)
{
    return fwd_common<float>(Q, K, V, O, LSE, B, H, N, d, scale, causal, blockmask, stream, true,
                             kMaxDWide);
}

fa_status fa_bwd_f32(const float *dO, const float *Q, const float *K, const float *V,
                     const float *O, const float *LSE, float *dQ, float *dK, float *dV, int B,
                     int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    return bwd_common<float>(dO, Q, K, V, O, LSE, dQ, dK, dV, B, H, N, d, scale, causal,
                             blockmask, workspace, workspace_bytes, stream, true, kMaxDWide);
}

const char *fa_status_str(fa_status s)
{
    switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_SHAPE: return "invalid shape";
    case FA_ERR_HEADDIM:
        return "unsupported head dimension (d must be a multiple of 8 in [8, 128]; in [8, 256] for fa_fwd, "
               "fa_bwd, fa_decode, fa_fwd_f32 and fa_bwd_f32)";
    case FA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite and > 0, causal 0 or 1, dropout probability in [0, 1)";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "HIP error";
    case FA_ERR_SCRATCH:
        return "problem needs more backward scratch than the no-allocation entry point's static "
               "array holds (FA_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

const char *fa_last_hip_error(void)
{
    return g_last_hip_error;
}

const char *fa_version(void)
{
    return "fa-gfx950 0.1.0";
}

}  // extern "C"
