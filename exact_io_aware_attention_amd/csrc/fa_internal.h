// Host-side interface between the C ABI layer (fa_api.cpp) and the kernel
// translation units. Arguments reaching these launchers are already
// validated: non-empty shapes, supported head dimension, aligned pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct Problem {
    int B, H, N, d;
    float scale;
    int causal;
    const uint8_t *mask;  // device pointer or nullptr
    hipStream_t stream;
    // dropout on P (dropout = 0: none): keep iff the element's Philox word
    // >= drop_threshold; kept weights times drop_inv_keep
    int dropout = 0;
    uint32_t drop_threshold = 0;
    uint64_t drop_seed = 0;
    float drop_inv_keep = 1.f;
};

// Scratch layout of the backward (offsets in bytes from the workspace base).
struct BwdWorkspace {
    size_t delta_off;  // float [B*H][N]: D_i = rowsum(dO o O)
    size_t lse2_off;   // float [B*H][N]: LSE_i * log2(e)
    size_t bytes;      // total
};
BwdWorkspace bwd_workspace_layout(int B, int H, int N, int d);

// Each launcher enqueues its kernels on p.stream and returns the
// hipGetLastError() status of the launches.
hipError_t launch_fwd_bf16(const Problem &p, const uint16_t *Q, const uint16_t *K,
                           const uint16_t *V, uint16_t *O, float *LSE);
hipError_t launch_bwd_bf16(const Problem &p, const uint16_t *dO, const uint16_t *Q,
                           const uint16_t *K, const uint16_t *V, const uint16_t *O,
                           const float *LSE, uint16_t *dQ, uint16_t *dK, uint16_t *dV,
                           void *workspace);
// The three phases of launch_bwd_bf16 (each one kernel), in the order they
// must run on one workspace: prep writes D and LSE*log2(e) that dq and dkdv
// read; dq and dkdv are independent of each other.
hipError_t launch_bwd_prep_bf16(const Problem &p, const uint16_t *dO, const uint16_t *O,
                                const float *LSE, void *workspace);
hipError_t launch_bwd_dq_bf16(const Problem &p, const uint16_t *dO, const uint16_t *Q,
                              const uint16_t *K, const uint16_t *V, uint16_t *dQ,
                              const void *workspace);
hipError_t launch_bwd_dkdv_bf16(const Problem &p, const uint16_t *dO, const uint16_t *Q,
                                const uint16_t *K, const uint16_t *V, uint16_t *dK,
                                uint16_t *dV, const void *workspace);
// Decode-shaped forward: Nq queries against Nk keys per head.
struct DecodeProblem {
    int B, H, Nq, Nk, d;
    float scale;
    int causal;  // queries at the last Nq positions: query i sees keys <= Nk - Nq + i
    hipStream_t stream;
};
// How the keys are split (a pure function of the shape) and the workspace it
// needs: per split, query and column an fp32 O, then per split and query an
// fp32 LSE (offset lpart_off).
struct DecodeSplit {
    int nsplit;        // key chunks per head
    int chunk;         // keys per chunk
    size_t lpart_off;  // byte offset of the LSE part
    size_t bytes;      // total
};
DecodeSplit decode_split(int B, int H, int Nq, int Nk, int d);
hipError_t launch_decode_bf16(const DecodeProblem &p, const uint16_t *Q, const uint16_t *K,
                              const uint16_t *V, uint16_t *O, float *LSE, void *workspace);

// FP8 forward: E4M3 Q, K, V with one descale each, bf16 O, fp32 LSE.
struct Fp8Problem {
    int B, H, N, d;  // d: 64 or 128
    float scale, q_descale, k_descale, v_descale;
    int causal;
    hipStream_t stream;
};
// Workspace of the FP8 forward: V^T tiles, [B*H][ceil(N/64)][d][64] bytes.
size_t fp8_workspace_bytes(int B, int H, int N, int d);
hipError_t launch_fwd_fp8(const Fp8Problem &p, const uint8_t *Q, const uint8_t *K,
                          const uint8_t *V, uint16_t *O, float *LSE, void *workspace);

hipError_t launch_fwd_f32(const Problem &p, const float *Q, const float *K, const float *V,
                          float *O, float *LSE);
// bf16 forward and backward for head dims in (128, 256] on the matrix
// cores (256-wide kernels; the backward rebuilds S in each of its dQ, dV
// and dK passes).
hipError_t launch_fwd_bf16_wide(const Problem &p, const uint16_t *Q, const uint16_t *K,
                                const uint16_t *V, uint16_t *O, float *LSE);
// dQ at d <= 128, and dK and dV in one pass at 64 < d <= 128, without
// dropout, in the slot-scheduled kernels (the -D and LSE * log2(e) rows of
// the workspace already written).
hipError_t launch_bwd_dq_bf16_slot(const Problem &p, const uint16_t *dO, const uint16_t *Q,
                                   const uint16_t *K, const uint16_t *V, uint16_t *dQ, const float *ndelta,
                                   const float *lse2);
hipError_t launch_bwd_dkdv_bf16_slot(const Problem &p, const uint16_t *dO, const uint16_t *Q,
                                     const uint16_t *K, const uint16_t *V, uint16_t *dK, uint16_t *dV,
                                     const float *ndelta, const float *lse2);
hipError_t launch_bwd_bf16_wide(const Problem &p, const uint16_t *dO, const uint16_t *Q,
                                const uint16_t *K, const uint16_t *V, const uint16_t *O,
                                const float *LSE, uint16_t *dQ, uint16_t *dK, uint16_t *dV,
                                void *workspace);
// Device address of the static scratch array of the no-allocation backward
// on the current device (looked up once per device); hipErrorInvalidValue if
// `bytes` exceeds its size.
hipError_t noalloc_scratch(size_t bytes, void **out);

hipError_t launch_bwd_f32(const Problem &p, const float *dO, const float *Q, const float *K,
                          const float *V, const float *O, const float *LSE, float *dQ,
                          float *dK, float *dV, void *workspace);

}  // namespace fa
