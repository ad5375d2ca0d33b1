/*
 * fa.h -- C ABI of the MI355X (gfx950) exact IO-aware attention library.
 *
 * The operation is exact scaled-dot-product attention, computed tile by tile
 * with an online softmax so that the N x N score and probability matrices
 * never reach device memory:
 *
 *   S = scale * Q K^T, masked;  P = softmax(S) row by row;  O = P V
 *
 * Definitions followed:
 *   - S, P, O: mstx.cn/posts/485 §二.1 "标准 Attention 的计算"; the 1/sqrt(d)
 *     scale as written in nanhubrain.csdn.net §二 "反向传播的代价".
 *   - tiling and the online max / exp-sum rescaling across key/value blocks:
 *     mstx.cn/posts/485 §三.1 "Tiling" and §三.2 "Online Softmax";
 *     lukebest.github.io FlashAttention, "算法要点".
 *   - one fused kernel QK^T -> softmax (+mask) -> PV:
 *     lukebest.github.io FlashAttention, "Kernel fusion".
 *   - backward by recomputation from Q, K, V and the saved row statistics:
 *     lukebest.github.io FlashAttention, "反向：重算而非存储";
 *     mstx.cn/posts/485 §三.3 "重计算".
 *   - causal mask P_ij = 0 for j > i (top-left aligned, diagonal kept):
 *     nanhubrain.csdn.net §三 "因果掩码下的锯齿形调度".
 *   - fixed block-sparse mask whose zero blocks are skipped:
 *     lukebest.github.io FlashAttention, "Block-Sparse FlashAttention".
 *
 * Common argument rules (all entry points):
 *   - Q, K, V, O, dO, dQ, dK, dV are DEVICE pointers to contiguous
 *     [B][H][N][d] tensors, d fastest, 16-byte aligned. In the bf16 entry
 *     points each element is a bf16 bit pattern (uint16); in the _f32 entry
 *     points each element is an IEEE float.
 *   - LSE is a DEVICE pointer to a contiguous [B][H][N] float tensor holding
 *     the natural-log log-sum-exp of each row of S: LSE_i = ln sum_j exp(S_ij).
 *     A row with no visible key gets O_i = 0 and LSE_i = -inf and contributes
 *     no gradient.
 *   - blockmask is NULL (dense) or a DEVICE pointer to uint8
 *     [ceil(N/128)][ceil(N/128)], row-major, nonzero = keep the 128 x 128
 *     block of (query block, key block). One mask serves every (b, h); it is
 *     combined with the causal mask by AND.
 *   - B, H, N >= 0 (any zero means an empty problem: FA_OK, nothing done);
 *     d a multiple of 8 in [8, 128] (d <= 64 runs in the 64-wide kernels and
 *     64 < d <= 128 in the 128-wide ones, the columns past d taken as zero:
 *     the cost is that of the padded width); fa_fwd, fa_fwd_f32 and
 *     fa_bwd_f32, fa_bwd and fa_decode also take 128 < d <= 256 (fa_fwd:
 *     all 256 columns of O in one workgroup; fa_bwd: dQ in one pass and
 *     dV and dK in a pass each, so S is rebuilt once more than at d <= 128,
 *     1.6x the method's contraction work); the backward phase,
 *     dropout and FP8 entry points stay at d <= 128 and return
 *     FA_ERR_HEADDIM past it;
 *     N * d < 2^30; scale finite and > 0; causal is 0 or 1.
 *   - stream is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously on it; argument checks happen synchronously, before any
 *     HIP call, and a failed check enqueues nothing.
 *   - Ownership: the caller owns every buffer. The library allocates and
 *     frees no device or host memory; backward scratch is passed in as
 *     `workspace` (fa_bwd_noalloc instead uses a static device array of the
 *     library, see there).
 *   - Errors are returned as fa_status; no exception crosses the ABI. After
 *     FA_ERR_HIP, fa_last_hip_error() describes the failure (thread-local).
 *   - Entry points keep no state between calls and may be called from
 *     several host threads on different streams (except fa_bwd_noalloc,
 *     whose calls on one GPU share its static scratch array).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,     /* B, H or N negative, or sizes overflow */
    FA_ERR_HEADDIM = 3,   /* d not supported */
    FA_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned */
    FA_ERR_SCALE = 5,     /* scale not finite or not > 0, causal not 0/1, or a
                             dropout probability outside [0, 1) */
    FA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than fa_bwd_workspace_bytes */
    FA_ERR_HIP = 7,       /* a HIP call failed; see fa_last_hip_error() */
    FA_ERR_SCRATCH = 8    /* fa_bwd_noalloc: the problem needs more scratch than
                             FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

#define FA_MASK_BLOCK 128

/* Forward, bf16 storage, fp32 softmax statistics and accumulation.
 * Reads Q, K, V (and blockmask); writes O (bf16) and LSE (float). */
fa_status fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE,
                 int B, int H, int N, int d, float scale, int causal,
                 const uint8_t *blockmask, void *stream);

/* Bytes of device scratch fa_bwd / fa_bwd_f32 need for this shape
 * (0 for an empty problem). The buffer needs no initialisation. */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward, bf16 storage. Given the forward's O and LSE and dO = dL/dO,
 * writes dQ, dK, dV (bf16) for the loss L, scale being a constant.
 * Reads dO, Q, K, V, O, LSE (and blockmask); workspace is device scratch of
 * at least fa_bwd_workspace_bytes(B, H, N, d) bytes, 256-byte aligned. */
fa_status fa_bwd(const void *dO, const void *Q, const void *K, const void *V,
                 const void *O, const float *LSE, void *dQ, void *dK, void *dV,
                 int B, int H, int N, int d, float scale, int causal,
                 const uint8_t *blockmask, void *workspace, size_t workspace_bytes,
                 void *stream);

/* The three phases of fa_bwd, one kernel each, for callers that schedule them
 * themselves (e.g. fa_bwd_dq and fa_bwd_dkdv on two streams) or time them.
 * fa_bwd_prep must complete on a workspace before fa_bwd_dq / fa_bwd_dkdv
 * read it; those two are independent of each other. Arguments as in fa_bwd.
 *   fa_bwd_prep: reads dO, O, LSE; writes the row statistics the other two
 *                read (-D_i with D_i = sum_k dO_ik O_ik, and LSE_i * log2(e))
 *                into the workspace.
 *   fa_bwd_dq:   reads dO, Q, K, V and the workspace; writes dQ.
 *   fa_bwd_dkdv: reads dO, Q, K, V and the workspace; writes dK and dV. */
fa_status fa_bwd_prep(const void *dO, const void *O, const float *LSE,
                      int B, int H, int N, int d,
                      void *workspace, size_t workspace_bytes, void *stream);
fa_status fa_bwd_dq(const void *dO, const void *Q, const void *K, const void *V, void *dQ,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t *blockmask, const void *workspace, size_t workspace_bytes,
                    void *stream);
fa_status fa_bwd_dkdv(const void *dO, const void *Q, const void *K, const void *V,
                      void *dK, void *dV, int B, int H, int N, int d, float scale, int causal,
                      const uint8_t *blockmask, const void *workspace, size_t workspace_bytes,
                      void *stream);

/* Size of the static device scratch array fa_bwd_noalloc uses (per GPU). */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation). The backward's scratch (two floats per row) lives
 * in a static device array of the library, FA_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends; this call
 * itself allocates nothing. Limit: fa_bwd_workspace_bytes(B, H, N, d) <=
 * FA_NOALLOC_SCRATCH_BYTES (B*H*N up to about 2 million rows), else
 * FA_ERR_SCRATCH before any HIP call. The array belongs to the GPU current on
 * the calling host thread, which must be the GPU of the tensors and the
 * stream. Every call on one GPU shares that GPU's array: calls must not
 * overlap in time on one GPU (different streams or host threads race on
 * it); calls ordered on one stream are safe, since each call rewrites every
 * entry it reads. Other arguments, results and errors as fa_bwd. */
fa_status fa_bwd_noalloc(const void *dO, const void *Q, const void *K, const void *V,
                         const void *O, const float *LSE, void *dQ, void *dK, void *dV,
                         int B, int H, int N, int d, float scale, int causal,
                         const uint8_t *blockmask, void *stream);

/* Forward with dropout on P (lukebest.github.io FlashAttention, "Kernel
 * fusion", lists dropout among the fused steps; the drawing rule is this
 * library's): element (i, j) of head bh = b*H + h is dropped iff word j % 4 of
 * Philox4x32-10(counter (j / 4, i, bh, 0), key (low 32 bits of seed, high 32
 * bits of seed)) is below floor(p_drop * 2^32) (Philox4x32-10: Salmon et al.,
 * SC 2011). Then O_i = sum_j P_ij Z_ij / (1 - p_drop) V_j with P the softmax
 * of the masked scores; LSE is that of P (no dropout), as fa_bwd_dropout
 * needs. p_drop in [0, 1) (0: same as fa_fwd); the same (p_drop, seed) must
 * be passed to fa_bwd_dropout. Other arguments and rules as fa_fwd. */
fa_status fa_fwd_dropout(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                         int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                         float p_drop, unsigned long long seed, void *stream);

/* Backward of fa_fwd_dropout (O is its output): dV = P~^T dO with
 * P~ = P o Z / (1 - p), dP = dO V^T, D_i = rowsum(dO o O),
 * dS = P o (Z o dP / (1 - p) - D), dQ = scale dS K, dK = scale dS^T Q; the
 * mask Z is drawn again from (p_drop, seed) by the same rule. Other arguments
 * and rules as fa_bwd (same workspace size). */
fa_status fa_bwd_dropout(const void *dO, const void *Q, const void *K, const void *V,
                         const void *O, const float *LSE, void *dQ, void *dK, void *dV, int B,
                         int H, int N, int d, float scale, int causal, const uint8_t *blockmask,
                         float p_drop, unsigned long long seed, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Bytes of device scratch fa_fwd_fp8 needs (0 for an empty problem or an
 * unsupported d): V^T in 64-key tiles, B*H*ceil(N/64)*64*d bytes. */
size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N, int d);

/* FP8 forward (lukebest.github.io FlashAttention, lineage table "谱系": the
 * third generation adds an FP8 forward). Q, K, V: [B][H][N][d] OCP E4M3 codes
 * (1 byte each; value = code * descale, one fp32 descale per tensor); O:
 * [B][H][N][d] bf16; LSE: [B][H][N] float. Computes the forward of the
 * decoded values: S = scale * Q K^T from the exact fp8 products accumulated
 * in fp32, fp32 online softmax, P rounded to E4M3 for the P V product, O and
 * LSE as fa_fwd. The error against exact attention of the decoded inputs is
 * that of rounding P to a 3-bit mantissa (relative error about 3% per
 * weight, in O's relative L2 about as much). d: 64 or 128; no block mask;
 * causal as fa_fwd. workspace: at least fa_fwd_fp8_workspace_bytes(B, H, N,
 * d) bytes of device memory, 256-byte aligned, owned by the caller (V is
 * transposed into it first). Descales must be finite and > 0
 * (FA_ERR_SCALE otherwise). */
fa_status fa_fwd_fp8(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                     int H, int N, int d, float scale, float q_descale, float k_descale,
                     float v_descale, int causal, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Bytes of device scratch fa_decode needs for this shape (0 for an empty
 * problem). It depends on the shape only. */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/* Decode-shaped forward, bf16: Nq queries per head against Nk keys of the
 * same head, for the few newest positions of a sequence attending to its
 * cached keys and values (lukebest.github.io FlashAttention, lineage table
 * "谱系", the FlashDecoding line: with few queries the keys are split into
 * chunks processed in parallel, and the chunk results are merged with the
 * online-softmax rule of mstx.cn/posts/485 §三.2).
 *   Q, O: [B][H][Nq][d] bf16;  K, V: [B][H][Nk][d] bf16;  LSE: [B][H][Nq]
 *   float, natural log.  O_i = softmax(scale q_i K^T) V over the keys query
 *   i sees: all of them, or with causal = 1 the keys j <= Nk - Nq + i (the
 *   queries are the last Nq positions; for Nq = Nk this is fa_fwd's causal
 *   rule). A query that sees no key gets O_i = 0, LSE_i = -inf.
 *   No block mask. Same head-dim, scale and alignment rules as fa_fwd, with
 *   Nq >= 0 and Nk >= 0 each meeting fa_fwd's limits on N.
 *   workspace: device memory of at least fa_decode_workspace_bytes(B, H, Nq,
 *   Nk, d) bytes, 256-byte aligned, owned by the caller; its contents on
 *   entry do not matter and calls sharing it must be ordered on one stream.
 *   Meant for small Nq (each 32-query block reads all of K and V once).
 *   Returns FA_ERR_WORKSPACE when the workspace is missing, misaligned or
 *   too small. */
fa_status fa_decode(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                    int H, int Nq, int Nk, int d, float scale, int causal, void *workspace,
                    size_t workspace_bytes, void *stream);

/* fp32 debug path: the same tiled online-softmax algorithm with every tensor
 * in float and fp32 arithmetic throughout. Same argument rules. */
fa_status fa_fwd_f32(const float *Q, const float *K, const float *V, float *O, float *LSE,
                     int B, int H, int N, int d, float scale, int causal,
                     const uint8_t *blockmask, void *stream);

fa_status fa_bwd_f32(const float *dO, const float *Q, const float *K, const float *V,
                     const float *O, const float *LSE, float *dQ, float *dK, float *dV,
                     int B, int H, int N, int d, float scale, int causal,
                     const uint8_t *blockmask, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Static text for a status code. */
const char *fa_status_str(fa_status s);

/* Text of the last HIP failure seen by this host thread ("" if none). */
const char *fa_last_hip_error(void);

/* Library version string. */
const char *fa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FA_H */
