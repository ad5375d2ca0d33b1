/*
 * CPU fp64 reference for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or helper with the GPU library and must never be used as a
 * fallback for it.
 *
 * What it computes is the plain definition, written out with every N x N
 * intermediate materialised (no tiling, no online softmax, no fusion):
 *
 *   S = scale * Q K^T                (mstx.cn/posts/485 §二.1 "标准 Attention 的计算";
 *                                     the 1/sqrt(d) factor is the one written in
 *                                     nanhubrain.csdn.net §二 "反向传播的代价")
 *   S_ij = -inf where j is not allowed for row i:
 *        causal: P_ij = 0 for j > i  (nanhubrain.csdn.net §三 "因果掩码下的锯齿形调度")
 *        fixed block mask: zero blocks are skipped
 *                                    (lukebest.github.io FlashAttention, "Block-Sparse FlashAttention")
 *   P = softmax(S) row by row, max-subtracted
 *                                    (cloud.baidu.com/article/7906313 §工作原理 "数学等价变换";
 *                                     mstx.cn/posts/485 §三.2 "标准 softmax")
 *   O = P V                          (mstx.cn/posts/485 §二.1)
 *   LSE_i = m_i + ln(l_i)            (the saved per-row statistic; the pages save
 *                                     (m, l), mstx.cn/posts/485 §三.3 "重计算")
 *
 * Backward, for a loss L with dL/dO = dO (the recompute method of
 * lukebest.github.io "反向：重算而非存储" reaches the same gradients):
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *   dS = P o (dP - D 1^T),  dQ = scale * dS K,  dK = scale * dS^T Q.
 * The printed gradient formula of cloud.baidu.com §工作原理 "梯度计算优化" is
 * garbled (a matrix product where a row sum belongs); the rule above is the
 * softmax Jacobian written out, and sum_j P_ij dP_ij = sum_k dO_ik O_ik holds
 * exactly because O_i = sum_j P_ij V_j.
 *
 * Convention for a row with no allowed key (not on the pages): O_i = 0,
 * LSE_i = -inf, and the row contributes nothing to any gradient.
 *
 * Layout: every tensor is contiguous [B][H][N][d] (d fastest), LSE is
 * [B][H][N]. The block mask is [nb][nb] row-major with nb = ceil(N/blk),
 * nonzero = keep, shared by all (b, h), and combined with causal by AND.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#include "oracle.h"

static int key_allowed(long i, long j, int causal, const unsigned char *mask,
                       long blk, long nb)
{
    if (causal && j > i)
        return 0;
    if (mask && mask[(i / blk) * nb + (j / blk)] == 0)
        return 0;
    return 1;
}

/* One row of the forward for one head: fills srow[0..N) with P_i. (row of P),
 * writes O_i and LSE_i. */
static void forward_row(const double *q, const double *k, const double *v,
                        long N, long d, double scale, int causal,
                        const unsigned char *mask, long blk, long nb, long i,
                        double *prow, double *orow, double *lse)
{
    double m = -INFINITY;
    for (long j = 0; j < N; ++j) {
        if (!key_allowed(i, j, causal, mask, blk, nb)) {
            prow[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (long c = 0; c < d; ++c)
            dot += q[i * d + c] * k[j * d + c];
        prow[j] = scale * dot;
        if (prow[j] > m)
            m = prow[j];
    }
    for (long c = 0; c < d; ++c)
        orow[c] = 0.0;
    if (m == -INFINITY) {
        for (long j = 0; j < N; ++j)
            prow[j] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (long j = 0; j < N; ++j) {
        double e = (prow[j] == -INFINITY) ? 0.0 : exp(prow[j] - m);
        prow[j] = e;
        l += e;
    }
    for (long j = 0; j < N; ++j)
        prow[j] /= l;
    for (long j = 0; j < N; ++j) {
        if (prow[j] == 0.0)
            continue;
        for (long c = 0; c < d; ++c)
            orow[c] += prow[j] * v[j * d + c];
    }
    *lse = m + log(l);
}

static int check_args(long B, long H, long N, long d, long blk)
{
    if (B < 0 || H < 0 || N < 0 || d <= 0 || blk <= 0)
        return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

int oracle_attention(const double *Q, const double *K, const double *V,
                     const double *dO, double *O, double *LSE,
                     double *dQ, double *dK, double *dV,
                     long B, long H, long N, long d, double scale, int causal,
                     const unsigned char *blockmask, long blk)
{
    int rc = check_args(B, H, N, d, blk);
    if (rc != ORACLE_OK)
        return rc;
    const long nb = (N + blk - 1) / blk;
    const int want_bwd = (dO != NULL);
    if (want_bwd && (dQ == NULL || dK == NULL || dV == NULL))
        return ORACLE_ERR_ARG;
    if (N == 0)
        return ORACLE_OK;

    double *P = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
    double *dS = want_bwd ? (double *)malloc(sizeof(double) * (size_t)N * (size_t)N) : NULL;
    double *D = want_bwd ? (double *)malloc(sizeof(double) * (size_t)N) : NULL;
    if (!P || (want_bwd && (!dS || !D))) {
        free(P); free(dS); free(D);
        return ORACLE_ERR_NOMEM;
    }

    for (long bh = 0; bh < B * H; ++bh) {
        const double *q = Q + bh * N * d, *k = K + bh * N * d, *v = V + bh * N * d;
        double *o = O + bh * N * d, *lse = LSE + bh * N;

        /* Forward: materialise every row of P. */
        #pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i)
            forward_row(q, k, v, N, d, scale, causal, blockmask, blk, nb, i,
                        P + i * N, o + i * d, lse + i);

        if (!want_bwd)
            continue;

        const double *dout = dO + bh * N * d;
        double *dq = dQ + bh * N * d, *dk = dK + bh * N * d, *dv = dV + bh * N * d;

        /* D_i = rowsum(dO o O); dP_ij = dO_i . V_j; dS = P o (dP - D);
         * dQ_i = scale * sum_j dS_ij K_j. */
        #pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i) {
            double Di = 0.0;
            for (long c = 0; c < d; ++c)
                Di += dout[i * d + c] * o[i * d + c];
            D[i] = Di;
            for (long j = 0; j < N; ++j) {
                double pij = P[i * N + j];
                if (pij == 0.0) {
                    dS[i * N + j] = 0.0;
                    continue;
                }
                double dp = 0.0;
                for (long c = 0; c < d; ++c)
                    dp += dout[i * d + c] * v[j * d + c];
                dS[i * N + j] = pij * (dp - Di);
            }
            for (long c = 0; c < d; ++c)
                dq[i * d + c] = 0.0;
            for (long j = 0; j < N; ++j) {
                double s = dS[i * N + j];
                if (s == 0.0)
                    continue;
                for (long c = 0; c < d; ++c)
                    dq[i * d + c] += s * k[j * d + c];
            }
            for (long c = 0; c < d; ++c)
                dq[i * d + c] *= scale;
        }

        /* dK_j = scale * sum_i dS_ij Q_i;  dV_j = sum_i P_ij dO_i. */
        #pragma omp parallel for schedule(dynamic, 16)
        for (long j = 0; j < N; ++j) {
            for (long c = 0; c < d; ++c) {
                dk[j * d + c] = 0.0;
                dv[j * d + c] = 0.0;
            }
            for (long i = 0; i < N; ++i) {
                double s = dS[i * N + j];
                double pij = P[i * N + j];
                if (s != 0.0)
                    for (long c = 0; c < d; ++c)
                        dk[j * d + c] += s * q[i * d + c];
                if (pij != 0.0)
                    for (long c = 0; c < d; ++c)
                        dv[j * d + c] += pij * dout[i * d + c];
            }
            for (long c = 0; c < d; ++c)
                dk[j * d + c] *= scale;
        }
    }
    free(P);
    free(dS);
    free(D);
    return ORACLE_OK;
}

int oracle_attention_rows(const double *Q, const double *K, const double *V,
                          long B, long H, long N, long d, double scale, int causal,
                          const unsigned char *blockmask, long blk,
                          const long *row_bh, const long *row_i, long nrows,
                          double *O_rows, double *LSE_rows)
{
    int rc = check_args(B, H, N, d, blk);
    if (rc != ORACLE_OK)
        return rc;
    for (long r = 0; r < nrows; ++r)
        if (row_bh[r] < 0 || row_bh[r] >= B * H || row_i[r] < 0 || row_i[r] >= N)
            return ORACLE_ERR_ARG;
    const long nb = (N + blk - 1) / blk;
    int nomem = 0;
    #pragma omp parallel
    {
        double *prow = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!prow) {
            #pragma omp atomic write
            nomem = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < nrows; ++r) {
                const long bh = row_bh[r];
                forward_row(Q + bh * N * d, K + bh * N * d, V + bh * N * d, N, d,
                            scale, causal, blockmask, blk, nb, row_i[r], prow,
                            O_rows + r * d, LSE_rows + r);
            }
        }
        free(prow);
    }
    return nomem ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011): a 4 x 32-bit counter and a 2 x 32-bit key give
 * 4 x 32 random bits. One round multiplies counter words 0 and 2 by the
 * constants 0xD2511F53 and 0xCD9E8D57 into 64-bit products, and the new
 * counter is (hi(c2 M1) ^ c1 ^ k0, lo(c2 M1), hi(c0 M0) ^ c3 ^ k1, lo(c0 M0));
 * between rounds the key is advanced by (0x9E3779B9, 0xBB67AE85).
 */
void oracle_philox4x32_10(const unsigned int ctr_in[4], const unsigned int key_in[2],
                          unsigned int out[4])
{
    unsigned int c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    unsigned int k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const unsigned long long p0 = (unsigned long long)0xD2511F53u * c[0];
        const unsigned long long p1 = (unsigned long long)0xCD9E8D57u * c[2];
        const unsigned int n0 = (unsigned int)(p1 >> 32) ^ c[1] ^ k0;
        const unsigned int n1 = (unsigned int)p1;
        const unsigned int n2 = (unsigned int)(p0 >> 32) ^ c[3] ^ k1;
        const unsigned int n3 = (unsigned int)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/*
 * Dropout mask (the drawing rule is this library's, the pages only place
 * dropout among the fused steps: lukebest.github.io FlashAttention, "Kernel
 * fusion"): element (i, j) of head bh is dropped iff word j % 4 of
 * Philox4x32-10(counter = (j / 4, i, bh, 0), key = (seed low, seed high)) is
 * below floor(p_drop * 2^32); kept weights are scaled by 1 / (1 - p_drop).
 */
static unsigned int drop_threshold(double p_drop)
{
    const double t = floor(p_drop * 4294967296.0);
    return t >= 4294967295.0 ? 4294967295u : (unsigned int)t;
}

int oracle_dropout_keep(long bh, long i, long j, double p_drop, unsigned long long seed)
{
    const unsigned int ctr[4] = {(unsigned int)(j / 4), (unsigned int)i, (unsigned int)bh, 0u};
    const unsigned int key[2] = {(unsigned int)seed, (unsigned int)(seed >> 32)};
    unsigned int w[4];
    oracle_philox4x32_10(ctr, key, w);
    return w[j % 4] >= drop_threshold(p_drop);
}

/*
 * Attention with dropout on P, forward and (dO != NULL) backward, written out
 * with N x N intermediates like oracle_attention (head bh of the arrays draws
 * its mask as head bh + bh_offset, so a slice of heads can be checked alone):
 *   P = softmax(S) (S as above, masks included), Z_ij in {0, 1} the mask,
 *   P~ = P o Z / (1 - p),  O = P~ V,  LSE from P's statistics (no dropout);
 *   dV = P~^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *   dS = P o (Z o dP / (1 - p) - D 1^T),  dQ = scale dS K,  dK = scale dS^T Q.
 * (D_i = sum_j P~_ij dP_ij because O_i = sum_j P~_ij V_j; dS is the softmax
 * Jacobian applied to the gradient reaching P, Z o dP / (1 - p).)
 */
int oracle_attention_dropout(const double *Q, const double *K, const double *V,
                             const double *dO, double *O, double *LSE,
                             double *dQ, double *dK, double *dV,
                             long B, long H, long N, long d, double scale, int causal,
                             const unsigned char *blockmask, long blk,
                             double p_drop, unsigned long long seed, long bh_offset)
{
    int rc = check_args(B, H, N, d, blk);
    if (rc != ORACLE_OK)
        return rc;
    if (!(p_drop >= 0.0 && p_drop < 1.0))
        return ORACLE_ERR_ARG;
    const int want_bwd = (dO != NULL);
    if (want_bwd && (dQ == NULL || dK == NULL || dV == NULL))
        return ORACLE_ERR_ARG;
    if (N == 0)
        return ORACLE_OK;
    const long nb = (N + blk - 1) / blk;
    const double inv_keep = 1.0 / (1.0 - p_drop);
    double *P = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
    double *Z = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
    double *D = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!P || !Z || !D) {
        free(P); free(Z); free(D);
        return ORACLE_ERR_NOMEM;
    }
    for (long bh = 0; bh < B * H; ++bh) {
        const double *q = Q + bh * N * d, *k = K + bh * N * d, *v = V + bh * N * d;
        double *o = O + bh * N * d, *lse = LSE + bh * N;
        #pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i) {
            /* P_i and LSE_i (O_i from forward_row is replaced below) */
            forward_row(q, k, v, N, d, scale, causal, blockmask, blk, nb, i,
                        P + i * N, o + i * d, lse + i);
            for (long j = 0; j < N; ++j)
                Z[i * N + j] = oracle_dropout_keep(bh + bh_offset, i, j, p_drop, seed) ? 1.0 : 0.0;
            for (long c = 0; c < d; ++c)
                o[i * d + c] = 0.0;
            for (long j = 0; j < N; ++j) {
                const double pt = P[i * N + j] * Z[i * N + j] * inv_keep;
                if (pt != 0.0)
                    for (long c = 0; c < d; ++c)
                        o[i * d + c] += pt * v[j * d + c];
            }
        }
        if (!want_bwd)
            continue;
        const double *dout = dO + bh * N * d;
        double *dq = dQ + bh * N * d, *dk = dK + bh * N * d, *dv = dV + bh * N * d;
        /* overwrite Z with dS row by row once D_i is known */
        #pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i) {
            double Di = 0.0;
            for (long c = 0; c < d; ++c)
                Di += o[i * d + c] * dout[i * d + c];
            D[i] = Di;
        }
        /* dV_j = sum_i P~_ij dO_i (before Z is overwritten) */
        #pragma omp parallel for schedule(dynamic, 16)
        for (long j = 0; j < N; ++j) {
            for (long c = 0; c < d; ++c)
                dv[j * d + c] = 0.0;
            for (long i = 0; i < N; ++i) {
                const double pt = inv_keep * Z[i * N + j] * P[i * N + j];
                if (pt != 0.0)
                    for (long c = 0; c < d; ++c)
                        dv[j * d + c] += pt * dout[i * d + c];
            }
        }
        #pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i) {
            for (long j = 0; j < N; ++j) {
                const double pij = P[i * N + j];
                double g = 0.0;
                if (pij != 0.0) {
                    double dp = 0.0;
                    for (long c = 0; c < d; ++c)
                        dp += v[j * d + c] * dout[i * d + c];
                    g = pij * (Z[i * N + j] * dp * inv_keep - D[i]);
                }
                Z[i * N + j] = g;  /* now dS */
            }
            for (long c = 0; c < d; ++c)
                dq[i * d + c] = 0.0;
            for (long j = 0; j < N; ++j) {
                const double ds = Z[i * N + j];
                if (ds != 0.0)
                    for (long c = 0; c < d; ++c)
                        dq[i * d + c] += ds * k[j * d + c];
            }
            for (long c = 0; c < d; ++c)
                dq[i * d + c] = scale * dq[i * d + c];
        }
        #pragma omp parallel for schedule(dynamic, 16)
        for (long j = 0; j < N; ++j) {
            for (long c = 0; c < d; ++c)
                dk[j * d + c] = 0.0;
            for (long i = 0; i < N; ++i) {
                const double ds = Z[i * N + j];
                if (ds != 0.0)
                    for (long c = 0; c < d; ++c)
                        dk[j * d + c] += ds * q[i * d + c];
            }
            for (long c = 0; c < d; ++c)
                dk[j * d + c] = scale * dk[j * d + c];
        }
    }
    free(P);
    free(Z);
    free(D);
    return ORACLE_OK;
}

/*
 * Decode-shaped forward: Nq queries against Nk keys of the same head (the
 * queries are the last Nq positions of a sequence whose first Nk positions
 * are the keys, as when the key/value cache of earlier steps is attended).
 * What is computed is the same definition as above, row by row:
 *   S_ij = scale * q_i . k_j,  P_i = softmax(S_i),  O_i = P_i V,
 *   LSE_i = max_j S_ij + ln sum_j exp(S_ij - max_j S_ij)
 * (mstx.cn/posts/485 §二.1 and §三.2), with the causal rule P_ij = 0 for
 * keys after the query's own position: query i sits at position
 * Nk - Nq + i, so key j is allowed iff j <= Nk - Nq + i (nanhubrain.csdn.net
 * §三's j > i rule with the query index shifted to its position; for
 * Nq = Nk it is that rule). No block mask. The split of the keys into chunks
 * whose partial results are merged afterwards is lukebest.github.io's
 * FlashDecoding line of the lineage table ("谱系"); this reference does not
 * split: it is the plain result the merged one must equal.
 */
static void decode_row(const double *q, const double *k, const double *v,
                       long nkeys, long d, double scale, double *srow,
                       double *orow, double *lse)
{
    for (long c = 0; c < d; ++c)
        orow[c] = 0.0;
    if (nkeys <= 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (long j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (long c = 0; c < d; ++c)
            dot += q[c] * k[j * d + c];
        srow[j] = scale * dot;
        if (srow[j] > m)
            m = srow[j];
    }
    double l = 0.0;
    for (long j = 0; j < nkeys; ++j) {
        srow[j] = exp(srow[j] - m);
        l += srow[j];
    }
    for (long j = 0; j < nkeys; ++j) {
        const double p = srow[j] / l;
        for (long c = 0; c < d; ++c)
            orow[c] += p * v[j * d + c];
    }
    *lse = log(l) + m;
}

int oracle_attention_kv(const double *Q, const double *K, const double *V,
                        double *O, double *LSE, long B, long H, long Nq, long Nk,
                        long d, double scale, int causal)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d <= 0)
        return ORACLE_ERR_ARG;
    int nomem = 0;
    #pragma omp parallel
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!srow) {
            #pragma omp atomic write
            nomem = 1;
        } else {
            #pragma omp for collapse(2) schedule(dynamic, 1)
            for (long bh = 0; bh < B * H; ++bh)
                for (long i = 0; i < Nq; ++i) {
                    long nkeys = Nk;
                    if (causal) {
                        const long last = Nk - Nq + i;  /* last allowed key */
                        nkeys = last + 1 < Nk ? last + 1 : Nk;
                    }
                    decode_row(Q + (bh * Nq + i) * d, K + bh * Nk * d, V + bh * Nk * d,
                               nkeys, d, scale, srow, O + (bh * Nq + i) * d, LSE + bh * Nq + i);
                }
        }
        free(srow);
    }
    return nomem ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

int oracle_num_threads(void)
{
    return omp_get_max_threads();
}
