/*
 * CPU fp64 attention reference (test infrastructure only; see oracle.c).
 * Tensors are contiguous [B][H][N][d] doubles, LSE is [B][H][N].
 * blockmask is NULL (dense) or [ceil(N/blk)][ceil(N/blk)] bytes, nonzero = keep.
 */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_OK = 0, ORACLE_ERR_ARG = 1, ORACLE_ERR_NOMEM = 2 };

/* Forward (and, when dO != NULL, backward) of exact attention.
 * O, LSE always written; dQ, dK, dV written when dO != NULL. */
int oracle_attention(const double *Q, const double *K, const double *V,
                     const double *dO, double *O, double *LSE,
                     double *dQ, double *dK, double *dV,
                     long B, long H, long N, long d, double scale, int causal,
                     const unsigned char *blockmask, long blk);

/* Forward for selected rows only: row r is query row_i[r] of head row_bh[r]
 * (head index b*H + h). Writes O_rows[r][0..d) and LSE_rows[r]. */
int oracle_attention_rows(const double *Q, const double *K, const double *V,
                          long B, long H, long N, long d, double scale, int causal,
                          const unsigned char *blockmask, long blk,
                          const long *row_bh, const long *row_i, long nrows,
                          double *O_rows, double *LSE_rows);

/* Forward of Nq queries against Nk keys per head: Q, O are [B][H][Nq][d],
 * K, V are [B][H][Nk][d], LSE is [B][H][Nq]. causal: query i is at position
 * Nk - Nq + i and sees keys j <= Nk - Nq + i (none when that is negative). */
int oracle_attention_kv(const double *Q, const double *K, const double *V,
                        double *O, double *LSE, long B, long H, long Nq, long Nk,
                        long d, double scale, int causal);

/* Philox4x32-10: counter ctr[4], key key[2] -> out[4]. */
void oracle_philox4x32_10(const unsigned int ctr[4], const unsigned int key[2],
                          unsigned int out[4]);

/* Dropout mask bit (1 = kept) of element (i, j) of head bh: word j % 4 of
 * Philox4x32-10((j / 4, i, bh, 0), (seed low, seed high)) >= floor(p 2^32). */
int oracle_dropout_keep(long bh, long i, long j, double p_drop, unsigned long long seed);

/* oracle_attention with dropout on P (kept weights scaled by 1 / (1 - p)). */
int oracle_attention_dropout(const double *Q, const double *K, const double *V,
                             const double *dO, double *O, double *LSE,
                             double *dQ, double *dK, double *dV,
                             long B, long H, long N, long d, double scale, int causal,
                             const unsigned char *blockmask, long blk,
                             double p_drop, unsigned long long seed, long bh_offset);

/* Number of OpenMP threads the reference runs with. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
