/*
 * oracle.c -- plain fp64 CPU oracle for Ring Self-Attention (RSA).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library. It shares no code, header,
 * table or helper with the HIP library; the two meet only through the seeded
 * inputs they are both given.
 *
 * What it computes (review page of "Sequence Parallelism: Making 4D
 * Parallelism Possible", ABSTRACT and proposed-method section): the sequence
 * is split into N chunks, one per device; each device holds the query chunk
 * of its rank, and key and value chunks travel around a ring so that every
 * query chunk meets every key chunk and every value chunk, producing the
 * ordinary self-attention output. The pages print no formula; the reading
 * taken here is the plain scaled-dot-product attention
 *
 *     O = softmax(Q K^T / sqrt(d) + M) V,
 *
 * with M = 0 for valid keys and -inf for padded keys (the key-padding mask is
 * the same for every head and query row). The oracle evaluates it through
 * RSA's own two stages, in the ring order of the query row's rank n:
 *
 *   stage 1 (keys):   for ring step t = 0..N-1, chunk c = (n - t) mod N,
 *                     score s_j = (q . k_j) / sqrt(d) for every key j of c;
 *   softmax over the full key length (all N chunks);
 *   stage 2 (values): for ring step t = 0..N-1, chunk c = (n - t) mod N,
 *                     O += P_j v_j for every key j of c.
 *
 * Backward (same page, proposed-method section: gradients also flow through
 * ring communication): the ordinary softmax-attention gradients of the loss
 * <O, dO>, accumulated over query chunks and ring steps in the same order.
 *
 * Causal variant (`causal` nonzero). The pages do not mention one; it
 * follows the standard autoregressive definition: the query at sequence
 * position i sees key j only if j <= i, on top of the key-padding mask. The
 * ring order is unchanged (chunks after the query's own are then entirely
 * hidden).
 *
 * Everything is fp64 with plain loops; no BLAS, no blocking, no reordering
 * beyond the ring order. Rows without a valid key give O = 0, lse = -inf and
 * zero gradients.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE 2
#define ORACLE_ERR_ALLOC 7

static int ring_chunk(int n, int t, int N) { return ((n - t) % N + N) % N; }

/*
 * Forward for the query rows of q ([B,H,Lq,d]); row i sits at absolute
 * sequence position qpos[i] (NULL: position i), which fixes its rank
 * n = qpos[i] / (L/N) and therefore its ring order. k, v: [B,H,L,d].
 * mask: [B,L], nonzero = valid key; NULL = all keys valid.
 * out: [B,H,Lq,d]; lse: [B,H,Lq] natural-log sum-exp of the scaled scores
 * (may be NULL). causal: hide keys j > qpos[i].
 */
int oracle_forward(const double* q, const double* k, const double* v,
                   const uint8_t* mask, int B, int H, int L, int d, int N,
                   int Lq, const int64_t* qpos, int causal, double* out, double* lse)
{
    if (B < 0 || H < 0 || L <= 0 || d <= 0 || N <= 0 || Lq < 0 || L % N != 0)
        return ORACLE_ERR_SHAPE;
    const int Lc = L / N;
    const double scale = 1.0 / sqrt((double)d);
    const int64_t rows = (int64_t)B * H * Lq;
    int status = ORACLE_OK;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        uint8_t* ok = (uint8_t*)malloc((size_t)L);
        if (!s || !ok) {
#pragma omp atomic write
            status = ORACLE_ERR_ALLOC;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t bh = r / Lq;
                const int i = (int)(r % Lq);
                const int b = (int)(bh / H);
                const int64_t pos = qpos ? qpos[i] : i;
                const int n = (int)(pos / Lc);
                const double* qi = q + r * d;
                const double* kh = k + bh * (int64_t)L * d;
                const double* vh = v + bh * (int64_t)L * d;
                const uint8_t* mb = mask ? mask + (int64_t)b * L : NULL;
                double* oi = out + r * d;

                /* stage 1: scores against every key chunk, in ring order */
                int any = 0;
                double m = -INFINITY;
                for (int t = 0; t < N; ++t) {
                    const int c = ring_chunk(n, t, N);
                    for (int j = c * Lc; j < (c + 1) * Lc; ++j) {
                        ok[j] = (mb ? (mb[j] != 0) : 1) && !(causal && j > pos);
                        if (!ok[j]) continue;
                        double dot = 0.0;
                        for (int x = 0; x < d; ++x) dot += qi[x] * kh[(int64_t)j * d + x];
                        s[j] = dot * scale;
                        if (!any || s[j] > m) m = s[j];
                        any = 1;
                    }
                }
                for (int x = 0; x < d; ++x) oi[x] = 0.0;
                if (!any) {
                    if (lse) lse[r] = -INFINITY;
                    continue;
                }
                /* softmax over the full key length: normaliser in ring order */
                double l = 0.0;
                for (int t = 0; t < N; ++t) {
                    const int c = ring_chunk(n, t, N);
                    for (int j = c * Lc; j < (c + 1) * Lc; ++j)
                        if (ok[j]) l += exp(s[j] - m);
                }
                /* stage 2: weighted values, in ring order */
                for (int t = 0; t < N; ++t) {
                    const int c = ring_chunk(n, t, N);
                    for (int j = c * Lc; j < (c + 1) * Lc; ++j) {
                        if (!ok[j]) continue;
                        const double p = exp(s[j] - m) / l;
                        for (int x = 0; x < d; ++x) oi[x] += p * vh[(int64_t)j * d + x];
                    }
                }
                if (lse) lse[r] = m + log(l);
            }
        }
        free(s);
        free(ok);
    }
    return status;
}

/*
 * Backward of the loss <O, dO> for the full sequence: q, k, v, dout, dq, dk,
 * dv are [B,H,L,d]; mask as in oracle_forward. For each head the oracle walks
 * query chunk n = 0..N-1 and, for each of its rows, the key chunks in the
 * ring order of rank n:
 *
 *   P_ij  = softmax_j(s_ij)              (recomputed from its own fp64 scores)
 *   O_i   = sum_j P_ij v_j
 *   D_i   = dO_i . O_i
 *   dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j += scale * dS_ij q_i,   dV_j += P_ij dO_i.
 *
 * causal: keys j > i are hidden from row i (P_ij = 0).
 */
int oracle_backward(const double* q, const double* k, const double* v,
                    const double* dout, const uint8_t* mask, int B, int H, int L,
                    int d, int N, int causal, double* dq, double* dk, double* dv)
{
    if (B < 0 || H < 0 || L <= 0 || d <= 0 || N <= 0 || L % N != 0)
        return ORACLE_ERR_SHAPE;
    const int Lc = L / N;
    const double scale = 1.0 / sqrt((double)d);
    const int64_t heads = (int64_t)B * H;
    const int64_t hsz = (int64_t)L * d;
    int status = ORACLE_OK;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        double* p = (double*)malloc(sizeof(double) * (size_t)L);
        uint8_t* ok = (uint8_t*)malloc((size_t)L);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s || !p || !ok || !o) {
#pragma omp atomic write
            status = ORACLE_ERR_ALLOC;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < heads; ++bh) {
                const int b = (int)(bh / H);
                const double* qh = q + bh * hsz;
                const double* kh = k + bh * hsz;
                const double* vh = v + bh * hsz;
                const double* gh = dout + bh * hsz;
                double* dqh = dq + bh * hsz;
                double* dkh = dk + bh * hsz;
                double* dvh = dv + bh * hsz;
                const uint8_t* mb = mask ? mask + (int64_t)b * L : NULL;
                memset(dqh, 0, sizeof(double) * (size_t)hsz);
                memset(dkh, 0, sizeof(double) * (size_t)hsz);
                memset(dvh, 0, sizeof(double) * (size_t)hsz);

                for (int n = 0; n < N; ++n) {
                    for (int i = n * Lc; i < (n + 1) * Lc; ++i) {
                        const double* qi = qh + (int64_t)i * d;
                        const double* gi = gh + (int64_t)i * d;
                        /* scores and softmax, keys visited in ring order */
                        int any = 0;
                        double m = -INFINITY;
                        for (int t = 0; t < N; ++t) {
                            const int c = ring_chunk(n, t, N);
                            for (int j = c * Lc; j < (c + 1) * Lc; ++j) {
                                ok[j] = (mb ? (mb[j] != 0) : 1) && !(causal && j > i);
                                if (!ok[j]) continue;
                                double dot = 0.0;
                                for (int x = 0; x < d; ++x) dot += qi[x] * kh[(int64_t)j * d + x];
                                s[j] = dot * scale;
                                if (!any || s[j] > m) m = s[j];
                                any = 1;
                            }
                        }
                        if (!any) continue; /* no valid key: zero gradients */
                        double l = 0.0;
                        for (int t = 0; t < N; ++t) {
                            const int c = ring_chunk(n, t, N);
                            for (int j = c * Lc; j < (c + 1) * Lc; ++j)
                                if (ok[j]) l += exp(s[j] - m);
                        }
                        for (int x = 0; x < d; ++x) o[x] = 0.0;
                        for (int t = 0; t < N; ++t) {
                            const int c = ring_chunk(n, t, N);
                            for (int j = c * Lc; j < (c + 1) * Lc; ++j) {
                                p[j] = ok[j] ? exp(s[j] - m) / l : 0.0;
                                for (int x = 0; x < d; ++x) o[x] += p[j] * vh[(int64_t)j * d + x];
                            }
                        }
                        double D = 0.0;
                        for (int x = 0; x < d; ++x) D += gi[x] * o[x];
                        for (int t = 0; t < N; ++t) {
                            const int c = ring_chunk(n, t, N);
                            for (int j = c * Lc; j < (c + 1) * Lc; ++j) {
                                if (!ok[j]) continue;
                                double dp = 0.0;
                                for (int x = 0; x < d; ++x) dp += gi[x] * vh[(int64_t)j * d + x];
                                const double ds = p[j] * (dp - D);
                                for (int x = 0; x < d; ++x) {
                                    dqh[(int64_t)i * d + x] += scale * ds * kh[(int64_t)j * d + x];
                                    dkh[(int64_t)j * d + x] += scale * ds * qi[x];
                                    dvh[(int64_t)j * d + x] += p[j] * gi[x];
                                }
                            }
                        }
                    }
                }
            }
        }
        free(s);
        free(p);
        free(ok);
        free(o);
    }
    return status;
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
