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
 * Dropout variant (drop_p8 > 0). The pages do not mention dropout either;
 * the reading taken is attention dropout on the softmax weights: with P the
 * softmax over the full key length (its normaliser, and so lse, unchanged),
 * each weight P_ij is kept with probability 1 - p and scaled by 1 / (1 - p),
 * or set to 0, and O_i = sum_j P_ij Z_ij v_j. The probability is quantised
 * to p = drop_p8 / 256, and the keep decision of weight (b, h, i, j) is a
 * fixed function of its indices, the seed and the offset, drawn from the
 * counter-based generator Philox-4x32-10 (below): see dropout_keep().
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
 * Philox-4xW-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section on
 * the Philox family: a counter of four W-bit words and a key of two. Each of
 * the 10 rounds multiplies counter words 0 and 2 by the constants M0 and M1
 * into a high and a low W-bit half (hi0:lo0 = M0 * c0, hi1:lo1 = M1 * c2)
 * and sets the counter to (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); between
 * rounds the key words are increased by the Weyl constants W0 and W1. The
 * output is the counter after 10 rounds. The 32-bit and 64-bit instances are
 * generated from this one definition.
 */
#define MUL32(a, b, hi, lo)                              \
    do {                                                 \
        const uint64_t pr_ = (uint64_t)(a) * (uint64_t)(b); \
        hi = (uint32_t)(pr_ >> 32);                      \
        lo = (uint32_t)pr_;                              \
    } while (0)
#define MUL64(a, b, hi, lo)                                                \
    do {                                                                   \
        const unsigned __int128 pr_ = (unsigned __int128)(a) * (b);        \
        hi = (uint64_t)(pr_ >> 64);                                        \
        lo = (uint64_t)pr_;                                                \
    } while (0)
#define PHILOX_4X_10(NAME, T, MUL, M0, M1, W0, W1)                              \
    void NAME(const T ctr[4], const T key[2], T out[4])                         \
    {                                                                           \
        T c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];                   \
        T k0 = key[0], k1 = key[1];                                             \
        for (int r = 0; r < 10; ++r) {                                          \
            T hi0, lo0, hi1, lo1;                                               \
            MUL(M0, c0, hi0, lo0);                                              \
            MUL(M1, c2, hi1, lo1);                                              \
            const T n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;                     \
            c0 = n0;                                                            \
            c1 = lo1;                                                           \
            c2 = n2;                                                            \
            c3 = lo0;                                                           \
            k0 += (T)(W0);                                                      \
            k1 += (T)(W1);                                                      \
        }                                                                       \
        out[0] = c0;                                                            \
        out[1] = c1;                                                            \
        out[2] = c2;                                                            \
        out[3] = c3;                                                            \
    }

PHILOX_4X_10(oracle_philox4x32_10, uint32_t, MUL32, 0xD2511F53u, 0xCD9E8D57u, 0x9E3779B9u, 0xBB67AE85u)
PHILOX_4X_10(oracle_philox4x64_10, uint64_t, MUL64, 0xD2E7470EE14C6C93ull, 0xCA5A826395121157ull,
             0x9E3779B97F4A7C15ull, 0xBB67AE8584CAA73Bull)

/*
 * Dropout keep decision for the attention weight of query position i and key
 * position j in head bh = b * H + h (positions in the sequence, so the
 * decision does not depend on N or on the ring order):
 *   counter = ((j / 32) * 2 + bit 2 of j,  i,  bh,  offset),  key = (seed low 32 bits, seed high 32 bits);
 *   x = Philox-4x32-10(counter, key);  u = byte (j mod 4) of word ((j / 8) mod 4) of x;
 *   kept iff u >= p8.
 * One counter covers the 16 keys of a 32-key block that share bit 2 of j,
 * for one query row; a kept weight is scaled by 256 / (256 - p8).
 */
static int dropout_keep(int p8, uint64_t seed, uint32_t offset, int64_t bh, int64_t i, int64_t j)
{
    if (p8 <= 0) return 1;
    const uint32_t ctr[4] = {(uint32_t)(((j >> 5) << 1) | ((j >> 2) & 1)), (uint32_t)i, (uint32_t)bh, offset};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t x[4];
    oracle_philox4x32_10(ctr, key, x);
    const uint32_t u = (x[(j >> 3) & 3] >> (8 * (j & 3))) & 0xffu;
    return u >= (uint32_t)p8;
}

/* Keep decisions of a block of weights (for tests): keep[r * nj + c] for
 * query position i0 + r and key position j0 + c of head bh. */
void oracle_dropout_keep(int p8, uint64_t seed, uint32_t offset, int64_t bh, int64_t i0, int ni, int64_t j0,
                         int nj, uint8_t* keep)
{
    for (int r = 0; r < ni; ++r)
        for (int c = 0; c < nj; ++c)
            keep[(int64_t)r * nj + c] = (uint8_t)dropout_keep(p8, seed, offset, bh, i0 + r, j0 + c);
}

/*
 * Forward for the query rows of q ([B,H,Lq,d]); row i sits at absolute
 * sequence position qpos[i] (NULL: position i), which fixes its rank
 * n = qpos[i] / (L/N) and therefore its ring order. k, v: [B,H,L,d].
 * mask: [B,L], nonzero = valid key; NULL = all keys valid.
 * out: [B,H,Lq,d]; lse: [B,H,Lq] natural-log sum-exp of the scaled scores
 * (may be NULL). causal: hide keys j > qpos[i]. drop_p8 in [0, 256): the
 * dropout probability times 256 (0: no dropout), with drop_seed and
 * drop_offset as in dropout_keep().
 */
int oracle_forward(const double* q, const double* k, const double* v,
                   const uint8_t* mask, int B, int H, int L, int d, int N,
                   int Lq, const int64_t* qpos, int causal, int drop_p8, uint64_t drop_seed,
                   uint32_t drop_offset, double* out, double* lse)
{
    if (B < 0 || H < 0 || L <= 0 || d <= 0 || N <= 0 || Lq < 0 || L % N != 0 || drop_p8 < 0 || drop_p8 > 255)
        return ORACLE_ERR_SHAPE;
    const double keep_scale = 256.0 / (256.0 - drop_p8);
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
                /* stage 2: weighted values, in ring order (dropout acts on
                   the normalised weights) */
                for (int t = 0; t < N; ++t) {
                    const int c = ring_chunk(n, t, N);
                    for (int j = c * Lc; j < (c + 1) * Lc; ++j) {
                        if (!ok[j]) continue;
                        double p = exp(s[j] - m) / l;
                        if (drop_p8 > 0) p *= dropout_keep(drop_p8, drop_seed, drop_offset, bh, pos, j) ? keep_scale : 0.0;
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
 *   Z_ij  = dropout factor: 256 / (256 - p8) if kept, else 0 (1 without dropout)
 *   O_i   = sum_j P_ij Z_ij v_j
 *   D_i   = dO_i . O_i
 *   dP_ij = Z_ij (dO_i . v_j)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j += scale * dS_ij q_i,   dV_j += P_ij Z_ij dO_i.
 *
 * causal: keys j > i are hidden from row i (P_ij = 0). drop_*: as in
 * oracle_forward (the same keep decisions).
 */
int oracle_backward(const double* q, const double* k, const double* v,
                    const double* dout, const uint8_t* mask, int B, int H, int L,
                    int d, int N, int causal, int drop_p8, uint64_t drop_seed, uint32_t drop_offset,
                    double* dq, double* dk, double* dv)
{
    if (B < 0 || H < 0 || L <= 0 || d <= 0 || N <= 0 || L % N != 0 || drop_p8 < 0 || drop_p8 > 255)
        return ORACLE_ERR_SHAPE;
    const double keep_scale = 256.0 / (256.0 - drop_p8);
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
        double* z = (double*)malloc(sizeof(double) * (size_t)L);
        if (!s || !p || !ok || !o || !z) {
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
                                z[j] = (drop_p8 > 0 && ok[j])
                                           ? (dropout_keep(drop_p8, drop_seed, drop_offset, bh, i, j) ? keep_scale : 0.0)
                                           : 1.0;
                                for (int x = 0; x < d; ++x) o[x] += p[j] * z[j] * vh[(int64_t)j * d + x];
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
                                const double ds = p[j] * (z[j] * dp - D);
                                for (int x = 0; x < d; ++x) {
                                    dqh[(int64_t)i * d + x] += scale * ds * kh[(int64_t)j * d + x];
                                    dkh[(int64_t)j * d + x] += scale * ds * qi[x];
                                    dvh[(int64_t)j * d + x] += p[j] * z[j] * gi[x];
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
        free(z);
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
