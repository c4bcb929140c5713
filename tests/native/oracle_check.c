/*
 * oracle_check.c -- runs the fp64 oracle (oracle/oracle.c) on small cases
 * under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_host_sanitizers.py builds it). Cases: every ring size of a
 * short sequence, key padding with fully masked rows, chunks shorter than
 * one key, one rank's rows through qpos, the causal variant, and the
 * backward, each without and with dropout. Each result is checked for
 * finiteness and for the two facts that hold whatever the inputs: a row without a visible key gives zeros
 * (lse -inf), and the forward does not depend on N.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_forward(const double* q, const double* k, const double* v, const uint8_t* mask, int B, int H, int L,
                   int d, int N, int Lq, const int64_t* qpos, int causal, int drop_p8, uint64_t drop_seed,
                   uint32_t drop_offset, double* out, double* lse);
int oracle_backward(const double* q, const double* k, const double* v, const double* dout, const uint8_t* mask,
                    int B, int H, int L, int d, int N, int causal, int drop_p8, uint64_t drop_seed,
                    uint32_t drop_offset, double* dq, double* dk, double* dv);

/* the dropout settings every case runs with (p8 = 0: none) */
static int P8 = 0;
static const uint64_t SEED = 0x0123456789ABCDEFull;
#define DROP P8, SEED, 7u

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); ++failures; } } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform_pm1(void) {   /* xorshift64*: inputs only */
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double* fill(size_t n) {
    double* a = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = uniform_pm1();
    return a;
}

static void run_case(int B, int H, int L, int d, int causal, const uint8_t* mask) {
    const size_t n = (size_t)B * H * L * d;
    double *q = fill(n), *k = fill(n), *v = fill(n), *g = fill(n);
    double *o1 = malloc(n * sizeof(double)), *oN = malloc(n * sizeof(double));
    double *l1 = malloc((size_t)B * H * L * sizeof(double)), *lN = malloc((size_t)B * H * L * sizeof(double));
    CHECK(oracle_forward(q, k, v, mask, B, H, L, d, 1, L, NULL, causal, DROP, o1, l1) == 0);
    for (int N = 1; N <= L; ++N) {
        if (L % N) continue;
        CHECK(oracle_forward(q, k, v, mask, B, H, L, d, N, L, NULL, causal, DROP, oN, lN) == 0);
        for (size_t i = 0; i < n; ++i) CHECK(isfinite(oN[i]) && fabs(oN[i] - o1[i]) < 1e-12);
        for (size_t r = 0; r < (size_t)B * H * L; ++r) {
            CHECK(lN[r] == l1[r] || fabs(lN[r] - l1[r]) < 1e-12);
            if (isinf(lN[r])) for (int x = 0; x < d; ++x) CHECK(oN[r * d + x] == 0.0);
        }
        /* the rows of one rank through qpos, with q holding only those rows */
        const int Lc = L / N, rank = N - 1;
        double* ql = malloc((size_t)B * H * Lc * d * sizeof(double));
        double* ol = malloc((size_t)B * H * Lc * d * sizeof(double));
        int64_t* pos = malloc((size_t)Lc * sizeof(int64_t));
        for (int i = 0; i < Lc; ++i) pos[i] = (int64_t)rank * Lc + i;
        for (int bh = 0; bh < B * H; ++bh)
            for (int i = 0; i < Lc; ++i)
                for (int x = 0; x < d; ++x)
                    ql[((size_t)bh * Lc + i) * d + x] = q[((size_t)bh * L + pos[i]) * d + x];
        CHECK(oracle_forward(ql, k, v, mask, B, H, L, d, N, Lc, pos, causal, DROP, ol, NULL) == 0);
        for (int bh = 0; bh < B * H; ++bh)
            for (int i = 0; i < Lc; ++i)
                for (int x = 0; x < d; ++x)
                    CHECK(fabs(ol[((size_t)bh * Lc + i) * d + x] - o1[((size_t)bh * L + pos[i]) * d + x]) < 1e-12);
        free(ql); free(ol); free(pos);
        double *dq = malloc(n * sizeof(double)), *dk = malloc(n * sizeof(double)), *dv = malloc(n * sizeof(double));
        CHECK(oracle_backward(q, k, v, g, mask, B, H, L, d, N, causal, DROP, dq, dk, dv) == 0);
        for (size_t i = 0; i < n; ++i) CHECK(isfinite(dq[i]) && isfinite(dk[i]) && isfinite(dv[i]));
        free(dq); free(dk); free(dv);
    }
    CHECK(oracle_forward(q, k, v, mask, B, H, L, d, 3, L, NULL, causal, DROP, oN, lN) == (L % 3 ? 2 : 0));
    free(q); free(k); free(v); free(g); free(o1); free(oN); free(l1); free(lN);
}

int main(void) {
    uint8_t mask[2 * 12];
    for (int j = 0; j < 12; ++j) {
        mask[j] = (uint8_t)(j < 7);          /* right padding */
        mask[12 + j] = (uint8_t)(j >= 3);    /* left padding: early causal rows see nothing */
    }
    uint8_t none[2 * 12] = {0};
    run_case(1, 2, 12, 4, 0, NULL);
    run_case(2, 2, 12, 3, 0, mask);
    run_case(2, 1, 12, 5, 1, mask);
    run_case(2, 1, 12, 2, 0, none);          /* every row without a key */
    run_case(1, 1, 1, 1, 1, NULL);
    P8 = 77;   /* the same cases with dropout */
    run_case(1, 2, 12, 4, 0, NULL);
    run_case(2, 2, 12, 3, 1, mask);
    run_case(2, 1, 12, 2, 0, none);
    if (failures) {
        fprintf(stderr, "%d oracle check(s) failed\n", failures);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
