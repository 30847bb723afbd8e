/* Drives every entry point of oracle/oracle.c on small inputs held in
 * exactly sized heap buffers, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: an out-of-bounds access, a use of freed
 * memory or undefined arithmetic in the oracle aborts with a report.
 * Exit status 0 when every call ran cleanly. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_fwd(const double*, const double*, const double*, double*, double*, int, const int*, const int*, int,
                int, double, int, double, uint32_t, uint64_t, int, const int*, const uint8_t*, int, int);
void oracle_bwd(const double*, const double*, const double*, const double*, double*, double*, double*, int,
                const int*, const int*, int, int, double, int, double, uint32_t, uint64_t, int, const int*,
                const uint8_t*, int, int);
void oracle_fwd_head_tiled(const double*, const double*, const double*, long, int, int, double, int, double,
                           uint32_t, uint64_t, int, int, int, int, double*, double*, long);
void oracle_decode(const double*, const double*, const double*, double*, double*, int, int, int, int, int,
                   const int*, double, int);
void oracle_rows_head(const double*, const double*, const double*, const double*, long, int, int, double, int,
                      int, const int*, double*, double*, double*);
void oracle_keep_mask(uint64_t, uint32_t, int, int, int, uint8_t*);

static double* rnd(size_t n, unsigned* st)
{
    double* x = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) {
        *st = *st * 1664525u + 1013904223u;
        x[i] = ((double)(*st >> 8) / (double)(1u << 24)) * 2.0 - 1.0;
    }
    return x;
}

static int finite_all(const double* x, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void)
{
    unsigned st = 12345u;
    const int H = 3, d = 8;
    /* varlen batch with empty sequences; every mode of the batch calls */
    const int lens[5] = {0, 7, 0, 19, 1};
    int starts[5], T = 0;
    for (int s = 0; s < 5; ++s) { starts[s] = T; T += lens[s]; }
    const size_t n = (size_t)T * H * d;
    double *q = rnd(n, &st), *k = rnd(n, &st), *v = rnd(n, &st), *g = rnd(n, &st);
    double *o = rnd(n, &st), *lse = rnd((size_t)T * H, &st);
    double *dq = rnd(n, &st), *dk = rnd(n, &st), *dv = rnd(n, &st);
    const int blk = 4, nb = 5;  /* ceil(19 / 4) */
    uint8_t* bm = (uint8_t*)malloc((size_t)5 * H * nb * nb);
    for (int i = 0; i < 5 * H * nb * nb; ++i) bm[i] = (uint8_t)((i * 7) % 3 != 0);
    const int sel[4] = {1, 2, 3, 0};
    for (int causal = 0; causal < 2; ++causal)
        for (int drop = 0; drop < 2; ++drop)
            for (int mask = 0; mask < 2; ++mask)
                for (int pick = 0; pick < 2; ++pick) {
                    const double p = drop ? 0.3 : 0.0;
                    const uint32_t t = drop ? (uint32_t)floor(0.3 * 65536.0) : 0u;
                    oracle_fwd(q, k, v, o, lse, 5, starts, lens, H, d, 0.35, causal, p, t, 99u, pick ? 2 : 0,
                               pick ? sel : NULL, mask ? bm : NULL, blk, nb);
                    oracle_bwd(q, k, v, g, dq, dk, dv, 5, starts, lens, H, d, 0.35, causal, p, t, 99u,
                               pick ? 2 : 0, pick ? sel : NULL, mask ? bm : NULL, blk, nb);
                }
    /* tiled recurrence on one head of the longest sequence, odd tiles (its
     * output rows share the inputs' stride) */
    double* ot = (double*)malloc(sizeof(double) * (18 * (size_t)H * d + d));
    double* lt = (double*)malloc(sizeof(double) * 19);
    oracle_fwd_head_tiled(q + (size_t)starts[3] * H * d, k + (size_t)starts[3] * H * d,
                          v + (size_t)starts[3] * H * d, (long)H * d, 19, d, 0.35, 1, 0.2,
                          (uint32_t)floor(0.2 * 65536.0), 5u, 3, 1, 3, 5, ot, lt, 1);
    for (int i = 0; i < 19; ++i)
        if (!finite_all(ot + (size_t)i * H * d, d)) return 2;
    /* decode with per-sequence cache lengths, including an empty cache */
    const int B = 3, nq = 2, nk = 11, lk[3] = {11, 0, 5};
    double *dqd = rnd((size_t)B * nq * H * d, &st), *kc = rnd((size_t)B * nk * H * d, &st);
    double *vc = rnd((size_t)B * nk * H * d, &st), *od = rnd((size_t)B * nq * H * d, &st);
    double* ld = rnd((size_t)B * nq * H, &st);
    oracle_decode(dqd, kc, vc, od, ld, B, H, nq, nk, d, lk, 0.5, 1);
    oracle_decode(dqd, kc, vc, od, ld, B, H, nq, nk, d, NULL, 0.5, 0);
    /* row subset of one head */
    const int rows[3] = {0, 9, 18};
    double *orow = (double*)malloc(sizeof(double) * 3 * d), *lrow = (double*)malloc(sizeof(double) * 3);
    double* qrow = (double*)malloc(sizeof(double) * 3 * d);
    for (int causal = 0; causal < 2; ++causal)
        oracle_rows_head(q + (size_t)starts[3] * H * d, k + (size_t)starts[3] * H * d,
                         v + (size_t)starts[3] * H * d, g + (size_t)starts[3] * H * d, (long)H * d, 19, d, 0.35,
                         causal, 3, rows, orow, lrow, qrow);
    if (!finite_all(orow, 3 * (size_t)d) || !finite_all(qrow, 3 * (size_t)d)) return 3;
    uint8_t* km = (uint8_t*)malloc(19 * 19);
    oracle_keep_mask(7u, 6553u, 2, 1, 19, km);
    free(q); free(k); free(v); free(g); free(o); free(lse); free(dq); free(dk); free(dv); free(bm);
    free(ot); free(lt); free(dqd); free(kc); free(vc); free(od); free(ld); free(orow); free(lrow); free(qrow);
    free(km);
    printf("oracle sanitizer run: clean\n");
    return 0;
}
