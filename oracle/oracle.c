/*
 * Plain fp64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant generator
 * with the GPU library.
 *
 * What it computes follows the three-step definition of attention on the
 * page "企业官网建设流程全解析" (dpshk.com lab write-up), section 2.1
 * ("三步计算背后的显存账本"): S = Q K^T, P = row softmax(S), O = P V.  The
 * scores are multiplied by the scale (1/sqrt(d) by default) before the
 * softmax, which is how the plain einsum reference in the code-comparison
 * section of the tiemojia.cn PyTorch article forms them.  Tensors
 * use the [batch, seq, heads, head_dim] layout named in section 4.2 of the
 * lab write-up.  Each (sequence, head) pair is computed on its own:
 *
 *   step 1  S[i][j] = scale * sum_c q[i][c] k[j][c]   for visible j
 *   step 2  P[i][j] = exp(S[i][j] - m_i) / sum_j' exp(S[i][j'] - m_i)
 *           (m_i = row max; a full two-pass softmax over the whole row)
 *           LSE_i   = m_i + ln sum_j exp(S[i][j] - m_i)
 *   dropout Z[i][j] = P[i][j] * keep(i,j) / (1 - p)   (else Z = P)
 *   step 3  O[i]    = sum_j Z[i][j] v[j]
 *
 * "Visible" means j <= i for causal attention, every j < L otherwise.
 * With a block mask (block-sparse attention, the block-sparse mode named in
 * section 5.2 of the coreui.cn FlashAttention-2 how-to), element (i, j) is
 * visible only if
 * in addition the mask entry of query block i / blk and key block j / blk is
 * nonzero.  A row with no visible key has O = 0, LSE = -inf and no gradient.
 * The N x N matrices S, P (and dP in the backward) are materialised per
 * head on purpose: this is the standard algorithm the tiled method is
 * exactly equivalent to (lab write-up section 3.2).
 *
 * The backward is the textbook analytic gradient of L = sum O*dO:
 *   dZ[i][j] = dO_i . v_j,  dP[i][j] = dZ[i][j] * keep/(1-p)
 *   dS[i][j] = P[i][j] (dP[i][j] - sum_k P[i][k] dP[i][k])
 *   dQ_i = scale sum_j dS[i][j] k_j,  dK_j = scale sum_i dS[i][j] q_i,
 *   dV_j = sum_i Z[i][j] dO_i.
 *
 * oracle_fwd_head_tiled() runs the online-softmax recurrences of the lab
 * write-up, section 3.2 (running row max m and row sum l, O rescaled by
 * e^{m - m_new} per column block, divided by l at the end), in fp64.  It
 * exists only to check that the tiled recurrence equals the definition.
 *
 * Dropout keep bits come from Philox-4x32-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), written here from
 * that paper: key = (seed low word, seed high word); counter =
 * (row i, col j / 8, head h, batch-or-sequence b).  The four 32-bit output
 * words are read as eight 16-bit values, value v = low half of word v/2 for
 * even v and high half for odd v; column j uses value j mod 8, and the
 * element is kept iff that value >= thresh, where the caller passes
 * thresh = floor(p * 2^16).  Row and column indices are local to the
 * sequence.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- Philox */

static void philox_round(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {            /* Weyl key schedule between rounds */
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        philox_round(c, k0, k1);
    }
    memcpy(out, c, sizeof(c));
}

int oracle_keep(uint64_t seed, uint32_t thresh, int b, int h, int i, int j)
{
    uint32_t ctr[4] = {(uint32_t)i, (uint32_t)j >> 3, (uint32_t)h, (uint32_t)b};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    uint32_t v = (j & 1) ? out[(j & 7) >> 1] >> 16 : out[(j & 7) >> 1] & 0xFFFFu;
    return v >= thresh;
}

/* Keep mask of one (b, h) head, row-major L x L bytes (1 = kept). */
void oracle_keep_mask(uint64_t seed, uint32_t thresh, int b, int h, int L, uint8_t* mask)
{
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < L; ++j)
            mask[(size_t)i * L + j] = (uint8_t)oracle_keep(seed, thresh, b, h, i, j);
}

/* --------------------------------------------------------- common pieces */

typedef struct {
    double scale;     /* multiplies q.k */
    int causal;
    int dropout;      /* 0: no dropout */
    double keep_scale;/* 1/(1-p) */
    uint32_t thresh;  /* floor(p * 2^16) */
    uint64_t seed;
    int b, h;         /* counter indices of this head */
    const uint8_t* bmask; /* NULL, or [nbq][nbk] block mask of this head */
    int blk, nbk;     /* block size (rows and columns), mask row length */
} head_args;

/* Columns 0 .. n_visible - 1 may be visible (causal prefix); visible() is
 * the full test. */
static int n_visible(const head_args* a, int i, int L) { return a->causal ? i + 1 : L; }
static int visible(const head_args* a, int i, int j)
{
    if (a->causal && j > i) return 0;
    return !a->bmask || a->bmask[(size_t)(i / a->blk) * a->nbk + j / a->blk] != 0;
}

static double dot(const double* x, const double* y, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += x[c] * y[c];
    return s;
}

/* Steps 1 and 2 for one head: fills P (L x L, zero where not visible) and lse. */
static void softmax_rows(const double* q, const double* k, long ld, int L, int d,
                         const head_args* a, double* P, double* lse)
{
    #pragma omp parallel for schedule(dynamic, 8)
    for (int i = 0; i < L; ++i) {
        double* row = P + (size_t)i * L;
        int nv = n_visible(a, i, L);
        double m = -INFINITY;
        int any = 0;
        for (int j = 0; j < nv; ++j) {
            if (!visible(a, i, j)) continue;
            row[j] = a->scale * dot(q + (size_t)i * ld, k + (size_t)j * ld, d);
            if (row[j] > m) m = row[j];
            any = 1;
        }
        if (!any) {                 /* no visible key: P = 0, LSE = -inf */
            for (int j = 0; j < L; ++j) row[j] = 0.0;
            if (lse) lse[i] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int j = 0; j < nv; ++j)
            if (visible(a, i, j)) sum += exp(row[j] - m);
        for (int j = 0; j < nv; ++j) row[j] = visible(a, i, j) ? exp(row[j] - m) / sum : 0.0;
        for (int j = nv; j < L; ++j) row[j] = 0.0;
        if (lse) lse[i] = m + log(sum);
    }
}

static double keep_factor(const head_args* a, int i, int j)
{
    if (!a->dropout) return 1.0;
    return oracle_keep(a->seed, a->thresh, a->b, a->h, i, j) ? a->keep_scale : 0.0;
}

/* --------------------------------------------------------------- forward */

/* One head.  q, k, v, o point at row 0 of the head; rows are ld elements
 * apart (ld = H*d for a [tokens, H, d] tensor).  lse is indexed lse[i*lse_ld]. */
void oracle_fwd_head(const double* q, const double* k, const double* v, long ld, int L, int d,
                     double scale, int causal, double dropout_p, uint32_t thresh, uint64_t seed,
                     int b, int h, const uint8_t* bmask, int blk, int nbk,
                     double* o, double* lse, long lse_ld)
{
    if (L <= 0) return;
    head_args a = {scale, causal, dropout_p > 0.0, 1.0 / (1.0 - dropout_p), thresh, seed, b, h,
                   bmask, blk, nbk};
    double* P = (double*)malloc(sizeof(double) * (size_t)L * L);
    double* l = (double*)malloc(sizeof(double) * (size_t)L);
    softmax_rows(q, k, ld, L, d, &a, P, l);
    #pragma omp parallel for schedule(dynamic, 8)
    for (int i = 0; i < L; ++i) {
        double* oi = o + (size_t)i * ld;
        for (int c = 0; c < d; ++c) oi[c] = 0.0;
        int nv = n_visible(&a, i, L);
        for (int j = 0; j < nv; ++j) {
            if (!visible(&a, i, j)) continue;
            double z = P[(size_t)i * L + j] * keep_factor(&a, i, j);
            const double* vj = v + (size_t)j * ld;
            for (int c = 0; c < d; ++c) oi[c] += z * vj[c];
        }
        lse[(size_t)i * lse_ld] = l[i];
    }
    free(l);
    free(P);
}

/* Online-softmax recurrence with Br x Bc blocks (fp64), for the
 * tiled-equals-definition check only. */
void oracle_fwd_head_tiled(const double* q, const double* k, const double* v, long ld, int L, int d,
                           double scale, int causal, double dropout_p, uint32_t thresh, uint64_t seed,
                           int b, int h, int Br, int Bc, double* o, double* lse, long lse_ld)
{
    if (L <= 0) return;
    head_args a = {scale, causal, dropout_p > 0.0, 1.0 / (1.0 - dropout_p), thresh, seed, b, h,
                   NULL, 1, 0};
    double* acc = (double*)malloc(sizeof(double) * (size_t)Br * d);
    double* m = (double*)malloc(sizeof(double) * (size_t)Br);
    double* l = (double*)malloc(sizeof(double) * (size_t)Br);
    double* s = (double*)malloc(sizeof(double) * (size_t)Br * Bc);
    for (int i0 = 0; i0 < L; i0 += Br) {
        int nr = L - i0 < Br ? L - i0 : Br;
        for (int r = 0; r < nr; ++r) { m[r] = -INFINITY; l[r] = 0.0; }
        memset(acc, 0, sizeof(double) * (size_t)nr * d);
        for (int j0 = 0; j0 < L; j0 += Bc) {
            int nc = L - j0 < Bc ? L - j0 : Bc;
            for (int r = 0; r < nr; ++r) {
                int i = i0 + r;
                /* S_ij block row and its local max over visible columns */
                double bm = -INFINITY;
                for (int t = 0; t < nc; ++t) {
                    int j = j0 + t;
                    if (causal && j > i) { s[(size_t)r * Bc + t] = -INFINITY; continue; }
                    double sv = scale * dot(q + (size_t)i * ld, k + (size_t)j * ld, d);
                    s[(size_t)r * Bc + t] = sv;
                    if (sv > bm) bm = sv;
                }
                if (bm == -INFINITY) continue;          /* block fully masked for this row */
                double m_new = m[r] > bm ? m[r] : bm;
                double alpha = exp(m[r] - m_new);       /* e^{m - m_new}; 0 on the first block */
                double* ar = acc + (size_t)r * d;
                for (int c = 0; c < d; ++c) ar[c] *= alpha;
                l[r] *= alpha;
                for (int t = 0; t < nc; ++t) {
                    double sv = s[(size_t)r * Bc + t];
                    if (sv == -INFINITY) continue;
                    double e = exp(sv - m_new);
                    l[r] += e;                           /* l excludes dropout */
                    double z = e * keep_factor(&a, i, j0 + t);
                    const double* vj = v + (size_t)(j0 + t) * ld;
                    for (int c = 0; c < d; ++c) ar[c] += z * vj[c];
                }
                m[r] = m_new;
            }
        }
        for (int r = 0; r < nr; ++r) {
            double* oi = o + (size_t)(i0 + r) * ld;
            for (int c = 0; c < d; ++c) oi[c] = acc[(size_t)r * d + c] / l[r];
            lse[(size_t)(i0 + r) * lse_ld] = m[r] + log(l[r]);
        }
    }
    free(s); free(l); free(m); free(acc);
}

/* -------------------------------------------------------------- backward */

void oracle_bwd_head(const double* q, const double* k, const double* v, const double* dout,
                     long ld, int L, int d, double scale, int causal, double dropout_p,
                     uint32_t thresh, uint64_t seed, int b, int h,
                     const uint8_t* bmask, int blk, int nbk,
                     double* dq, double* dk, double* dv)
{
    if (L <= 0) return;
    head_args a = {scale, causal, dropout_p > 0.0, 1.0 / (1.0 - dropout_p), thresh, seed, b, h,
                   bmask, blk, nbk};
    size_t LL = (size_t)L * L;
    double* P = (double*)malloc(sizeof(double) * LL);
    double* dS = (double*)malloc(sizeof(double) * LL);
    double* Z = (double*)malloc(sizeof(double) * LL);
    softmax_rows(q, k, ld, L, d, &a, P, NULL);
    /* dP and dS, one row at a time */
    #pragma omp parallel for schedule(dynamic, 8)
    for (int i = 0; i < L; ++i) {
        int nv = n_visible(&a, i, L);
        double* dsr = dS + (size_t)i * L;
        double* zr = Z + (size_t)i * L;
        const double* pr = P + (size_t)i * L;
        double rowdot = 0.0;
        for (int j = 0; j < nv; ++j) {
            if (!visible(&a, i, j)) { dsr[j] = 0.0; zr[j] = 0.0; continue; }
            double kf = keep_factor(&a, i, j);
            double dp = dot(dout + (size_t)i * ld, v + (size_t)j * ld, d) * kf;
            dsr[j] = dp;
            zr[j] = pr[j] * kf;
            rowdot += pr[j] * dp;
        }
        for (int j = 0; j < nv; ++j) dsr[j] = pr[j] * (dsr[j] - rowdot);  /* 0 where invisible */
        for (int j = nv; j < L; ++j) { dsr[j] = 0.0; zr[j] = 0.0; }
    }
    /* dQ = scale dS K */
    #pragma omp parallel for schedule(dynamic, 8)
    for (int i = 0; i < L; ++i) {
        double* g = dq + (size_t)i * ld;
        for (int c = 0; c < d; ++c) g[c] = 0.0;
        for (int j = 0; j < L; ++j) {
            double w = dS[(size_t)i * L + j];
            if (w == 0.0) continue;
            const double* kj = k + (size_t)j * ld;
            for (int c = 0; c < d; ++c) g[c] += w * kj[c];
        }
        for (int c = 0; c < d; ++c) g[c] *= scale;
    }
    /* dK = scale dS^T Q,  dV = Z^T dO */
    #pragma omp parallel for schedule(dynamic, 8)
    for (int j = 0; j < L; ++j) {
        double* gk = dk + (size_t)j * ld;
        double* gv = dv + (size_t)j * ld;
        for (int c = 0; c < d; ++c) { gk[c] = 0.0; gv[c] = 0.0; }
        for (int i = 0; i < L; ++i) {
            double w = dS[(size_t)i * L + j];
            double z = Z[(size_t)i * L + j];
            const double* qi = q + (size_t)i * ld;
            const double* gi = dout + (size_t)i * ld;
            for (int c = 0; c < d; ++c) { gk[c] += w * qi[c]; gv[c] += z * gi[c]; }
        }
        for (int c = 0; c < d; ++c) gk[c] *= scale;
    }
    free(Z); free(dS); free(P);
}

/* ---------------------------------------------------- whole-batch drivers */

/* Tensors are [tokens, H, d] (contiguous); sequence s occupies tokens
 * starts[s] .. starts[s] + lens[s] - 1.  lse is [tokens, H].  If sel is not
 * NULL only the nsel (sequence, head) pairs sel[2t], sel[2t+1] are computed;
 * other outputs are left untouched. */
static void run_pairs(int nseq, const int* starts, const int* lens, int H, int nsel, const int* sel,
                      void (*fn)(int s, int h, void* ctx), void* ctx)
{
    int npairs = sel ? nsel : nseq * H;
    if (npairs == 1) {               /* one head: let the head function use the threads */
        fn(sel ? sel[0] : 0, sel ? sel[1] : 0, ctx);
        return;
    }
    #pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < npairs; ++t) {
        int s = sel ? sel[2 * t] : t / H;
        int h = sel ? sel[2 * t + 1] : t % H;
        fn(s, h, ctx);
    }
    (void)starts; (void)lens;
}

typedef struct {
    const double *q, *k, *v, *dout;
    double *o, *lse, *dq, *dk, *dv;
    const int *starts, *lens;
    int H, d, causal;
    double scale, p;
    uint32_t thresh;
    uint64_t seed;
    const uint8_t* bmask;   /* NULL, or [nseq][H][nb][nb] */
    int blk, nb;
} batch_ctx;

static const uint8_t* head_mask(const batch_ctx* c, int s, int h)
{
    return c->bmask ? c->bmask + ((size_t)s * c->H + h) * (size_t)c->nb * c->nb : NULL;
}

static void fwd_one(int s, int h, void* vctx)
{
    batch_ctx* c = (batch_ctx*)vctx;
    long ld = (long)c->H * c->d;
    size_t off = (size_t)c->starts[s] * ld + (size_t)h * c->d;
    oracle_fwd_head(c->q + off, c->k + off, c->v + off, ld, c->lens[s], c->d, c->scale, c->causal,
                    c->p, c->thresh, c->seed, s, h, head_mask(c, s, h), c->blk, c->nb, c->o + off,
                    c->lse + (size_t)c->starts[s] * c->H + h, c->H);
}

static void bwd_one(int s, int h, void* vctx)
{
    batch_ctx* c = (batch_ctx*)vctx;
    long ld = (long)c->H * c->d;
    size_t off = (size_t)c->starts[s] * ld + (size_t)h * c->d;
    oracle_bwd_head(c->q + off, c->k + off, c->v + off, c->dout + off, ld, c->lens[s], c->d,
                    c->scale, c->causal, c->p, c->thresh, c->seed, s, h,
                    head_mask(c, s, h), c->blk, c->nb, c->dq + off, c->dk + off, c->dv + off);
}

/* bmask: NULL, or a [nseq][H][nb][nb] uint8 block mask with blocks of blk
 * rows and columns (nb = ceil(max sequence length / blk)). */
void oracle_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                int nseq, const int* starts, const int* lens, int H, int d, double scale, int causal,
                double dropout_p, uint32_t thresh, uint64_t seed, int nsel, const int* sel,
                const uint8_t* bmask, int blk, int nb)
{
    batch_ctx c = {q, k, v, NULL, o, lse, NULL, NULL, NULL, starts, lens, H, d, causal,
                   scale, dropout_p, thresh, seed, bmask, blk, nb};
    run_pairs(nseq, starts, lens, H, nsel, sel, fwd_one, &c);
}

void oracle_bwd(const double* q, const double* k, const double* v, const double* dout,
                double* dq, double* dk, double* dv,
                int nseq, const int* starts, const int* lens, int H, int d, double scale, int causal,
                double dropout_p, uint32_t thresh, uint64_t seed, int nsel, const int* sel,
                const uint8_t* bmask, int blk, int nb)
{
    batch_ctx c = {q, k, v, dout, NULL, NULL, dq, dk, dv, starts, lens, H, d, causal,
                   scale, dropout_p, thresh, seed, bmask, blk, nb};
    run_pairs(nseq, starts, lens, H, nsel, sel, bwd_one, &c);
}

/* ------------------------------------------------------------ KV-cache decode */

/* Decode step of inference with a KV cache (the cache use described in
 * section 6.1 of the lab write-up): nq new query tokens attend to the lk
 * cached keys and values of their sequence, the new tokens being the last nq
 * positions of it, so that with causal masking query t (0 <= t < nq) sees
 * keys j <= lk - nq + t (bottom-right alignment).  Steps 1-3 as above on the
 * nq x lk score matrix.  q, o: [B, nq, H, d]; k, v: [B, nk_max, H, d] of
 * which the first lk[b] tokens are valid; lse: [B, nq, H].  A query that
 * sees no key gets O = 0, LSE = -inf. */
void oracle_decode(const double* q, const double* k, const double* v, double* o, double* lse,
                   int B, int H, int nq, int nk_max, int d, const int* lk, double scale, int causal)
{
    #pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            int L = lk ? lk[b] : nk_max;
            double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
            for (int t = 0; t < nq; ++t) {
                const double* qt = q + (((size_t)b * nq + t) * H + h) * d;
                double* ot = o + (((size_t)b * nq + t) * H + h) * d;
                int nv = causal ? L - nq + t + 1 : L;
                if (nv > L) nv = L;
                for (int c = 0; c < d; ++c) ot[c] = 0.0;
                if (nv <= 0) { lse[((size_t)b * nq + t) * H + h] = -INFINITY; continue; }
                double m = -INFINITY;
                for (int j = 0; j < nv; ++j) {
                    s[j] = scale * dot(qt, k + (((size_t)b * nk_max + j) * H + h) * d, d);
                    if (s[j] > m) m = s[j];
                }
                double sum = 0.0;
                for (int j = 0; j < nv; ++j) sum += exp(s[j] - m);
                for (int j = 0; j < nv; ++j) {
                    double pj = exp(s[j] - m) / sum;
                    const double* vj = v + (((size_t)b * nk_max + j) * H + h) * d;
                    for (int c = 0; c < d; ++c) ot[c] += pj * vj[c];
                }
                lse[((size_t)b * nq + t) * H + h] = m + log(sum);
            }
            free(s);
        }
}

/* Selected query rows of one head, for sequences too long to hold P:
 * for each listed row i, the definition restricted to that row (no dropout,
 * no block mask) -- s_j = scale q_i.k_j over the visible keys j, m = max s,
 * p_j = e^{s_j - m} / sum_j e^{s_j - m}, o_i = sum_j p_j v_j and
 * LSE_i = m + ln sum_j e^{s_j - m} (lab write-up, section 2.1); and, when
 * dout is given, the same analytic backward as oracle_bwd_head restricted
 * to row i: D_i = dO_i.o_i, dp_j = dO_i.v_j, dS_j = p_j (dp_j - D_i),
 * dQ_i = scale sum_j dS_j k_j.  q, k, v, dout hold rows of one head with
 * ld elements between tokens; o, dq are [nrows][d], lse [nrows]. */
void oracle_rows_head(const double* q, const double* k, const double* v, const double* dout, long ld, int L,
                      int d, double scale, int causal, int nrows, const int* rows, double* o, double* lse,
                      double* dq)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        const int i = rows[r];
        const int nv = causal ? i + 1 : L;
        double* p = (double*)malloc(sizeof(double) * (size_t)nv);
        double m = -INFINITY;
        for (int j = 0; j < nv; ++j) {
            p[j] = scale * dot(q + (size_t)i * ld, k + (size_t)j * ld, d);
            if (p[j] > m) m = p[j];
        }
        double sum = 0.0;
        for (int j = 0; j < nv; ++j) sum += exp(p[j] - m);
        for (int j = 0; j < nv; ++j) p[j] = exp(p[j] - m) / sum;
        lse[r] = m + log(sum);
        double* oi = o + (size_t)r * d;
        for (int c = 0; c < d; ++c) oi[c] = 0.0;
        for (int j = 0; j < nv; ++j)
            for (int c = 0; c < d; ++c) oi[c] += p[j] * v[(size_t)j * ld + c];
        if (dout) {
            const double* g = dout + (size_t)i * ld;
            const double D = dot(g, oi, d);
            double* dqi = dq + (size_t)r * d;
            for (int c = 0; c < d; ++c) dqi[c] = 0.0;
            for (int j = 0; j < nv; ++j) {
                const double ds = p[j] * (dot(g, v + (size_t)j * ld, d) - D);
                for (int c = 0; c < d; ++c) dqi[c] += scale * ds * k[(size_t)j * ld + c];
            }
        }
        free(p);
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
