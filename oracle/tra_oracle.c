/*
 * tra_oracle.c -- plain, slow, fp64 CPU oracle for entropy-radius block-sparse
 * spatiotemporal self-attention over a (T, H, W) video token grid.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or execute this file or the library built from it; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header, table or constant generator with the HIP path.
 *
 * What it computes (per head, batch 1, all arithmetic in IEEE fp64):
 *
 *   tokens      q, k, v are [heads][T][H][W][d] bfloat16 bit patterns, widened
 *               exactly to fp64.  Token (t, y, x) belongs to block
 *               (t, y / s, x / s) with s = sqrt(block): an s x s spatial tile
 *               inside one frame.  Tiles are counted ceil(H/s) x ceil(W/s)
 *               per frame; cells past the grid edge are not tokens.
 *               (Token Radius Attention for Efficient Video Generation,
 *               "The TRA Pipeline": tile-major layout so that spatial
 *               neighbours share a block.)
 *   probe       pooled means Qbar_b, Kbar_b over the real tokens of each
 *               block; logits s_bc = Qbar_b . Kbar_c / sqrt(d) over all nb
 *               blocks; p_b = softmax(s_b); H_b = -sum_c p_bc ln p_bc;
 *               Hn_b = H_b / ln(nb) (0 when nb = 1).
 *               (Same page, "Insight I" and "The TRA Pipeline:
 *               Entropy-to-Budget": attention entropy decides how much a query
 *               needs; here measured on block-pooled queries and keys.)
 *   radius      r_b = min(r_min + floor(Hn_b * (r_max - r_min + 1)), r_max):
 *               a linear quantiser of normalised entropy onto the integer
 *               radii r_min..r_max.  (Same page, "Budget-to-Radius": entropy
 *               becomes a per-query radius.)
 *   mask        M[i][j] = 1 iff max(|t_i - t_j|, |y_i/s - y_j/s|,
 *               |x_i/s - x_j/s|) <= r_blk(i): Chebyshev distance on block
 *               coordinates (frame, tile row, tile column) against the
 *               query's own block radius, built per query row from token
 *               coordinates.  (Same page, "Insight II": a query-centred
 *               neighbourhood in space, limited in time; Radial Attention to
 *               Accelerate Video Generation, "The idea behind Radial
 *               Attention": attention decays with spatiotemporal distance.)
 *   attention   o_i = sum_j w_ij v_j with w_ij = exp(s_ij - m_i) / sum_j
 *               exp(s_ij - m_i) over the keys with M[i][j] = 1,
 *               s_ij = q_i . k_j / sqrt(d), m_i = max_j s_ij: exact softmax
 *               attention restricted to the kept key blocks.
 *               (AB-Attention speeds up video diffusion transformers up to
 *               2.23x, first paragraph: dynamic block-sparse attention
 *               computes exact attention only on the chosen key/value
 *               blocks.)
 *   block lists L(qb) = ascending list of key blocks kb whose Chebyshev
 *               block distance from qb is <= r_qb -- exactly the blocks that
 *               hold a key of some query row of qb under M.
 *
 * A radius of ORC_RADIUS_INF (INT32_MAX) is the dense case: every key kept.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_RADIUS_INF 2147483647
#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-4)

typedef struct {
    int T, H, W, s, nby, nbx;
    long nb, N;
} orc_grid;

static double orc_lut[65536];
static int orc_lut_ready = 0;

/* bfloat16 bit pattern -> fp64, exact: a bf16 is the upper half of a binary32. */
static void orc_init_lut(void)
{
    if (orc_lut_ready) return;
    for (uint32_t h = 0; h < 65536u; ++h) {
        uint32_t u = h << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        orc_lut[h] = (double)f;
    }
    orc_lut_ready = 1;
}

static int orc_grid_make(orc_grid *g, int T, int H, int W, int block)
{
    if (T < 1 || H < 1 || W < 1 || block < 1) return ORC_EINVAL;
    int s = 0;
    while ((s + 1) * (s + 1) <= block) ++s;
    if (s * s != block) return ORC_EINVAL;
    g->T = T; g->H = H; g->W = W; g->s = s;
    g->nby = (H + s - 1) / s;
    g->nbx = (W + s - 1) / s;
    g->nb = (long)T * g->nby * g->nbx;
    g->N = (long)T * H * W;
    return ORC_OK;
}

static long orc_labs(long a) { return a < 0 ? -a : a; }

/* Chebyshev distance between the blocks of tokens (ti,yi,xi) and (tj,yj,xj). */
static long orc_block_cheb(const orc_grid *g, int ti, int yi, int xi, int tj, int yj, int xj)
{
    long dt = orc_labs((long)ti - tj);
    long dy = orc_labs((long)(yi / g->s) - (yj / g->s));
    long dx = orc_labs((long)(xi / g->s) - (xj / g->s));
    long m = dt > dy ? dt : dy;
    return m > dx ? m : dx;
}

/* Linear quantiser of normalised entropy onto r_min..r_max. */
int orc_radius(double h_norm, int r_min, int r_max)
{
    if (r_min == ORC_RADIUS_INF && r_max == ORC_RADIUS_INF) return ORC_RADIUS_INF;
    long R = (long)r_max - (long)r_min + 1;
    long r = (long)r_min + (long)floor(h_norm * (double)R);
    if (r > r_max) r = r_max;
    return (int)r;
}

/* Mean of x over the real tokens of each block: out[heads][nb][d]. */
int orc_pool(const uint16_t *x, int T, int H, int W, int heads, int d, int block, double *out)
{
    orc_grid g;
    if (!x || !out || heads < 1 || d < 1 || orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    orc_init_lut();
    long *count = (long *)calloc((size_t)g.nb, sizeof(long));
    if (!count) return ORC_ENOMEM;
    for (int t = 0; t < T; ++t)
        for (int y = 0; y < H; ++y)
            for (int xx = 0; xx < W; ++xx)
                count[((long)t * g.nby + y / g.s) * g.nbx + xx / g.s] += 1;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < heads; ++h) {
        double *o = out + (size_t)h * g.nb * d;
        memset(o, 0, sizeof(double) * (size_t)g.nb * d);
        const uint16_t *xh = x + (size_t)h * g.N * d;
        long n = 0;
        for (int t = 0; t < T; ++t)
            for (int y = 0; y < H; ++y)
                for (int xx = 0; xx < W; ++xx, ++n) {
                    long b = ((long)t * g.nby + y / g.s) * g.nbx + xx / g.s;
                    for (int c = 0; c < d; ++c) o[b * d + c] += orc_lut[xh[n * d + c]];
                }
        for (long b = 0; b < g.nb; ++b)
            for (int c = 0; c < d; ++c) o[b * d + c] /= (double)count[b];
    }
    free(count);
    return ORC_OK;
}

/*
 * Pooled-entropy probe and radius per (head, block).
 * h_norm[heads][nb] (fp64) and radius[heads][nb] (int32).
 * r_min == r_max == ORC_RADIUS_INF is the dense case: every radius infinite,
 * h_norm left at 0.
 */
int orc_probe(const uint16_t *q, const uint16_t *k, int T, int H, int W, int heads, int d,
              int block, int r_min, int r_max, double *h_norm, int32_t *radius)
{
    orc_grid g;
    if (!q || !k || !h_norm || !radius || heads < 1 || d < 1) return ORC_EINVAL;
    if (orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    int dense = (r_min == ORC_RADIUS_INF && r_max == ORC_RADIUS_INF);
    if (!dense && (r_min < 0 || r_max < r_min)) return ORC_EINVAL;
    if (dense) {
        for (long i = 0; i < (long)heads * g.nb; ++i) { h_norm[i] = 0.0; radius[i] = ORC_RADIUS_INF; }
        return ORC_OK;
    }
    size_t pooled = (size_t)heads * g.nb * d;
    double *qb = (double *)malloc(sizeof(double) * pooled);
    double *kb = (double *)malloc(sizeof(double) * pooled);
    if (!qb || !kb) { free(qb); free(kb); return ORC_ENOMEM; }
    int rc = orc_pool(q, T, H, W, heads, d, block, qb);
    if (!rc) rc = orc_pool(k, T, H, W, heads, d, block, kb);
    if (rc) { free(qb); free(kb); return rc; }
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    const double log_nb = log((double)g.nb);
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)g.nb);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for collapse(2) schedule(dynamic, 8)
        for (int h = 0; h < heads; ++h)
            for (long b = 0; b < g.nb; ++b) {
                if (!s) continue;
                const double *qv = qb + ((size_t)h * g.nb + b) * d;
                double m = -INFINITY;
                for (long c = 0; c < g.nb; ++c) {
                    const double *kv = kb + ((size_t)h * g.nb + c) * d;
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += qv[i] * kv[i];
                    s[c] = acc * inv_sqrt_d;
                    if (s[c] > m) m = s[c];
                }
                double Z = 0.0;
                for (long c = 0; c < g.nb; ++c) Z += exp(s[c] - m);
                double Hb = 0.0;
                for (long c = 0; c < g.nb; ++c) {
                    double p = exp(s[c] - m) / Z;
                    if (p > 0.0) Hb -= p * log(p);
                }
                double hn = g.nb > 1 ? Hb / log_nb : 0.0;
                h_norm[(size_t)h * g.nb + b] = hn;
                radius[(size_t)h * g.nb + b] = orc_radius(hn, r_min, r_max);
            }
        free(s);
    }
    free(qb);
    free(kb);
    return fail ? ORC_ENOMEM : ORC_OK;
}

/*
 * Key-block lists: for every (head, query block) the ascending key blocks
 * within the query block's Chebyshev radius.  idx[heads][nb][maxcnt] (only the
 * first cnt entries of a row are written), cnt[heads][nb].
 */
int orc_block_lists(const int32_t *radius, int T, int H, int W, int heads, int block,
                    long maxcnt, int32_t *idx, int32_t *cnt)
{
    orc_grid g;
    if (!radius || !idx || !cnt || heads < 1 || maxcnt < 1) return ORC_EINVAL;
    if (orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int h = 0; h < heads; ++h)
        for (long qb = 0; qb < g.nb; ++qb) {
            long r = radius[(size_t)h * g.nb + qb];
            int tq = (int)(qb / ((long)g.nby * g.nbx));
            int byq = (int)((qb / g.nbx) % g.nby);
            int bxq = (int)(qb % g.nbx);
            long c = 0;
            int32_t *row = idx + ((size_t)h * g.nb + qb) * maxcnt;
            if (r < 0) {
#pragma omp atomic write
                bad = 1;
                cnt[(size_t)h * g.nb + qb] = 0;
                continue;
            }
            for (long kb = 0; kb < g.nb; ++kb) {
                int tk = (int)(kb / ((long)g.nby * g.nbx));
                int byk = (int)((kb / g.nbx) % g.nby);
                int bxk = (int)(kb % g.nbx);
                long dt = orc_labs((long)tq - tk), dy = orc_labs((long)byq - byk), dx = orc_labs((long)bxq - bxk);
                long m = dt > dy ? dt : dy;
                m = m > dx ? m : dx;
                if (m <= r) {
                    if (c >= maxcnt) {
#pragma omp atomic write
                        bad = 1;
                        break;
                    }
                    row[c++] = (int32_t)kb;
                }
            }
            cnt[(size_t)h * g.nb + qb] = (int32_t)c;
        }
    return bad ? ORC_EINVAL : ORC_OK;
}

/*
 * Masked softmax attention for selected query rows.
 * rows[n] = head * N + token (token = (t*H + y)*W + x); out[n][d] fp64.
 * radius[heads][nb] gives each query block's radius (ORC_RADIUS_INF = dense).
 */
int orc_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       int T, int H, int W, int heads, int d, int block,
                       const int32_t *radius, long nrows, const int64_t *rows, double *out)
{
    orc_grid g;
    if (!q || !k || !v || !radius || !rows || !out || heads < 1 || d < 1 || nrows < 0) return ORC_EINVAL;
    if (orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    for (long n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= (int64_t)heads * g.N) return ORC_EINVAL;
    orc_init_lut();
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)g.N);
        long *js = (long *)malloc(sizeof(long) * (size_t)g.N);
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !js || !qi || !acc) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long n = 0; n < nrows; ++n) {
            if (!s || !js || !qi || !acc) continue;
            int h = (int)(rows[n] / g.N);
            long i = rows[n] % g.N;
            int ti = (int)(i / ((long)H * W)), yi = (int)((i / W) % H), xi = (int)(i % W);
            long bi = ((long)ti * g.nby + yi / g.s) * g.nbx + xi / g.s;
            long r = radius[(size_t)h * g.nb + bi];
            const uint16_t *qh = q + (size_t)h * g.N * d;
            const uint16_t *kh = k + (size_t)h * g.N * d;
            const uint16_t *vh = v + (size_t)h * g.N * d;
            for (int c = 0; c < d; ++c) qi[c] = orc_lut[qh[i * d + c]];
            /* explicit token mask row, then the logits of the kept keys */
            long cnt = 0;
            double m = -INFINITY;
            for (int tj = 0; tj < T; ++tj) {
                if (orc_labs((long)ti - tj) > r) continue; /* no key of this frame passes */
                for (int yj = 0; yj < H; ++yj)
                    for (int xj = 0; xj < W; ++xj) {
                        if (orc_block_cheb(&g, ti, yi, xi, tj, yj, xj) > r) continue;
                        long j = ((long)tj * H + yj) * W + xj;
                        const uint16_t *kj = kh + (size_t)j * d;
                        double dot = 0.0;
                        for (int c = 0; c < d; ++c) dot += qi[c] * orc_lut[kj[c]];
                        s[cnt] = dot * inv_sqrt_d;
                        js[cnt] = j;
                        if (s[cnt] > m) m = s[cnt];
                        ++cnt;
                    }
            }
            double Z = 0.0;
            for (int c = 0; c < d; ++c) acc[c] = 0.0;
            for (long e = 0; e < cnt; ++e) {
                double w = exp(s[e] - m);
                Z += w;
                const uint16_t *vj = vh + (size_t)js[e] * d;
                for (int c = 0; c < d; ++c) acc[c] += w * orc_lut[vj[c]];
            }
            double *o = out + (size_t)n * d;
            for (int c = 0; c < d; ++c) o[c] = acc[c] / Z;
        }
        free(s); free(js); free(qi); free(acc);
    }
    return fail ? ORC_ENOMEM : ORC_OK;
}

/* Masked softmax attention for every token: out[heads][T][H][W][d] fp64. */
int orc_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  int T, int H, int W, int heads, int d, int block,
                  const int32_t *radius, double *out)
{
    orc_grid g;
    if (heads < 1 || orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    long nrows = (long)heads * g.N;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)nrows);
    if (!rows) return ORC_ENOMEM;
    for (long n = 0; n < nrows; ++n) rows[n] = n;
    int rc = orc_attention_rows(q, k, v, T, H, W, heads, d, block, radius, nrows, rows, out);
    free(rows);
    return rc;
}

/*
 * Token-level radius policy (Token Radius Attention for Efficient Video
 * Generation, "Insight I", "Insight II" and "The TRA Pipeline":
 * Entropy-to-Budget, Budget-to-Radius, Fused CUDA Kernels), per head:
 *
 *   entropy     H_i = -sum_j p_ij ln p_ij with p_i = softmax_j(q_i . k_j / sqrt(d))
 *               over every real key token j: the entropy of query i's dense
 *               attention row (the warm-up step).
 *   budget      b_i = tau exp(H_i) keys, clamped to [1, N]: exp(H_i) is the
 *               row's effective number of keys, and b_i / N the retained
 *               fraction the page writes as tau exp(H_i) / N.
 *   radius      base radius r0_i with sum_{t'} pi (r0_i phi(|t' - t_i|))^2 = b_i
 *               over the T frames, phi(delta) = exp(-gamma delta):
 *               r0_i = sqrt(b_i / (pi S(t_i))), S(t) = sum_{t'} exp(-2 gamma |t' - t|).
 *   support     key token j is in query i's support iff
 *               (y_j - y_i)^2 + (x_j - x_i)^2 <= (r0_i phi(|t_j - t_i|))^2:
 *               a disk in every frame, shrinking with temporal distance.
 *   voting      key block K is kept for query block Q iff at least min_votes
 *               real query tokens of Q have a real key token of K in their
 *               support; lists ascending.
 *   attention   exact softmax attention of each query over every real key
 *               token of the blocks in its block's list.
 */

/* Entropy of the dense attention row of each selected query row (head * N + token). */
int orc_token_entropy_rows(const uint16_t *q, const uint16_t *k, int T, int H, int W, int heads,
                           int d, int block, long nrows, const int64_t *rows, double *ent)
{
    orc_grid g;
    if (!q || !k || !rows || !ent || heads < 1 || d < 1 || nrows < 0) return ORC_EINVAL;
    if (orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    for (long n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= (int64_t)heads * g.N) return ORC_EINVAL;
    orc_init_lut();
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)g.N);
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qi) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long n = 0; n < nrows; ++n) {
            if (!s || !qi) continue;
            int h = (int)(rows[n] / g.N);
            long i = rows[n] % g.N;
            const uint16_t *qh = q + (size_t)h * g.N * d;
            const uint16_t *kh = k + (size_t)h * g.N * d;
            for (int c = 0; c < d; ++c) qi[c] = orc_lut[qh[i * d + c]];
            double m = -INFINITY;
            for (long j = 0; j < g.N; ++j) {
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qi[c] * orc_lut[kh[j * d + c]];
                s[j] = dot * inv_sqrt_d;
                if (s[j] > m) m = s[j];
            }
            double Z = 0.0;
            for (long j = 0; j < g.N; ++j) Z += exp(s[j] - m);
            double Hi = 0.0;
            for (long j = 0; j < g.N; ++j) {
                double p = exp(s[j] - m) / Z;
                if (p > 0.0) Hi -= p * log(p);
            }
            ent[n] = Hi;
        }
        free(s); free(qi);
    }
    return fail ? ORC_ENOMEM : ORC_OK;
}

/* Base radius of every token from its entropy: ent, r0 are [heads][N]. */
int orc_token_radius(const double *ent, int T, int H, int W, int heads, double tau,
                     double gamma, double *r0)
{
    if (!ent || !r0 || T < 1 || H < 1 || W < 1 || heads < 1 || !(tau > 0.0) || !(gamma >= 0.0))
        return ORC_EINVAL;
    const long N = (long)T * H * W;
    const double pi = 3.14159265358979323846;
    for (int h = 0; h < heads; ++h)
        for (long i = 0; i < N; ++i) {
            int ti = (int)(i / ((long)H * W));
            double S = 0.0;
            for (int t = 0; t < T; ++t) S += exp(-2.0 * gamma * (double)orc_labs((long)t - ti));
            double b = tau * exp(ent[(size_t)h * N + i]);
            if (b < 1.0) b = 1.0;
            if (b > (double)N) b = (double)N;
            r0[(size_t)h * N + i] = sqrt(b / (pi * S));
        }
    return ORC_OK;
}

/*
 * Voting lists for the selected (head * nb + query block) rows, by the
 * definition: every real query token of the block against every real key token
 * of every key block.  r0 is [heads][N]; the support test uses the squared
 * radius times r2_scale (1 for the definition; 1 -+ eps brackets rounding).
 * idx[nrows][maxcnt] (first cnt entries written), cnt[nrows].
 */
int orc_token_lists(const double *r0, int T, int H, int W, int heads, int block, double gamma,
                    int min_votes, double r2_scale, long nrows, const int64_t *rows, long maxcnt,
                    int32_t *idx, int32_t *cnt)
{
    orc_grid g;
    if (!r0 || !rows || !idx || !cnt || heads < 1 || maxcnt < 1 || min_votes < 1) return ORC_EINVAL;
    if (orc_grid_make(&g, T, H, W, block) || !(gamma >= 0.0)) return ORC_EINVAL;
    for (long n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= (int64_t)heads * g.nb) return ORC_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long n = 0; n < nrows; ++n) {
        int h = (int)(rows[n] / g.nb);
        long qb = rows[n] % g.nb;
        int tq = (int)(qb / ((long)g.nby * g.nbx));
        int byq = (int)((qb / g.nbx) % g.nby), bxq = (int)(qb % g.nbx);
        long c = 0;
        for (long kb = 0; kb < g.nb; ++kb) {
            int tk = (int)(kb / ((long)g.nby * g.nbx));
            int byk = (int)((kb / g.nbx) % g.nby), bxk = (int)(kb % g.nbx);
            double phi = exp(-gamma * (double)orc_labs((long)tk - tq));
            int votes = 0;
            for (int yi = byq * g.s; yi < (byq + 1) * g.s && yi < H; ++yi)
                for (int xi = bxq * g.s; xi < (bxq + 1) * g.s && xi < W; ++xi) {
                    double r = r0[(size_t)h * g.N + ((long)tq * H + yi) * W + xi] * phi;
                    double r2 = r * r * r2_scale;
                    int hit = 0;
                    for (int yj = byk * g.s; yj < (byk + 1) * g.s && yj < H && !hit; ++yj)
                        for (int xj = bxk * g.s; xj < (bxk + 1) * g.s && xj < W && !hit; ++xj) {
                            double dy = (double)(yj - yi), dx = (double)(xj - xi);
                            if (dy * dy + dx * dx <= r2) hit = 1;
                        }
                    votes += hit;
                }
            if (votes >= min_votes) {
                if (c >= maxcnt) {
#pragma omp atomic write
                    bad = 1;
                    break;
                }
                idx[(size_t)n * maxcnt + c++] = (int32_t)kb;
            }
        }
        cnt[n] = (int32_t)c;
    }
    return bad ? ORC_EINVAL : ORC_OK;
}

/*
 * Softmax attention of selected rows over explicit key-block lists:
 * idx[heads][nb][maxcnt], cnt[heads][nb]; entries outside [0, nb) are skipped,
 * every other entry adds all real tokens of its block once more (a duplicate
 * counts twice); an empty row gives zeros.  lw[heads][nb][maxcnt] (or NULL)
 * adds the entry's log-weight to the logits of its keys: the entry's keys
 * count exp(lw) times in numerator and denominator.  out[nrows][d] fp64.
 */
int orc_attention_lists_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             int T, int H, int W, int heads, int d, int block,
                             const int32_t *idx, const int32_t *cnt, const double *lw, long maxcnt,
                             long nrows, const int64_t *rows, double *out)
{
    orc_grid g;
    if (!q || !k || !v || !idx || !cnt || !rows || !out || heads < 1 || d < 1 || maxcnt < 1)
        return ORC_EINVAL;
    if (orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    for (long n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= (int64_t)heads * g.N) return ORC_EINVAL;
    orc_init_lut();
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int fail = 0;
#pragma omp parallel
    {
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!qi || !acc) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long n = 0; n < nrows; ++n) {
            if (!qi || !acc) continue;
            int h = (int)(rows[n] / g.N);
            long i = rows[n] % g.N;
            int ti = (int)(i / ((long)H * W)), yi = (int)((i / W) % H), xi = (int)(i % W);
            long bi = ((long)ti * g.nby + yi / g.s) * g.nbx + xi / g.s;
            const uint16_t *qh = q + (size_t)h * g.N * d;
            const uint16_t *kh = k + (size_t)h * g.N * d;
            const uint16_t *vh = v + (size_t)h * g.N * d;
            for (int c = 0; c < d; ++c) qi[c] = orc_lut[qh[i * d + c]];
            long m_ = cnt[(size_t)h * g.nb + bi];
            if (m_ < 0) m_ = 0;
            if (m_ > maxcnt) m_ = maxcnt;
            const int32_t *row = idx + ((size_t)h * g.nb + bi) * maxcnt;
            const double *lrow = lw ? lw + ((size_t)h * g.nb + bi) * maxcnt : NULL;
            /* two passes over the listed keys: max, then weights */
            double m = -INFINITY;
            for (int pass = 0; pass < 2; ++pass) {
                double Z = 0.0;
                for (int c = 0; c < d; ++c) acc[c] = 0.0;
                for (long e = 0; e < m_; ++e) {
                    long kb = row[e];
                    if (kb < 0 || kb >= g.nb) continue;
                    int tk = (int)(kb / ((long)g.nby * g.nbx));
                    int byk = (int)((kb / g.nbx) % g.nby), bxk = (int)(kb % g.nbx);
                    const double bias = lrow ? lrow[e] : 0.0;
                    for (int yj = byk * g.s; yj < (byk + 1) * g.s && yj < H; ++yj)
                        for (int xj = bxk * g.s; xj < (bxk + 1) * g.s && xj < W; ++xj) {
                            long j = ((long)tk * H + yj) * W + xj;
                            double dot = 0.0;
                            for (int c = 0; c < d; ++c) dot += qi[c] * orc_lut[kh[(size_t)j * d + c]];
                            double sj = dot * inv_sqrt_d + bias;
                            if (pass == 0) {
                                if (sj > m) m = sj;
                            } else {
                                double w = exp(sj - m);
                                Z += w;
                                for (int c = 0; c < d; ++c) acc[c] += w * orc_lut[vh[(size_t)j * d + c]];
                            }
                        }
                }
                if (pass == 1) {
                    double *o = out + (size_t)n * d;
                    for (int c = 0; c < d; ++c) o[c] = Z > 0.0 ? acc[c] / Z : 0.0;
                }
            }
        }
        free(qi); free(acc);
    }
    return fail ? ORC_ENOMEM : ORC_OK;
}

/*
 * Sampling with inclusion-probability weighting (AB-Attention speeds up video
 * diffusion transformers up to 2.23x, second paragraph: key blocks are sampled
 * in proportion to importance estimates and reweighted by inverse inclusion
 * probability, so that one pass estimates dense attention), per head and
 * query block Q:
 *   importance  p_QK = softmax_K(Qbar_Q . Kbar_K / sqrt(d)) over all nb key
 *               blocks, Qbar / Kbar the means over real tokens (one query
 *               cluster per block);
 *   inclusion   pi_QK = min(1, m p_QK) for an expected budget of m blocks;
 *               pi_QQ = 1 (the own block is always kept);
 *   sample      K kept iff u_QK < pi_QK, u[heads][nb][nb] caller-supplied
 *               uniforms in [0, 1);
 *   weight      lw_QK = -ln pi_QK, added to the logits of K's keys: the
 *               self-normalised inverse-inclusion estimate of dense attention.
 * pi_scale multiplies pi before the comparison (1 for the definition; 1 -+ eps
 * brackets rounding).  idx, lw [heads][nb][maxcnt], cnt [heads][nb]; ascending.
 */
int orc_sip_lists(const uint16_t *q, const uint16_t *k, const double *u, int T, int H, int W,
                  int heads, int d, int block, double m, double pi_scale, long maxcnt,
                  int32_t *idx, int32_t *cnt, double *lw)
{
    orc_grid g;
    if (!q || !k || !u || !idx || !cnt || !lw || heads < 1 || d < 1 || maxcnt < 1 || !(m >= 0.0))
        return ORC_EINVAL;
    if (orc_grid_make(&g, T, H, W, block)) return ORC_EINVAL;
    size_t pooled = (size_t)heads * g.nb * d;
    double *qb = (double *)malloc(sizeof(double) * pooled);
    double *kb = (double *)malloc(sizeof(double) * pooled);
    if (!qb || !kb) { free(qb); free(kb); return ORC_ENOMEM; }
    int rc = orc_pool(q, T, H, W, heads, d, block, qb);
    if (!rc) rc = orc_pool(k, T, H, W, heads, d, block, kb);
    if (rc) { free(qb); free(kb); return rc; }
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)g.nb);
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(2) schedule(dynamic, 8)
        for (int h = 0; h < heads; ++h)
            for (long b = 0; b < g.nb; ++b) {
                if (!s) continue;
                const double *qv = qb + ((size_t)h * g.nb + b) * d;
                double mx = -INFINITY;
                for (long c = 0; c < g.nb; ++c) {
                    const double *kv = kb + ((size_t)h * g.nb + c) * d;
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += qv[i] * kv[i];
                    s[c] = acc * inv_sqrt_d;
                    if (s[c] > mx) mx = s[c];
                }
                double Z = 0.0;
                for (long c = 0; c < g.nb; ++c) Z += exp(s[c] - mx);
                long n = 0;
                size_t row = (size_t)h * g.nb + b;
                for (long c = 0; c < g.nb; ++c) {
                    double pi = c == b ? 1.0 : m * exp(s[c] - mx) / Z;
                    if (pi > 1.0) pi = 1.0;
                    if (u[row * g.nb + c] < pi * pi_scale) {
                        if (n >= maxcnt) {
#pragma omp atomic write
                            bad = 1;
                            break;
                        }
                        idx[row * maxcnt + n] = (int32_t)c;
                        lw[row * maxcnt + n] = -log(pi);
                        ++n;
                    }
                }
                cnt[row] = (int32_t)n;
            }
        free(s);
    }
    free(qb);
    free(kb);
    return bad ? ORC_EINVAL : ORC_OK;
}

int orc_num_threads(void) { return omp_get_max_threads(); }
