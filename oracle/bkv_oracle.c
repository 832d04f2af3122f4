/*
 * bkv_oracle.c -- CPU oracle for the BeaconKV eviction step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under long_reasoning_decode_amd/) never calls it and shares no
 * code, header, table or constant with it.
 *
 * Sources (cited by page title and section; "Notes" below means the reading
 * notes "BeaconKV：用历史查询代表保护长推理的远程回看" on liuzhao09.github.io,
 * "Summary" means the rcap.io post "BeaconKV: Key-Value Cache Compression
 * Guided by Beacon Queries"):
 *   Notes §2.1, Eq. 4-6     attention weights w_{tau,j}, max and mean pooling
 *   Notes §2.2, App. Alg. 1 farthest point sampling (FPS), and its prefill use
 *   Notes §2.2, Eq. 9       continual FPS buffer bounds B_Q^min / B_Q^max
 *   Notes §2.2, App. Alg. 2 cycle: freeze beacons, collect recents, evict,
 *                           merge beacons + recents by FPS
 *   Notes §2.3, Eq. 7-8     RoPE realignment, GQA max-pool score, keep set
 *   Summary, pseudocode     per-step order: append, FPS when >= 32, evict
 *
 * Precision.  Scores are computed in fp64 (their plain definition).  Two
 * steps produce integers or bf16 codes from floating point, so they are
 * specified in fp32 with a fixed operation order, which the GPU kernels
 * reproduce exactly:
 *   - RoPE rotation of a bf16 query, rounded to bf16 (round to nearest even);
 *   - FPS cosines, mean cosines and argmin decisions.
 * This file must be compiled with -ffp-contract=off (see oracle/build.py).
 *
 * Pins: every function here is checked in tests/test_oracle_*.py against
 * closed forms, hand-derived cases, library routines or brute force.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Configuration of one call: its own definition, not the library's struct. */
typedef struct {
    int n_layers, batch, hq, hkv, d;
    int cap;          /* rows allocated per unit's K/V */
    int budget;       /* B_KV^min: rows kept */
    int n_prefix;     /* forced prefix keep */
    int n_recent_kv;  /* forced recent-window keep */
    int n_beacon;     /* B_Q^min */
    int n_recent_q;   /* recent queries; B_Q^max = n_beacon + n_recent_q */
    int causal;       /* recent query i sees only slots <= N - n_recent_q + i */
    int qcap;         /* rows allocated per query buffer (>= B_Q^max) */
    int pool_mean;    /* 0: max pooling (Eq. 7); 1: mean pooling (Eq. 6) */
    int beacon_src;   /* 0: continual FPS; 1: initial queries; 2: random history (reservoir) */
    unsigned seed;    /* key of the random-history draws */
    double theta;     /* RoPE base */
    /* Global unit index of each unit passed, for calls on a sample of the
     * workload's units: the random-history draws are keyed by the global
     * buffer index u * G + h.  NULL: the units passed are 0, 1, ... */
    const long long *unit_ids;
} bkvo_cfg;

static long long global_unit(const bkvo_cfg *c, int u) { return c->unit_ids ? c->unit_ids[u] : (long long)u; }

enum { BKVO_SRC_FPS = 0, BKVO_SRC_INITIAL = 1, BKVO_SRC_RANDOM = 2, BKVO_SRC_NAIVE = 3 };

int bkvo_reservoir_slot(unsigned seed, long long uq, int n, int n_beacon);

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32.                                                            */

static float bf2f(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f2u(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* Round an fp32 value to the nearest bf16, ties to the even code.
 * Written from the definition: the two bf16 neighbours are the truncation
 * and the next code away from zero; pick the nearer in exact (fp64)
 * arithmetic, on a tie the one whose last mantissa bit is 0.  NaN maps to a
 * quiet NaN of the same sign; values that round beyond the largest finite
 * bf16 become infinity (the next code above 0x7F7F is 0x7F80). */
uint16_t bkvo_f32_to_bf16(float f)
{
    uint32_t u = f2u(f);
    if (isnan(f))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint16_t lo = (uint16_t)(u >> 16);          /* truncation toward zero */
    if ((u & 0xFFFFu) == 0)
        return lo;                               /* exact */
    uint16_t hi = (uint16_t)(lo + 1);            /* next code away from zero */
    double x = fabs((double)f);
    double vlo = fabs((double)bf2f(lo));
    double vhi;
    if ((hi & 0x7FFFu) == 0x7F80u)               /* rounding up reaches inf */
        vhi = ldexp(1.0, 128);                   /* the value inf stands for */
    else
        vhi = fabs((double)bf2f(hi));
    double dlo = x - vlo, dhi = vhi - x;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;                  /* tie: even code */
}

/* ------------------------------------------------------------------------ */
/* RoPE (Notes §2.3: beacons rotated to step t, recents to their own
 * positions).  The pages only name RoPE(q, t); the convention taken is the
 * one of the model families they evaluate: pairs (i, i + d/2) rotated by the
 * angle p * theta^(-2i/d), i < d/2.                                         */

/* cs[((p - p0) * (d/2) + i) * 2 + {0,1}] = {cos, sin} of p * theta^(-2i/d),
 * computed in fp64 and rounded to fp32. */
void bkvo_rope_table(double theta, int d, int p0, int p1, float *cs)
{
    int h = d / 2;
    for (int p = p0; p < p1; ++p) {
        for (int i = 0; i < h; ++i) {
            double freq = pow(theta, -2.0 * (double)i / (double)d);
            double ang = (double)p * freq;
            float *o = cs + ((size_t)(p - p0) * h + i) * 2;
            o[0] = (float)cos(ang);
            o[1] = (float)sin(ang);
        }
    }
}

/* Rotate one bf16 row by the fp32 table row cs_p (d/2 {cos, sin} pairs), in
 * fp32 with each product and sum rounded separately, then round to bf16. */
static void rope_row_with(const uint16_t *x, int d, const float *cs_p, uint16_t *y)
{
    int h = d / 2;
    for (int i = 0; i < h; ++i) {
        float c = cs_p[2 * i], s = cs_p[2 * i + 1];
        float a = bf2f(x[i]), b = bf2f(x[i + h]);
        float ac = a * c, bs = b * s, bc = b * c, as = a * s;
        float y0 = ac - bs;
        float y1 = bc + as;
        y[i] = bkvo_f32_to_bf16(y0);
        y[i + h] = bkvo_f32_to_bf16(y1);
    }
}

/* Rotate one row at position p (table row computed on the spot). */
void bkvo_rope_row(const uint16_t *x, int d, double theta, int p, uint16_t *y)
{
    float *cs = (float *)malloc(sizeof(float) * (size_t)d);
    bkvo_rope_table(theta, d, p, p + 1, cs);
    rope_row_with(x, d, cs, y);
    free(cs);
}

/* ------------------------------------------------------------------------ */
/* FPS (Notes §2.2, App. Alg. 1).
 *   a_i = (1/n) sum_j cos(q_i, q_j);  p = argmin_i a_i;  I = {p};
 *   S_j = cos(q_j, q_p);  repeat: r = argmin_{j not in I} S_j,
 *   I <- I + {r},  S_j <- max(S_j, cos(q_j, q_r)),  until |I| = m.
 * fp32, fixed order:
 *   dot_ij = fmaf over k = 0..d-1 ascending, starting from +0;
 *   nrm_i  = sqrtf(dot_ii);
 *   cos_ij = 0 if nrm_i or nrm_j is 0, else dot_ij / (nrm_i * nrm_j);
 *   a_i    = (cos_i0 + cos_i1 + ... + cos_i(n-1), left to right) / n;
 * the sum in a_i includes j = i (the page's sum runs over all N); every
 * argmin takes the lowest index among equal values.  If n <= m no sampling
 * happens and the selection is 0..n-1.
 * Writes the selected indices in selection order; returns their count.     */
int bkvo_fps(const uint16_t *X, int n, int d, int m, int *sel)
{
    if (n <= 0 || m <= 0) return 0;
    if (n <= m) {
        for (int i = 0; i < n; ++i) sel[i] = i;
        return n;
    }
    float *x = (float *)malloc(sizeof(float) * (size_t)n * d);
    float *cs = (float *)malloc(sizeof(float) * (size_t)n * n);
    float *nrm = (float *)malloc(sizeof(float) * (size_t)n);
    float *S = (float *)malloc(sizeof(float) * (size_t)n);
    char *taken = (char *)calloc((size_t)n, 1);
    for (int i = 0; i < n * d; ++i) x[i] = bf2f(X[i]);

    for (int i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int k = 0; k < d; ++k) acc = fmaf(x[i * d + k], x[i * d + k], acc);
        nrm[i] = sqrtf(acc);
    }
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < n; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < d; ++k) acc = fmaf(x[i * d + k], x[j * d + k], acc);
            float c;
            if (nrm[i] == 0.0f || nrm[j] == 0.0f) c = 0.0f;
            else c = acc / (nrm[i] * nrm[j]);
            cs[i * n + j] = c;
        }
    }
    /* seed: lowest mean cosine */
    int p = 0;
    float best = 0.0f;
    for (int i = 0; i < n; ++i) {
        float s = 0.0f;
        for (int j = 0; j < n; ++j) s = s + cs[i * n + j];
        float a = s / (float)n;
        if (i == 0 || a < best) { best = a; p = i; }
    }
    int cnt = 0;
    sel[cnt++] = p;
    taken[p] = 1;
    for (int j = 0; j < n; ++j) S[j] = cs[j * n + p];
    while (cnt < m) {
        int r = -1;
        float bv = 0.0f;
        for (int j = 0; j < n; ++j) {
            if (taken[j]) continue;
            if (r < 0 || S[j] < bv) { r = j; bv = S[j]; }
        }
        sel[cnt++] = r;
        taken[r] = 1;
        for (int j = 0; j < n; ++j) {
            float c = cs[j * n + r];
            if (c > S[j]) S[j] = c;
        }
    }
    free(x); free(cs); free(nrm); free(S); free(taken);
    return cnt;
}

/* Diagnostic twin of bkvo_fps in fp64 (same steps, fp64 arithmetic).  For
 * each pick it also reports the margin: the gap between the chosen value and
 * the next-best candidate (a_i for the seed, S_j afterwards).  A pick whose
 * margin is tiny is one where rounding may legitimately decide. */
int bkvo_fps_f64(const uint16_t *X, int n, int d, int m, int *sel, double *margin)
{
    if (n <= 0 || m <= 0) return 0;
    if (n <= m) {
        for (int i = 0; i < n; ++i) { sel[i] = i; if (margin) margin[i] = INFINITY; }
        return n;
    }
    double *x = (double *)malloc(sizeof(double) * (size_t)n * d);
    double *cs = (double *)malloc(sizeof(double) * (size_t)n * n);
    double *nrm = (double *)malloc(sizeof(double) * (size_t)n);
    double *S = (double *)malloc(sizeof(double) * (size_t)n);
    char *taken = (char *)calloc((size_t)n, 1);
    for (int i = 0; i < n * d; ++i) x[i] = (double)bf2f(X[i]);
    for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += x[i * d + k] * x[i * d + k];
        nrm[i] = sqrt(acc);
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += x[i * d + k] * x[j * d + k];
            cs[i * n + j] = (nrm[i] == 0.0 || nrm[j] == 0.0) ? 0.0 : acc / (nrm[i] * nrm[j]);
        }
    double *a = (double *)malloc(sizeof(double) * (size_t)n);
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int j = 0; j < n; ++j) s += cs[i * n + j];
        a[i] = s / n;
    }
    int p = 0;
    for (int i = 1; i < n; ++i) if (a[i] < a[p]) p = i;
    double second = INFINITY;
    for (int i = 0; i < n; ++i) if (i != p && a[i] < second) second = a[i];
    int cnt = 0;
    if (margin) margin[cnt] = second - a[p];
    sel[cnt++] = p;
    taken[p] = 1;
    for (int j = 0; j < n; ++j) S[j] = cs[j * n + p];
    while (cnt < m) {
        int r = -1;
        for (int j = 0; j < n; ++j) {
            if (taken[j]) continue;
            if (r < 0 || S[j] < S[r]) r = j;
        }
        double sec = INFINITY;
        for (int j = 0; j < n; ++j) if (!taken[j] && j != r && S[j] < sec) sec = S[j];
        if (margin) margin[cnt] = sec - S[r];
        sel[cnt++] = r;
        taken[r] = 1;
        for (int j = 0; j < n; ++j) if (cs[j * n + r] > S[j]) S[j] = cs[j * n + r];
    }
    free(x); free(cs); free(nrm); free(S); free(taken); free(a);
    return cnt;
}

/* ------------------------------------------------------------------------ */
/* FPS over a long query set: the prefill initialisation (Notes §2.2: at
 * prefill the first representatives are sampled from the prompt's queries,
 * with the steps of App. Alg. 1).  The steps and fp32 operations are those of
 * bkvo_fps except the seed.  With n in the thousands the n x n mean cosines
 * cost O(n^2 d); they are taken instead from the identity
 *   a_i = (1/n) sum_j cos(q_i, q_j) = (1/n) u_i . sum_j u_j,  u_j = q_j / |q_j|,
 * which holds exactly in real arithmetic (cos is the dot product of the unit
 * rows; a zero row has u = 0, matching cos = 0).  fp32, fixed order:
 *   nrm_j  = sqrtf(fmaf chain of q_j . q_j over k ascending, from +0);
 *   inv_j  = 1 / nrm_j, or 0 when nrm_j is 0;   u_j[k] = q_j[k] * inv_j;
 *   s[k]   = pairwise sum of u_j[k] over j (pairwise_sum below);
 *   a_i    = (fmaf chain of u_i[k] * s[k] over k ascending, from +0) / n;
 * then p = argmin a_i and the S updates of bkvo_fps, with cos_ij =
 * dot_ij / (nrm_i * nrm_j) computed from the bf16 rows as there.          */

/* Pairwise (cascade) summation of x[lo .. lo + len), len a power of two:
 * the sum of the left half plus the sum of the right half; terms at or
 * beyond n are zero.  The result does not depend on how far the range is
 * padded, since a zero subtree adds +0. */
static float pairwise_sum(const float *x, size_t stride, int n, int lo, int len)
{
    if (lo >= n) return 0.0f;
    if (len == 1) return x[(size_t)lo * stride];
    int h = len / 2;
    return pairwise_sum(x, stride, n, lo, h) + pairwise_sum(x, stride, n, lo + h, h);
}

/* Pairwise sum of x[0 .. n) (exported for its own pins). */
float bkvo_pairwise_sum(const float *x, int n)
{
    int len = 1;
    while (len < n) len *= 2;
    return n > 0 ? pairwise_sum(x, 1, n, 0, len) : 0.0f;
}

int bkvo_fps_long(const uint16_t *X, int n, int d, int m, int *sel)
{
    if (n <= 0 || m <= 0) return 0;
    if (n <= m) {
        for (int i = 0; i < n; ++i) sel[i] = i;
        return n;
    }
    float *x = (float *)malloc(sizeof(float) * (size_t)n * d);
    float *u = (float *)malloc(sizeof(float) * (size_t)n * d);
    float *nrm = (float *)malloc(sizeof(float) * (size_t)n);
    float *ssum = (float *)malloc(sizeof(float) * (size_t)d);
    float *S = (float *)malloc(sizeof(float) * (size_t)n);
    char *taken = (char *)calloc((size_t)n, 1);
    for (size_t i = 0; i < (size_t)n * d; ++i) x[i] = bf2f(X[i]);
    for (int j = 0; j < n; ++j) {
        float acc = 0.0f;
        for (int k = 0; k < d; ++k) acc = fmaf(x[(size_t)j * d + k], x[(size_t)j * d + k], acc);
        nrm[j] = sqrtf(acc);
        float inv = nrm[j] == 0.0f ? 0.0f : 1.0f / nrm[j];
        for (int k = 0; k < d; ++k) u[(size_t)j * d + k] = x[(size_t)j * d + k] * inv;
    }
    int len = 1;
    while (len < n) len *= 2;
    for (int k = 0; k < d; ++k) ssum[k] = pairwise_sum(u + k, (size_t)d, n, 0, len);
    /* seed: lowest mean cosine */
    int p = 0;
    float best = 0.0f;
    for (int i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int k = 0; k < d; ++k) acc = fmaf(u[(size_t)i * d + k], ssum[k], acc);
        float a = acc / (float)n;
        if (i == 0 || a < best) { best = a; p = i; }
    }
    int cnt = 0;
    sel[cnt++] = p;
    taken[p] = 1;
    int r = p;
    for (int j = 0; j < n; ++j) S[j] = -INFINITY;
    while (cnt < m) {
        /* fold in the cosines to the last pick, then take the farthest row */
        for (int j = 0; j < n; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < d; ++k) acc = fmaf(x[(size_t)j * d + k], x[(size_t)r * d + k], acc);
            float c = (nrm[j] == 0.0f || nrm[r] == 0.0f) ? 0.0f : acc / (nrm[j] * nrm[r]);
            if (c > S[j]) S[j] = c;
        }
        int nx = -1;
        float bv = 0.0f;
        for (int j = 0; j < n; ++j) {
            if (taken[j]) continue;
            if (nx < 0 || S[j] < bv) { nx = j; bv = S[j]; }
        }
        r = nx;
        sel[cnt++] = r;
        taken[r] = 1;
    }
    free(x); free(u); free(nrm); free(ssum); free(S); free(taken);
    return cnt;
}

/* FPS exactly as the page defines it (Notes §2.2, App. Alg. 1), in fp64,
 * with no shortcut: every mean cosine a_i = (1/n) sum_j cos(q_i, q_j) is
 * summed from the n cosines of row i (O(n^2 d)); the greedy steps keep
 * S_j = max over the rows taken of cos(q_j, q_r) and take the untaken row
 * of smallest S (lowest index on ties).  Cosines are computed on the fly
 * (memory O(n d)).  This is the reference for FPS over many rows that does
 * not share the fp32 operation order of bkvo_fps_long.
 *
 * Replay: when forced is non-NULL, step s takes forced[s] instead of its own
 * argmin (the rows taken so far are then those of the replayed selection),
 * and regret[s] is the fp64 value of the row taken minus the smallest value
 * over the untaken rows (a_i at the seed, S_j afterwards): 0 where the replay
 * takes an optimal row, +INFINITY where forced[s] is out of range or already
 * taken (the replay then goes on from the optimal row, which sel records).
 * margin[s] (nullable) is the gap between the smallest and the second
 * smallest value at that step (+INFINITY with one candidate): the room fp
 * rounding has to decide the step either way.  sel receives the rows taken.
 * Returns the number of steps, min(n, m) (the selection 0..n-1 with zero
 * regret and infinite margins when n <= m).                              */
static double cos64(const double *x, const double *nrm, int d, int i, int j)
{
    if (nrm[i] == 0.0 || nrm[j] == 0.0) return 0.0;
    double acc = 0.0;
    for (int k = 0; k < d; ++k) acc += x[(size_t)i * d + k] * x[(size_t)j * d + k];
    return acc / (nrm[i] * nrm[j]);
}

int bkvo_fps_plain(const uint16_t *X, int n, int d, int m, const int *forced, int *sel, double *regret,
                   double *margin)
{
    if (n <= 0 || m <= 0) return 0;
    if (n <= m) {
        for (int i = 0; i < n; ++i) {
            sel[i] = i;
            if (regret) regret[i] = 0.0;
            if (margin) margin[i] = INFINITY;
        }
        return n;
    }
    double *x = (double *)malloc(sizeof(double) * (size_t)n * d);
    double *nrm = (double *)malloc(sizeof(double) * (size_t)n);
    double *v = (double *)malloc(sizeof(double) * (size_t)n);   /* a_i, then S_j */
    char *taken = (char *)calloc((size_t)n, 1);
    for (size_t i = 0; i < (size_t)n * d; ++i) x[i] = (double)bf2f(X[i]);
    for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += x[(size_t)i * d + k] * x[(size_t)i * d + k];
        nrm[i] = sqrt(acc);
    }
    for (int i = 0; i < n; ++i) {
        double sum = 0.0;
        for (int j = 0; j < n; ++j) sum += cos64(x, nrm, d, i, j);
        v[i] = sum / n;
    }
    int cnt = 0;
    while (cnt < m) {
        /* the best and second-best untaken values (first index on ties) */
        int best = -1;
        double second = INFINITY;
        for (int j = 0; j < n; ++j) {
            if (taken[j]) continue;
            if (best < 0 || v[j] < v[best]) {
                if (best >= 0) second = v[best];
                best = j;
            } else if (v[j] < second) {
                second = v[j];
            }
        }
        int r = forced ? forced[cnt] : best;
        double rg;
        if (r < 0 || r >= n || taken[r]) {
            rg = INFINITY;
            r = best;   /* continue the replay from the optimal row */
        } else {
            rg = v[r] - v[best];
        }
        if (regret) regret[cnt] = rg;
        if (margin) margin[cnt] = second - v[best];
        sel[cnt++] = r;
        taken[r] = 1;
        if (cnt == 1) {   /* S_j starts as the cosine to the seed */
            for (int j = 0; j < n; ++j) v[j] = cos64(x, nrm, d, j, r);
        } else {
            for (int j = 0; j < n; ++j) {
                double c = cos64(x, nrm, d, j, r);
                if (c > v[j]) v[j] = c;
            }
        }
    }
    free(x); free(nrm); free(v); free(taken);
    return cnt;
}

/* Prefill initialisation of nbuf query buffers (global indices from buf0)
 * from their prompt queries q_prompt[b][0 .. P), under the beacon source src:
 *   FPS     -- the buffer becomes FPS_long(prompt, n_beacon), survivors in
 *              ascending prompt order, count min(P, n_beacon);
 *   initial -- the first min(P, n_beacon) prompt rows, count min(P, n_beacon);
 *   random  -- the prompt rows offered in order to the reservoir, count P.
 * sel_out[b][i] (nullable): the i-th pick (FPS) or the prompt row held in
 * slot i (the other sources), -1 past the last.
 * q_prompt: [nbuf][P][d]; qbuf: [nbuf][qcap][d]; qcount: [nbuf].           */
void bkvo_prefill(int nbuf, int P, int d, int n_beacon, int qcap, int src, unsigned seed, long long buf0,
                  const uint16_t *q_prompt, uint16_t *qbuf, int32_t *qcount, int32_t *sel_out)
{
    int *sel = (int *)malloc(sizeof(int) * (size_t)(n_beacon + 1));
    char *keep = (char *)malloc((size_t)(P > 0 ? P : 1));
    for (int b = 0; b < nbuf; ++b) {
        const uint16_t *src_rows = q_prompt + (size_t)b * P * d;
        uint16_t *buf = qbuf + (size_t)b * qcap * d;
        int got;
        if (src == BKVO_SRC_FPS) {
            got = bkvo_fps_long(src_rows, P, d, n_beacon, sel);
            memset(keep, 0, (size_t)(P > 0 ? P : 1));
            for (int i = 0; i < got; ++i) keep[sel[i]] = 1;
            int w = 0;
            for (int i = 0; i < P; ++i)
                if (keep[i]) { memcpy(buf + (size_t)w * d, src_rows + (size_t)i * d, sizeof(uint16_t) * (size_t)d); ++w; }
            qcount[b] = w;
        } else if (src == BKVO_SRC_INITIAL) {
            got = P < n_beacon ? P : n_beacon;
            for (int i = 0; i < got; ++i) sel[i] = i;
            memcpy(buf, src_rows, sizeof(uint16_t) * (size_t)got * d);
            qcount[b] = got;
        } else {
            got = P < n_beacon ? P : n_beacon;
            for (int i = 0; i < n_beacon; ++i) sel[i] = -1;
            for (int n = 0; n < P; ++n) {
                int j = bkvo_reservoir_slot(seed, buf0 + b, n, n_beacon);
                if (j >= 0) {
                    memcpy(buf + (size_t)j * d, src_rows + (size_t)n * d, sizeof(uint16_t) * (size_t)d);
                    sel[j] = n;
                }
            }
            qcount[b] = P;
        }
        if (sel_out)
            for (int i = 0; i < n_beacon; ++i) sel_out[(size_t)b * n_beacon + i] = i < got ? sel[i] : -1;
    }
    free(sel);
    free(keep);
}

/* ------------------------------------------------------------------------ */
/* Continual FPS buffer update (Notes §2.2, Eq. 9; Summary, pseudocode).
 * For each query buffer b: append q_new[b] at slot qcount[b] and increment;
 * if the count reaches B_Q^max = n_beacon + n_recent_q, replace the buffer
 * by FPS(buffer, n_beacon), survivors kept in ascending slot order, and set
 * the count to n_beacon.  sel_out[b][0..n_beacon) receives the selection
 * order, or -1 when no sampling ran (sel_out may be NULL).
 * qbuf: [nbuf][qcap][d] bf16; qcount: [nbuf]; q_new: [nbuf][d].            */
void bkvo_fps_update(int nbuf, int qcap, int d, int n_beacon, int n_recent_q,
                     uint16_t *qbuf, int32_t *qcount, const uint16_t *q_new,
                     int32_t *sel_out)
{
    int bqmax = n_beacon + n_recent_q;
    int *sel = (int *)malloc(sizeof(int) * (size_t)(bqmax + 1));
    uint16_t *tmp = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)qcap * d);
    for (int b = 0; b < nbuf; ++b) {
        uint16_t *buf = qbuf + (size_t)b * qcap * d;
        int c = qcount[b];
        /* a valid buffer holds fewer than B_Q^max rows between calls */
        if (c < 0) c = 0;
        if (c > bqmax - 1) c = bqmax - 1;
        memcpy(buf + (size_t)c * d, q_new + (size_t)b * d, sizeof(uint16_t) * (size_t)d);
        c += 1;
        if (sel_out)
            for (int i = 0; i < n_beacon; ++i) sel_out[(size_t)b * n_beacon + i] = -1;
        if (c >= bqmax) {
            int got = bkvo_fps(buf, c, d, n_beacon, sel);
            if (sel_out)
                for (int i = 0; i < got; ++i) sel_out[(size_t)b * n_beacon + i] = sel[i];
            /* survivors in ascending slot order */
            char *keep = (char *)calloc((size_t)c, 1);
            for (int i = 0; i < got; ++i) keep[sel[i]] = 1;
            int w = 0;
            for (int i = 0; i < c; ++i)
                if (keep[i]) {
                    memcpy(tmp + (size_t)w * d, buf + (size_t)i * d, sizeof(uint16_t) * (size_t)d);
                    ++w;
                }
            memcpy(buf, tmp, sizeof(uint16_t) * (size_t)w * d);
            free(keep);
            c = w;
        }
        qcount[b] = c;
    }
    free(sel);
    free(tmp);
}

/* Compression at the freeze point of a cycle (Notes §2.2 App. Alg. 2: the
 * beacons a cycle is scored with stand for every query it collected).  Each
 * buffer whose count (clamped to [0, B_Q^max - 1] as in bkvo_fps_update)
 * exceeds n_beacon becomes FPS(buffer, n_beacon), survivors in ascending slot
 * order, count n_beacon; the others are left alone (sel_out -1s).  With
 * n_beacon = 0 every non-empty buffer is emptied.                         */
void bkvo_fps_compress(int nbuf, int qcap, int d, int n_beacon, int n_recent_q,
                       uint16_t *qbuf, int32_t *qcount, int32_t *sel_out)
{
    int bqmax = n_beacon + n_recent_q;
    int *sel = (int *)malloc(sizeof(int) * (size_t)(bqmax + 1));
    uint16_t *tmp = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)qcap * d);
    for (int b = 0; b < nbuf; ++b) {
        uint16_t *buf = qbuf + (size_t)b * qcap * d;
        int c = qcount[b];
        if (c < 0) c = 0;
        if (c > bqmax - 1) c = bqmax - 1;
        if (sel_out)
            for (int i = 0; i < n_beacon; ++i) sel_out[(size_t)b * n_beacon + i] = -1;
        if (c <= n_beacon) continue;
        if (n_beacon == 0) { qcount[b] = 0; continue; }
        int got = bkvo_fps(buf, c, d, n_beacon, sel);
        if (sel_out)
            for (int i = 0; i < got; ++i) sel_out[(size_t)b * n_beacon + i] = sel[i];
        char *keep = (char *)calloc((size_t)c, 1);
        for (int i = 0; i < got; ++i) keep[sel[i]] = 1;
        int w = 0;
        for (int i = 0; i < c; ++i)
            if (keep[i]) {
                memcpy(tmp + (size_t)w * d, buf + (size_t)i * d, sizeof(uint16_t) * (size_t)d);
                ++w;
            }
        memcpy(buf, tmp, sizeof(uint16_t) * (size_t)w * d);
        free(keep);
        qcount[b] = w;
    }
    free(sel);
    free(tmp);
}

/* ------------------------------------------------------------------------ */
/* Other sources of beacons (the ablations of Notes §3.2 Fig. 6 and §3.4
 * Table 3), with the same buffer, count and cycle as continual FPS:
 *   initial  -- Initial+Recent: the beacons are the first n_beacon queries the
 *               buffer is offered and never change (later queries are
 *               ignored; the merge keeps the buffer);
 *   random   -- random history: the beacons are a uniform random sample of
 *               n_beacon of all queries offered so far, kept by reservoir
 *               sampling (Vitter's Algorithm R).  The count is the number of
 *               queries offered; the n-th (0-based) goes to slot n while
 *               n < n_beacon, else to slot j = floor(r (n + 1) / 2^32) if
 *               j < n_beacon, with r a 32-bit draw.  Collection-phase queries
 *               are offered as they come, the cycle's recent queries at the
 *               merge, in ring order, so the beacons stay frozen while the
 *               recents are collected (App. Alg. 2).
 * The draws r are the first output word of Philox4x32-10 (Salmon, Moraes,
 * Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with
 * counter (n, buffer index, 0, 0) and key (seed, 0).                       */

/* Philox4x32-10: ten rounds; in each, the counter words (c0, c1, c2, c3)
 * become (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)),
 * and the key is then bumped by the Weyl constants. */
void bkvo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0; k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Reservoir slot of the n-th query offered to buffer uq, or -1 (dropped). */
int bkvo_reservoir_slot(unsigned seed, long long uq, int n, int n_beacon)
{
    if (n < n_beacon) return n;
    uint32_t ctr[4] = {(uint32_t)n, (uint32_t)uq, 0u, 0u}, key[2] = {seed, 0u}, out[4];
    bkvo_philox4x32_10(ctr, key, out);
    uint32_t j = (uint32_t)(((uint64_t)out[0] * (uint64_t)((uint32_t)n + 1u)) >> 32);
    return j < (uint32_t)n_beacon ? (int)j : -1;
}

/* Offer one pre-RoPE query to buffer uq (rows buf, count *cnt) under the
 * initial or random rule. */
static void offer(const bkvo_cfg *c, long long uq, uint16_t *buf, int32_t *cnt, const uint16_t *q)
{
    int d = c->d, n = *cnt < 0 ? 0 : *cnt;
    if (c->beacon_src == BKVO_SRC_INITIAL) {
        if (n < c->n_beacon) {
            memcpy(buf + (size_t)n * d, q, sizeof(uint16_t) * (size_t)d);
            *cnt = n + 1;
        }
        return;
    }
    int j = bkvo_reservoir_slot(c->seed, uq, n, c->n_beacon);
    if (j >= 0) memcpy(buf + (size_t)j * d, q, sizeof(uint16_t) * (size_t)d);
    *cnt = n + 1;
}

/* The per-step buffer update under the configured source, for nbuf buffers
 * whose global indices start at buf0: continual FPS (bkvo_fps_update), or one
 * offer per buffer.  sel_out (nullable) as for bkvo_fps_update (-1s when no
 * sampling ran, always for the other sources). */
void bkvo_beacon_update(const bkvo_cfg *c, int nbuf, long long buf0, uint16_t *qbuf, int32_t *qcount,
                        const uint16_t *q_new, int32_t *sel_out)
{
    if (c->beacon_src == BKVO_SRC_FPS) {
        bkvo_fps_update(nbuf, c->qcap, c->d, c->n_beacon, c->n_recent_q, qbuf, qcount, q_new, sel_out);
        return;
    }
    if (c->beacon_src == BKVO_SRC_NAIVE) {   /* the beacons come from the history at each eviction */
        if (sel_out)
            for (size_t i = 0; i < (size_t)nbuf * c->n_beacon; ++i) sel_out[i] = -1;
        return;
    }
    for (int b = 0; b < nbuf; ++b) {
        offer(c, buf0 + b, qbuf + (size_t)b * c->qcap * c->d, qcount + b, q_new + (size_t)b * c->d);
        if (sel_out)
            for (int i = 0; i < c->n_beacon; ++i) sel_out[(size_t)b * c->n_beacon + i] = -1;
    }
}

/* ------------------------------------------------------------------------ */
/* Attention weights of one observation row (Notes §2.1, Eq. 4), fp64:
 *   z_j = (q . k_j) / sqrt(d) for visible j <= vis (j < N);
 *   w_j = exp(z_j - c),  c = m + ln sum_l exp(z_l - m),  m = max_l z_l;
 *   w_j = 0 for j > vis.  Returns c (or -inf if nothing is visible).      */
double bkvo_row_weights(const uint16_t *q, const uint16_t *K, int N, int d, int vis, double *w)
{
    int last = vis < N - 1 ? vis : N - 1;
    double inv = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int j = 0; j <= last; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += (double)bf2f(q[k]) * (double)bf2f(K[(size_t)j * d + k]);
        w[j] = acc * inv;
        if (w[j] > m) m = w[j];
    }
    if (last < 0) {
        for (int j = 0; j < N; ++j) w[j] = 0.0;
        return -INFINITY;
    }
    double l = 0.0;
    for (int j = 0; j <= last; ++j) l += exp(w[j] - m);
    double c = m + log(l);
    for (int j = 0; j <= last; ++j) w[j] = exp(w[j] - c);
    for (int j = last + 1; j < N; ++j) w[j] = 0.0;
    return c;
}

/* ------------------------------------------------------------------------ */
/* Per-unit arrays.  A unit is one (layer, batch, KV head); its q-heads are
 * the G = hq / hkv heads h with h / G equal to the KV head.  All per-unit
 * inputs are passed unit-major:
 *   K, V       [U][cap][d]           bf16, K holds post-RoPE keys
 *   qbuf       [U][G][qcap][d]       pre-RoPE buffers (modified by merge)
 *   qcount     [U][G]                (modified by merge)
 *   q_recent   [U][G][n_recent_q][d] pre-RoPE recent queries
 *   pos_recent [U][n_recent_q]       positions of the recent queries
 *   t          [U]                   current step (beacons are rotated to it)
 * Outputs: scores [U][N] fp64, idx [U][budget] (-1 beyond min(N, budget)),
 * moved [U] (#{r : idx[r] != r}), fps_sel [U][G][n_beacon].               */

typedef struct {
    const bkvo_cfg *cfg;
    int N;
    uint16_t *K, *V, *qbuf;
    int32_t *qcount;
    const uint16_t *q_recent;
    const int32_t *pos_recent, *t;
    double *scores;
    int32_t *idx, *moved, *fps_sel;
    int do_score, do_select, do_compact, do_merge;
    int u0, u1;
} unit_job;

/* Beacons at an eviction are the current representatives: the first
 * min(qcount, n_beacon) buffer rows, which hold the last FPS or merge output.
 * Rows appended after it (slots >= n_beacon) form the buffer's recent set,
 * which the cycle clears when the beacons are frozen (Notes §2.2, App. Alg. 2). */
static int n_beacons_of(const bkvo_cfg *c, int qcount)
{
    int nb = qcount < c->n_beacon ? qcount : c->n_beacon;
    return nb < 0 ? 0 : nb;
}

/* Fold one observation row's weights into the unit's score. */
static void pool_row(const bkvo_cfg *c, const double *w, int N, double *score)
{
    for (int j = 0; j < N; ++j) {
        if (c->pool_mean) score[j] += w[j];
        else if (w[j] > score[j]) score[j] = w[j];
    }
}

/* Score of one unit (Notes §2.3, Eq. 7): max over the group's heads and all
 * their observation rows of the row's attention weight.
 * With pool_mean the max becomes the mean of Notes §2.1 Eq. 6, taken over the
 * same rows of all the group's heads (the Max/Mean ablation of Notes §3.3
 * Table 2 pools both over the queries and over the heads).  A row's weight on
 * a key it does not see is 0, and the divisor counts every observation row:
 * sum over the heads h of min(qcount_h, n_beacon) + n_recent_q. */
static void score_unit(const bkvo_cfg *c, int N, int u, const uint16_t *K,
                       const uint16_t *qbuf, const int32_t *qcount,
                       const uint16_t *q_recent, const int32_t *pos_recent,
                       const int32_t *t, double *score)
{
    int d = c->d, G = c->hq / c->hkv;
    double *w = (double *)malloc(sizeof(double) * (size_t)N);
    uint16_t *qh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    for (int j = 0; j < N; ++j) score[j] = 0.0;
    const uint16_t *Ku = K + (size_t)u * c->cap * d;
    int rows = 0;
    for (int h = 0; h < G; ++h) {
        const uint16_t *buf = qbuf + ((size_t)u * G + h) * c->qcap * d;
        int nb = n_beacons_of(c, qcount[(size_t)u * G + h]);
        for (int s = 0; s < nb; ++s) {
            bkvo_rope_row(buf + (size_t)s * d, d, c->theta, t[u], qh);
            bkvo_row_weights(qh, Ku, N, d, N - 1, w);
            pool_row(c, w, N, score);
            ++rows;
        }
        const uint16_t *rec = q_recent + ((size_t)u * G + h) * c->n_recent_q * d;
        for (int i = 0; i < c->n_recent_q; ++i) {
            ++rows;
            int vis = c->causal ? N - c->n_recent_q + i : N - 1;
            if (vis < 0) continue;
            bkvo_rope_row(rec + (size_t)i * d, d, c->theta,
                          pos_recent[(size_t)u * c->n_recent_q + i], qh);
            bkvo_row_weights(qh, Ku, N, d, vis, w);
            pool_row(c, w, N, score);
        }
    }
    if (c->pool_mean && rows > 0)
        for (int j = 0; j < N; ++j) score[j] /= rows;
    free(w);
    free(qh);
}

typedef struct { double s; int j; } cand;

static int cand_cmp(const void *a, const void *b)
{
    const cand *x = (const cand *)a, *y = (const cand *)b;
    if (x->s > y->s) return -1;     /* higher score first */
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);  /* then lower index */
}

/* Keep set (Notes §2.3, Eq. 8), 0-based:
 *   I_keep = [0, n_prefix) U [N - n_recent_kv, N);
 *   k_sel = budget - |I_keep|;  I_final = sort(I_keep U TopK(score, k_sel,
 *   excluding I_keep)), ranking by score descending, then index ascending.
 * If N <= budget everything is kept.  Writes idx[0..min(N,budget)) ascending
 * and -1 after that.  Returns #{r : idx[r] != r}. */
int bkvo_select(const double *score, int N, int budget, int n_prefix, int n_recent_kv, int32_t *idx)
{
    if (N <= budget) {
        for (int r = 0; r < budget; ++r) idx[r] = r < N ? r : -1;
        return 0;
    }
    char *keep = (char *)calloc((size_t)N, 1);
    int np = n_prefix < N ? n_prefix : N;
    int rs = N - n_recent_kv < 0 ? 0 : N - n_recent_kv;
    int nk = 0;
    for (int j = 0; j < N; ++j)
        if (j < np || j >= rs) { keep[j] = 1; ++nk; }
    int k_sel = budget - nk;
    cand *cs = (cand *)malloc(sizeof(cand) * (size_t)N);
    int nc = 0;
    for (int j = 0; j < N; ++j)
        if (!keep[j]) { cs[nc].s = score[j]; cs[nc].j = j; ++nc; }
    qsort(cs, (size_t)nc, sizeof(cand), cand_cmp);
    for (int i = 0; i < k_sel && i < nc; ++i) keep[cs[i].j] = 1;
    int r = 0, moved = 0;
    for (int j = 0; j < N && r < budget; ++j)
        if (keep[j]) { idx[r] = j; if (j != r) ++moved; ++r; }
    for (; r < budget; ++r) idx[r] = -1;
    free(keep);
    free(cs);
    return moved;
}

/* In-place compaction (Notes §2.3, Eq. 8: K^ = K[:, I_final, :], same for V):
 * row r of the result is row idx[r] of the input, r < count of valid idx. */
static void compact_rows(uint16_t *X, int d, int N, const int32_t *idx, int budget)
{
    uint16_t *tmp = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)budget * d);
    int n = 0;
    for (int r = 0; r < budget; ++r) {
        if (idx[r] < 0 || idx[r] >= N) break;
        memcpy(tmp + (size_t)r * d, X + (size_t)idx[r] * d, sizeof(uint16_t) * (size_t)d);
        ++n;
    }
    memcpy(X, tmp, sizeof(uint16_t) * (size_t)n * d);
    free(tmp);
}

/* Merge at the end of a cycle (Notes §2.2, App. Alg. 2): the beacons and the
 * recent queries, both pre-RoPE, are joined (beacons first, then recents in
 * order) and FPS(., n_beacon) gives the next cycle's buffer, survivors in
 * candidate order; the count becomes their number. */
static void merge_unit(const bkvo_cfg *c, int u, uint16_t *qbuf, int32_t *qcount,
                       const uint16_t *q_recent, int32_t *fps_sel)
{
    int d = c->d, G = c->hq / c->hkv;
    if (c->beacon_src != BKVO_SRC_FPS) {
        /* initial, naive: nothing changes; random: the recents are offered in ring order */
        for (int h = 0; h < G; ++h) {
            size_t b = (size_t)u * G + h;
            if (c->beacon_src == BKVO_SRC_RANDOM)
                for (int i = 0; i < c->n_recent_q; ++i)
                    offer(c, global_unit(c, u) * G + h, qbuf + b * c->qcap * d, qcount + b,
                          q_recent + (b * c->n_recent_q + i) * d);
            if (fps_sel)
                for (int i = 0; i < c->n_beacon; ++i) fps_sel[b * c->n_beacon + i] = -1;
        }
        return;
    }
    int nmax = c->n_beacon + c->n_recent_q;
    uint16_t *X = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(nmax + 1) * d);
    int *sel = (int *)malloc(sizeof(int) * (size_t)(nmax + 1));
    for (int h = 0; h < G; ++h) {
        size_t b = (size_t)u * G + h;
        uint16_t *buf = qbuf + b * c->qcap * d;
        int nb = n_beacons_of(c, qcount[b]);
        memcpy(X, buf, sizeof(uint16_t) * (size_t)nb * d);
        memcpy(X + (size_t)nb * d, q_recent + b * c->n_recent_q * d,
               sizeof(uint16_t) * (size_t)c->n_recent_q * d);
        int n = nb + c->n_recent_q;
        int got = bkvo_fps(X, n, d, c->n_beacon, sel);
        if (fps_sel) {
            for (int i = 0; i < c->n_beacon; ++i)
                fps_sel[b * c->n_beacon + i] = i < got ? sel[i] : -1;
        }
        char *keep = (char *)calloc((size_t)(n > 0 ? n : 1), 1);
        for (int i = 0; i < got; ++i) keep[sel[i]] = 1;
        int w = 0;
        for (int i = 0; i < n; ++i)
            if (keep[i]) { memcpy(buf + (size_t)w * d, X + (size_t)i * d, sizeof(uint16_t) * (size_t)d); ++w; }
        qcount[b] = w;
        free(keep);
    }
    free(X);
    free(sel);
}

static void *run_units(void *arg)
{
    unit_job *J = (unit_job *)arg;
    const bkvo_cfg *c = J->cfg;
    int N = J->N, d = c->d;
    double *sc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    int32_t *ix = (int32_t *)malloc(sizeof(int32_t) * (size_t)c->budget);
    for (int u = J->u0; u < J->u1; ++u) {
        double *s = J->scores ? J->scores + (size_t)u * N : sc;
        int32_t *ii = J->idx ? J->idx + (size_t)u * c->budget : ix;
        if (J->do_score)
            score_unit(c, N, u, J->K, J->qbuf, J->qcount, J->q_recent, J->pos_recent, J->t, s);
        if (J->do_select) {
            int mv = bkvo_select(s, N, c->budget, c->n_prefix, c->n_recent_kv, ii);
            if (J->moved) J->moved[u] = mv;
        }
        if (J->do_compact) {
            compact_rows(J->K + (size_t)u * c->cap * d, d, N, ii, c->budget);
            compact_rows(J->V + (size_t)u * c->cap * d, d, N, ii, c->budget);
        }
        if (J->do_merge)
            merge_unit(c, u, J->qbuf, J->qcount, J->q_recent, J->fps_sel);
    }
    free(sc);
    free(ix);
    return NULL;
}

static void run_parallel(unit_job base, int U, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > U) nthreads = U > 0 ? U : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    unit_job *jobs = (unit_job *)malloc(sizeof(unit_job) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = base;
        jobs[i].u0 = (int)((long)U * i / nthreads);
        jobs[i].u1 = (int)((long)U * (i + 1) / nthreads);
        pthread_create(&th[i], NULL, run_units, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
}

/* Scores only: scores[U][N] (fp64). */
void bkvo_score(const bkvo_cfg *cfg, int U, int N, const uint16_t *K,
                const uint16_t *qbuf, const int32_t *qcount, const uint16_t *q_recent,
                const int32_t *pos_recent, const int32_t *t, double *scores, int nthreads)
{
    unit_job J;
    memset(&J, 0, sizeof J);
    J.cfg = cfg; J.N = N;
    J.K = (uint16_t *)K; J.qbuf = (uint16_t *)qbuf; J.qcount = (int32_t *)qcount;
    J.q_recent = q_recent; J.pos_recent = pos_recent; J.t = t;
    J.scores = scores;
    J.do_score = 1;
    run_parallel(J, U, nthreads);
}

/* The whole eviction of Notes §2.2 App. Alg. 2 / §2.3 Eq. 7-8 for U units:
 * score, keep set, in-place compaction of K and V, then the merge FPS of the
 * buffers.  Any output pointer may be NULL. */
void bkvo_evict(const bkvo_cfg *cfg, int U, int N, uint16_t *K, uint16_t *V,
                uint16_t *qbuf, int32_t *qcount, const uint16_t *q_recent,
                const int32_t *pos_recent, const int32_t *t,
                int32_t *idx, double *scores, int32_t *moved, int32_t *fps_sel,
                int nthreads)
{
    unit_job J;
    memset(&J, 0, sizeof J);
    J.cfg = cfg; J.N = N;
    J.K = K; J.V = V; J.qbuf = qbuf; J.qcount = qcount;
    J.q_recent = q_recent; J.pos_recent = pos_recent; J.t = t;
    J.scores = scores; J.idx = idx; J.moved = moved; J.fps_sel = fps_sel;
    J.do_score = J.do_select = J.do_compact = J.do_merge = 1;
    run_parallel(J, U, nthreads);
}

/* Merge step alone (for checking the buffer update in isolation). */
void bkvo_merge(const bkvo_cfg *cfg, int U, uint16_t *qbuf, int32_t *qcount,
                const uint16_t *q_recent, int32_t *fps_sel)
{
    for (int u = 0; u < U; ++u) merge_unit(cfg, u, qbuf, qcount, q_recent, fps_sel);
}

/* Compaction alone, given keep indices (idx[U][budget], -1 terminated). */
void bkvo_compact(const bkvo_cfg *cfg, int U, int N, uint16_t *K, uint16_t *V, const int32_t *idx)
{
    for (int u = 0; u < U; ++u) {
        compact_rows(K + (size_t)u * cfg->cap * cfg->d, cfg->d, N, idx + (size_t)u * cfg->budget, cfg->budget);
        compact_rows(V + (size_t)u * cfg->cap * cfg->d, cfg->d, N, idx + (size_t)u * cfg->budget, cfg->budget);
    }
}

/* ------------------------------------------------------------------------ */
/* Streaming decode cycle (Notes §2.2, App. Alg. 2; Summary, pseudocode) for
 * U units whose caches have the same length L.  Each decode step s < S, per
 * unit u (inputs step-major: k_new, v_new [S][U][d], q_new [S][U][G][d],
 * pos [S][U], the position of step s's token in u's sequence):
 *   1. the new key, rotated to its position, and the new value become row L
 *      of the unit's K and V;
 *   2. while L < cap - n_recent_q (the cycle's collection phase) each of the
 *      unit's G query buffers takes its new pre-RoPE query by the continual
 *      FPS update; in the last n_recent_q steps before the cache is full the
 *      buffers stay frozen (their first rows are the cycle's beacons) and the
 *      query goes to recent slot i = L - (cap - n_recent_q) with its position;
 *      at the first of these steps a buffer still holding more than n_beacon
 *      rows is compressed to n_beacon by FPS (bkvo_fps_compress), so that the
 *      beacons stand for every query the cycle collected;
 *   3. L grows by one; when it reaches cap the unit is evicted with N = cap
 *      and t = this step's position -- scores, keep set, compaction, merge
 *      FPS of beacons and recents -- and L becomes budget.
 * Naive full-history beacons (beacon_src NAIVE, Notes §3.2 Fig. 7): every
 * step's query is also appended to its head's history hist [U][G][hcap][d]
 * (counts hcount [U][G]; a full history takes no more rows), the buffers are
 * not updated in the collection phase, and at each eviction, before the
 * scores, each buffer becomes the FPS of its history without the cycle's
 * n_recent_q recent queries, rows [0, hcount - n_recent_q), taken as the
 * prefill sampling takes a prompt (bkvo_fps_long; survivors in ascending
 * history order); the merge leaves it alone.
 * State, in/out, unit-major as for bkvo_evict: K, V [U][cap][d], qbuf
 * [U][G][qcap][d], qcount [U][G], q_recent [U][G][n_recent_q][d],
 * pos_recent [U][n_recent_q]; *L_io is the shared cache length.  idx_hist
 * [max_ev][U][budget] and score_hist [max_ev][U][cap] (nullable) receive the
 * first max_ev evictions' keep sets and scores.  Returns the number of
 * evictions.                                                               */
typedef struct {
    const bkvo_cfg *cfg;
    int U, S, L0;
    const uint16_t *k_new, *v_new, *q_new;
    const int32_t *pos;
    uint16_t *K, *V, *qbuf, *q_recent;
    int32_t *qcount, *pos_recent, *t;
    int32_t *idx_hist;
    double *score_hist;
    int max_ev;
    uint16_t *hist;     /* naive source: query history [U][G][hcap][d] */
    int32_t *hcount;    /* [U][G] */
    int hcap;
    int u0, u1;
    int n_ev, L_end;
} stream_job;

/* Buffer of one head from FPS over the first n rows of its history (the
 * prefill sampling of bkvo_prefill). */
static void history_beacons(const bkvo_cfg *c, const uint16_t *hist, int n, uint16_t *buf, int32_t *cnt)
{
    bkvo_prefill(1, n, c->d, c->n_beacon, c->qcap, BKVO_SRC_FPS, 0u, 0, hist, buf, cnt, NULL);
}

static void *run_stream_units(void *arg)
{
    stream_job *J = (stream_job *)arg;
    const bkvo_cfg *c = J->cfg;
    int d = c->d, G = c->hq / c->hkv, U = J->U, nrq = c->n_recent_q;
    int ring0 = c->cap - nrq;
    double *sc = (double *)malloc(sizeof(double) * (size_t)c->cap);
    int32_t *ix = (int32_t *)malloc(sizeof(int32_t) * (size_t)(c->budget > 0 ? c->budget : 1));
    for (int u = J->u0; u < J->u1; ++u) {
        int L = J->L0, ne = 0;
        uint16_t *Ku = J->K + (size_t)u * c->cap * d;
        uint16_t *Vu = J->V + (size_t)u * c->cap * d;
        for (int s = 0; s < J->S; ++s) {
            size_t su = (size_t)s * U + u;
            int p = J->pos[su];
            bkvo_rope_row(J->k_new + su * d, d, c->theta, p, Ku + (size_t)L * d);
            memcpy(Vu + (size_t)L * d, J->v_new + su * d, sizeof(uint16_t) * (size_t)d);
            const uint16_t *qn = J->q_new + su * G * d;
            if (c->beacon_src == BKVO_SRC_NAIVE)
                for (int h = 0; h < G; ++h) {
                    int32_t *hc = J->hcount + (size_t)u * G + h;
                    int n = *hc < 0 ? 0 : *hc;
                    if (n < J->hcap) {
                        memcpy(J->hist + (((size_t)u * G + h) * J->hcap + n) * d, qn + (size_t)h * d,
                               sizeof(uint16_t) * (size_t)d);
                        *hc = n + 1;
                    }
                }
            if (L < ring0) {
                bkvo_beacon_update(c, G, global_unit(c, u) * G, J->qbuf + (size_t)u * G * c->qcap * d,
                                   J->qcount + (size_t)u * G, qn, NULL);
            } else {
                int i = L - ring0;
                if (i == 0 && c->beacon_src == BKVO_SRC_FPS)   /* freeze */
                    bkvo_fps_compress(G, c->qcap, d, c->n_beacon, nrq, J->qbuf + (size_t)u * G * c->qcap * d,
                                      J->qcount + (size_t)u * G, NULL);
                for (int h = 0; h < G; ++h)
                    memcpy(J->q_recent + (((size_t)u * G + h) * nrq + i) * d, qn + (size_t)h * d,
                           sizeof(uint16_t) * (size_t)d);
                J->pos_recent[(size_t)u * nrq + i] = p;
            }
            L += 1;
            if (L == c->cap) {
                J->t[u] = p;
                if (c->beacon_src == BKVO_SRC_NAIVE)
                    for (int h = 0; h < G; ++h) {
                        size_t b = (size_t)u * G + h;
                        int n = J->hcount[b] - nrq;
                        history_beacons(c, J->hist + b * J->hcap * d, n > 0 ? n : 0, J->qbuf + b * c->qcap * d,
                                        J->qcount + b);
                    }
                score_unit(c, c->cap, u, J->K, J->qbuf, J->qcount, J->q_recent, J->pos_recent, J->t, sc);
                bkvo_select(sc, c->cap, c->budget, c->n_prefix, c->n_recent_kv, ix);
                compact_rows(Ku, d, c->cap, ix, c->budget);
                compact_rows(Vu, d, c->cap, ix, c->budget);
                merge_unit(c, u, J->qbuf, J->qcount, J->q_recent, NULL);
                if (ne < J->max_ev) {
                    if (J->idx_hist)
                        memcpy(J->idx_hist + ((size_t)ne * U + u) * c->budget, ix,
                               sizeof(int32_t) * (size_t)c->budget);
                    if (J->score_hist)
                        memcpy(J->score_hist + ((size_t)ne * U + u) * c->cap, sc, sizeof(double) * (size_t)c->cap);
                }
                ++ne;
                L = c->budget < c->cap ? c->budget : c->cap;
            }
        }
        J->n_ev = ne;
        J->L_end = L;
    }
    free(sc);
    free(ix);
    return NULL;
}

int bkvo_stream(const bkvo_cfg *cfg, int U, int S, const uint16_t *k_new, const uint16_t *v_new,
                const uint16_t *q_new, const int32_t *pos, uint16_t *K, uint16_t *V, int32_t *L_io,
                uint16_t *qbuf, int32_t *qcount, uint16_t *q_recent, int32_t *pos_recent,
                int32_t *idx_hist, double *score_hist, int max_ev, uint16_t *hist, int32_t *hcount, int hcap,
                int nthreads)
{
    if (U <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > U) nthreads = U;
    int32_t *t = (int32_t *)calloc((size_t)U, sizeof(int32_t));
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    stream_job *jobs = (stream_job *)malloc(sizeof(stream_job) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) {
        stream_job *J = &jobs[i];
        memset(J, 0, sizeof *J);
        J->cfg = cfg; J->U = U; J->S = S; J->L0 = *L_io;
        J->k_new = k_new; J->v_new = v_new; J->q_new = q_new; J->pos = pos;
        J->K = K; J->V = V; J->qbuf = qbuf; J->q_recent = q_recent;
        J->qcount = qcount; J->pos_recent = pos_recent; J->t = t;
        J->idx_hist = idx_hist; J->score_hist = score_hist; J->max_ev = max_ev;
        J->hist = hist; J->hcount = hcount; J->hcap = hcap;
        J->u0 = (int)((long)U * i / nthreads);
        J->u1 = (int)((long)U * (i + 1) / nthreads);
        J->L_end = J->L0;
        pthread_create(&th[i], NULL, run_stream_units, J);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    int n_ev = jobs[0].n_ev;
    *L_io = jobs[0].L_end;
    free(th);
    free(jobs);
    free(t);
    return n_ev;
}

/* ------------------------------------------------------------------------ */
/* Decode attention of one step over the (compressed) cache (Notes §2.1, the
 * second formula: the new token's query attends over [K || k] and takes the
 * softmax-weighted sum of [V || v]; the new key and value are already rows of
 * the cache).  For query buffer uq = u * G + h, the bf16 pre-RoPE query
 * q[uq] is rotated to the unit's position pos[u] (bkvo_rope_row) and
 *   out[uq][k] = sum_{j < L} w_j V[u][j][k],  w = softmax_j(q . K[u][j] / sqrt(d)),
 * in fp64 (bkvo_row_weights).  scale[uq][k] = sum_j w_j |V[u][j][k]|, the
 * magnitude against which an fp32 evaluation's rounding is judged.
 * K, V: [U][cap][d]; q: [U][G][d]; out, scale: [U][G][d].                   */
void bkvo_decode_attention(const bkvo_cfg *c, int U, int L, const uint16_t *K, const uint16_t *V,
                           const uint16_t *q, const int32_t *pos, double *out, double *scale)
{
    int d = c->d, G = c->hq / c->hkv;
    double *w = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    uint16_t *qr = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    for (int u = 0; u < U; ++u) {
        const uint16_t *Ku = K + (size_t)u * c->cap * d, *Vu = V + (size_t)u * c->cap * d;
        for (int h = 0; h < G; ++h) {
            size_t uq = (size_t)u * G + h;
            bkvo_rope_row(q + uq * d, d, c->theta, pos[u], qr);
            bkvo_row_weights(qr, Ku, L, d, L - 1, w);
            for (int k = 0; k < d; ++k) {
                double acc = 0.0, mag = 0.0;
                for (int j = 0; j < L; ++j) {
                    double v = (double)bf2f(Vu[(size_t)j * d + k]);
                    acc += w[j] * v;
                    mag += w[j] * fabs(v);
                }
                out[uq * d + k] = acc;
                if (scale) scale[uq * d + k] = mag;
            }
        }
    }
    free(w);
    free(qr);
}

int bkvo_cfg_size(void) { return (int)sizeof(bkvo_cfg); }
