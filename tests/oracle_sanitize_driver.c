/*
 * Exercise every oracle entry point on small random inputs and edge shapes,
 * built together with the oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitized.py (CPU only).
 * Any out-of-bounds access, leak or undefined operation aborts the program.
 */
#include "../oracle/bkv_oracle.c"

#include <stdio.h>

static uint32_t rng = 12345u;
static float frand(void)
{
    rng = rng * 1664525u + 1013904223u;
    return ((float)(rng >> 8) / 16777216.0f) * 2.0f - 1.0f;
}
static void fill_bf16(uint16_t *x, size_t n, float scale)
{
    for (size_t i = 0; i < n; ++i) x[i] = bkvo_f32_to_bf16(scale * frand());
}

static void run_case(int hq, int hkv, int d, int N, int budget, int npf, int nrkv, int nb, int nrq, int S)
{
    bkvo_cfg c;
    memset(&c, 0, sizeof c);
    c.n_layers = 1; c.batch = 1; c.hq = hq; c.hkv = hkv; c.d = d; c.cap = N; c.budget = budget;
    c.n_prefix = npf; c.n_recent_kv = nrkv; c.n_beacon = nb; c.n_recent_q = nrq; c.causal = 1;
    c.qcap = 32; c.theta = 10000.0;
    int U = hkv, G = hq / hkv;
    size_t kv = (size_t)U * N * d;
    uint16_t *K = malloc(kv * 2), *V = malloc(kv * 2);
    uint16_t *qbuf = malloc((size_t)U * G * c.qcap * d * 2);
    uint16_t *qr = malloc((size_t)U * G * (nrq > 0 ? nrq : 1) * d * 2);
    int32_t *qc = malloc(sizeof(int32_t) * U * G), *pos = malloc(sizeof(int32_t) * U * (nrq > 0 ? nrq : 1));
    int32_t *t = malloc(sizeof(int32_t) * U);
    fill_bf16(K, kv, 3.0f); fill_bf16(V, kv, 1.0f);
    fill_bf16(qbuf, (size_t)U * G * c.qcap * d, 2.0f);
    fill_bf16(qr, (size_t)U * G * (nrq > 0 ? nrq : 1) * d, 2.0f);
    for (int i = 0; i < U * G; ++i) qc[i] = (i * 7) % (nb + 2);
    for (int u = 0; u < U; ++u) {
        t[u] = 500 + u;
        for (int i = 0; i < nrq; ++i) pos[u * nrq + i] = t[u] - nrq + 1 + i;
    }
    int32_t *idx = malloc(sizeof(int32_t) * U * (budget > 0 ? budget : 1));
    double *sc = malloc(sizeof(double) * U * N);
    int32_t *moved = malloc(sizeof(int32_t) * U), *sel = malloc(sizeof(int32_t) * U * G * (nb > 0 ? nb : 1));
    bkvo_score(&c, U, N, K, qbuf, qc, qr, pos, t, sc, 2);
    bkvo_evict(&c, U, N, K, V, qbuf, qc, qr, pos, t, idx, sc, moved, sel, 2);
    bkvo_merge(&c, U, qbuf, qc, qr, sel);
    bkvo_compact(&c, U, N, K, V, idx);

    /* buffer update and fp64 FPS on the same buffers */
    uint16_t *qn = malloc((size_t)U * G * d * 2);
    fill_bf16(qn, (size_t)U * G * d, 2.0f);
    for (int i = 0; i < U * G; ++i) qc[i] = (nb + nrq) - 1;
    bkvo_fps_update(U * G, c.qcap, d, nb, nrq, qbuf, qc, qn, sel);
    int sel32[33];
    double mar[33];
    bkvo_fps_f64(qbuf, 32, d, nb, sel32, mar);
    bkvo_fps(qbuf, 1, d, 1, sel32);
    bkvo_fps(qbuf, 5, d, 0, sel32);
    double reg[33];
    bkvo_fps_plain(qbuf, 32, d, nb, NULL, sel32, reg, mar);
    bkvo_fps_plain(qbuf, 32, d, nb, sel32, sel32, reg, NULL);
    bkvo_fps_plain(qbuf, 3, d, 5, NULL, sel32, NULL, NULL);
    for (int i = 0; i < U * G; ++i) qc[i] = (i % (nb + nrq + 3)) - 1;
    bkvo_fps_compress(U * G, c.qcap, d, nb, nrq, qbuf, qc, sel);
    bkvo_fps_compress(U * G, c.qcap, d, 0, nrq, qbuf, qc, NULL);

    /* a short stream from an empty cache, under each source of beacons */
    for (int src = 0; src < 4 && S > 0; ++src) {
        c.beacon_src = src;
        c.seed = 99u;
        uint16_t *kn = malloc((size_t)S * U * d * 2), *vn = malloc((size_t)S * U * d * 2);
        uint16_t *qs = malloc((size_t)S * U * G * d * 2);
        int32_t *ps = malloc(sizeof(int32_t) * S * U);
        fill_bf16(kn, (size_t)S * U * d, 1.0f); fill_bf16(vn, (size_t)S * U * d, 1.0f);
        fill_bf16(qs, (size_t)S * U * G * d, 2.0f);
        for (int s = 0; s < S * U; ++s) ps[s] = s / U;
        memset(qc, 0, sizeof(int32_t) * U * G);
        int32_t L = 0;
        int32_t *ih = malloc(sizeof(int32_t) * 4 * U * (budget > 0 ? budget : 1));
        double *sh = malloc(sizeof(double) * 4 * U * N);
        int hcap = S;
        uint16_t *hist = malloc((size_t)U * G * hcap * d * 2);
        int32_t *hc = calloc((size_t)U * G, sizeof(int32_t));
        bkvo_stream(&c, U, S, kn, vn, qs, ps, K, V, &L, qbuf, qc, qr, pos, ih, sh, 4, hist, hc, hcap, 2);
        free(kn); free(vn); free(qs); free(ps); free(ih); free(sh); free(hist); free(hc);
    }
    free(K); free(V); free(qbuf); free(qr); free(qc); free(pos); free(t); free(idx); free(sc);
    free(moved); free(sel); free(qn);
}

/* mean pooling, with and without the causal mask */
static void c_mean_case(void)
{
    bkvo_cfg c;
    memset(&c, 0, sizeof c);
    c.n_layers = 1; c.batch = 1; c.hq = 4; c.hkv = 2; c.d = 64; c.cap = 20; c.budget = 12;
    c.n_prefix = 2; c.n_recent_kv = 4; c.n_beacon = 3; c.n_recent_q = 4; c.qcap = 8; c.theta = 10000.0;
    c.pool_mean = 1;
    uint16_t K[2 * 20 * 64], qb[4 * 8 * 64], qr[4 * 4 * 64];
    int32_t qc[4] = {3, 1, 0, 5}, pos[2 * 4] = {1, 2, 3, 4, 5, 6, 7, 8}, t[2] = {9, 10};
    double sc[2 * 20];
    fill_bf16(K, sizeof K / 2, 2.0f); fill_bf16(qb, sizeof qb / 2, 2.0f); fill_bf16(qr, sizeof qr / 2, 2.0f);
    for (int causal = 0; causal < 2; ++causal) {
        c.causal = causal;
        bkvo_score(&c, 2, 20, K, qb, qc, qr, pos, t, sc, 2);
        bkvo_score(&c, 2, 2, K, qb, qc, qr, pos, t, sc, 1);
    }
}

int main(void)
{
    float cs[64 * 2];
    uint16_t x[64], y[64];
    fill_bf16(x, 64, 1.0f);
    bkvo_rope_table(1e4, 64, 0, 2, cs);
    bkvo_rope_row(x, 64, 1e4, 77, y);
    double w[50];
    bkvo_row_weights(x, x, 1, 64, -1, w);
    double s0[40];
    int32_t id[40];
    for (int i = 0; i < 40; ++i) s0[i] = (i % 3) * 0.25;
    bkvo_select(s0, 40, 20, 4, 8, id);
    bkvo_select(s0, 10, 20, 4, 8, id);
    /* G = 2, d = 64; G = 1; G = 4, d = 128; no recents; no beacons; nothing to evict; stream cadence */
    run_case(4, 2, 64, 160, 128, 8, 16, 16, 16, 200);
    run_case(3, 3, 64, 33, 128, 4, 16, 16, 16, 0);
    run_case(4, 1, 128, 97, 64, 4, 16, 16, 16, 0);
    run_case(2, 1, 64, 70, 40, 4, 8, 16, 0, 90);
    run_case(2, 1, 64, 70, 40, 4, 8, 0, 16, 0);
    run_case(2, 2, 64, 48, 40, 2, 4, 31, 1, 120);
    c_mean_case();
    /* prefill sampling: empty, shorter than the buffer, long */
    for (int P = 0; P <= 300; P += 150) {
        int P1 = P == 150 ? 9 : P;
        uint16_t *qp = malloc((size_t)3 * (P1 > 0 ? P1 : 1) * 64 * 2), *qb = malloc((size_t)3 * 32 * 64 * 2);
        int32_t qcnt[3], sl[3 * 16];
        fill_bf16(qp, (size_t)3 * (P1 > 0 ? P1 : 1) * 64, 2.0f);
        for (int src = 0; src < 3; ++src) bkvo_prefill(3, P1, 64, 16, 32, src, 7u, 5, qp, qb, qcnt, sl);
        free(qp); free(qb);
    }
    {   /* decode attention, including a one-row cache */
        bkvo_cfg c;
        memset(&c, 0, sizeof c);
        c.hq = 4; c.hkv = 2; c.d = 64; c.cap = 30; c.theta = 10000.0;
        uint16_t K[2 * 30 * 64], V[2 * 30 * 64], q[4 * 64];
        int32_t pos[2] = {5, 40};
        double o[4 * 64], sc[4 * 64];
        fill_bf16(K, sizeof K / 2, 2.0f); fill_bf16(V, sizeof V / 2, 1.0f); fill_bf16(q, sizeof q / 2, 2.0f);
        bkvo_decode_attention(&c, 2, 30, K, V, q, pos, o, sc);
        bkvo_decode_attention(&c, 2, 1, K, V, q, pos, o, NULL);
    }
    float ps[5] = {1.0f, 2.0f, 3.0f, 4.0f, 5.0f};
    bkvo_pairwise_sum(ps, 5);
    bkvo_pairwise_sum(ps, 0);
    printf("ok\n");
    return 0;
}
