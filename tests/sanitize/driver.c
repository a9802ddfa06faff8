/*
 * Host-code driver for the sanitizer test (tests/test_sanitizers.py): runs
 * the library's host format functions (lut_weight_quantized_amd/csrc/
 * lut6_format.cpp) and every entry of the CPU oracle (oracle/lut6_oracle.c)
 * on small shapes -- ragged row subsets, odd head counts, a ragged chunk of
 * the recurrence, refusals -- with every buffer allocated at its exact size,
 * so that AddressSanitizer sees any access past an end and
 * UndefinedBehaviorSanitizer any overflow or bad shift.  It checks a few
 * results too (pack/unpack round trip, library and oracle packing agree),
 * and prints "sanitize driver ok" at the end.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* library host functions (C ABI) */
size_t lut6_packed_bytes(int64_t N, int64_t K);
size_t lut6_table_bytes(int64_t N);
int lut6_pack(const uint8_t *idx, uint8_t *packed, int64_t N, int64_t K);
int lut6_unpack(const uint8_t *packed, uint8_t *idx, int64_t N, int64_t K);
const char *lut6_status_string(int status);

/* oracle */
double ora_f16_to_f64(uint16_t h);
uint16_t ora_f64_to_f16(double v);
int ora_pack(const uint8_t *idx, uint8_t *packed, int64_t n, int64_t k);
int ora_unpack(const uint8_t *packed, uint8_t *idx, int64_t n, int64_t k);
int ora_dequant(const uint8_t *packed, const uint16_t *tables, uint16_t *w, int64_t n, int64_t k);
int ora_linear(const uint16_t *x, const uint8_t *packed, const uint16_t *tables, int64_t L, int64_t K,
               int64_t N, double in_scale, int epilogue, const int64_t *rows, int64_t n_rows,
               int threads, double *y_exact, void *y_out);
int ora_int8_linear(const uint16_t *x, const int8_t *q, const uint16_t *qs, int64_t L, int64_t K,
                    int64_t N, double in_scale, int epilogue, const int64_t *rows, int64_t n_rows,
                    int threads, double *y_exact, void *y_out);
int ora_int8_dequant(const int8_t *q, const uint16_t *qs, uint16_t *w, int64_t n, int64_t k);
int ora_quantize(const uint16_t *w, uint8_t *packed, uint16_t *tables, int64_t n, int64_t k,
                 int64_t g0, int64_t g1, double *sse);
int ora_km_centres(const uint16_t *w, int64_t n, int64_t k, int64_t g, int rounds, double *centres);
int ora_attention(const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v,
                  int64_t ldv, int64_t L, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                  const int64_t *rows, int64_t n_rows, int threads, double *o_exact, uint16_t *o_out,
                  double *o_abs, double *v_abs);
int ora_gated_delta(const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v,
                    int64_t ldv, const float *g, const float *beta, int64_t ldg, int64_t L, int64_t Hk,
                    int64_t Hv, int64_t dk, int64_t dv, const float *state_in, int threads,
                    double *o_exact, uint16_t *o_out, double *o_abs, double *state_out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng_state >> 33);
}
static double urand(void) { return (rnd() + 0.5) / 2147483648.0; }   /* (0, 1) */
static uint16_t h16(double v) { return ora_f64_to_f16(v); }

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

#define CHECK(cond)                                                            \
    do {                                                                       \
        if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); exit(1); } \
    } while (0)

static void format_and_linear(int64_t L, int64_t K, int64_t N)
{
    const int64_t pb = (int64_t)lut6_packed_bytes(N, K);
    uint8_t *idx = xmalloc((size_t)(N * K)), *back = xmalloc((size_t)(N * K));
    uint8_t *p1 = xmalloc((size_t)pb), *p2 = xmalloc((size_t)pb);
    for (int64_t i = 0; i < N * K; ++i) idx[i] = (uint8_t)(rnd() & 63);
    CHECK(lut6_pack(idx, p1, N, K) == 0);
    CHECK(ora_pack(idx, p2, N, K) == 0);
    CHECK(memcmp(p1, p2, (size_t)pb) == 0);
    CHECK(lut6_unpack(p1, back, N, K) == 0);
    CHECK(memcmp(idx, back, (size_t)(N * K)) == 0);
    CHECK(ora_unpack(p2, back, N, K) == 0);
    CHECK(memcmp(idx, back, (size_t)(N * K)) == 0);

    uint16_t *tab = xmalloc(lut6_table_bytes(N));
    for (int64_t i = 0; i < N / 16 * 64; ++i) tab[i] = h16((urand() - 0.5) * 0.04);
    uint16_t *w = xmalloc((size_t)(N * K) * 2);
    CHECK(ora_dequant(p2, tab, w, N, K) == 0);
    uint16_t *x = xmalloc((size_t)(L * K) * 2);
    for (int64_t i = 0; i < L * K; ++i) x[i] = h16(urand() * 4.0 - 2.0);
    /* every epilogue, all rows and a ragged subset, several thread counts */
    int64_t rows[3] = {0, L / 2, L - 1};
    for (int epi = 0; epi < (N % 32 ? 2 : 3); ++epi) {
        const int64_t n_out = epi == 2 ? N / 2 : N;
        for (int sub = 0; sub < 2; ++sub) {
            const int64_t nr = sub ? 3 : L;
            double *ye = xmalloc((size_t)(nr * n_out) * 8);
            void *yo = xmalloc((size_t)(nr * n_out) * (epi == 0 ? 4 : 2));
            CHECK(ora_linear(x, p2, tab, L, K, N, 16.0, epi, sub ? rows : NULL, nr, 1 + sub * 4, ye, yo) == 0);
            free(ye);
            free(yo);
        }
    }
    /* refusals never write */
    {
        double ye1;
        uint16_t yo1;
        CHECK(ora_linear(x, p2, tab, L, K, N, 1.0, 5, NULL, L, 1, &ye1, &yo1) != 0);
        CHECK(ora_linear(x, p2, tab, L, K, N, 1.0, 0, rows, -1, 1, &ye1, &yo1) != 0);
    }
    CHECK(lut6_pack(idx, p1, N, K + 1) != 0);
    idx[N * K - 1] = 64;
    CHECK(lut6_pack(idx, p1, N, K) != 0);
    free(idx); free(back); free(p1); free(p2); free(tab); free(w); free(x);
}

static void int8_variant(int64_t L, int64_t K, int64_t N)
{
    int8_t *q = xmalloc((size_t)(N * K));
    uint16_t *qs = xmalloc((size_t)(N * (K / 32)) * 2);
    for (int64_t i = 0; i < N * K; ++i) q[i] = (int8_t)(rnd() & 255);
    for (int64_t i = 0; i < N * (K / 32); ++i) qs[i] = h16(1e-3 + urand() * 1e-3);
    uint16_t *w = xmalloc((size_t)(N * K) * 2);
    CHECK(ora_int8_dequant(q, qs, w, N, K) == 0);
    uint16_t *x = xmalloc((size_t)(L * K) * 2);
    for (int64_t i = 0; i < L * K; ++i) x[i] = h16(urand() - 0.5);
    int64_t rows[2] = {L - 1, 0};
    for (int epi = 0; epi < 3; ++epi) {
        const int64_t n_out = epi == 2 ? N / 2 : N;
        double *ye = xmalloc((size_t)(2 * n_out) * 8);
        void *yo = xmalloc((size_t)(2 * n_out) * (epi == 0 ? 4 : 2));
        CHECK(ora_int8_linear(x, q, qs, L, K, N, 2.0, epi, rows, 2, 3, ye, yo) == 0);
        free(ye);
        free(yo);
    }
    free(q); free(qs); free(w); free(x);
}

static void quantize(int64_t N, int64_t K)
{
    uint16_t *w = xmalloc((size_t)(N * K) * 2);
    for (int64_t i = 0; i < N * K; ++i) w[i] = h16((urand() - 0.5) * 0.1);
    uint8_t *packed = xmalloc((size_t)lut6_packed_bytes(N, K));
    uint16_t *tables = xmalloc(lut6_table_bytes(N));
    double sse[41], c[64];
    CHECK(ora_quantize(w, packed, tables, N, K, 0, N / 16, sse) == 0);
    CHECK(ora_km_centres(w, N, K, N / 16 - 1, 3, c) == 0);
    CHECK(ora_km_centres(w, N, K, N / 16, 3, c) != 0);
    free(w); free(packed); free(tables);
}

static void attention(int64_t L, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D)
{
    const int64_t ldq = Hq * D + 8, ldk = Hkv * D + 16, ldv = Hkv * D;
    uint16_t *q = xmalloc((size_t)((L - 1) * ldq + Hq * D) * 2);
    uint16_t *k = xmalloc((size_t)((Lk - 1) * ldk + Hkv * D) * 2);
    uint16_t *v = xmalloc((size_t)((Lk - 1) * ldv + Hkv * D) * 2);
    for (int64_t i = 0; i < (L - 1) * ldq + Hq * D; ++i) q[i] = h16(urand() - 0.5);
    for (int64_t i = 0; i < (Lk - 1) * ldk + Hkv * D; ++i) k[i] = h16(urand() - 0.5);
    for (int64_t i = 0; i < (Lk - 1) * ldv + Hkv * D; ++i) v[i] = h16(urand() - 0.5);
    int64_t rows[2] = {0, L - 1};
    double *oe = xmalloc((size_t)(2 * Hq * D) * 8), *oa = xmalloc((size_t)(2 * Hq * D) * 8);
    double *va = xmalloc((size_t)(2 * Hq * D) * 8);
    uint16_t *oo = xmalloc((size_t)(2 * Hq * D) * 2);
    CHECK(ora_attention(q, ldq, k, ldk, v, ldv, L, Lk, Hq, Hkv, D, rows, 2, 2, oe, oo, oa, va) == 0);
    free(q); free(k); free(v); free(oe); free(oa); free(va); free(oo);
}

static void gated_delta(int64_t L, int64_t Hk, int64_t Hv, int64_t d)
{
    const int64_t ldq = Hk * d, ldk = Hk * d + 8, ldv = Hv * d, ldg = Hv + 3;
    uint16_t *q = xmalloc((size_t)(L * ldq) * 2), *k = xmalloc((size_t)((L - 1) * ldk + Hk * d) * 2);
    uint16_t *v = xmalloc((size_t)(L * ldv) * 2);
    float *g = xmalloc((size_t)((L - 1) * ldg + Hv) * 4), *be = xmalloc((size_t)((L - 1) * ldg + Hv) * 4);
    float *s0 = xmalloc((size_t)(Hv * d * d) * 4);
    for (int64_t i = 0; i < L * ldq; ++i) q[i] = h16((urand() - 0.5) * 0.2);
    for (int64_t i = 0; i < (L - 1) * ldk + Hk * d; ++i) k[i] = h16((urand() - 0.5) * 0.2);
    for (int64_t i = 0; i < L * ldv; ++i) v[i] = h16(urand() - 0.5);
    for (int64_t i = 0; i < (L - 1) * ldg + Hv; ++i) { g[i] = (float)(-0.5 * urand()); be[i] = (float)urand(); }
    for (int64_t i = 0; i < Hv * d * d; ++i) s0[i] = (float)(urand() - 0.5);
    double *oe = xmalloc((size_t)(L * Hv * d) * 8), *oa = xmalloc((size_t)(L * Hv * d) * 8);
    uint16_t *oo = xmalloc((size_t)(L * Hv * d) * 2);
    double *so = xmalloc((size_t)(Hv * d * d) * 8);
    CHECK(ora_gated_delta(q, ldq, k, ldk, v, ldv, g, be, ldg, L, Hk, Hv, d, d, s0, 3, oe, oo, oa, so) == 0);
    free(q); free(k); free(v); free(g); free(be); free(s0); free(oe); free(oa); free(oo); free(so);
}

int main(void)
{
#ifdef SANITIZE_CONTROL
    {
        /* control build: one read past the end, which the sanitizer must report */
        volatile uint8_t *buf = xmalloc(8);
        volatile uint8_t past = buf[8];
        (void)past;
    }
#endif
    for (int s = -1; s < 12; ++s) CHECK(lut6_status_string(s) != NULL);
    CHECK(lut6_packed_bytes(16, 6) == 0 && lut6_table_bytes(20) == 0);
    for (uint32_t h = 0; h < 65536; ++h) (void)ora_f64_to_f16(ora_f16_to_f64((uint16_t)h));
    format_and_linear(5, 64, 32);
    format_and_linear(17, 192, 96);
    format_and_linear(1, 4, 16);
    int8_variant(7, 64, 64);
    int8_variant(3, 128, 32);
    quantize(32, 64);
    quantize(16, 4);
    attention(5, 9, 4, 2, 16);
    attention(1, 1, 2, 1, 8);
    gated_delta(6, 1, 2, 8);
    gated_delta(1, 2, 4, 4);
    printf("sanitize driver ok\n");
    return 0;
}
