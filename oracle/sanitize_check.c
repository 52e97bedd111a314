/*
 * sanitize_check.c -- a small driver that runs every function of
 * kvarn_oracle.c on small inputs, edge cases included, for a gcc build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (the CPU test suite builds
 * and runs it). It checks only properties that hold by construction (the
 * rotation is its own inverse, pack/unpack round trips, codes in [0, 3],
 * decode of a one-token cache returns that token's value row); the oracle's
 * numerical pins live in the Python tests. Exit status 0 = all checks held
 * and no sanitizer report (the sanitizers abort on their first finding).
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle itself.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double kvo_hadamard_entry(int i, int k);
int kvo_rotate(const double *x, int rows, int d, double *y);
int kvo_balance(const double *y, int T, int D, int iters, double *r, double *c, double *eps);
int kvo_quantize_block(const double *x, int T, int D, int iters, uint8_t *codes, double *rp,
                       double *c, double *u, double *eps);
int kvo_quantize_tensor(const double *x, int B, int H, int T, int D, int chunk, int iters,
                        uint8_t *codes, double *rp, double *c, double *u, double *eps);
int kvo_append(const double *x, int B, int H, int D, const int *pos, uint8_t *codes,
               double *rp, double *c, int cap, int chunk, double *u_out);
int kvo_pack(const uint8_t *codes, int B, int H, int T, int D, int chunk, int kind,
             uint8_t *out);
int kvo_unpack(const uint8_t *packed, int B, int H, int T, int D, int chunk, int kind,
               uint8_t *out);
int kvo_dequant(const uint8_t *codes, const double *rp, const double *c, int n, int D,
                int chunk, double *out);
int kvo_token_error(const double *x, const double *xhat, int n, int D, double *ratio,
                    double *cosine);
int kvo_decode_attn(const double *q, int B, int Hq, int Hkv, int D, const uint8_t *k_codes,
                    const double *k_rp, const double *k_c, const uint8_t *v_codes,
                    const double *v_rp, const double *v_c, int cap, int chunk,
                    const int *lens, double scale, double *out);

static int failures = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

/* xorshift64 uniform in [-1, 1) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 4503599627370496.0 - 1.0;
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void run_dim(int D, int chunk, int T) {
    const int B = 2, H = 2, cap = T + chunk, iters = 4;
    const size_t nx = (size_t)B * H * T * D;
    double *x = xmalloc(nx * sizeof(double));
    for (size_t i = 0; i < nx; ++i) x[i] = uniform() * (1.0 + (double)(i % 7));
    /* a zero token row and a zero channel in the first block */
    memset(x, 0, (size_t)D * sizeof(double));
    for (int t = 0; t < chunk; ++t) x[(size_t)t * D + 1] = 0.0;

    /* rotation: entries, involution */
    double *y = xmalloc(nx * sizeof(double)), *z = xmalloc(nx * sizeof(double));
    CHECK(kvo_hadamard_entry(3, 5) == -1.0);
    CHECK(kvo_rotate(x, B * H * T, D, y) == 0);
    CHECK(kvo_rotate(y, B * H * T, D, z) == 0);
    for (size_t i = 0; i < nx; ++i) CHECK(fabs(z[i] - x[i]) <= 1e-12 * (1.0 + fabs(x[i])));

    /* balancing, and the error paths of bad arguments */
    double *r = xmalloc((size_t)chunk * sizeof(double)), *c = xmalloc((size_t)D * sizeof(double));
    double eps[4];
    CHECK(kvo_balance(y, chunk, D, iters, r, c, eps) == 0);
    CHECK(kvo_balance(y, chunk, D, 0, r, c, NULL) == 0);
    CHECK(kvo_balance(NULL, chunk, D, iters, r, c, eps) != 0);
    CHECK(kvo_rotate(x, 1, 3, y) != 0);

    /* whole-tensor quantization, all outputs */
    const int nch = T / chunk;
    uint8_t *codes = xmalloc(nx);
    double *rp = xmalloc((size_t)B * H * T * sizeof(double));
    double *cs = xmalloc((size_t)B * H * nch * D * sizeof(double));
    double *u = xmalloc(nx * sizeof(double));
    double *ep = xmalloc((size_t)B * H * nch * iters * sizeof(double));
    CHECK(kvo_quantize_tensor(x, B, H, T, D, chunk, iters, codes, rp, cs, u, ep) == 0);
    CHECK(kvo_quantize_tensor(x, B, H, T, D, chunk, 0, codes, rp, cs, NULL, NULL) == 0);
    CHECK(kvo_quantize_tensor(x, B, H, T, D, chunk, iters, codes, rp, cs, u, ep) == 0);
    for (size_t i = 0; i < nx; ++i) CHECK(codes[i] <= 3);
    CHECK(rp[0] == 0.0); /* the zero token */

    /* non-finite input is refused */
    double keep = x[5];
    x[5] = NAN;
    CHECK(kvo_quantize_block(x, chunk, D, iters, codes, rp, cs, u, ep) == -2);
    x[5] = keep;

    /* pack / unpack round trip, both kinds */
    uint8_t *packed = xmalloc(nx / 4), *back = xmalloc(nx);
    for (int kind = 0; kind < 2; ++kind) {
        CHECK(kvo_pack(codes, B, H, T, D, chunk, kind, packed) == 0);
        CHECK(kvo_unpack(packed, B, H, T, D, chunk, kind, back) == 0);
        CHECK(memcmp(codes, back, nx) == 0);
    }

    /* a cache of capacity T + chunk: the quantized tokens, then appends that
     * open the next chunk, then skipped positions */
    uint8_t *kc = xmalloc((size_t)B * H * cap * D);
    double *krp = xmalloc((size_t)B * H * cap * sizeof(double));
    double *kcs = xmalloc((size_t)B * H * (cap / chunk) * D * sizeof(double));
    memset(kc, 2, (size_t)B * H * cap * D);
    memset(krp, 0, (size_t)B * H * cap * sizeof(double));
    for (size_t i = 0; i < (size_t)B * H * (cap / chunk) * D; ++i) kcs[i] = 1.0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            size_t bh = (size_t)b * H + h;
            memcpy(kc + bh * cap * D, codes + bh * T * D, (size_t)T * D);
            memcpy(krp + bh * cap, rp + bh * T, (size_t)T * sizeof(double));
            memcpy(kcs + bh * (cap / chunk) * D, cs + bh * nch * D,
                   (size_t)nch * D * sizeof(double));
        }
    double *xn = xmalloc((size_t)B * H * D * sizeof(double)), *un = xmalloc((size_t)B * H * D * sizeof(double));
    for (size_t i = 0; i < (size_t)B * H * D; ++i) xn[i] = uniform();
    int pos[2] = {T, T};
    CHECK(kvo_append(xn, B, H, D, pos, kc, krp, kcs, cap, chunk, un) == 0);
    pos[0] = T + 1;
    pos[1] = -1;
    CHECK(kvo_append(xn, B, H, D, pos, kc, krp, kcs, cap, chunk, NULL) == 0);
    pos[0] = cap;
    CHECK(kvo_append(xn, B, H, D, pos, kc, krp, kcs, cap, chunk, NULL) == 0);

    /* dequant and the per-token error of every token of (0, 0) */
    double *xh = xmalloc((size_t)T * D * sizeof(double));
    double *ratio = xmalloc((size_t)T * sizeof(double)), *cosine = xmalloc((size_t)T * sizeof(double));
    CHECK(kvo_dequant(kc, krp, kcs, T, D, chunk, xh) == 0);
    CHECK(kvo_token_error(x, xh, T, D, ratio, cosine) == 0);
    CHECK(ratio[0] == 1.0 && cosine[0] == 1.0); /* both zero: (1, 1) */
    for (int t = 1; t < T; ++t) CHECK(cosine[t] > 0.5 && cosine[t] <= 1.0 + 1e-12);

    /* decode: valid, one-token and out-of-range lengths */
    const int G = 2, Hq = H * G;
    double *q = xmalloc((size_t)B * Hq * D * sizeof(double)), *o = xmalloc((size_t)B * Hq * D * sizeof(double));
    for (size_t i = 0; i < (size_t)B * Hq * D; ++i) q[i] = uniform();
    int lens[2] = {T + 2, 1};
    CHECK(kvo_decode_attn(q, B, Hq, H, D, kc, krp, kcs, kc, krp, kcs, cap, chunk, lens,
                          1.0 / sqrt((double)D), o) == 0);
    double *v0 = xmalloc((size_t)D * sizeof(double));
    CHECK(kvo_dequant(kc + (size_t)1 * H * cap * D, krp + (size_t)1 * H * cap, kcs + (size_t)1 * H * (cap / chunk) * D, 1, D, chunk, v0) == 0);
    for (int j = 0; j < D; ++j) CHECK(fabs(o[((size_t)1 * Hq) * D + j] - v0[j]) <= 1e-12 * (1.0 + fabs(v0[j])));
    lens[0] = 0;
    lens[1] = cap + 1;
    CHECK(kvo_decode_attn(q, B, Hq, H, D, kc, krp, kcs, kc, krp, kcs, cap, chunk, lens,
                          1.0 / sqrt((double)D), o) == 0);
    for (size_t i = 0; i < (size_t)B * Hq * D; ++i) CHECK(o[i] == 0.0);

    free(x); free(y); free(z); free(r); free(c); free(codes); free(rp); free(cs); free(u);
    free(ep); free(packed); free(back); free(kc); free(krp); free(kcs); free(xn); free(un);
    free(xh); free(ratio); free(cosine); free(q); free(o); free(v0);
}

int main(void) {
    run_dim(128, 128, 256);
    run_dim(64, 128, 256);
    run_dim(256, 128, 128);
    run_dim(8, 4, 8);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitize check ok\n");
    return 0;
}
