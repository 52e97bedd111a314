/*
 * kvarn_oracle.c -- plain, slow CPU reference of the KVarN KV-cache quantizer
 * and of the attention step that consumes the quantized cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, includes or
 * calls this file. It is built by gcc into liboracle_kvarn.so and loaded (via
 * ctypes, from oracle/__init__.py) only by tests/, by the smoke check and by
 * the CPU-baseline leg of bench.py. It shares no code, header, table or
 * constant with the HIP path.
 *
 * Everything is fp64, scalar, unblocked and written in the order the method
 * states it. Sources (web pages about arXiv 2606.03458, "KVarN:
 * Variance-Normalized KV-Cache Quantization Mitigates Error Accumulation in
 * Reasoning Tasks"):
 *   [abstract]  the paper's abstract as carried by the codewithpapers.app
 *               record of arXiv 2606.03458;
 *   [HIW-1]     rndamp.com article on KVarN, section "How It Works", item 1
 *               (incoherence processing via Hadamard rotation);
 *   [HIW-2]     same article, "How It Works", item 2 (dual-scaling variance
 *               normalization);
 *   [Numbers]   same article, section "Numbers" (two scales, second scale
 *               fused into the dequantization kernel);
 *   [Problem]   same article, section "The Problem" (errors flow from one
 *               decoding step into the next).
 * Where the pages leave a step open, the reading taken is stated at the step
 * (tags SC-n) and listed in the design notes of the repository.
 *
 * Parity pins (tests/test_oracle_*.py): the rotation against
 * scipy.linalg.hadamard and its closed forms; the balancing against the
 * rank-one closed form and its invariants; the code choice against brute-force
 * enumeration; the packing against hand-written bytes; the attention against
 * torch's scaled_dot_product_attention in fp64 and its special cases.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KVO_OK 0
#define KVO_ERR_ARG (-1)
#define KVO_ERR_NONFINITE (-2)
#define KVO_ERR_NOMEM (-3)

static int is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

static int parity_of(unsigned v) {
    int p = 0;
    while (v) {
        p ^= (int)(v & 1u);
        v >>= 1;
    }
    return p;
}

/* Sylvester-order Hadamard matrix entry: H[i][k] = (-1)^popcount(i AND k).
 * [HIW-1] names a Hadamard transform along the channel axis; SC-1 takes the
 * Sylvester (natural) order with no sign diagonal. */
double kvo_hadamard_entry(int i, int k) {
    return parity_of((unsigned)(i & k)) ? -1.0 : 1.0;
}

/* Rotation of each row of x[rows][d] by H_d / sqrt(d) (SC-1), written as the
 * matrix product it is defined by:  y[r][k] = sum_j x[r][j] H[j][k] / sqrt(d).
 * H is symmetric and H H = d I, so applying this twice returns the input: the
 * same call un-rotates. */
int kvo_rotate(const double *x, int rows, int d, double *y) {
    if (!x || !y || rows < 0 || !is_pow2(d)) return KVO_ERR_ARG;
    const double s = 1.0 / sqrt((double)d);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)d);
    if (!tmp) return KVO_ERR_NOMEM;
    for (int r = 0; r < rows; ++r) {
        const double *xr = x + (size_t)r * d;
        for (int k = 0; k < d; ++k) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j) acc += xr[j] * kvo_hadamard_entry(j, k);
            tmp[k] = acc * s;
        }
        memcpy(y + (size_t)r * d, tmp, sizeof(double) * (size_t)d);
    }
    free(tmp);
    return KVO_OK;
}

/* Dual-scaling variance normalization of one block y[T][D] [HIW-2],
 * [abstract]: alternately balance the token (row) and channel (column) axes
 * so that the variance of y_ij / (r_i c_j) becomes about uniform.
 *
 * SC-4: "variance" is the uncentred mean of squares, P_ij = y_ij^2 (no mean
 *       is removed; the pages mention two scales and no offset).
 * SC-5: start from c = 1; one iteration = a row step then a column step;
 *       `iters` iterations, no early exit:
 *         row step     r_i^2 = (1/D) sum_j P_ij / c_j^2
 *         column step  c_j^2 = (1/T) sum_i P_ij / r_i^2
 *       A zero row (column) sum gives r_i = 1 (c_j = 1).
 * eps[k] (if not NULL) records, after iteration k, the largest deviation of a
 * non-zero row's normalized mean square from 1:
 *         max_i | (1/D) sum_j P_ij / (r_i^2 c_j^2) - 1 |.
 * r[T] holds the final row scales (1 for every row when iters == 0). */
int kvo_balance(const double *y, int T, int D, int iters, double *r, double *c,
                double *eps) {
    if (!y || !r || !c || T <= 0 || D <= 0 || iters < 0) return KVO_ERR_ARG;
    for (int j = 0; j < D; ++j) c[j] = 1.0;
    for (int i = 0; i < T; ++i) r[i] = 1.0;
    for (int it = 0; it < iters; ++it) {
        for (int i = 0; i < T; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j) {
                double p = y[(size_t)i * D + j] * y[(size_t)i * D + j];
                acc += p / (c[j] * c[j]);
            }
            acc /= (double)D;
            r[i] = acc > 0.0 ? sqrt(acc) : 1.0;
        }
        for (int j = 0; j < D; ++j) {
            double acc = 0.0;
            for (int i = 0; i < T; ++i) {
                double p = y[(size_t)i * D + j] * y[(size_t)i * D + j];
                acc += p / (r[i] * r[i]);
            }
            acc /= (double)T;
            c[j] = acc > 0.0 ? sqrt(acc) : 1.0;
        }
        if (eps) {
            double worst = 0.0;
            for (int i = 0; i < T; ++i) {
                double acc = 0.0, raw = 0.0;
                for (int j = 0; j < D; ++j) {
                    double p = y[(size_t)i * D + j] * y[(size_t)i * D + j];
                    raw += p;
                    acc += p / (r[i] * r[i] * c[j] * c[j]);
                }
                if (raw == 0.0) continue;
                double dev = fabs(acc / (double)D - 1.0);
                if (dev > worst) worst = dev;
            }
            eps[it] = worst;
        }
    }
    return KVO_OK;
}

/* 2-bit code of one normalized value u (SC-6, SC-8): the four levels are
 * {-1.5, -0.5, +0.5, +1.5} in units of the step, code = level + 1.5, i.e. the
 * nearest level with ties going to the upper one:  code = floor(u + 2),
 * clamped to [0, 3]. */
static uint8_t code_of(double u) {
    double f = floor(u + 2.0);
    if (f < 0.0) f = 0.0;
    if (f > 3.0) f = 3.0;
    return (uint8_t)f;
}

/* Range step and coding of one token row y[D] against column scales c[D]
 * (SC-7): the row step r'_i = max_j |y_ij / c_j| / 2 is the smallest step for
 * which no element leaves the 4-level grid; u_ij = y_ij / (r'_i c_j) lies in
 * [-2, 2]. A zero row has r' = 0, u = 0, code 2. Returns r'. */
static double code_row(const double *y, const double *c, int D, uint8_t *codes,
                       double *u) {
    double m = 0.0;
    for (int j = 0; j < D; ++j) {
        double a = fabs(y[j] / c[j]);
        if (a > m) m = a;
    }
    double rp = m / 2.0;
    for (int j = 0; j < D; ++j) {
        double uj = rp > 0.0 ? y[j] / (rp * c[j]) : 0.0;
        if (u) u[j] = uj;
        codes[j] = code_of(uj);
    }
    return rp;
}

static int all_finite(const double *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* The whole quantizer for one block x[T][D] (one layer, sequence, kv-head,
 * tensor and chunk; SC-3): rotate [HIW-1], balance [HIW-2], then the range
 * step and 2-bit codes [abstract]. Outputs: codes[T][D] (one code per byte),
 * rp[T] (row scale r'), c[D] (column scale), u[T][D] (pre-rounding value, may
 * be NULL), eps[iters] (may be NULL). */
int kvo_quantize_block(const double *x, int T, int D, int iters, uint8_t *codes,
                       double *rp, double *c, double *u, double *eps) {
    if (!x || !codes || !rp || !c || T <= 0 || !is_pow2(D) || iters < 0)
        return KVO_ERR_ARG;
    if (!all_finite(x, (size_t)T * D)) return KVO_ERR_NONFINITE;
    double *y = (double *)malloc(sizeof(double) * (size_t)T * D);
    double *r = (double *)malloc(sizeof(double) * (size_t)T);
    if (!y || !r) {
        free(y);
        free(r);
        return KVO_ERR_NOMEM;
    }
    int st = kvo_rotate(x, T, D, y);
    if (st == KVO_OK) st = kvo_balance(y, T, D, iters, r, c, eps);
    if (st == KVO_OK)
        for (int i = 0; i < T; ++i)
            rp[i] = code_row(y + (size_t)i * D, c, D, codes + (size_t)i * D,
                             u ? u + (size_t)i * D : NULL);
    free(y);
    free(r);
    return st;
}

/* Quantize a dense tensor x[B][H][T][D] chunk by chunk (chunk tokens per
 * block, SC-3). Outputs are unpacked: codes[B][H][T][D], rp[B][H][T],
 * c[B][H][T/chunk][D], u like codes (may be NULL), eps[B][H][T/chunk][iters]
 * (may be NULL). */
int kvo_quantize_tensor(const double *x, int B, int H, int T, int D, int chunk,
                        int iters, uint8_t *codes, double *rp, double *c,
                        double *u, double *eps) {
    if (B < 0 || H < 0 || chunk <= 0 || T % chunk != 0) return KVO_ERR_ARG;
    int nch = T / chunk;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int k = 0; k < nch; ++k) {
                size_t bh = (size_t)b * H + h;
                size_t tok0 = bh * T + (size_t)k * chunk;
                int st = kvo_quantize_block(
                    x + tok0 * D, chunk, D, iters, codes + tok0 * D, rp + tok0,
                    c + (bh * nch + k) * D, u ? u + tok0 * D : NULL,
                    eps ? eps + (bh * nch + k) * (size_t)iters : NULL);
                if (st != KVO_OK) return st;
            }
    return KVO_OK;
}

/* One new token per (sequence, kv-head) during decoding ([Problem]: the cache
 * grows one token per step). SC-11: the token is coded at once against the
 * column scales of the chunk it falls in; when it opens a chunk
 * (pos % chunk == 0) that chunk's column scales are copied from the previous
 * chunk of the same sequence and head, or set to 1 for the first chunk. The
 * row scale is the token's own range step (SC-7).
 * x[B][H][D]; pos[B] (a position outside [0, cap) skips that sequence);
 * codes[B][H][cap][D] unpacked, rp[B][H][cap], c[B][H][cap/chunk][D];
 * u_out[B][H][D] (may be NULL) receives the pre-rounding values. */
int kvo_append(const double *x, int B, int H, int D, const int *pos,
               uint8_t *codes, double *rp, double *c, int cap, int chunk,
               double *u_out) {
    if (!x || !pos || !codes || !rp || !c || !is_pow2(D) || chunk <= 0 ||
        cap % chunk != 0)
        return KVO_ERR_ARG;
    if (!all_finite(x, (size_t)B * H * D)) return KVO_ERR_NONFINITE;
    int nch = cap / chunk;
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    if (!y) return KVO_ERR_NOMEM;
    for (int b = 0; b < B; ++b) {
        int p = pos[b];
        if (p < 0 || p >= cap) continue;
        int k = p / chunk;
        for (int h = 0; h < H; ++h) {
            size_t bh = (size_t)b * H + h;
            double *cc = c + (bh * nch + k) * D;
            if (p % chunk == 0)
                for (int j = 0; j < D; ++j)
                    cc[j] = k > 0 ? c[(bh * nch + k - 1) * D + j] : 1.0;
            kvo_rotate(x + bh * D, 1, D, y);
            rp[bh * cap + p] = code_row(y, cc, D, codes + (bh * cap + p) * D,
                                        u_out ? u_out + bh * D : NULL);
        }
    }
    free(y);
    return KVO_OK;
}

/* Packed 2-bit layout of one chunk (SC-10), four codes per byte, lowest bits
 * first:
 *   kind 0 (K), token-major : token t owns D/4 bytes; channel j sits in byte
 *                             j/4 at bits 2*(j%4).
 *   kind 1 (V), channel-major: channel j owns chunk/4 bytes; token t sits in
 *                             byte t/4 at bits 2*(t%4).
 * codes[B][H][T][D] unpacked -> packed[B][H][T/chunk][chunk*D/4]. */
int kvo_pack(const uint8_t *codes, int B, int H, int T, int D, int chunk,
             int kind, uint8_t *packed) {
    if (!codes || !packed || chunk <= 0 || T % chunk || D % 4 || chunk % 4 ||
        (kind != 0 && kind != 1))
        return KVO_ERR_ARG;
    size_t per_chunk = (size_t)chunk * D / 4;
    int nch = T / chunk;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int k = 0; k < nch; ++k) {
                size_t bh = (size_t)b * H + h;
                uint8_t *out = packed + (bh * nch + k) * per_chunk;
                memset(out, 0, per_chunk);
                for (int t = 0; t < chunk; ++t)
                    for (int j = 0; j < D; ++j) {
                        unsigned v =
                            codes[(bh * T + (size_t)k * chunk + t) * D + j] & 3u;
                        size_t byte;
                        int shift;
                        if (kind == 0) {
                            byte = (size_t)t * (D / 4) + j / 4;
                            shift = 2 * (j % 4);
                        } else {
                            byte = (size_t)j * (chunk / 4) + t / 4;
                            shift = 2 * (t % 4);
                        }
                        out[byte] |= (uint8_t)(v << shift);
                    }
            }
    return KVO_OK;
}

/* Inverse of kvo_pack. */
int kvo_unpack(const uint8_t *packed, int B, int H, int T, int D, int chunk,
               int kind, uint8_t *codes) {
    if (!codes || !packed || chunk <= 0 || T % chunk || D % 4 || chunk % 4 ||
        (kind != 0 && kind != 1))
        return KVO_ERR_ARG;
    size_t per_chunk = (size_t)chunk * D / 4;
    int nch = T / chunk;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int k = 0; k < nch; ++k) {
                size_t bh = (size_t)b * H + h;
                const uint8_t *in = packed + (bh * nch + k) * per_chunk;
                for (int t = 0; t < chunk; ++t)
                    for (int j = 0; j < D; ++j) {
                        size_t byte;
                        int shift;
                        if (kind == 0) {
                            byte = (size_t)t * (D / 4) + j / 4;
                            shift = 2 * (j % 4);
                        } else {
                            byte = (size_t)j * (chunk / 4) + t / 4;
                            shift = 2 * (t % 4);
                        }
                        codes[(bh * T + (size_t)k * chunk + t) * D + j] =
                            (uint8_t)((in[byte] >> shift) & 3u);
                    }
            }
    return KVO_OK;
}

/* Reconstruction of tokens [0, n) of one (sequence, head) cache in the
 * ORIGINAL basis: yhat_tj = (code_tj - 1.5) r'_t c_{chunk(t), j} (the two
 * scales of [Numbers]), then x_hat = rotate(yhat) (the rotation is its own
 * inverse). codes[n][D], rp[n], c[ceil(n/chunk)][D] -> out[n][D]. */
int kvo_dequant(const uint8_t *codes, const double *rp, const double *c, int n,
                int D, int chunk, double *out) {
    if (!codes || !rp || !c || !out || n < 0 || !is_pow2(D) || chunk <= 0)
        return KVO_ERR_ARG;
    for (int t = 0; t < n; ++t)
        for (int j = 0; j < D; ++j)
            out[(size_t)t * D + j] = ((double)codes[(size_t)t * D + j] - 1.5) *
                                     rp[t] * c[(size_t)(t / chunk) * D + j];
    return kvo_rotate(out, n, D, out);
}

/* Per-token magnitude and direction of a reconstruction. The rndamp article
 * on KVarN, "The Problem", attributes the K error to wrong token magnitudes
 * rather than to directional distortion, and its "How It Works" closing
 * paragraph says the method minimizes the magnitude component. Reading taken
 * (the pages give no formula): for each of the n tokens,
 *   ratio_t  = ||xhat_t|| / ||x_t||                       (magnitude)
 *   cosine_t = <xhat_t, x_t> / (||xhat_t|| ||x_t||)       (direction)
 * Degenerate tokens: both zero -> (1, 1); x zero, xhat not -> (+inf, 0);
 * xhat zero, x not -> (0, 0). x[n][D], xhat[n][D] -> ratio[n], cosine[n]. */
int kvo_token_error(const double *x, const double *xhat, int n, int D,
                    double *ratio, double *cosine) {
    if (!x || !xhat || !ratio || !cosine || n < 0 || D <= 0) return KVO_ERR_ARG;
    for (int t = 0; t < n; ++t) {
        const double *a = x + (size_t)t * D, *b = xhat + (size_t)t * D;
        double aa = 0.0, bb = 0.0, ab = 0.0;
        for (int j = 0; j < D; ++j) {
            aa += a[j] * a[j];
            bb += b[j] * b[j];
            ab += a[j] * b[j];
        }
        if (aa == 0.0 && bb == 0.0) {
            ratio[t] = 1.0;
            cosine[t] = 1.0;
        } else if (aa == 0.0) {
            ratio[t] = INFINITY;
            cosine[t] = 0.0;
        } else if (bb == 0.0) {
            ratio[t] = 0.0;
            cosine[t] = 0.0;
        } else {
            ratio[t] = sqrt(bb) / sqrt(aa);
            cosine[t] = ab / (sqrt(aa) * sqrt(bb));
        }
    }
    return KVO_OK;
}

/* Decode attention over the reconstructed cache (SC-12): for each sequence b
 * and query head h, kv-head g = h / (Hq / Hkv) (grouped-query attention);
 * K_hat, V_hat of (b, g) over tokens [0, len_b) in the original basis;
 *   s_t = scale * <q_h, K_hat_t>,  p = softmax(s),  o = sum_t p_t V_hat_t.
 * Plain dense fp64 attention: no scale folding, no rotated-domain shortcut.
 * A length outside [1, cap] gives a zero output row.
 * q[B][Hq][D]; k_codes/v_codes[B][Hkv][cap][D] unpacked; k_rp/v_rp[B][Hkv][cap];
 * k_c/v_c[B][Hkv][cap/chunk][D]; lens[B]; out[B][Hq][D]. */
int kvo_decode_attn(const double *q, int B, int Hq, int Hkv, int D,
                    const uint8_t *k_codes, const double *k_rp, const double *k_c,
                    const uint8_t *v_codes, const double *v_rp, const double *v_c,
                    int cap, int chunk, const int *lens, double scale, double *out) {
    if (!q || !k_codes || !k_rp || !k_c || !v_codes || !v_rp || !v_c || !lens ||
        !out || Hkv <= 0 || Hq % Hkv || !is_pow2(D) || chunk <= 0 || cap % chunk)
        return KVO_ERR_ARG;
    int group = Hq / Hkv, nch = cap / chunk;
    double *kh = (double *)malloc(sizeof(double) * (size_t)cap * D);
    double *vh = (double *)malloc(sizeof(double) * (size_t)cap * D);
    double *s = (double *)malloc(sizeof(double) * (size_t)cap);
    if (!kh || !vh || !s) {
        free(kh);
        free(vh);
        free(s);
        return KVO_ERR_NOMEM;
    }
    for (int b = 0; b < B; ++b) {
        int n = lens[b];
        for (int g = 0; g < Hkv; ++g) {
            size_t bg = (size_t)b * Hkv + g;
            int ok = n >= 1 && n <= cap;
            if (ok) {
                kvo_dequant(k_codes + bg * cap * D, k_rp + bg * cap,
                            k_c + bg * nch * D, n, D, chunk, kh);
                kvo_dequant(v_codes + bg * cap * D, v_rp + bg * cap,
                            v_c + bg * nch * D, n, D, chunk, vh);
            }
            for (int hh = 0; hh < group; ++hh) {
                int h = g * group + hh;
                const double *qh = q + ((size_t)b * Hq + h) * D;
                double *o = out + ((size_t)b * Hq + h) * D;
                for (int j = 0; j < D; ++j) o[j] = 0.0;
                if (!ok) continue;
                double mx = -INFINITY;
                for (int t = 0; t < n; ++t) {
                    double acc = 0.0;
                    for (int j = 0; j < D; ++j) acc += qh[j] * kh[(size_t)t * D + j];
                    s[t] = scale * acc;
                    if (s[t] > mx) mx = s[t];
                }
                double den = 0.0;
                for (int t = 0; t < n; ++t) {
                    s[t] = exp(s[t] - mx);
                    den += s[t];
                }
                for (int t = 0; t < n; ++t) {
                    double p = s[t] / den;
                    for (int j = 0; j < D; ++j) o[j] += p * vh[(size_t)t * D + j];
                }
            }
        }
    }
    free(kh);
    free(vh);
    free(s);
    return KVO_OK;
}
