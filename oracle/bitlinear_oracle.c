/*
 * Plain CPU oracle for the BitNet b1.58 BitLinear (W1.58A8) path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP implementation.
 *
 * Every function is the plain definition written out, one element at a time,
 * in the order the pages state it.  Where the pages run their listings in
 * PyTorch's default dtype, the arithmetic here is IEEE binary32 with one
 * rounding per operation (the file must be compiled with -ffp-contract=off
 * and without -ffast-math; x86-64 SSE evaluates float in float).  Sums whose
 * order the pages leave open are computed exactly (order-free) and rounded
 * once.
 *
 * Sources (pages by title and section):
 *  [P1] "BitNet論文分析：1-Bit LLMの時代" (youngju.dev): sections
 *       "1-Bit重みとSign関数", "Absmean量子化関数",
 *       "BitNet b1.58：三値重みのイノベーション" (BitLinear_b158 listing),
 *       "bitnet.cpp推論フレームワーク / アーキテクチャ概要" (I2_S codes).
 *  [P2] "BitNet — 1-bit Transformersの実装ライブラリ" (ai-heartland.com):
 *       "BitLinearの仕組み：量子化フロー".
 *  [P3] "BitNet.cpp 深度解析" (dashen-tech.com): §2.3 I2_S format,
 *       §3.1 integer matmul as sum_pos - sum_neg.
 *  [P5] "BitNet b1.58 2B4T" news (reinforz.co.jp): W1.58A8, ReLU², no bias.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q 127.0f   /* activation code range [-127, 127] (symmetric reading) */
#define ORC_EPS 1e-5f  /* the listings add 1e-5 to the scale before dividing   */

/* ------------------------------------------------------------------------ */
/* Exact summation.  Shewchuk's non-overlapping partials ("Adaptive Precision
 * Floating-Point Arithmetic", 1997), finished with the round-half-even
 * correction of Python's math.fsum.  Returns the exact sum of the terms
 * rounded once to binary64.  Used for the absmean of [P1] "Absmean量子化関数"
 * (the mean of |W| over the whole tensor) and for the mean square of RMSNorm.
 * All terms fed here are exactly representable in binary64.                */
typedef struct {
    double *p;
    int n, cap;
} orc_partials;

static void orc_partials_init(orc_partials *s) {
    s->cap = 64;
    s->n = 0;
    s->p = (double *)malloc(sizeof(double) * (size_t)s->cap);
}

static void orc_partials_add(orc_partials *s, double x) {
    int i = 0;
    for (int j = 0; j < s->n; ++j) {
        double y = s->p[j];
        if (fabs(x) < fabs(y)) { double t = x; x = y; y = t; }
        double hi = x + y;
        double lo = y - (hi - x);
        if (lo != 0.0) s->p[i++] = lo;
        x = hi;
    }
    if (i >= s->cap) {
        s->cap *= 2;
        s->p = (double *)realloc(s->p, sizeof(double) * (size_t)s->cap);
    }
    s->p[i] = x;
    s->n = i + 1;
}

static double orc_partials_round(orc_partials *s) {
    int n = s->n;
    double hi = 0.0, lo = 0.0;
    if (n > 0) {
        hi = s->p[--n];
        while (n > 0) {
            double x = hi;
            double y = s->p[--n];
            hi = x + y;
            double yr = hi - x;
            lo = y - yr;
            if (lo != 0.0) break;
        }
        /* If the dropped tail has the same sign as lo, the rounding above
         * was a half-way case decided the wrong way: redo it. */
        if (n > 0 && ((lo < 0.0 && s->p[n - 1] < 0.0) ||
                      (lo > 0.0 && s->p[n - 1] > 0.0))) {
            double y = lo * 2.0;
            double x = hi + y;
            double yr = x - hi;
            if (y == yr) hi = x;
        }
    }
    free(s->p);
    s->p = NULL;
    return hi;
}

/* Exact sum of |w_i| over n binary32 values, rounded once to binary64. */
double orc_abs_sum_exact(const float *w, int64_t n) {
    orc_partials s;
    orc_partials_init(&s);
    for (int64_t i = 0; i < n; ++i) orc_partials_add(&s, fabs((double)w[i]));
    return orc_partials_round(&s);
}

/* Exact sum of x_i^2 over n binary32 values, rounded once to binary64.
 * Each square of a binary32 value is exact in binary64. */
double orc_sq_sum_exact(const float *x, int64_t n) {
    orc_partials s;
    orc_partials_init(&s);
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        orc_partials_add(&s, v * v);
    }
    return orc_partials_round(&s);
}

/* ------------------------------------------------------------------------ */
/* [P1] "Absmean量子化関数": the per-tensor weight scale is the mean of |W|
 * over all n = N*K entries.  Defined here as the exact sum rounded to
 * binary64, divided by n in binary64, rounded to binary32. */
float orc_weight_scale(const float *w, int64_t n) {
    if (n <= 0) return 0.0f;
    double s = orc_abs_sum_exact(w, n);
    return (float)(s / (double)n);
}

/* [P1] "Absmean量子化関数": divide by (scale + 1e-5), round half to even,
 * clamp to [-1, 1].  Output one int8 in {-1, 0, +1} per weight. */
void orc_ternarize(const float *w, int64_t n, float gamma, int8_t *t) {
    float d = gamma + ORC_EPS;
    for (int64_t i = 0; i < n; ++i) {
        float q = w[i] / d;
        float r = nearbyintf(q); /* default rounding mode: half to even */
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        t[i] = (int8_t)r;
    }
}

/* [P1] "1-Bit重みとSign関数": +1 where w >= 0 (including -0.0), else -1. */
void orc_binarize(const float *w, int64_t n, int8_t *t) {
    for (int64_t i = 0; i < n; ++i) t[i] = (w[i] >= 0.0f) ? (int8_t)1 : (int8_t)-1;
}

/* ------------------------------------------------------------------------ */
/* Packed 2-bit layout.  [P1] "アーキテクチャ概要" and [P3] §2.3: 2 bits per
 * weight, code 00 = -1, 01 = 0, 10 = +1, sixteen weights per 32-bit word.
 * Layout used here (the pages leave the bit order open):
 *   row n holds Kp = K rounded up to 64 weights as Kp/16 words;
 *   word j covers weights 16j .. 16j+15;
 *   weight 16j + 4s + b sits in byte b of the word, at bits 2s and 2s+1;
 *   weights k >= K are padding and hold code 01 (zero). */
int64_t orc_padded_k(int64_t K) { return (K + 63) / 64 * 64; }

void orc_pack(const int8_t *t, int64_t N, int64_t K, uint32_t *packed) {
    int64_t kp = orc_padded_k(K);
    int64_t words = kp / 16;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < words; ++j) {
            uint32_t word = 0;
            for (int64_t k = 16 * j; k < 16 * j + 16; ++k) {
                uint32_t code = 1u;
                if (k < K) code = (uint32_t)(t[n * K + k] + 1);
                int64_t r = k - 16 * j;
                int64_t s = r / 4, b = r % 4;
                word |= code << (8 * b + 2 * s);
            }
            packed[n * words + j] = word;
        }
    }
}

/* Inverse of orc_pack.  Returns the number of code-11 fields found (never
 * emitted by the packer) plus the number of padding fields that are not 01. */
int64_t orc_unpack(const uint32_t *packed, int64_t N, int64_t K, int8_t *t) {
    int64_t kp = orc_padded_k(K);
    int64_t words = kp / 16;
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < kp; ++k) {
            int64_t j = k / 16, r = k % 16;
            int64_t s = r / 4, b = r % 4;
            uint32_t code = (packed[n * words + j] >> (8 * b + 2 * s)) & 3u;
            if (code == 3u) { ++bad; continue; }
            if (k < K) t[n * K + k] = (int8_t)((int)code - 1);
            else if (code != 1u) ++bad;
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Packed 1-bit layout for the binary variant ([P1] "1-Bit重みとSign関数":
 * W_b = Sign(W) has two values, so one bit per weight suffices; [P2] counts
 * the 1-bit memory saving).  Layout used here:
 *   row n holds Kb = K rounded up to 128 weights as Kb/32 words;
 *   word j covers weights 32j .. 32j+31;
 *   weight 32j + 4s + b (s = 0..7, b = 0..3) is bit 8b + s of the word;
 *   the bit is 1 for +1 and 0 for -1; weights k >= K are padding, bit 0. */
int64_t orc_padded_k1(int64_t K) { return (K + 127) / 128 * 128; }

/* t holds only -1 and +1; returns the number of other values met (packed
 * as -1). */
int64_t orc_pack1(const int8_t *t, int64_t N, int64_t K, uint32_t *packed) {
    int64_t kb = orc_padded_k1(K);
    int64_t words = kb / 32;
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < words; ++j) {
            uint32_t word = 0;
            for (int64_t k = 32 * j; k < 32 * j + 32; ++k) {
                uint32_t bit = 0u;
                if (k < K) {
                    int8_t v = t[n * K + k];
                    if (v == 1) bit = 1u;
                    else if (v != -1) ++bad;
                }
                int64_t r = k - 32 * j;
                int64_t s = r / 4, b = r % 4;
                word |= bit << (8 * b + s);
            }
            packed[n * words + j] = word;
        }
    }
    return bad;
}

/* Inverse of orc_pack1.  Returns the number of padding bits that are set. */
int64_t orc_unpack1(const uint32_t *packed, int64_t N, int64_t K, int8_t *t) {
    int64_t kb = orc_padded_k1(K);
    int64_t words = kb / 32;
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < kb; ++k) {
            int64_t j = k / 32, r = k % 32;
            int64_t s = r / 4, b = r % 4;
            uint32_t bit = (packed[n * words + j] >> (8 * b + s)) & 1u;
            if (k < K) t[n * K + k] = bit ? (int8_t)1 : (int8_t)-1;
            else if (bit) ++bad;
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* [P1] "BitNet b1.58" activation_quant: per token (row) scale = max |x| over
 * the row; x * Q / (scale + 1e-5), evaluated left to right, rounded half to
 * even, clamped.  Q = 127 and the clamp is [-127, 127] (symmetric range of
 * [P2] "BitLinearの仕組み").  Also returns the row sum of the codes. */
void orc_act_quant(const float *x, int64_t M, int64_t K, int8_t *q, float *gamma,
                   int32_t *rowsum) {
    for (int64_t m = 0; m < M; ++m) {
        const float *xr = x + m * K;
        float g = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xr[k]);
            if (a > g) g = a;
        }
        float d = g + ORC_EPS;
        int32_t rs = 0;
        for (int64_t k = 0; k < K; ++k) {
            float v = (xr[k] * ORC_Q) / d;
            float r = nearbyintf(v);
            if (r > ORC_Q) r = ORC_Q;
            if (r < -ORC_Q) r = -ORC_Q;
            q[m * K + k] = (int8_t)r;
            rs += (int32_t)r;
        }
        gamma[m] = g;
        if (rowsum) rowsum[m] = rs;
    }
}

/* [P1] "BitNet a4.8": activations in 4 bits, with the top fraction of the
 * values (the outliers) split off and kept in 8 bits.  Reading taken here
 * (the page gives no formulas): per token row, the n_out entries of largest
 * |x| (ties to the lower index) are outliers; they are quantised like
 * activation_quant with Q = 127 and their own scale g8 = their max |x|; all
 * other entries are quantised with Q = 7 (symmetric 4-bit range [-7, 7]) and
 * the scale g4 = max |x| over them.  Each code vector is zero where the
 * other one holds the entry.  outlier [M][K] receives 1 at the outliers. */
static const float *orc_sort_row;

static int orc_outlier_order(const void *a, const void *b) {
    int64_t i = *(const int64_t *)a, j = *(const int64_t *)b;
    float u = fabsf(orc_sort_row[i]), v = fabsf(orc_sort_row[j]);
    if (u > v) return -1;
    if (u < v) return 1;
    return (i < j) ? -1 : (i > j);
}

void orc_act_quant_a48(const float *x, int64_t M, int64_t K, int64_t n_out, int8_t *q4,
                       float *g4, int32_t *rs4, int8_t *q8, float *g8, int32_t *rs8,
                       uint8_t *outlier) {
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
    if (n_out > K) n_out = K;
    if (n_out < 0) n_out = 0;
    for (int64_t m = 0; m < M; ++m) {
        const float *xr = x + m * K;
        uint8_t *out = outlier + m * K;
        for (int64_t k = 0; k < K; ++k) order[k] = k;
        orc_sort_row = xr;
        qsort(order, (size_t)K, sizeof(int64_t), orc_outlier_order);
        for (int64_t k = 0; k < K; ++k) out[k] = 0;
        for (int64_t j = 0; j < n_out; ++j) out[order[j]] = 1;
        float a8 = 0.0f, a4 = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xr[k]);
            if (out[k]) { if (a > a8) a8 = a; }
            else if (a > a4) a4 = a;
        }
        float d8 = a8 + ORC_EPS, d4 = a4 + ORC_EPS;
        int32_t s4 = 0, s8 = 0;
        for (int64_t k = 0; k < K; ++k) {
            int8_t c4 = 0, c8 = 0;
            if (out[k]) {
                float r = nearbyintf((xr[k] * ORC_Q) / d8);
                if (r > ORC_Q) r = ORC_Q;
                if (r < -ORC_Q) r = -ORC_Q;
                c8 = (int8_t)r;
            } else {
                float r = nearbyintf((xr[k] * 7.0f) / d4);
                if (r > 7.0f) r = 7.0f;
                if (r < -7.0f) r = -7.0f;
                c4 = (int8_t)r;
            }
            q4[m * K + k] = c4;
            q8[m * K + k] = c8;
            s4 += c4;
            s8 += c8;
        }
        g4[m] = a4;
        g8[m] = a8;
        if (rs4) rs4[m] = s4;
        if (rs8) rs8[m] = s8;
    }
    free(order);
}

/* The a4.8 output: each part dequantised as [P1]'s listing does
 * (output * (w_scale * x_scale) / Q, left to right), then the two added. */
void orc_dequant_a48(const int32_t *acc4, const float *g4, const int32_t *acc8, const float *g8,
                     float gamma_w, int64_t M, int64_t N, float *y) {
    for (int64_t m = 0; m < M; ++m) {
        float s4 = gamma_w * g4[m], s8 = gamma_w * g8[m];
        for (int64_t n = 0; n < N; ++n) {
            float y4 = ((float)acc4[m * N + n] * s4) / 7.0f;
            float y8 = ((float)acc8[m * N + n] * s8) / ORC_Q;
            y[m * N + n] = y4 + y8;
        }
    }
}

/* [P1] F.linear(x_q, w_q) with no bias ([P5]): acc[m][n] = sum_k q[m][k] *
 * t[n][k], an exact integer sum.  W is [N][K] (out, in) as in the listings'
 * nn.Parameter(out_features, in_features). */
void orc_int_linear(const int8_t *q, const int8_t *t, int64_t M, int64_t N, int64_t K,
                    int32_t *acc) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int32_t)q[m * K + k] * (int32_t)t[n * K + k];
            acc[m * N + n] = s;
        }
    }
}

/* [P1] dequant: output * (w_scale * x_scale) / Q, left to right. */
void orc_dequant(const int32_t *acc, const float *gamma_x, float gamma_w, int64_t M,
                 int64_t N, float *y) {
    for (int64_t m = 0; m < M; ++m) {
        float s = gamma_w * gamma_x[m];
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = ((float)acc[m * N + n] * s) / ORC_Q;
    }
}

/* [P1] nn.RMSNorm over the last dimension: y = x * rsqrt(mean(x^2) + eps) * g.
 * mean(x^2) is the exact sum rounded to binary64, divided by D in binary64,
 * rounded to binary32; rsqrt is a correctly rounded sqrt followed by a
 * correctly rounded reciprocal.  g may be NULL (ones). */
void orc_rmsnorm(const float *x, const float *g, float eps, int64_t M, int64_t D, float *y) {
    for (int64_t m = 0; m < M; ++m) {
        const float *xr = x + m * D;
        double s = orc_sq_sum_exact(xr, D);
        float ms = (float)(s / (double)D);
        float r = 1.0f / sqrtf(ms + eps);
        for (int64_t k = 0; k < D; ++k) {
            float v = xr[k] * r;
            y[m * D + k] = g ? v * g[k] : v;
        }
    }
}

/* [P5] ReLU² feed-forward with the gated structure: h = relu(g)^2 * u. */
void orc_relu2_mul(const float *g, const float *u, int64_t n, float *h) {
    for (int64_t i = 0; i < n; ++i) {
        float a = g[i] > 0.0f ? g[i] : 0.0f;
        h[i] = (a * a) * u[i];
    }
}

/* One BitLinear from float activations and unpacked ternary weights:
 * quantise x per token, integer linear, dequantise. */
void orc_bitlinear(const float *x, int64_t M, int64_t K, const int8_t *t, float gamma_w,
                   int64_t N, int8_t *q, float *gamma_x, int32_t *rowsum, int32_t *acc,
                   float *y) {
    orc_act_quant(x, M, K, q, gamma_x, rowsum);
    orc_int_linear(q, t, M, N, K, acc);
    orc_dequant(acc, gamma_x, gamma_w, M, N, y);
}

/* The feed-forward block: RMSNorm(D) -> int8 quant -> gate and up BitLinears
 * (D -> F) -> relu(gate)^2 * up -> int8 requant -> down BitLinear (F -> D).
 * With subln != 0 the down BitLinear normalises its input first, as every
 * BitLinear of [P1] "BitNet b1.58" does (self.norm before the activation
 * quantiser; the sub-layer norm of [P4] "正規化で分散を安定させる" and [P5]):
 * hn = RMSNorm(h) over F with weight subln_w (NULL: ones) and subln_eps, and
 * the requantisation reads hn instead of h.
 * Internal tensors are returned for inspection; the caller provides
 *   xn [M][D], qx [M][D], gx [M], hx [M][F], hn [M][F] (used only with
 *   subln), qh [M][F], gh [M], y [M][D]. */
void orc_ffn(const float *x, int64_t M, int64_t D, int64_t F, const float *norm_w,
             float norm_eps, const int8_t *tg, float sg, const int8_t *tu, float su,
             const int8_t *td, float sd, int subln, const float *subln_w, float subln_eps,
             float *xn, int8_t *qx, float *gx, float *hx, float *hn, int8_t *qh, float *gh,
             float *y) {
    orc_rmsnorm(x, norm_w, norm_eps, M, D, xn);
    orc_act_quant(xn, M, D, qx, gx, NULL);
    int32_t *acc_g = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * F));
    int32_t *acc_u = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * F));
    float *yg = (float *)malloc(sizeof(float) * (size_t)(M * F));
    float *yu = (float *)malloc(sizeof(float) * (size_t)(M * F));
    int32_t *acc_d = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * D));
    orc_int_linear(qx, tg, M, F, D, acc_g);
    orc_int_linear(qx, tu, M, F, D, acc_u);
    orc_dequant(acc_g, gx, sg, M, F, yg);
    orc_dequant(acc_u, gx, su, M, F, yu);
    orc_relu2_mul(yg, yu, M * F, hx);
    if (subln) {
        orc_rmsnorm(hx, subln_w, subln_eps, M, F, hn);
        orc_act_quant(hn, M, F, qh, gh, NULL);
    } else {
        orc_act_quant(hx, M, F, qh, gh, NULL);
    }
    orc_int_linear(qh, td, M, D, F, acc_d);
    orc_dequant(acc_d, gh, sd, M, D, y);
    free(acc_g);
    free(acc_u);
    free(yg);
    free(yu);
    free(acc_d);
}

/* Threads the OpenMP loops above will use (reported with timings). */
int orc_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
