/* Drives every function of the C oracle on small inputs, including the
 * degenerate ones (zero rows, all-equal rows, K not a multiple of 64 or
 * 128, n_out of 0 and of K), for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Checks the round trips it can check on its
 * own; the sanitizers report any out-of-bounds access, leak or undefined
 * operation.  Exits non-zero on a failed check. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_abs_sum_exact(const float *w, int64_t n);
double orc_sq_sum_exact(const float *x, int64_t n);
float orc_weight_scale(const float *w, int64_t n);
void orc_ternarize(const float *w, int64_t n, float gamma, int8_t *t);
void orc_binarize(const float *w, int64_t n, int8_t *t);
int64_t orc_padded_k(int64_t K);
void orc_pack(const int8_t *t, int64_t N, int64_t K, uint32_t *packed);
int64_t orc_unpack(const uint32_t *packed, int64_t N, int64_t K, int8_t *t);
int64_t orc_padded_k1(int64_t K);
int64_t orc_pack1(const int8_t *t, int64_t N, int64_t K, uint32_t *packed);
int64_t orc_unpack1(const uint32_t *packed, int64_t N, int64_t K, int8_t *t);
void orc_act_quant(const float *x, int64_t M, int64_t K, int8_t *q, float *gamma, int32_t *rowsum);
void orc_act_quant_a48(const float *x, int64_t M, int64_t K, int64_t n_out, int8_t *q4, float *g4,
                       int32_t *rs4, int8_t *q8, float *g8, int32_t *rs8, uint8_t *outlier);
void orc_dequant_a48(const int32_t *acc4, const float *g4, const int32_t *acc8, const float *g8,
                     float gamma_w, int64_t M, int64_t N, float *y);
void orc_int_linear(const int8_t *q, const int8_t *t, int64_t M, int64_t N, int64_t K, int32_t *acc);
void orc_dequant(const int32_t *acc, const float *gamma_x, float gamma_w, int64_t M, int64_t N,
                 float *y);
void orc_rmsnorm(const float *x, const float *g, float eps, int64_t M, int64_t D, float *y);
void orc_relu2_mul(const float *g, const float *u, int64_t n, float *h);
void orc_bitlinear(const float *x, int64_t M, int64_t K, const int8_t *t, float gamma_w, int64_t N,
                   int8_t *q, float *gamma_x, int32_t *rowsum, int32_t *acc, float *y);
void orc_ffn(const float *x, int64_t M, int64_t D, int64_t F, const float *norm_w, float norm_eps,
             const int8_t *tg, float sg, const int8_t *tu, float su, const int8_t *td, float sd,
             int subln, const float *subln_w, float subln_eps, float *xn, int8_t *qx, float *gx,
             float *hx, float *hn, int8_t *qh, float *gh, float *y);

static uint64_t st = 0x243F6A8885A308D3ull;
static float frand(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (float)((int64_t)(st >> 11) - (1ll << 52)) / (float)(1ll << 52);
}
#define NEW(T, n) ((T *)calloc((size_t)(n) > 0 ? (size_t)(n) : 1, sizeof(T)))

static int layer(int64_t M, int64_t K, int64_t N) {
    float *w = NEW(float, N * K), *x = NEW(float, M * K);
    for (int64_t i = 0; i < N * K; ++i) w[i] = 0.02f * frand();
    for (int64_t i = 0; i < M * K; ++i) x[i] = frand();
    if (M > 1)
        for (int64_t k = 0; k < K; ++k) x[K + k] = 0.0f;         /* zero row */
    if (M > 2)
        for (int64_t k = 0; k < K; ++k) x[2 * K + k] = 1.5f;     /* all equal */
    const float g = orc_weight_scale(w, N * K);
    int8_t *t = NEW(int8_t, N * K), *tb = NEW(int8_t, N * K), *t2 = NEW(int8_t, N * K);
    orc_ternarize(w, N * K, g, t);
    orc_binarize(w, N * K, tb);
    const int64_t kp = orc_padded_k(K), kb = orc_padded_k1(K);
    uint32_t *p = NEW(uint32_t, N * kp / 16), *p1 = NEW(uint32_t, N * kb / 32);
    orc_pack(t, N, K, p);
    int bad = orc_unpack(p, N, K, t2) != 0 || memcmp(t, t2, (size_t)(N * K)) != 0;
    orc_pack1(tb, N, K, p1);
    bad |= orc_unpack1(p1, N, K, t2) != 0 || memcmp(tb, t2, (size_t)(N * K)) != 0;
    int8_t *q = NEW(int8_t, M * K), *q4 = NEW(int8_t, M * K), *q8 = NEW(int8_t, M * K);
    float *gx = NEW(float, M), *g4 = NEW(float, M), *g8 = NEW(float, M), *y = NEW(float, M * N);
    int32_t *rs = NEW(int32_t, M), *r4 = NEW(int32_t, M), *r8 = NEW(int32_t, M);
    int32_t *acc = NEW(int32_t, M * N), *acc8 = NEW(int32_t, M * N);
    uint8_t *out = NEW(uint8_t, M * K);
    orc_bitlinear(x, M, K, t, g, N, q, gx, rs, acc, y);
    orc_act_quant(x, M, K, q, gx, rs);
    const int64_t nouts[4] = {0, 1, K / 3, K};
    for (int i = 0; i < 4; ++i) {
        orc_act_quant_a48(x, M, K, nouts[i], q4, g4, r4, q8, g8, r8, out);
        orc_int_linear(q4, t, M, N, K, acc);
        orc_int_linear(q8, t, M, N, K, acc8);
        orc_dequant_a48(acc, g4, acc8, g8, g, M, N, y);
    }
    orc_dequant(acc, gx, g, M, N, y);
    (void)orc_sq_sum_exact(x, M * K);
    (void)orc_abs_sum_exact(w, N * K);
    free(w); free(x); free(t); free(tb); free(t2); free(p); free(p1); free(q); free(q4); free(q8);
    free(gx); free(g4); free(g8); free(y); free(rs); free(r4); free(r8); free(acc); free(acc8);
    free(out);
    return bad;
}

static int ffn(int64_t M, int64_t D, int64_t F, int subln) {
    float *x = NEW(float, M * D), *nw = NEW(float, D), *sw = NEW(float, F);
    for (int64_t i = 0; i < M * D; ++i) x[i] = frand();
    for (int64_t i = 0; i < D; ++i) nw[i] = 1.0f + 0.1f * frand();
    for (int64_t i = 0; i < F; ++i) sw[i] = 1.0f + 0.1f * frand();
    int8_t *tg = NEW(int8_t, F * D), *tu = NEW(int8_t, F * D), *td = NEW(int8_t, D * F);
    for (int64_t i = 0; i < F * D; ++i) {
        tg[i] = (int8_t)((st >> 3) % 3) - 1; frand();
        tu[i] = (int8_t)((st >> 5) % 3) - 1; frand();
        td[i] = (int8_t)((st >> 7) % 3) - 1; frand();
    }
    float *xn = NEW(float, M * D), *gx = NEW(float, M), *hx = NEW(float, M * F), *hn = NEW(float, M * F);
    float *gh = NEW(float, M), *y = NEW(float, M * D), *h2 = NEW(float, M * F);
    int8_t *qx = NEW(int8_t, M * D), *qh = NEW(int8_t, M * F);
    orc_ffn(x, M, D, F, subln ? NULL : nw, 1e-6f, tg, 0.02f, tu, 0.03f, td, 0.01f, subln,
            subln ? sw : NULL, 1e-6f, xn, qx, gx, hx, hn, qh, gh, y);
    orc_rmsnorm(x, NULL, 1e-6f, M, D, xn);
    orc_relu2_mul(hx, hx, M * F, h2);
    free(x); free(nw); free(sw); free(tg); free(tu); free(td); free(xn); free(gx); free(hx);
    free(hn); free(gh); free(y); free(h2); free(qx); free(qh);
    return 0;
}

int main(void) {
    int bad = 0;
    const int64_t shapes[][3] = {{1, 1, 1}, {3, 15, 17}, {4, 63, 5}, {2, 64, 3}, {5, 65, 9},
                                 {3, 127, 4}, {3, 129, 7}, {6, 300, 11}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        bad |= layer(shapes[i][0], shapes[i][1], shapes[i][2]);
    bad |= ffn(3, 64, 96, 0) | ffn(2, 100, 70, 1) | ffn(1, 8, 8, 1);
    float z[5] = {0, 0, 0, 0, 0};
    bad |= orc_weight_scale(z, 5) != 0.0f;
    printf("%s\n", bad ? "FAIL" : "ok");
    return bad;
}
