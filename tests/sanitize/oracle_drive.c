/*
 * oracle_drive.c -- runs every function of the CPU oracle (oracle/sage_oracle.c)
 * on small seeded inputs and their edge cases (empty and ragged lengths,
 * all-zero blocks, special floats, splits, causal masks, Nq != Nkv), so that
 * an AddressSanitizer / UndefinedBehaviorSanitizer build can check the
 * oracle's memory accesses and arithmetic.  Test infrastructure: built and
 * run by tests/test_sanitizers.py; exits non-zero on a failed sanity check.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float orc_f16_decode(uint16_t h);
uint16_t orc_f16_encode(float f);
float orc_bf16_decode(uint16_t h);
uint16_t orc_bf16_encode(float f);
float orc_e4m3_decode(uint8_t b);
uint8_t orc_e4m3_encode_sat(float f);
void orc_decode16(const uint16_t* in, float* out, int64_t n, int dtype);
void orc_encode16(const float* in, uint16_t* out, int64_t n, int dtype);
void orc_decode_e4m3(const uint8_t* in, float* out, int64_t n);
void orc_encode_e4m3(const float* in, uint8_t* out, int64_t n);
void orc_channel_mean(const float* x, int64_t n, int d, float* mu);
void orc_smooth(const float* x, const float* mu, int64_t n, int d, float* xs);
void orc_quant_int8_blocks(const float* xs, int64_t n, int d, int blk, int8_t* codes,
                           float* scales);
void orc_quant_fp8_channels(const float* vs, int64_t n, int d, uint8_t* codes, float* scales);
void orc_delta_s(const float* mu_q, const float* ks, int64_t n_kv, int d, float* ds);
void orc_block_mean(const float* x, int64_t n, int d, int blk, float* mu);
void orc_smooth_blocks(const float* x, const float* mu, int64_t n, int d, int blk, float* xs);
void orc_mu_code(const float* x, int d, int8_t* hi, int8_t* lo, float* scale);
void orc_delta_s_block(const float* ds_seq, const int8_t* hi, const int8_t* lo, float scale,
                       const int8_t* kc, const float* k_scale, int64_t nkv, int d, int blk,
                       float* ds);
void orc_qk_int32(const int8_t* qc, const int8_t* kc, int64_t nq, int64_t nkv, int d,
                  int32_t* s);
void orc_attn_recipe_rows(const int8_t* qc, const float* q_scale, const int8_t* kc,
                          const float* k_scale, const uint8_t* vc, const float* v_scale,
                          const float* delta_s, const float* mu_v, int64_t nq, int64_t nkv, int d,
                          float sm_scale, int causal, int bkv, int blk, int64_t split,
                          const int64_t* rows, int64_t nrows, float* out, float* lse, float* tie);
void orc_attn_recipe_half_rows(const int8_t* qc, const float* q_scale, const int8_t* kc,
                               const float* k_scale, const uint16_t* vh, int bf16,
                               const float* delta_s, const float* mu_v, int64_t nq, int64_t nkv,
                               int d, float sm_scale, int causal, int bkv, int blk, int64_t split,
                               const int64_t* rows, int64_t nrows, float* out, float* lse,
                               float* tie);
void orc_attn_exact_rows(const float* q, const float* k, const float* v, int64_t nq, int64_t nkv,
                         int d, double sm_scale, int causal, const int64_t* rows, int64_t nrows,
                         double* out, double* lse);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double unif(void) {
    rng_state += 0x9e3779b97f4a7c15ull;
    uint64_t z = rng_state;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static float randn(void) {
    double u = unif(), v = unif();
    if (u < 1e-300) u = 1e-300;
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static int fails = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++fails;                                                    \
        }                                                               \
    } while (0)

static void codecs(void) {
    for (uint32_t h = 0; h < 65536; ++h) {
        float a = orc_f16_decode((uint16_t)h), b = orc_bf16_decode((uint16_t)h);
        if (!isnan(a)) CHECK(orc_f16_encode(a) == (uint16_t)h || a == 0.0f);
        if (!isnan(b)) CHECK(orc_bf16_encode(b) == (uint16_t)h || b == 0.0f);
    }
    for (int b = 0; b < 256; ++b) {
        float x = orc_e4m3_decode((uint8_t)b);
        if (!isnan(x)) CHECK(orc_e4m3_encode_sat(x) == (uint8_t)b || x == 0.0f);
    }
    const float special[] = {NAN, INFINITY, -INFINITY, 0.0f, -0.0f, 1e-45f, -1e-45f, 1e-40f,
                             65504.0f, 65520.0f, 3.4e38f, 448.0f, 464.0f, 1e30f, -1e30f};
    for (size_t i = 0; i < sizeof(special) / sizeof(special[0]); ++i) {
        (void)orc_f16_encode(special[i]);
        (void)orc_bf16_encode(special[i]);
        (void)orc_e4m3_encode_sat(special[i]);
    }
    float f[7] = {1.f, -2.f, 0.5f, 3e5f, -1e-9f, 448.f, 0.f};
    uint16_t h[7];
    uint8_t e[7];
    float g[7];
    for (int dt = 0; dt < 2; ++dt) {
        orc_encode16(f, h, 7, dt);
        orc_decode16(h, g, 7, dt);
    }
    orc_encode_e4m3(f, e, 7);
    orc_decode_e4m3(e, g, 7);
    orc_encode16(f, h, 0, 0);
}

static void prepass_and_attention(int nq, int nkv, int d, int blk, int causal, int64_t split) {
    float* q = malloc(sizeof(float) * (size_t)(nq ? nq : 1) * d);
    float* k = malloc(sizeof(float) * (size_t)(nkv ? nkv : 1) * d);
    float* v = malloc(sizeof(float) * (size_t)(nkv ? nkv : 1) * d);
    for (int i = 0; i < nq * d; ++i) q[i] = randn() + 2.0f;
    for (int i = 0; i < nkv * d; ++i) k[i] = randn() * 2.0f;
    for (int i = 0; i < nkv * d; ++i) v[i] = randn();
    if (nkv > blk)   /* an all-zero K block and an all-zero V channel */
        for (int i = 0; i < blk * d; ++i) k[i] = 0.0f;
    for (int j = 0; j < nkv; ++j) v[j * d + 1] = 0.0f;

    float* mu = malloc(sizeof(float) * d);
    float* ks = malloc(sizeof(float) * (size_t)(nkv ? nkv : 1) * d);
    float* vs = malloc(sizeof(float) * (size_t)(nkv ? nkv : 1) * d);
    orc_channel_mean(k, nkv, d, mu);
    orc_smooth(k, mu, nkv, d, ks);
    orc_smooth(v, NULL, nkv, d, vs);
    const int nbq = (nq + blk - 1) / blk, nbk = (nkv + blk - 1) / blk;
    int8_t* qc = malloc((size_t)(nq ? nq : 1) * d);
    int8_t* kc = malloc((size_t)(nkv ? nkv : 1) * d);
    uint8_t* vc = malloc((size_t)(nkv ? nkv : 1) * d);
    uint16_t* vh = malloc(sizeof(uint16_t) * (size_t)(nkv ? nkv : 1) * d);
    float* qsc = malloc(sizeof(float) * (nbq ? nbq : 1));
    float* ksc = malloc(sizeof(float) * (nbk ? nbk : 1));
    float* vsc = malloc(sizeof(float) * d);
    float* ds = malloc(sizeof(float) * (nkv ? nkv : 1));
    float* ds2 = malloc(sizeof(float) * (nkv ? nkv : 1));
    orc_quant_int8_blocks(ks, nkv, d, blk, kc, ksc);
    orc_quant_fp8_channels(vs, nkv, d, vc, vsc);
    orc_encode16(vs, vh, (int64_t)nkv * d, 1);
    /* per-block Q smoothing */
    float* mub = malloc(sizeof(float) * (size_t)(nbq ? nbq : 1) * d);
    float* qs = malloc(sizeof(float) * (size_t)(nq ? nq : 1) * d);
    float* mubar = malloc(sizeof(float) * d);
    float* dev = malloc(sizeof(float) * d);
    int8_t* hi = malloc(d);
    int8_t* lo = malloc(d);
    orc_channel_mean(q, nq, d, mubar);
    orc_block_mean(q, nq, d, blk, mub);
    orc_smooth_blocks(q, mub, nq, d, blk, qs);
    orc_quant_int8_blocks(qs, nq, d, blk, qc, qsc);
    orc_delta_s(mubar, ks, nkv, d, ds);
    for (int b = 0; b < nbq; ++b) {
        float sc;
        for (int c = 0; c < d; ++c) dev[c] = mub[b * d + c] - mubar[c];
        orc_mu_code(dev, d, hi, lo, &sc);
        for (int c = 0; c < d; ++c) CHECK(hi[c] >= -127 && hi[c] <= 127 && lo[c] >= -64 && lo[c] <= 64);
        orc_delta_s_block(ds, hi, lo, sc, kc, ksc, nkv, d, blk, ds2);
        orc_delta_s_block(NULL, hi, lo, sc, kc, ksc, nkv, d, blk, ds2);
    }
    {
        float zero[4] = {0, 0, 0, 0}, sc = 1.0f;
        int8_t zh[4], zl[4];
        orc_mu_code(zero, 4, zh, zl, &sc);
        CHECK(sc == 0.0f && zh[0] == 0 && zl[3] == 0);
    }
    int32_t* s = malloc(sizeof(int32_t) * (size_t)(nq ? nq : 1) * (nkv ? nkv : 1));
    orc_qk_int32(qc, kc, nq, nkv, d, s);

    int64_t* rows = malloc(sizeof(int64_t) * (nq ? nq : 1));
    for (int i = 0; i < nq; ++i) rows[i] = i;
    float* out = malloc(sizeof(float) * (size_t)(nq ? nq : 1) * d);
    float* lse = malloc(sizeof(float) * (nq ? nq : 1));
    float* tie = malloc(sizeof(float) * (size_t)(nq ? nq : 1) * d);
    double* oe = malloc(sizeof(double) * (size_t)(nq ? nq : 1) * d);
    double* le = malloc(sizeof(double) * (nq ? nq : 1));
    const float sm = 1.0f / sqrtf((float)d);
    orc_attn_recipe_rows(qc, qsc, kc, ksc, vc, vsc, ds, mu, nq, nkv, d, sm, causal, 128, blk, split,
                         rows, nq, out, lse, tie);
    for (int i = 0; i < nq * d; ++i) CHECK(isfinite(out[i]));
    orc_attn_recipe_rows(qc, qsc, kc, ksc, vc, vsc, NULL, NULL, nq, nkv, d, sm, causal, 128, blk,
                         split, rows, nq, out, NULL, NULL);
    for (int bf = 0; bf < 2; ++bf)
        orc_attn_recipe_half_rows(qc, qsc, kc, ksc, vh, bf, ds, NULL, nq, nkv, d, sm, causal, 128,
                                  blk, split, rows, nq, out, lse, tie);
    orc_attn_exact_rows(q, k, v, nq, nkv, d, sm, causal, rows, nq, oe, le);
    orc_attn_exact_rows(q, k, v, nq, nkv, d, sm, causal, rows, 0, oe, NULL);

    free(q); free(k); free(v); free(mu); free(ks); free(vs); free(qc); free(kc); free(vc);
    free(vh); free(qsc); free(ksc); free(vsc); free(ds); free(ds2); free(mub); free(qs);
    free(mubar); free(dev); free(hi); free(lo); free(s); free(rows); free(out); free(lse);
    free(tie); free(oe); free(le);
}

int main(void) {
    codecs();
    const int shapes[][6] = {
        /* nq, nkv, d, blk, causal, split */
        {0, 0, 64, 64, 0, 0},     {1, 0, 64, 64, 1, 0},     {0, 5, 64, 64, 0, 0},
        {1, 1, 64, 64, 1, 0},     {17, 17, 64, 32, 0, 0},   {33, 70, 96, 64, 1, 0},
        {64, 50, 128, 64, 0, 0},  {130, 300, 64, 64, 1, 128}, {200, 70, 64, 32, 1, 0},
        {3, 900, 128, 64, 1, 256}, {65, 129, 96, 32, 0, 384},
    };
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        prepass_and_attention(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3],
                              shapes[i][4], shapes[i][5]);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle drive: ok\n");
    return 0;
}
