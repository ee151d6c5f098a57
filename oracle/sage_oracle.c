/*
 * sage_oracle.c -- plain, slow, scalar CPU oracle for the SageAttention /
 * SageAttention2 quantized attention forward pass (INT8 Q.K^T; FP8 P.V, or
 * 16-bit P.V in the first SageAttention's variant).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker of the HIP
 * library: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code, header, table or constant
 * generator with the GPU path and never includes a HIP header.  Build:
 *     gcc -O2 -ffp-contract=off -fPIC -shared -pthread sage_oracle.c -lm
 * (no -ffast-math, default rounding mode, IEEE denormals).
 *
 * Sources (web pages; cited by title and section):
 *  [PKG]   "sageattention" package page -- "What it is and what it does":
 *          smoothing, per-block quantization of Q and K, head dims 64/96/128,
 *          Nq != Nkv, GQA; "Quickstart": sageattn(q, k, v, tensor_layout,
 *          is_causal, smooth_k).
 *  [BLOG]  ComfyUI blog on SageAttention, list "main roles and features",
 *          item 2 ("keeping accuracy"): smoothing lowers quantization error;
 *          QK is computed in INT8 and PV in FP8, with different granularities.
 *  [SA2]   "SageAttention2: technical report" summary -- "Main concepts",
 *          item 2: Q and V are smoothed by subtracting their channel mean
 *          before quantization; item 3: the INT8+FP8 precision branch.
 *  [SA1]   SA1 abstract (llama.cpp discussion #9901): attention is O(N^2) and
 *          the method quantizes attention itself.
 *  [GUIDE] "SageAttention量化加速框架" install guide, section 3.1 (benchmark
 *          scripts): the qk_int8_pv_fp16 kernel, INT8 Q.K^T with a 16-bit
 *          P.V; [PKG] "What it is and what it does": FP16 accumulators.
 *
 * Every step below follows the plainest reading of those pages; where they
 * are silent the comment says which choice is taken.  Floating point: the
 * recipe functions use FP32 exactly as the method's GPU arithmetic is
 * specified (so that quantized codes are decided in the same precision on
 * both sides); the exact reference (orc_attn_exact_rows) is FP64 throughout.
 *
 * Pins: codecs are checked against numpy/torch conversions and their
 * definitions; the channel mean against closed forms; quantizers against
 * round-trip bounds; int32 Q.K^T against brute force; the recipe against
 * textbook special cases and FP64 attention (tests/test_oracle_*.py).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Codecs, written from the format definitions.                              */
/* ------------------------------------------------------------------------ */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
ORC_EXPORT float orc_f16_decode(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)       v = ldexp((double)m, -24);               /* subnormal  */
    else if (e == 31) v = m ? NAN : INFINITY;
    else              v = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -v : v);
}

/* Round-to-nearest-even encode of an FP32 value into binary16. */
ORC_EXPORT uint16_t orc_f16_encode(float f) {
    uint32_t u = f2u(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    float a = fabsf(f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0f) return (uint16_t)(sign | 0x7c00);     /* rounds to inf */
    /* Work in double: a is exact there; scale to integer units of the target
       ulp and round half to even with nearbyint (default mode = RNE). */
    double da = (double)a;
    if (da < ldexp(1.0, -14)) {                                 /* subnormal  */
        double q = nearbyint(da * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)q);                  /* q<=1024 ok */
    }
    int e; double fr = frexp(da, &e);                           /* da=fr*2^e  */
    double q = nearbyint(fr * 2048.0);                          /* 1024..2048 */
    if (q == 2048.0) { q = 1024.0; e += 1; }
    int ef = e - 1 + 15;
    if (ef >= 31) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (ef << 10) | ((int)q - 1024));
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
ORC_EXPORT float orc_bf16_decode(uint16_t h) { return u2f((uint32_t)h << 16); }

ORC_EXPORT uint16_t orc_bf16_encode(float f) {
    if (isnan(f)) return (uint16_t)((f2u(f) >> 16) | 0x40);
    double a = fabs((double)f);
    uint16_t sign = (uint16_t)((f2u(f) >> 16) & 0x8000);
    if (a == 0.0) return sign;
    if (isinf(f)) return (uint16_t)(sign | 0x7f80);
    if (a < ldexp(1.0, -126)) {                                 /* subnormal  */
        double q = nearbyint(a * ldexp(1.0, 133));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e; double fr = frexp(a, &e);
    double q = nearbyint(fr * 256.0);                           /* 128..256   */
    if (q == 256.0) { q = 128.0; e += 1; }
    int ef = e - 1 + 127;
    if (ef >= 255) return (uint16_t)(sign | 0x7f80);
    return (uint16_t)(sign | (ef << 7) | ((int)q - 128));
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
   infinities, S.1111.111 is NaN, largest finite 448, subnormals 2^-9..      */
ORC_EXPORT float orc_e4m3_decode(uint8_t b) {
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0)       v = ldexp((double)m, -9);
    else                   v = ldexp((double)(8 + m), e - 10);
    return (float)(s ? -v : v);
}

/* RNE encode with saturation to +-448 (OCP e4m3fn, the FP8 flavour gfx950
   converts to natively; the pages say only "FP8").  NaN maps to 0x7f. */
ORC_EXPORT uint8_t orc_e4m3_encode_sat(float f) {
    if (isnan(f)) return 0x7f;
    uint8_t sign = (f2u(f) >> 31) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (a >= 448.0) return (uint8_t)(sign | 0x7e);              /* saturate   */
    if (a < ldexp(1.0, -6)) {                                   /* subnormal  */
        double q = nearbyint(a * 512.0);                        /* 0..8       */
        return (uint8_t)(sign | (uint8_t)q);                    /* 8 = 2^-6 ok*/
    }
    int e; double fr = frexp(a, &e);
    double q = nearbyint(fr * 16.0);                            /* 8..16      */
    if (q == 16.0) { q = 8.0; e += 1; }
    int ef = e - 1 + 7;
    if (ef > 15 || (ef == 15 && q - 8 >= 7)) return (uint8_t)(sign | 0x7e);
    return (uint8_t)(sign | (ef << 3) | ((int)q - 8));
}

/* Bulk decoders: dtype 0 = fp16, 1 = bf16. */
ORC_EXPORT void orc_decode16(const uint16_t* in, float* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype ? orc_bf16_decode(in[i]) : orc_f16_decode(in[i]);
}
ORC_EXPORT void orc_encode16(const float* in, uint16_t* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype ? orc_bf16_encode(in[i]) : orc_f16_encode(in[i]);
}
ORC_EXPORT void orc_decode_e4m3(const uint8_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(in[i]);
}
ORC_EXPORT void orc_encode_e4m3(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode_sat(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Pre-pass: smoothing and quantization ([PKG], [BLOG] item 2, [SA2] item 2) */
/* ------------------------------------------------------------------------ */

/* Per-channel mean over all n tokens of one (sequence, head) -- the pages
   fix neither the scope nor the summation order; this order is a reading.
   x is [n][d] row-major FP32 (exactly decoded inputs).  Order: tokens are
   grouped in chunks of 64 aligned to the sequence start; each chunk is summed
   token by token in FP32, the chunk sums are added in chunk order in FP32,
   and the total is divided by n with one correctly rounded FP32 division.  */
ORC_EXPORT void orc_channel_mean(const float* x, int64_t n, int d, float* mu) {
    for (int c = 0; c < d; ++c) {
        float total = 0.0f;
        for (int64_t t0 = 0; t0 < n; t0 += 64) {
            float part = 0.0f;
            int64_t t1 = t0 + 64 < n ? t0 + 64 : n;
            for (int64_t t = t0; t < t1; ++t) part = part + x[t * d + c];
            total = total + part;
        }
        mu[c] = n > 0 ? total / (float)n : 0.0f;
    }
}

/* x_s = fl32(x - mu) per element (the smoothed value stays FP32; it is not
   re-rounded to the input dtype).
   mu == NULL means no smoothing (x_s = x). */
ORC_EXPORT void orc_smooth(const float* x, const float* mu, int64_t n, int d, float* xs) {
    for (int64_t t = 0; t < n; ++t)
        for (int c = 0; c < d; ++c)
            xs[t * d + c] = mu ? x[t * d + c] - mu[c] : x[t * d + c];
}

/* The quotients k/a of the quantizers below (k = 127, 448 or 16256 over an
   absmax a) leave the FP32 range once a falls below k/FLT_MAX, about
   10^-36 .. 10^-34 (reachable with bf16 inputs); the inverse scale would be
   infinite and the codes sign-only (and NaN for zeros).  For the INT8 Q/K
   blocks and the 15-bit deviation code, where a < 2^-100 the values and a
   are therefore scaled by 2^64 before the quotient: exact there (subnormals
   included), and the codes are then those the same block gets at any other
   power-of-two scale.  Above 2^-100 the factor is 1 and changes nothing.
   (V channels that small count as zero instead: orc_quant_fp8_channels.)   */
static float tiny_rescale(float a) { return a < 0x1p-100f ? 0x1p64f : 1.0f; }

/* Per-block symmetric INT8 quantization (block size, absmax scale, rounding
   and the zero block are readings where the pages are silent): blocks of `blk` tokens
   aligned to the sequence start (the last one may be short).  a = max |x_s|
   over the block; a == 0 gives scale 0 and zero codes; otherwise
   inv = fl32(127/a), scale = fl32(a/127), code = clamp(rne(fl32(x_s*inv)),
   -127, 127) (with the rescale of tiny_rescale: inv = fl32(127/(a*r)),
   code from fl32((x_s*r)*inv)).  codes: [n][d]; scales: [ceil(n/blk)].      */
ORC_EXPORT void orc_quant_int8_blocks(const float* xs, int64_t n, int d, int blk,
                                      int8_t* codes, float* scales) {
    for (int64_t b0 = 0, bi = 0; b0 < n; b0 += blk, ++bi) {
        int64_t b1 = b0 + blk < n ? b0 + blk : n;
        float a = 0.0f;
        for (int64_t t = b0; t < b1; ++t)
            for (int c = 0; c < d; ++c) {
                float v = fabsf(xs[t * d + c]);
                if (v > a) a = v;
            }
        if (a == 0.0f) {
            scales[bi] = 0.0f;
            for (int64_t t = b0; t < b1; ++t)
                for (int c = 0; c < d; ++c) codes[t * d + c] = 0;
            continue;
        }
        const float r = tiny_rescale(a);
        float inv = 127.0f / (a * r);
        scales[bi] = a / 127.0f;
        for (int64_t t = b0; t < b1; ++t)
            for (int c = 0; c < d; ++c) {
                float y = (xs[t * d + c] * r) * inv;
                float r = nearbyintf(y);                      /* RNE         */
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                codes[t * d + c] = (int8_t)r;
            }
    }
}

/* Per-channel FP8 E4M3 quantization of (smoothed) V (per channel: a V scale
   must be constant along the contracted token axis): per
   channel c, a = max over the n tokens of |v_s|; a == 0 gives scale 0 and
   zero codes, and so does a < 2^-100 (a channel that small counts as zero:
   the output moves by less than 2^-100); otherwise inv = fl32(448/a),
   scale = fl32(a/448) and code = e4m3_rne_sat(fl32(v_s*inv)).
   codes: [n][d]; scales: [d].                                               */
ORC_EXPORT void orc_quant_fp8_channels(const float* vs, int64_t n, int d,
                                       uint8_t* codes, float* scales) {
    for (int c = 0; c < d; ++c) {
        float a = 0.0f;
        for (int64_t t = 0; t < n; ++t) {
            float v = fabsf(vs[t * d + c]);
            if (v > a) a = v;
        }
        if (a < 0x1p-100f) {
            scales[c] = 0.0f;
            for (int64_t t = 0; t < n; ++t) codes[t * d + c] = 0;
            continue;
        }
        float inv = 448.0f / a;
        scales[c] = a / 448.0f;
        for (int64_t t = 0; t < n; ++t)
            codes[t * d + c] = orc_e4m3_encode_sat(vs[t * d + c] * inv);
    }
}

/* Score bias that compensates Q smoothing: subtracting mu_q from every
   query changes each score q_i.k_j by mu_q.k_j, which depends on j, so it is
   added back: ds_j = sum_c mu_q[c] * k_s[j][c], accumulated in FP32 in
   ascending c.  k_s: [n_kv][d]; ds: [n_kv].                                 */
ORC_EXPORT void orc_delta_s(const float* mu_q, const float* ks, int64_t n_kv, int d,
                            float* ds) {
    for (int64_t j = 0; j < n_kv; ++j) {
        float acc = 0.0f;
        for (int c = 0; c < d; ++c) acc = acc + mu_q[c] * ks[j * d + c];
        ds[j] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Per-block Q smoothing ([SA2] "Main concepts" item 2 subtracts the channel */
/* mean of Q; the pages fix neither the span of the mean nor how the score   */
/* compensation is formed -- the choices below are readings).               */
/* ------------------------------------------------------------------------ */

/* Channel means of each quantization block of Q: blocks of `blk` tokens
   aligned to the sequence start (the last one may be short).  Per block and
   channel, the block's tokens are summed in order in FP32 and the sum is
   divided by the block's token count with one correctly rounded FP32
   division.  x [n][d]; mu [ceil(n/blk)][d].                                 */
ORC_EXPORT void orc_block_mean(const float* x, int64_t n, int d, int blk, float* mu) {
    for (int64_t b0 = 0, bi = 0; b0 < n; b0 += blk, ++bi) {
        int64_t b1 = b0 + blk < n ? b0 + blk : n;
        for (int c = 0; c < d; ++c) {
            float sum = 0.0f;
            for (int64_t t = b0; t < b1; ++t) sum = sum + x[t * d + c];
            mu[bi * d + c] = sum / (float)(b1 - b0);
        }
    }
}

/* x_s = fl32(x - mu_b) with mu_b the mean of the token's own block. */
ORC_EXPORT void orc_smooth_blocks(const float* x, const float* mu, int64_t n, int d, int blk,
                                  float* xs) {
    for (int64_t t = 0; t < n; ++t)
        for (int c = 0; c < d; ++c) xs[t * d + c] = x[t * d + c] - mu[(t / blk) * d + c];
}

/* A block mean's deviation from the sequence mean as an integer code of 15
   bits with one FP32 scale, so that the block's share of the score
   compensation is an integer product with the INT8 key codes: for the
   vector x (x = fl32(mu_b - mu_q) per channel), a = max_c |x_c|; a == 0
   gives scale 0 and zero codes; otherwise inv = fl32(16256/a),
   scale = fl32(a/16256) (16256 = 127*128), and per channel y = fl32(x_c*inv),
   hi = clamp(rne(y/128), -127, 127), lo = rne(y - 128*hi) (|lo| <= 64), so
   that x_c ~ scale*(128*hi + lo) within scale/2 (tiny_rescale as for INT8).
   hi, lo: [d] int8.                                                         */
ORC_EXPORT void orc_mu_code(const float* x, int d, int8_t* hi, int8_t* lo, float* scale) {
    float a = 0.0f;
    for (int c = 0; c < d; ++c) {
        float v = fabsf(x[c]);
        if (v > a) a = v;
    }
    if (a == 0.0f) {
        *scale = 0.0f;
        for (int c = 0; c < d; ++c) hi[c] = lo[c] = 0;
        return;
    }
    const float r = tiny_rescale(a);
    float inv = 16256.0f / (a * r);
    *scale = a / 16256.0f;
    for (int c = 0; c < d; ++c) {
        float y = (x[c] * r) * inv;
        float h = nearbyintf(y / 128.0f);                  /* exact scaling */
        if (h > 127.0f) h = 127.0f;
        if (h < -127.0f) h = -127.0f;
        float l = nearbyintf(y - 128.0f * h);              /* exact difference */
        hi[c] = (int8_t)h;
        lo[c] = (int8_t)l;
    }
}

/* The score compensation of one Q block smoothed by its own mean mu_b.
   Subtracting mu_b from the block's queries changes each score q_i.k_j by
   mu_b.k_j = mu_q.k_j + (mu_b - mu_q).k_j.  The first term is the sequence's
   compensation ds_seq_j (orc_delta_s, from the unquantized K_s); the block's
   deviation is added from its code and the same INT8 key codes the scores
   use: ds_j = fl32(ds_seq_j + fl32(fl32(T_j) * fl32(scale * k_scale[j/blk])))
   with the exact integer T_j = sum_c (128*hi_c + lo_c) * kc[j][c].
   ds_seq [nkv] (NULL: 0); kc [nkv][d]; k_scale per `blk` keys; ds [nkv].    */
ORC_EXPORT void orc_delta_s_block(const float* ds_seq, const int8_t* hi, const int8_t* lo,
                                  float scale, const int8_t* kc, const float* k_scale,
                                  int64_t nkv, int d, int blk, float* ds) {
    for (int64_t j = 0; j < nkv; ++j) {
        int64_t T = 0;
        for (int c = 0; c < d; ++c)
            T += (128 * (int64_t)hi[c] + (int64_t)lo[c]) * (int64_t)kc[j * d + c];
        float f = scale * k_scale[j / blk];
        float corr = (float)T * f;
        ds[j] = ds_seq ? ds_seq[j] + corr : corr;
    }
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* S = Qc . Kc^T in int32 ([BLOG] item 2: QK in INT8).  qc [nq][d],
   kc [nkv][d], s [nq][nkv].  |S| <= d*127^2 < 2^24 for d <= 128.           */
ORC_EXPORT void orc_qk_int32(const int8_t* qc, const int8_t* kc, int64_t nq, int64_t nkv,
                             int d, int32_t* s) {
    for (int64_t i = 0; i < nq; ++i)
        for (int64_t j = 0; j < nkv; ++j) {
            int32_t acc = 0;
            for (int c = 0; c < d; ++c) acc += (int32_t)qc[i * d + c] * (int32_t)kc[j * d + c];
            s[i * nkv + j] = acc;
        }
}

/* Last key index visible to query row i (inclusive), or nkv-1 if not causal.
   Causal masking is aligned bottom-right: row i sees j <= i + nkv - nq. */
static int64_t last_visible(int64_t i, int64_t nq, int64_t nkv, int causal) {
    if (!causal) return nkv - 1;
    int64_t lim = i + nkv - nq;
    return lim < nkv - 1 ? lim : nkv - 1;
}

/* Same-recipe forward for selected query rows of one (sequence, q-head).
 *   qc, q_scale : int8 codes [nq][d], FP32 scale per 64-token block
 *   kc, k_scale : int8 codes [nkv][d], FP32 scale per 64-token block
 *   vdec        : the decoded V operand [nkv][d] (exact in FP32)
 *   out_scale   : FP32 [d] factor applied to acc at the end, or NULL (1)
 *   p_mode      : how p becomes the P.V operand (P_FP8 or P_F16 / P_BF16)
 *   delta_s     : FP32 [nkv] Q-smoothing compensation, or NULL; with
 *                 ds_rows > 0, FP32 [ceil(nq/ds_rows)][nkv]: row i takes
 *                 row i / ds_rows (one compensation per Q block)
 *   mu_v        : FP32 [d] V mean to add back at the output, or NULL
 *   bkv         : key-tile width of the online softmax (p^ depends on it)
 *   split       : keys per split (a multiple of bkv), or 0 for one split
 *   rows[nrows] : query rows to compute; out [nrows][d] FP32, lse [nrows]
 *   tie         : [nrows][d] FP32 or NULL: the rounding-tie bound below
 * Steps: s = fl32(S)*(sq*sk*sm_scale) (+ ds_j*sm_scale); the keys are cut into
 * splits of `split` keys, and in each split, for each key tile in order:
 * m' = max(m, max s), alpha = e^(m-m'), p = e^(s-m') (FP32),
 * l = alpha*l + sum p (from the FP32 p), p^ = the P.V operand made from p,
 * acc = alpha*acc + sum p^ * v, starting from m = -inf, l = 0, acc = 0.
 * The splits are then merged as partial softmax results (the log-sum-exp
 * merge of flash-decoding): M = max m_s, w_s = e^(m_s - M), L = sum w_s l_s,
 * A = sum w_s acc_s (in split order); o = A*out_scale/L (+ mu_v).  One split
 * is the plain online softmax.  A row that sees no key gives o = 0 and
 * lse = -inf.  LSE = M + ln L, the natural log of sum_j e^(s_j) over the
 * scores as the recipe forms them.
 *
 * Rounding-tie bound.  p^ is a code picked by rounding p (times 448 for E4M3)
 * in FP32.  The plain FP32 evaluations of the exponent (another order of its
 * products, log2 units, a hardware exp2 within an ulp, a row maximum taken a
 * few units in its last place higher) move p by a few parts in 2^24 of the
 * terms' magnitudes, so every code that p rounds to within that window
 * (tie_window, relative) is a correct result of the recipe.  Per key the
 * bound adds the spread of those codes (the largest minus the smallest)
 * times |v| per channel, carried through the rescales and the split merge
 * like acc, and scaled like the output (out_scale / L).  The spread is one
 * code step where a rounding midpoint lies within the window and 0 where
 * none does; where the scores are so large that the window itself spans
 * several codes (a row maximum of 2^16 or more in log2 units, whose own unit
 * in the last place is then 2^-7 or coarser), it spans them all, the top
 * code 448 included.  The same window moves each p itself, and so the row
 * sum L: an evaluation whose p_j lie within e^(+-window_j) of the oracle's
 * has a sum between L - LD and L + LU (LD = sum p_j (1 - e^-window_j),
 * LU = sum p_j (e^window_j - 1), carried like l), which scales the whole row
 * even where every code stays (a nearly one-hot row whose top p is 1 + 2^-9
 * rather than 1 keeps the code 448 but divides by a larger L).  The factors
 * that rescale a code after it is picked (alpha between key tiles, e^(m_s - M)
 * in the split merge) are differences of such maxima, within the same window
 * of 1: per key tacc therefore also takes the largest code in the window times
 * (e^window - 1) times |v|.  The bound is tacc * |out_scale| / (L - LD) +
 * |o - mu_v| * max(LD / (L - LD), LU / (L + LU)). */
enum { P_FP8 = 0, P_F16 = 1, P_BF16 = 2 };

/* Relative window within which a rounding midpoint counts as a tie: twice the
 * unit roundoff per rounding, six roundings per term, over the magnitudes of
 * the exponent's terms (terms = |score product| + |Q-smoothing bias|, and the
 * row maximum m; natural-log units), plus a constant for the exponential and
 * the P scale. */
static double tie_window(double terms, double m) {
    return ldexp(1.0, -23) * (6.0 * (terms + fabs(m)) + 16.0);
}

/* The operand format's value nearest x >= 0 in the format's own units (p*448
 * for E4M3, saturating at 448; p for fp16/bf16), round to nearest even. */
static double operand_round(double x, int p_mode) {
    const float f = (float)x;
    switch (p_mode) {
    case P_FP8: return orc_e4m3_decode(orc_e4m3_encode_sat(f));
    case P_F16: return orc_f16_decode(orc_f16_encode(f));
    default:    return orc_bf16_decode(orc_bf16_encode(f));
    }
}

/* Spread of p's operand over the window: the code of p moved up by the
 * window less the code of p moved down by it (in the operand's units, as
 * p_operand returns it). */
static float tie_step(float p, int p_mode, double window) {
    const double x = p_mode == P_FP8 ? (double)(p * 448.0f) : (double)p;
    if (x <= 0.0) return 0.0f;
    const double lo = window < 1.0 ? x * (1.0 - window) : 0.0;
    return (float)(operand_round(x * (1.0 + window), p_mode) - operand_round(lo, p_mode));
}

static float p_operand(float p, int p_mode) {
    switch (p_mode) {
    case P_FP8: return orc_e4m3_decode(orc_e4m3_encode_sat(p * 448.0f));
    case P_F16: return orc_f16_decode(orc_f16_encode(p));
    default:    return orc_bf16_decode(orc_bf16_encode(p));
    }
}

static void recipe_rows(const int8_t* qc, const float* q_scale, const int8_t* kc,
                        const float* k_scale, const float* vdec, const float* out_scale,
                        int p_mode, const float* delta_s_all, int64_t ds_rows,
                        const float* mu_v, int64_t nq,
                        int64_t nkv, int d, float sm_scale, int causal, int bkv, int blk,
                        int64_t split, const int64_t* rows, int64_t nrows, float* out,
                        float* lse, float* tie) {
    const int64_t span = split > 0 ? split : (nkv > 0 ? nkv : 1);
    const int64_t nsplit = nkv > 0 ? (nkv + span - 1) / span : 1;
    float* s = (float*)malloc(sizeof(float) * (size_t)(bkv > 0 ? bkv : 1));
    float* mag = (float*)malloc(sizeof(float) * (size_t)(bkv > 0 ? bkv : 1));
    float* accs = (float*)malloc(sizeof(float) * (size_t)d * (size_t)nsplit);
    float* ms = (float*)malloc(sizeof(float) * (size_t)nsplit);
    float* ls = (float*)malloc(sizeof(float) * (size_t)nsplit);
    float* acc = (float*)malloc(sizeof(float) * (size_t)d);
    float* ties = (float*)malloc(sizeof(float) * (size_t)d * (size_t)nsplit);
    float* tacc = (float*)malloc(sizeof(float) * (size_t)d);
    double* lus = (double*)malloc(sizeof(double) * (size_t)nsplit);
    double* lds = (double*)malloc(sizeof(double) * (size_t)nsplit);
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        int64_t jmax = last_visible(i, nq, nkv, causal);
        float sq = q_scale[i / blk];
        const float* delta_s =
            delta_s_all && ds_rows > 0 ? delta_s_all + (i / ds_rows) * nkv : delta_s_all;
        for (int64_t sp = 0; sp < nsplit; ++sp) {
            float* a = accs + sp * d;
            float* ta = ties + sp * d;
            float m = -INFINITY, l = 0.0f;
            double lu = 0.0, ld = 0.0;      /* the window of l, up and down */
            for (int c = 0; c < d; ++c) a[c] = ta[c] = 0.0f;
            int64_t k_end = (sp + 1) * span - 1 < jmax ? (sp + 1) * span - 1 : jmax;
            for (int64_t t0 = sp * span; t0 <= k_end; t0 += bkv) {
                int64_t t1 = t0 + bkv - 1 < k_end ? t0 + bkv - 1 : k_end;
                int64_t nt = t1 - t0 + 1;
                float mt = -INFINITY;
                for (int64_t j = t0; j <= t1; ++j) {
                    int32_t S = 0;
                    for (int c = 0; c < d; ++c)
                        S += (int32_t)qc[i * d + c] * (int32_t)kc[j * d + c];
                    float comb = sq * k_scale[j / blk];
                    comb = comb * sm_scale;
                    float sv = (float)S * comb;
                    if (tie) mag[j - t0] = fabsf(sv) + (delta_s ? fabsf(delta_s[j] * sm_scale) : 0.0f);
                    if (delta_s) sv = sv + delta_s[j] * sm_scale;
                    s[j - t0] = sv;
                    if (sv > mt) mt = sv;
                }
                float mn = m > mt ? m : mt;
                float alpha = (m == -INFINITY) ? 0.0f : (float)exp((double)(m - mn));
                float psum = 0.0f;
                double pu = 0.0, pd = 0.0;
                for (int c = 0; c < d; ++c) a[c] = alpha * a[c];
                if (tie)
                    for (int c = 0; c < d; ++c) ta[c] = alpha * ta[c];
                for (int64_t jj = 0; jj < nt; ++jj) {
                    float p = (float)exp((double)(s[jj] - mn));
                    psum = psum + p;
                    float ph = p_operand(p, p_mode);
                    if (tie) {
                        const double wdw = tie_window(mag[jj], mn);
                        pu += (double)p * expm1(wdw);
                        pd -= (double)p * expm1(-wdw);
                        const float st = tie_step(p, p_mode, wdw);
                        /* the code spread, and the largest code scaled by the
                           window of the factors that rescale it */
                        const float kt = (float)((double)st + ((double)ph + st) * expm1(wdw));
                        if (kt > 0.0f) {
                            const float* vrow = vdec + (t0 + jj) * d;
                            for (int c = 0; c < d; ++c) ta[c] = ta[c] + kt * fabsf(vrow[c]);
                        }
                    }
                    if (ph == 0.0f) continue;     /* a zero product leaves acc as is */
                    const float* vrow = vdec + (t0 + jj) * d;
                    for (int c = 0; c < d; ++c) a[c] = a[c] + ph * vrow[c];
                }
                l = alpha * l + psum;
                lu = (double)alpha * lu + pu;
                ld = (double)alpha * ld + pd;
                m = mn;
            }
            ms[sp] = m;
            ls[sp] = l;
            lus[sp] = lu;
            lds[sp] = ld;
        }
        /* merge the splits */
        float M = -INFINITY, L = 0.0f;
        double LU = 0.0, LD = 0.0;
        for (int64_t sp = 0; sp < nsplit; ++sp)
            if (ms[sp] > M) M = ms[sp];
        for (int c = 0; c < d; ++c) acc[c] = tacc[c] = 0.0f;
        if (M != -INFINITY) {
            for (int64_t sp = 0; sp < nsplit; ++sp) {
                if (ms[sp] == -INFINITY) continue;   /* a split without visible keys */
                float w = (float)exp((double)(ms[sp] - M));
                L = L + w * ls[sp];
                LU += (double)w * lus[sp];
                LD += (double)w * lds[sp];
                for (int c = 0; c < d; ++c) acc[c] = acc[c] + w * accs[sp * d + c];
                if (tie)
                    for (int c = 0; c < d; ++c) tacc[c] = tacc[c] + w * ties[sp * d + c];
            }
        }
        float* o = out + r * d;
        if (jmax < 0 || L == 0.0f) {
            for (int c = 0; c < d; ++c) o[c] = 0.0f;
            if (tie)
                for (int c = 0; c < d; ++c) tie[r * d + c] = 0.0f;
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        for (int c = 0; c < d; ++c) {
            float val = (out_scale ? acc[c] * out_scale[c] : acc[c]) / L;
            if (tie) {
                const double lo = (double)L - LD;
                const double rel = fmax(LD / lo, LU / ((double)L + LU));
                tie[r * d + c] = (float)((double)tacc[c] * (out_scale ? fabsf(out_scale[c]) : 1.0f) / lo
                                         + fabs((double)val) * rel);
            }
            if (mu_v) val = val + mu_v[c];
            o[c] = val;
        }
        if (lse) lse[r] = M + logf(L);
    }
    free(s);
    free(mag);
    free(accs);
    free(ms);
    free(ls);
    free(acc);
    free(ties);
    free(tacc);
    free(lus);
    free(lds);
}

/* The INT8-QK / FP8-PV recipe ([BLOG] item 2, [SA2] item 3):
 *   vc, v_scale : e4m3 codes [nkv][d] (logical row-major), FP32 scale per
 *                 channel; p^ = e4m3(p*448) (static scale 448), and the end
 *                 factor is v_scale/448. */
ORC_EXPORT void orc_attn_recipe_rows(const int8_t* qc, const float* q_scale,
                                     const int8_t* kc, const float* k_scale,
                                     const uint8_t* vc, const float* v_scale,
                                     const float* delta_s, const float* mu_v,
                                     int64_t nq, int64_t nkv, int d, float sm_scale,
                                     int causal, int bkv, int blk, int64_t split,
                                     const int64_t* rows, int64_t nrows,
                                     float* out, float* lse, float* tie) {
    /* decode every V code once; dec(v^) is exact in FP32 */
    float* vdec = (float*)malloc(sizeof(float) * (size_t)(nkv > 0 ? nkv : 1) * (size_t)d);
    float* fac = (float*)malloc(sizeof(float) * (size_t)d);
    for (int64_t j = 0; j < nkv * d; ++j) vdec[j] = orc_e4m3_decode(vc[j]);
    for (int c = 0; c < d; ++c) fac[c] = v_scale[c] / 448.0f;
    recipe_rows(qc, q_scale, kc, k_scale, vdec, fac, P_FP8, delta_s, 0, mu_v, nq, nkv, d, sm_scale,
                causal, bkv, blk, split, rows, nrows, out, lse, tie);
    free(vdec);
    free(fac);
}

/* The same with one compensation per Q block (per-block Q smoothing):
 * delta_s is FP32 [ceil(nq/ds_rows)][nkv] and row i takes row i / ds_rows. */
ORC_EXPORT void orc_attn_recipe_rows_blockds(const int8_t* qc, const float* q_scale,
                                             const int8_t* kc, const float* k_scale,
                                             const uint8_t* vc, const float* v_scale,
                                             const float* delta_s, int64_t ds_rows,
                                             const float* mu_v, int64_t nq, int64_t nkv, int d,
                                             float sm_scale, int causal, int bkv, int blk,
                                             int64_t split, const int64_t* rows, int64_t nrows,
                                             float* out, float* lse, float* tie) {
    float* vdec = (float*)malloc(sizeof(float) * (size_t)(nkv > 0 ? nkv : 1) * (size_t)d);
    float* fac = (float*)malloc(sizeof(float) * (size_t)d);
    for (int64_t j = 0; j < nkv * d; ++j) vdec[j] = orc_e4m3_decode(vc[j]);
    for (int c = 0; c < d; ++c) fac[c] = v_scale[c] / 448.0f;
    recipe_rows(qc, q_scale, kc, k_scale, vdec, fac, P_FP8, delta_s, ds_rows, mu_v, nq, nkv, d,
                sm_scale, causal, bkv, blk, split, rows, nrows, out, lse, tie);
    free(vdec);
    free(fac);
}

/* The INT8-QK / 16-bit-PV recipe of the first SageAttention (package page
 * "What it is and what it does": FP16 accumulators; the install guide's
 * benchmark section names the qk_int8_pv_fp16 kernel):
 *   vh   : V operand [nkv][d] as fp16 (bf16 = 0) or bf16 (bf16 = 1) bit
 *          patterns (the input V, or v - mu_v rounded to that type);
 *   p^ = p rounded to the same 16-bit type (no scale: p <= 1), and no end
 *   factor. */
ORC_EXPORT void orc_attn_recipe_half_rows(const int8_t* qc, const float* q_scale,
                                          const int8_t* kc, const float* k_scale,
                                          const uint16_t* vh, int bf16,
                                          const float* delta_s, const float* mu_v,
                                          int64_t nq, int64_t nkv, int d, float sm_scale,
                                          int causal, int bkv, int blk, int64_t split,
                                          const int64_t* rows, int64_t nrows,
                                          float* out, float* lse, float* tie) {
    float* vdec = (float*)malloc(sizeof(float) * (size_t)(nkv > 0 ? nkv : 1) * (size_t)d);
    for (int64_t j = 0; j < nkv * d; ++j)
        vdec[j] = bf16 ? orc_bf16_decode(vh[j]) : orc_f16_decode(vh[j]);
    recipe_rows(qc, q_scale, kc, k_scale, vdec, NULL, bf16 ? P_BF16 : P_F16, delta_s, 0, mu_v, nq,
                nkv, d, sm_scale, causal, bkv, blk, split, rows, nrows, out, lse, tie);
    free(vdec);
}

/* Exact softmax attention in FP64 ([SA1]: the quantity the method
 * approximates).  q [nq][d], k [nkv][d], v [nkv][d] are the exactly decoded
 * inputs; t_ij = sm_scale * q_i.k_j over visible j; o_i = sum_j w_ij v_j with
 * w the softmax of t over visible j.  Rows with no visible key give 0.
 * out [nrows][d] FP64; lse [nrows] FP64 natural-log (or NULL).             */
ORC_EXPORT void orc_attn_exact_rows(const float* q, const float* k, const float* v,
                                    int64_t nq, int64_t nkv, int d, double sm_scale,
                                    int causal, const int64_t* rows, int64_t nrows,
                                    double* out, double* lse) {
    double* t = (double*)malloc(sizeof(double) * (size_t)(nkv > 0 ? nkv : 1));
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        int64_t jmax = last_visible(i, nq, nkv, causal);
        double* o = out + r * d;
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        if (jmax < 0) { if (lse) lse[r] = -INFINITY; continue; }
        double mx = -INFINITY;
        for (int64_t j = 0; j <= jmax; ++j) {
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += (double)q[i * d + c] * (double)k[j * d + c];
            t[j] = sm_scale * dot;
            if (t[j] > mx) mx = t[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j <= jmax; ++j) { t[j] = exp(t[j] - mx); den += t[j]; }
        for (int64_t j = 0; j <= jmax; ++j) {
            double w = t[j] / den;
            for (int c = 0; c < d; ++c) o[c] += w * (double)v[j * d + c];
        }
        if (lse) lse[r] = mx + log(den);
    }
    free(t);
}
