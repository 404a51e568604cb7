/*
 * kvarn_oracle.c -- plain, slow CPU reference of the KVarN quantize and
 * decode-attention path, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP implementation, and the product
 * path never calls it.
 *
 * Sources (cited by page and section):
 *  [R] evermx.com review "KVarN vLLM KV-cache quantization", second paragraph:
 *      per fixed-size KV tile, four stages -- raw fp16 tile, Hadamard rotation
 *      across channels (orthonormal, scores preserved), iterative variance
 *      normalization (per-channel and per-token spreads equalized in turn,
 *      Sinkhorn style, on log-scales), then asymmetric
 *      round-to-nearest with the scales folded back in at read time;
 *      preset kvarn_k4v2_g128 = 4-bit keys, 2-bit values, 128-token tiles;
 *      fourth paragraph: MLA latent quantized to int4.
 *  [G] gmlx documentation "KV cache quantization", section "The two schemes":
 *      each head rotated with a Hadamard transform; records of 128 tokens
 *      whose token and channel spreads are evened out; first 128 tokens and the
 *      newest --kv-tail-tokens tokens (default 1024) stay fp16; widths
 *      2,3,4,5,6,8.  Section "Which layers quantize": head dims 128/256/512.
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function that implements it.  Readings in brief:
 *   - Hadamard = natural-order Sylvester matrix scaled by 1/sqrt(D), no sign
 *     randomisation; rotation acts on each token row: Y = X . H.
 *   - "standard deviation" = root mean square about zero, population (/N);
 *     one iteration = column step then row step; log-scales start at 0.
 *   - per-token asymmetric RTN: scale s = (max-min)/(2^b-1), zero-point = min
 *     (a float offset); round half to even; clamp to [0, 2^b-1].
 *   - stored values: per-token fp16 scale and zero-point, per-channel fp16
 *     column scale; codes bit-packed LSB-first.
 *
 * Record format (one quantized page x one KV head x K or V), little-endian:
 *   bytes [0, T*D*b/8)           codes, element e in bits [e*b, e*b+b) of the
 *                                byte stream, LSB first.  Token-major order
 *                                (e = t*D + j) or channel-major (e = j*T + t).
 *   then 4*T bytes               per token t: scale S_t (fp16), zero Zp_t (fp16)
 *   then 2*D bytes               per channel j: column scale C_j (fp16)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 / bfloat16 conversions, written from the format        */
/* definitions (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits;  */
/* bfloat16 = upper 16 bits of binary32).                                    */
/* ------------------------------------------------------------------------ */

double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return sign ? -v : v;
}

/* Round-to-nearest-even conversion of a double to binary16.  Values at or
 * beyond the overflow threshold (65520) become infinity. */
uint16_t orc_double_to_half(double x)
{
    uint16_t sign = 0;
    if (isnan(x))
        return 0x7e00;
    if (signbit(x)) {
        sign = 0x8000;
        x = -x;
    }
    if (x == 0.0)
        return sign;
    if (x >= 65520.0)
        return sign | 0x7c00;
    int e;
    frexp(x, &e);               /* x = m * 2^e, m in [0.5, 1) */
    int ue = e - 1;             /* x = 1.f * 2^ue */
    double q;                   /* quantum of the target format at x */
    if (ue < -14)
        q = ldexp(1.0, -24);    /* subnormal range */
    else
        q = ldexp(1.0, ue - 10);
    double n = nearbyint(x / q);  /* RNE on the integer multiple of q */
    double r = n * q;
    /* re-encode r (which may have rounded up to the next binade) */
    if (r >= 65520.0)
        return sign | 0x7c00;
    if (r < ldexp(1.0, -14)) {
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    }
    frexp(r, &e);
    ue = e - 1;
    uint16_t frac = (uint16_t)((r / ldexp(1.0, ue) - 1.0) * 1024.0);
    return sign | (uint16_t)((ue + 15) << 10) | frac;
}

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static int popcount_int(unsigned v)
{
    int c = 0;
    while (v) {
        c += v & 1u;
        v >>= 1;
    }
    return c;
}

/* ------------------------------------------------------------------------ */
/* Stage 2: Hadamard rotation across channels [R ¶2; G "The two schemes"].  */
/* Reading: the natural-order Sylvester matrix, entry (k, j) equal to       */
/* (-1)^popcount(k & j) / sqrt(D); it is symmetric and orthonormal.         */
/* ------------------------------------------------------------------------ */

void orc_hadamard_matrix(int D, double *H)
{
    double s = 1.0 / sqrt((double)D);
    for (int k = 0; k < D; k++)
        for (int j = 0; j < D; j++)
            H[(int64_t)k * D + j] = (popcount_int((unsigned)(k & j)) & 1) ? -s : s;
}

/* Y = X . H applied to every token row of a T x D tile: the +-1 signs of
 * the Sylvester matrix are summed first and the sum is divided by sqrt(D)
 * once.  For fp16 inputs every partial sum is exact in fp64 (an fp16 value
 * is an integer multiple of 2^-24 below 2^16, and D <= 2^9 of them need at
 * most 49 bits), so Y is the exact rotation rounded once; in particular a
 * channel that the rotation cancels comes out exactly zero. */
void orc_rotate(int T, int D, const double *X, double *Y)
{
    const double rt = sqrt((double)D);
    double *S = (double *)malloc(sizeof(double) * (size_t)D * D);  /* +-1 signs, symmetric */
    for (int k = 0; k < D; k++)
        for (int j = 0; j < D; j++)
            S[(int64_t)k * D + j] = (popcount_int((unsigned)(k & j)) & 1) ? -1.0 : 1.0;
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < D; j++) {
            double acc = 0.0;
            for (int k = 0; k < D; k++)
                acc += X[(int64_t)t * D + k] * S[(int64_t)j * D + k];
            Y[(int64_t)t * D + j] = acc / rt;
        }
    }
    free(S);
}

/* ------------------------------------------------------------------------ */
/* Stage 3: iterative variance normalization [R ¶2; G "The two schemes"].   */
/* Channel spreads and token spreads are divided out in turn, the scales    */
/* kept as logarithms, as in Sinkhorn's matrix balancing.  Readings:        */
/*   - log-scales lr (per token row) and lc (per channel column) start at 0; */
/*   - the normalized tile is Z_ij = Y_ij * exp(-lr_i - lc_j);              */
/*   - one iteration = a column step (lc_j += ln sigma of column j of Z)    */
/*     followed by a row step (lr_i += ln sigma of row i of Z, with the     */
/*     updated lc);                                                         */
/*   - sigma_mode 0: sigma = sqrt(mean of squares) (about zero, /N);        */
/*     sigma_mode 1: centred population standard deviation (kept only to    */
/*     show why the first reading is taken: it does not converge);          */
/*   - a sigma that is zero or not finite leaves that log-scale unchanged;  */
/*   - final_row_step = 0 stops after the last column step (used to show    */
/*     that the last row step cannot change a stored value).                */
/* ------------------------------------------------------------------------ */

static double sigma_of(const double *v, int n, int stride, int mode)
{
    double s1 = 0.0, s2 = 0.0;
    for (int i = 0; i < n; i++) {
        double x = v[(int64_t)i * stride];
        s1 += x;
        s2 += x * x;
    }
    if (mode == 0)
        return sqrt(s2 / n);
    double mean = s1 / n;
    double var = 0.0;
    for (int i = 0; i < n; i++) {
        double d = v[(int64_t)i * stride] - mean;
        var += d * d;
    }
    return sqrt(var / n);
}

void orc_normalize(int T, int D, const double *Y, int n_iters, int final_row_step,
                   int sigma_mode, double *lr, double *lc)
{
    double *Z = (double *)malloc(sizeof(double) * (size_t)T * D);
    for (int i = 0; i < T; i++)
        lr[i] = 0.0;
    for (int j = 0; j < D; j++)
        lc[j] = 0.0;
    for (int it = 0; it < n_iters; it++) {
        /* column step */
        for (int i = 0; i < T; i++)
            for (int j = 0; j < D; j++)
                Z[(int64_t)i * D + j] = Y[(int64_t)i * D + j] * exp(-lr[i] - lc[j]);
        for (int j = 0; j < D; j++) {
            double sg = sigma_of(Z + j, T, D, sigma_mode);
            if (sg > 0.0 && isfinite(sg))
                lc[j] += log(sg);
        }
        if (it == n_iters - 1 && !final_row_step)
            break;
        /* row step, using the updated column log-scales */
        for (int i = 0; i < T; i++)
            for (int j = 0; j < D; j++)
                Z[(int64_t)i * D + j] = Y[(int64_t)i * D + j] * exp(-lr[i] - lc[j]);
        for (int i = 0; i < T; i++) {
            double sg = sigma_of(Z + (int64_t)i * D, D, 1, sigma_mode);
            if (sg > 0.0 && isfinite(sg))
                lr[i] += log(sg);
        }
    }
    free(Z);
}

/* ------------------------------------------------------------------------ */
/* Stage 4: asymmetric round-to-nearest [R ¶2].  Per token row of the tile  */
/* divided by its column scales, W_ij = Y_ij / exp(lc_j):                    */
/*   mn_i = min_j W_ij, s_i = (max_j W_ij - mn_i) / (2^b - 1),              */
/*   u_ij = (W_ij - mn_i) / s_i  (0 when s_i = 0),                          */
/*   q_ij = clamp(round-half-even(u_ij), 0, 2^b - 1).                       */
/* The row log-scale lr_i multiplies both the row range and the row         */
/* minimum, so it cancels from q, s and mn; the stored per-token scale and  */
/* zero-point are therefore s_i and mn_i of W.                              */
/* ------------------------------------------------------------------------ */

void orc_rtn(int T, int D, const double *Y, const double *lc, int bits,
             uint8_t *codes, double *s_out, double *mn_out, double *u_out)
{
    int qmax = (1 << bits) - 1;
    double *W = (double *)malloc(sizeof(double) * (size_t)D);
    for (int i = 0; i < T; i++) {
        for (int j = 0; j < D; j++)
            W[j] = Y[(int64_t)i * D + j] / exp(lc[j]);
        double mn = W[0], mx = W[0];
        for (int j = 1; j < D; j++) {
            if (W[j] < mn) mn = W[j];
            if (W[j] > mx) mx = W[j];
        }
        double s = (mx - mn) / qmax;
        for (int j = 0; j < D; j++) {
            double u = s > 0.0 ? (W[j] - mn) / s : 0.0;
            double r = nearbyint(u);
            if (r < 0.0) r = 0.0;
            if (r > qmax) r = qmax;
            codes[(int64_t)i * D + j] = (uint8_t)r;
            if (u_out)
                u_out[(int64_t)i * D + j] = u;
        }
        s_out[i] = s;
        mn_out[i] = mn;
    }
    free(W);
}

/* ------------------------------------------------------------------------ */
/* Bit packing: element e occupies bits [e*b, e*b + b) of the byte stream,  */
/* least significant bit first.  Written one bit at a time.                 */
/* ------------------------------------------------------------------------ */

void orc_pack(const uint8_t *vals, int64_t n, int bits, uint8_t *out)
{
    memset(out, 0, (size_t)((n * bits + 7) / 8));
    for (int64_t e = 0; e < n; e++)
        for (int k = 0; k < bits; k++) {
            int64_t pos = e * bits + k;
            if ((vals[e] >> k) & 1)
                out[pos / 8] |= (uint8_t)(1u << (pos % 8));
        }
}

void orc_unpack(const uint8_t *in, int64_t n, int bits, uint8_t *vals)
{
    for (int64_t e = 0; e < n; e++) {
        unsigned v = 0;
        for (int k = 0; k < bits; k++) {
            int64_t pos = e * bits + k;
            v |= (unsigned)((in[pos / 8] >> (pos % 8)) & 1) << k;
        }
        vals[e] = (uint8_t)v;
    }
}

int64_t orc_record_bytes(int T, int D, int bits)
{
    return (int64_t)T * D * bits / 8 + 4 * (int64_t)T + 2 * (int64_t)D;
}

static void put_u16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}

static uint16_t get_u16(const uint8_t *p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* Position of the code of token t, channel j in a record's code stream.
 * Token-major: e = t D + j.  Channel-major: tokens in blocks of TB =
 * min(T, 64); block by block, each channel's TB codes in a row:
 * e = (t / TB) TB D + j TB + t % TB (for T <= 64 simply j T + t).  The pages
 * leave the order open; this one makes the codes of one 64-token block a
 * contiguous run. */
static int64_t code_pos(int T, int D, int t, int j, int channel_major)
{
    if (!channel_major)
        return (int64_t)t * D + j;
    int TB = T < 64 ? T : 64;
    return (int64_t)(t / TB) * TB * D + (int64_t)j * TB + t % TB;
}

/* ------------------------------------------------------------------------ */
/* One record: fp16 tile -> stages 2..4 -> packed bytes.                    */
/* Outputs (optional, may be NULL): u (T*D), lc (D), lr (T) for the checks. */
/* ------------------------------------------------------------------------ */

int orc_quantize_record(const uint16_t *x16, int T, int D, int bits, int n_iters,
                        int channel_major, uint8_t *record, double *u_out,
                        double *lc_out, double *lr_out)
{
    size_t nel = (size_t)T * D;
    double *X = (double *)malloc(sizeof(double) * nel);
    double *Y = (double *)malloc(sizeof(double) * nel);
    double *lr = (double *)malloc(sizeof(double) * T);
    double *lc = (double *)malloc(sizeof(double) * D);
    double *s = (double *)malloc(sizeof(double) * T);
    double *mn = (double *)malloc(sizeof(double) * T);
    uint8_t *q = (uint8_t *)malloc(nel);
    uint8_t *qo = (uint8_t *)malloc(nel);

    for (size_t e = 0; e < nel; e++)            /* stage 1: raw fp16 tile */
        X[e] = orc_half_to_double(x16[e]);
    orc_rotate(T, D, X, Y);                     /* stage 2 */
    orc_normalize(T, D, Y, n_iters, 1, 0, lr, lc);   /* stage 3 */
    orc_rtn(T, D, Y, lc, bits, q, s, mn, u_out); /* stage 4 */

    for (int t = 0; t < T; t++)
        for (int j = 0; j < D; j++) {
            qo[code_pos(T, D, t, j, channel_major)] = q[(int64_t)t * D + j];
        }
    int64_t cbytes = (int64_t)T * D * bits / 8;
    orc_pack(qo, (int64_t)nel, bits, record);
    for (int t = 0; t < T; t++) {
        put_u16(record + cbytes + 4 * t, orc_double_to_half(s[t]));
        put_u16(record + cbytes + 4 * t + 2, orc_double_to_half(mn[t]));
    }
    for (int j = 0; j < D; j++)
        put_u16(record + cbytes + 4 * T + 2 * j, orc_double_to_half(exp(lc[j])));
    if (lc_out)
        memcpy(lc_out, lc, sizeof(double) * D);
    if (lr_out)
        memcpy(lr_out, lr, sizeof(double) * T);

    free(X); free(Y); free(lr); free(lc); free(s); free(mn); free(q); free(qo);
    return 0;
}

/* Read back a record into the original (unrotated) basis, reading the
 * stored fp16 values: Yhat_tj = C_j * (S_t * q_tj + Zp_t), Xhat = Yhat . H
 * (H is symmetric and its own inverse). */
void orc_dequantize_record(const uint8_t *record, int T, int D, int bits,
                           int channel_major, double *Xhat)
{
    size_t nel = (size_t)T * D;
    uint8_t *qo = (uint8_t *)malloc(nel);
    double *Yh = (double *)malloc(sizeof(double) * nel);
    int64_t cbytes = (int64_t)T * D * bits / 8;
    orc_unpack(record, (int64_t)nel, bits, qo);
    for (int t = 0; t < T; t++) {
        double S = orc_half_to_double(get_u16(record + cbytes + 4 * t));
        double Z = orc_half_to_double(get_u16(record + cbytes + 4 * t + 2));
        for (int j = 0; j < D; j++) {
            double C = orc_half_to_double(get_u16(record + cbytes + 4 * T + 2 * j));
            Yh[(int64_t)t * D + j] = C * (S * qo[code_pos(T, D, t, j, channel_major)] + Z);
        }
    }
    orc_rotate(T, D, Yh, Xhat);
    free(qo);
    free(Yh);
}

/* ------------------------------------------------------------------------ */
/* Paged cache.  cfg[] = {T, D, k_bits, v_bits, n_iters, sink, tail, H, mla} */
/* fp16 pool: [n_fpages][H][T][D]; record pools: [n_qpages][H][bytes].      */
/* Keys are stored token-major, values channel-major; an MLA latent has     */
/* one token-major record per token that serves as both key and value.     */
/* ------------------------------------------------------------------------ */

enum { C_T, C_D, C_KB, C_VB, C_IT, C_SINK, C_TAIL, C_H, C_MLA, C_N };

/* Quantize page pairs (src fp16 page -> dst record page), all heads, K
 * and V.  Independent records are spread over threads. */
int orc_quantize_pages(const int32_t *cfg, const uint16_t *k16, const uint16_t *v16,
                       const int32_t *src, const int32_t *dst, int n,
                       uint8_t *krec, uint8_t *vrec, int n_threads)
{
    int T = cfg[C_T], D = cfg[C_D], H = cfg[C_H], mla = cfg[C_MLA];
    int nkinds = mla ? 1 : 2;
    int64_t kb = orc_record_bytes(T, D, cfg[C_KB]);
    int64_t vb = orc_record_bytes(T, D, cfg[C_VB]);
    int64_t total = (int64_t)n * H * nkinds;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t w = 0; w < total; w++) {
        int kind = (int)(w % nkinds);
        int h = (int)((w / nkinds) % H);
        int i = (int)(w / nkinds / H);
        const uint16_t *tile = (kind == 0 ? k16 : v16) +
                               ((int64_t)src[i] * H + h) * T * D;
        if (kind == 0)
            orc_quantize_record(tile, T, D, cfg[C_KB], cfg[C_IT], 0,
                                krec + ((int64_t)dst[i] * H + h) * kb, NULL, NULL, NULL);
        else
            orc_quantize_record(tile, T, D, cfg[C_VB], cfg[C_IT], 1,
                                vrec + ((int64_t)dst[i] * H + h) * vb, NULL, NULL, NULL);
    }
    return 0;
}

/* Number of quantized records of a sequence of L tokens: whole T-token
 * records starting after the fp16 sink, leaving at least `tail` newest
 * tokens in fp16 [G "The two schemes"]. */
int orc_quantized_pages(const int32_t *cfg, int L)
{
    int T = cfg[C_T], sink = cfg[C_SINK], tail = cfg[C_TAIL];
    if (L - sink - tail < T)
        return 0;
    return (L - sink - tail) / T;
}

/* ------------------------------------------------------------------------ */
/* Decode attention, by its plain definition: for each requested (batch b,  */
/* query head h) with KV head g = h / (Hq / H), read back every token       */
/* t < L of the sequence -- dequantized record values (rotated back to the  */
/* original basis) in the quantized region, the stored fp16 values in the   */
/* sink and tail -- then out = sum_t softmax_t(sm_scale * <q, k_t>) v_t,    */
/* with a max-subtracted softmax in double precision.                       */
/* q: [batch][Hq][D], float32 (q_is_bf16 = 0) or bfloat16 (1), raw bits.    */
/* pairs: n_pairs (b, h) pairs; out: [n_pairs][D].                          */
/* ------------------------------------------------------------------------ */

/* Read back every token t < La of sequence b, KV head g: dequantized record
 * values (rotated back to the original basis) for pages in the quantized
 * region of a sequence of Lr tokens, the stored fp16 values elsewhere (sink,
 * tail, and tokens past Lr).  Kh, Vh: at least ceil(La / T) * T * D doubles
 * each. */
static void read_back(const int32_t *cfg, const uint8_t *krec, const uint8_t *vrec,
                      const uint16_t *k16, const uint16_t *v16,
                      const int32_t *block_table, int max_pages, int b, int g, int Lr, int La,
                      double *Kh, double *Vh)
{
    int T = cfg[C_T], D = cfg[C_D], H = cfg[C_H], mla = cfg[C_MLA];
    int sink_pages = cfg[C_SINK] / T;
    int64_t kb = orc_record_bytes(T, D, cfg[C_KB]);
    int64_t vb = orc_record_bytes(T, D, cfg[C_VB]);
    int nq = orc_quantized_pages(cfg, Lr);
    int npages = (La + T - 1) / T;
    for (int p = 0; p < npages; p++) {
        int id = block_table[(int64_t)b * max_pages + p];
        int quant = (p >= sink_pages) && (p < sink_pages + nq);
        double *kd = Kh + (int64_t)p * T * D, *vd = Vh + (int64_t)p * T * D;
        if (quant) {
            orc_dequantize_record(krec + ((int64_t)id * H + g) * kb, T, D, cfg[C_KB], 0, kd);
            if (mla)
                memcpy(vd, kd, sizeof(double) * (size_t)T * D);
            else
                orc_dequantize_record(vrec + ((int64_t)id * H + g) * vb, T, D, cfg[C_VB], 1, vd);
        } else {
            const uint16_t *ks = k16 + ((int64_t)id * H + g) * T * D;
            const uint16_t *vs = (mla ? k16 : v16) + ((int64_t)id * H + g) * T * D;
            for (int64_t e = 0; e < (int64_t)T * D; e++) {
                kd[e] = orc_half_to_double(ks[e]);
                vd[e] = orc_half_to_double(vs[e]);
            }
        }
    }
}

/* The query vector of (b, h), widened exactly to double. */
static void load_query(const void *q, int q_is_bf16, int Hq, int D, int b, int h, double *qv)
{
    for (int j = 0; j < D; j++) {
        int64_t idx = ((int64_t)b * Hq + h) * D + j;
        if (q_is_bf16)
            qv[j] = orc_bf16_to_double(((const uint16_t *)q)[idx]);
        else
            qv[j] = (double)((const float *)q)[idx];
    }
}

/* out = sum_{t < L} softmax_t(sm_scale * <q, k_t>) v_t, max-subtracted
 * softmax in double precision; zeros when L = 0. */
static void attend(const double *qv, const double *Kh, const double *Vh, int L, int D,
                   double sm_scale, double *out)
{
    double *sc = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double m = -INFINITY;
    for (int t = 0; t < L; t++) {
        double acc = 0.0;
        for (int j = 0; j < D; j++)
            acc += qv[j] * Kh[(int64_t)t * D + j];
        sc[t] = sm_scale * acc;
        if (sc[t] > m)
            m = sc[t];
    }
    double l = 0.0;
    for (int t = 0; t < L; t++) {
        sc[t] = exp(sc[t] - m);
        l += sc[t];
    }
    for (int j = 0; j < D; j++) {
        double acc = 0.0;
        for (int t = 0; t < L; t++)
            acc += sc[t] * Vh[(int64_t)t * D + j];
        out[j] = L > 0 ? acc / l : 0.0;
    }
    free(sc);
}

int orc_decode(const int32_t *cfg, const uint8_t *krec, const uint8_t *vrec,
               const uint16_t *k16, const uint16_t *v16,
               const int32_t *block_table, const int32_t *seq_lens, int max_pages,
               const void *q, int q_is_bf16, int Hq, double sm_scale,
               const int32_t *pairs, int n_pairs, double *out, int n_threads)
{
    int T = cfg[C_T], D = cfg[C_D], H = cfg[C_H];
    int G = Hq / H;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int pi = 0; pi < n_pairs; pi++) {
        int b = pairs[2 * pi], h = pairs[2 * pi + 1];
        int L = seq_lens[b];
        int npages = (L + T - 1) / T;
        double *qv = (double *)malloc(sizeof(double) * D);
        double *Kh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        double *Vh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        load_query(q, q_is_bf16, Hq, D, b, h, qv);
        read_back(cfg, krec, vrec, k16, v16, block_table, max_pages, b, h / G, L, L, Kh, Vh);
        attend(qv, Kh, Vh, L, D, sm_scale, out + (int64_t)pi * D);
        free(qv); free(Kh); free(Vh);
    }
    return 0;
}

/* The same definition for whole query-head groups: for each requested
 * (b, g) the tokens of KV head g are read back once and attended by each of
 * its G = Hq / H query heads h = g G .. g G + G - 1.
 * groups: n_groups (b, g) pairs; out: [n_groups][G][D]. */
int orc_decode_groups(const int32_t *cfg, const uint8_t *krec, const uint8_t *vrec,
                      const uint16_t *k16, const uint16_t *v16,
                      const int32_t *block_table, const int32_t *seq_lens, int max_pages,
                      const void *q, int q_is_bf16, int Hq, double sm_scale,
                      const int32_t *groups, int n_groups, double *out, int n_threads)
{
    int T = cfg[C_T], D = cfg[C_D], H = cfg[C_H];
    int G = Hq / H;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int gi = 0; gi < n_groups; gi++) {
        int b = groups[2 * gi], g = groups[2 * gi + 1];
        int L = seq_lens[b];
        int npages = (L + T - 1) / T;
        double *qv = (double *)malloc(sizeof(double) * D);
        double *Kh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        double *Vh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        read_back(cfg, krec, vrec, k16, v16, block_table, max_pages, b, g, L, L, Kh, Vh);
        for (int k = 0; k < G; k++) {
            load_query(q, q_is_bf16, Hq, D, b, g * G + k, qv);
            attend(qv, Kh, Vh, L, D, sm_scale, out + ((int64_t)gi * G + k) * D);
        }
        free(qv); free(Kh); free(Vh);
    }
    return 0;
}

/* Verify-step decode, by its plain definition: M query tokens per sequence,
 * token i of sequence b at position L_b + i (L_b = seq_lens[b], the
 * committed tokens; the M tokens are appended after them), causal among
 * themselves [G "Speed and speculative decoding"]:
 *   out(b, i, h) = sum_{t <= L_b + i} softmax_t(sm_scale * <q(b, i, h), k_t>) v_t,
 * the tokens read back as in orc_decode with the quantized region of a
 * sequence of L_b tokens (tokens from L_b on are fp16).
 * q: [batch][M][Hq][D]; rows: n (b, i, h) triples; out: [n][D]. */
int orc_decode_mq(const int32_t *cfg, const uint8_t *krec, const uint8_t *vrec,
                  const uint16_t *k16, const uint16_t *v16,
                  const int32_t *block_table, const int32_t *seq_lens, int max_pages,
                  const void *q, int q_is_bf16, int M, int Hq, double sm_scale,
                  const int32_t *rows, int n_rows, double *out, int n_threads)
{
    int T = cfg[C_T], D = cfg[C_D], H = cfg[C_H];
    int G = Hq / H;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int ri = 0; ri < n_rows; ri++) {
        int b = rows[3 * ri], i = rows[3 * ri + 1], h = rows[3 * ri + 2];
        int Lr = seq_lens[b];
        int La = Lr + i + 1;
        if (La > max_pages * T)
            La = max_pages * T;
        int npages = (La + T - 1) / T;
        double *qv = (double *)malloc(sizeof(double) * D);
        double *Kh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        double *Vh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        load_query(q, q_is_bf16, Hq, D, b * M + i, h, qv);
        read_back(cfg, krec, vrec, k16, v16, block_table, max_pages, b, h / G, Lr, La, Kh, Vh);
        attend(qv, Kh, Vh, La, D, sm_scale, out + (int64_t)ri * D);
        free(qv); free(Kh); free(Vh);
    }
    return 0;
}

/* MLA with a rope sidecar.  An MLA model's key has two parts: the
 * compressed latent, which this method quantizes to int4 [R ¶4] and which
 * is also the value, and a small rotary-position key beside it (64 wide in
 * DeepSeek-style MLA), which stays fp16 (a reading of the 2.77x capacity
 * figure of [R ¶4]: the rope key kept 16-bit is consistent with it).  Plain definition, per requested row (b, i, h):
 *   key t = (x_t, r_t), value t = x_t, query = (q_lat[D], q_rope[R]),
 *   score_t = sm_scale * (<q_lat, x_t> + <q_rope, r_t>),
 *   out = sum_t softmax_t(score_t) x_t,
 * with x_t read back as in orc_decode (quantized region of the seq_lens[b]
 * committed tokens) and r_t, fp16, from the rope pool paired with the
 * region of t's page: rope_q [n_qpages][T][R] (indexed like the record
 * pool) for quantized pages, rope_f [n_fpages][T][R] for fp16 pages.
 * causal = 0: M = 1 and every row attends the seq_lens tokens (a decode
 * step); causal = 1: token i at position seq_lens[b] + i attends the tokens
 * up to and including itself (a verify step, as orc_decode_mq).
 * q: [batch][M][Hq][D + R]; rows: n (b, i, h) triples; out: [n][D]. */
int orc_decode_rope(const int32_t *cfg, const uint8_t *krec, const uint16_t *k16,
                    const uint16_t *rope_q, const uint16_t *rope_f, int R,
                    const int32_t *block_table, const int32_t *seq_lens, int max_pages,
                    const void *q, int q_is_bf16, int M, int causal, int Hq, double sm_scale,
                    const int32_t *rows, int n_rows, double *out, int n_threads)
{
    int T = cfg[C_T], D = cfg[C_D];
    int W = D + R;
    int sink_pages = cfg[C_SINK] / T;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int ri = 0; ri < n_rows; ri++) {
        int b = rows[3 * ri], i = rows[3 * ri + 1], h = rows[3 * ri + 2];
        int Lr = seq_lens[b];
        int La = causal ? Lr + i + 1 : Lr;
        if (La > max_pages * T)
            La = max_pages * T;
        int npages = (La + T - 1) / T;
        int nq = orc_quantized_pages(cfg, Lr);
        double *qv = (double *)malloc(sizeof(double) * W);
        double *Kh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        double *Vh = (double *)malloc(sizeof(double) * (size_t)npages * T * D + 8);
        double *sc = (double *)malloc(sizeof(double) * (size_t)(La > 0 ? La : 1));
        load_query(q, q_is_bf16, Hq, W, b * M + i, h, qv);
        read_back(cfg, krec, NULL, k16, NULL, block_table, max_pages, b, 0, Lr, La, Kh, Vh);
        double m = -INFINITY;
        for (int t = 0; t < La; t++) {
            int p = t / T;
            int id = block_table[(int64_t)b * max_pages + p];
            int quant = (p >= sink_pages) && (p < sink_pages + nq);
            const uint16_t *rt = (quant ? rope_q : rope_f) + ((int64_t)id * T + t % T) * R;
            double acc = 0.0;
            for (int j = 0; j < D; j++)
                acc += qv[j] * Kh[(int64_t)t * D + j];
            for (int r = 0; r < R; r++)
                acc += qv[D + r] * orc_half_to_double(rt[r]);
            sc[t] = sm_scale * acc;
            if (sc[t] > m)
                m = sc[t];
        }
        double l = 0.0;
        for (int t = 0; t < La; t++) {
            sc[t] = exp(sc[t] - m);
            l += sc[t];
        }
        for (int j = 0; j < D; j++) {
            double acc = 0.0;
            for (int t = 0; t < La; t++)
                acc += sc[t] * Vh[(int64_t)t * D + j];
            out[(int64_t)ri * D + j] = La > 0 ? acc / l : 0.0;
        }
        free(qv); free(Kh); free(Vh); free(sc);
    }
    return 0;
}
