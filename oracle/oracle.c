/*
 * CPU oracle for the IndexCache sparse-attention path -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, obviously correct C. Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg load this library; the product path never
 * does. It shares no code, header or table with the HIP library.
 *
 * What it computes (every step is the plain definition, in fp64):
 *   O0  decoders for OCP fp8 e4m3fn and bf16 bytes;
 *   O1  lightning-indexer scores     I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[base_t+s,:])
 *       ("Hy4 IndexCache cross-layer index reuse", Jargon: "Indexer", "DSA");
 *   O2  top-k selection: the k' = min(k, n_t) positions with the largest
 *       score, lower position first among equal scores ("Jargon: Top-k
 *       selection"); a full sort is the library step;
 *   O3  sparse MLA with a per-head softmax sink over the selected latent rows
 *       (GitHub issue "rtx6kpro #90", bullets on the learnable per-head sink
 *       and on the 576-wide MLA row: 512 latent + 64 RoPE), two-pass softmax.
 * The layer-stack rule (O4: shared layers reuse the index of the last
 * preceding full layer, issue #90 "Indexer:" bullet) lives in __init__.py.
 *   O5  the gated head output that follows the attention (issue #90, bullet on
 *       the elementwise sigmoid gate): each head's latent output is first
 *       decompressed by its value up-projection wv_b, then multiplied
 *       elementwise by sigmoid of the gate pre-activation, before o_proj.
 *   O6  the cache write that precedes the path: the new token's indexer key
 *       (LayerNorm with bias, interleaved RoPE on its trailing span, fp8
 *       cast) and its latent row (latent as given, interleaved RoPE on the
 *       trailing 64 entries).
 *
 * Readings where the pages are silent are listed with each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- O0 ---- */

/* OCP 8-bit float E4M3 ("fn" variant): 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits. Exponent field 0 encodes subnormals m/8 * 2^-6. The
 * all-ones exponent with all-ones mantissa (0x7F, 0xFF) is NaN; there is no
 * infinity, so exponent 15 with mantissa 0..6 is an ordinary normal number. */
double orc_fp8_e4m3fn_to_double(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int m = b & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* bf16 is the upper half of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

void orc_decode_fp8(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_fp8_e4m3fn_to_double(src[i]);
}

void orc_decode_bf16(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_bf16_to_double(src[i]);
}

/* ---------------------------------------------------------------- O1 ---- */

/* Indexer scores for T queries.
 *   q_idx [T, H_I, D_I] fp8, w [T, H_I] fp32, k_idx [rows, D_I] fp8
 *   query t sees cache rows base[t] .. base[t] + n[t] - 1 (position s is
 *   sequence-local), out [T, ld] fp64, entries s >= n[t] are left untouched.
 * Reading: one key vector per cached token, shared by all indexer heads, and a
 * non-negative weight per (query, head); no further scale factors. */
void orc_indexer_scores(int32_t T, int32_t H_I, int32_t D_I,
                        const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                        const int64_t *base, const int32_t *n, double *out, int64_t ld)
{
    for (int32_t t = 0; t < T; ++t) {
        double *qd = (double *)malloc(sizeof(double) * (size_t)H_I * D_I);
        orc_decode_fp8(q_idx + (int64_t)t * H_I * D_I, qd, (int64_t)H_I * D_I);
        int32_t nt = n[t];
#pragma omp parallel for schedule(static)
        for (int32_t s = 0; s < nt; ++s) {
            double kd[1024];
            const uint8_t *krow = k_idx + (base[t] + s) * (int64_t)D_I;
            for (int32_t d = 0; d < D_I; ++d)
                kd[d] = orc_fp8_e4m3fn_to_double(krow[d]);
            double I = 0.0;
            for (int32_t h = 0; h < H_I; ++h) {
                double dot = 0.0;
                for (int32_t d = 0; d < D_I; ++d)
                    dot += qd[(int64_t)h * D_I + d] * kd[d];
                if (dot > 0.0)
                    I += (double)w[(int64_t)t * H_I + h] * dot;
            }
            out[(int64_t)t * ld + s] = I;
        }
        free(qd);
    }
}

/* ---------------------------------------------------------------- O2 ---- */

typedef struct {
    float score;
    int32_t pos;
} orc_cand;

/* larger score first; among equal scores the lower position first */
static int orc_cmp_rank(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *b = (const orc_cand *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

static int orc_cmp_i32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Top-k over fp32 scores [T, ld]; query t considers positions 0 .. n[t]-1.
 * idx [T, k]: the selected positions in ascending order, then -1 padding.
 * When n[t] <= k every position is kept. Scores are compared as fp32 values,
 * so -0 and +0 are equal. */
void orc_topk(int32_t T, const float *scores, int64_t ld, const int32_t *n, int32_t k, int32_t *idx)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        int32_t nt = n[t];
        int32_t *row = idx + (int64_t)t * k;
        int32_t keep = nt < k ? nt : k;
        if (nt <= k) {
            for (int32_t i = 0; i < k; ++i)
                row[i] = i < nt ? i : -1;
            continue;
        }
        orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)nt);
        for (int32_t s = 0; s < nt; ++s) {
            c[s].score = scores[(int64_t)t * ld + s];
            c[s].pos = s;
        }
        qsort(c, (size_t)nt, sizeof(orc_cand), orc_cmp_rank);
        for (int32_t i = 0; i < keep; ++i)
            row[i] = c[i].pos;
        qsort(row, (size_t)keep, sizeof(int32_t), orc_cmp_i32);
        for (int32_t i = keep; i < k; ++i)
            row[i] = -1;
        free(c);
    }
}

/* ---------------------------------------------------------------- O3 ---- */

/* Sparse MLA with a per-head sink, for T queries and H heads.
 *   q [T, H, D_qk] bf16, kv [rows, D_qk] bf16 (the latent row; its first D_v
 *   entries are the value), idx [T, k] sequence-local positions (-1 = empty),
 *   sink [H] fp32, out [T, H, D_v] fp64.
 * For each (t, h), over the valid entries j of idx[t]:
 *   s_j = scale * <q[t,h,:], kv[base_t + idx_j, :]>
 *   m   = max(sink_h, max_j s_j)
 *   out = sum_j exp(s_j - m) kv[base_t+idx_j, :D_v] / (exp(sink_h - m) + sum_j exp(s_j - m))
 * Readings: the sink is a logit in the units of the scaled scores, it only
 * enlarges the denominator and carries no value; the scale covers the whole
 * 576-wide dot (latent and RoPE parts); the value is the leading D_v entries of
 * the same latent row (absorbed-MLA form). An empty selection gives zeros. */
void orc_sparse_mla(int32_t T, int32_t H, int32_t D_qk, int32_t D_v,
                    const uint16_t *q, const uint16_t *kv, const int64_t *base,
                    const int32_t *idx, int32_t k, const float *sink, double scale, double *out)
{
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            const int32_t *row = idx + (int64_t)t * k;
            double *qd = (double *)malloc(sizeof(double) * (size_t)D_qk);
            double *s = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
            double *o = out + ((int64_t)t * H + h) * D_v;
            orc_decode_bf16(q + ((int64_t)t * H + h) * D_qk, qd, D_qk);
            /* pass 1: scores and their maximum (the sink takes part in it) */
            double m = (double)sink[h];
            for (int32_t j = 0; j < k; ++j) {
                if (row[j] < 0)
                    continue;
                const uint16_t *kr = kv + (base[t] + row[j]) * (int64_t)D_qk;
                double dot = 0.0;
                for (int32_t d = 0; d < D_qk; ++d)
                    dot += qd[d] * orc_bf16_to_double(kr[d]);
                s[j] = scale * dot;
                if (s[j] > m)
                    m = s[j];
            }
            /* pass 2: normalised weighted sum of the value rows */
            double den = exp((double)sink[h] - m);
            for (int32_t v = 0; v < D_v; ++v)
                o[v] = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                if (row[j] < 0)
                    continue;
                const uint16_t *kr = kv + (base[t] + row[j]) * (int64_t)D_qk;
                double p = exp(s[j] - m);
                den += p;
                for (int32_t v = 0; v < D_v; ++v)
                    o[v] += p * orc_bf16_to_double(kr[v]);
            }
            for (int32_t v = 0; v < D_v; ++v)
                o[v] /= den;
            free(qd);
            free(s);
        }
    }
}

/* ---------------------------------------------------------------- O5 ---- */

/* Gated head output (issue #90, sigmoid-gate bullet: the gate multiplies the
 * decompressed per-head attention output, so wv_b is applied first):
 *   out[t,h,e] = sigmoid(gate[t,h,e]) * sum_c wv_b[h,e,c] * o[t,h,c]
 * o [T,H,D_v], wv_b [H,D_o,D_v], gate [T,H,D_o] as bf16 bytes; out fp64.
 * sigmoid(x) = 1 / (1 + e^-x). */
void orc_gated_output(int32_t T, int32_t H, int32_t D_v, int32_t D_o, const uint16_t *o, const uint16_t *wv_b,
                      const uint16_t *gate, double *out)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            const uint16_t *ot = o + ((int64_t)t * H + h) * D_v;
            for (int32_t e = 0; e < D_o; ++e) {
                const uint16_t *wr = wv_b + ((int64_t)h * D_o + e) * D_v;
                double acc = 0.0;
                for (int32_t c = 0; c < D_v; ++c)
                    acc += orc_bf16_to_double(wr[c]) * orc_bf16_to_double(ot[c]);
                const double g = orc_bf16_to_double(gate[((int64_t)t * H + h) * D_o + e]);
                out[((int64_t)t * H + h) * D_o + e] = acc / (1.0 + exp(-g));
            }
        }
    }
}

/* ---------------------------------------------------------------- O6 ---- */

/* The cache write that precedes the path: for each new token, its indexer key
 * and its latent row are stored in the two caches (issue #90: the "Indexer:"
 * bullet puts the key through a LayerNorm with bias whose eps is the model's
 * RMS-norm eps; the RoPE bullet says the rotary embedding is interleaved,
 * i.e. not NeoX style; the first paragraph fixes the 576-wide latent row as
 * 512 latent entries plus 64 RoPE entries).
 * Readings: the rotary angles come as a table (cos and sin per position and
 * frequency), so no base or scaling rule is assumed; the rotated span of the
 * indexer key is its trailing D_rope entries, the same place as in the latent
 * row; the key is stored as a plain fp8 cast, without a scale, as the indexer
 * reads it. */

/* fp8 e4m3fn code of a real value: the nearest finite code, ties to the code
 * with even mantissa; magnitudes past 448 take 448 (the format has no
 * infinity, so the cast saturates). The 127 non-negative finite codes are
 * scanned in increasing value. The sign is kept (-0 gives 0x80); NaN gives
 * 0x7F. */
uint8_t orc_encode_fp8_e4m3fn(double x)
{
    if (isnan(x))
        return 0x7F;
    const int sign = signbit(x) ? 0x80 : 0;
    if (isinf(x))
        return (uint8_t)(sign | 0x7E);              /* no infinity: the largest finite magnitude */
    const double a = fabs(x);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double d = fabs(orc_fp8_e4m3fn_to_double((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

/* Interleaved rotary embedding of one span of D_rope entries at position p:
 * entries 2i and 2i+1 form a pair that turns by the angle whose cosine is
 * rope[p, i] and whose sine is rope[p, D_rope/2 + i]. */
static void orc_rope_interleaved(double *x, int32_t D_rope, const float *rope, int32_t p)
{
    const float *cs = rope + (int64_t)p * D_rope;
    for (int32_t i = 0; i < D_rope / 2; ++i) {
        const double c = cs[i], s = cs[D_rope / 2 + i];
        const double x0 = x[2 * i], x1 = x[2 * i + 1];
        x[2 * i] = x0 * c - x1 * s;
        x[2 * i + 1] = x1 * c + x0 * s;
    }
}

/* Indexer key of each new token:
 *   y = (x - mean(x)) / sqrt(var(x) + eps) * ln_w + ln_b, var the mean squared
 *       deviation (LayerNorm with bias);
 *   the trailing D_rope entries of y rotate at position pos[t];
 *   code = fp8 e4m3fn of y, the decision taken on y rounded to fp32 (the
 *          precision the stored code is computed in).
 * k_pre [T, D_I] bf16, ln_w and ln_b [D_I] fp32, rope [*, D_rope] fp32,
 * pos [T]; y [T, D_I] fp64 and code [T, D_I] are outputs. */
void orc_index_key(int32_t T, int32_t D_I, int32_t D_rope, const uint16_t *k_pre, const float *ln_w,
                   const float *ln_b, double eps, const float *rope, const int32_t *pos, double *y, uint8_t *code)
{
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
        double *yt = y + (int64_t)t * D_I;
        double mean = 0.0, var = 0.0;
        for (int32_t d = 0; d < D_I; ++d) {
            yt[d] = orc_bf16_to_double(k_pre[(int64_t)t * D_I + d]);
            mean += yt[d];
        }
        mean /= D_I;
        for (int32_t d = 0; d < D_I; ++d)
            var += (yt[d] - mean) * (yt[d] - mean);
        var /= D_I;
        const double inv = 1.0 / sqrt(var + eps);
        for (int32_t d = 0; d < D_I; ++d)
            yt[d] = (yt[d] - mean) * inv * (double)ln_w[d] + (double)ln_b[d];
        if (D_rope > 0)
            orc_rope_interleaved(yt + (D_I - D_rope), D_rope, rope, pos[t]);
        for (int32_t d = 0; d < D_I; ++d)
            code[(int64_t)t * D_I + d] = orc_encode_fp8_e4m3fn((double)(float)yt[d]);
    }
}

/* Latent row of each new token: the leading D_qk - D_rope entries (the
 * compressed latent, which is also the value) are stored as given; the
 * trailing D_rope entries rotate at position pos[t].
 * kv_pre [T, D_qk] bf16 -> out [T, D_qk] fp64. */
void orc_latent_row(int32_t T, int32_t D_qk, int32_t D_rope, const uint16_t *kv_pre, const float *rope,
                    const int32_t *pos, double *out)
{
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
        double *ot = out + (int64_t)t * D_qk;
        for (int32_t d = 0; d < D_qk; ++d)
            ot[d] = orc_bf16_to_double(kv_pre[(int64_t)t * D_qk + d]);
        if (D_rope > 0)
            orc_rope_interleaved(ot + (D_qk - D_rope), D_rope, rope, pos[t]);
    }
}
