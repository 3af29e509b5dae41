/* The C oracle's functions on small deterministic inputs, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer: every buffer access and
 * every integer and float-to-int conversion on these paths is checked. The
 * values themselves are pinned by the oracle's own tests; this only asks
 * that the code runs clean. Exit status 0 when it does. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double orc_fp8_e4m3fn_to_double(uint8_t b);
double orc_bf16_to_double(uint16_t b);
void orc_decode_fp8(const uint8_t *src, double *dst, int64_t n);
void orc_decode_bf16(const uint16_t *src, double *dst, int64_t n);
void orc_indexer_scores(int32_t T, int32_t H_I, int32_t D_I, const uint8_t *q_idx, const float *w,
                        const uint8_t *k_idx, const int64_t *base, const int32_t *n, double *out, int64_t ld);
void orc_topk(int32_t T, const float *scores, int64_t ld, const int32_t *n, int32_t k, int32_t *idx);
void orc_sparse_mla(int32_t T, int32_t H, int32_t D_qk, int32_t D_v, const uint16_t *q, const uint16_t *kv,
                    const int64_t *base, const int32_t *idx, int32_t k, const float *sink, double scale,
                    double *out);
void orc_gated_output(int32_t T, int32_t H, int32_t D_v, int32_t D_o, const uint16_t *o, const uint16_t *wv_b,
                      const uint16_t *gate, double *out);
uint8_t orc_encode_fp8_e4m3fn(double x);
void orc_index_key(int32_t T, int32_t D_I, int32_t D_rope, const uint16_t *k_pre, const float *ln_w,
                   const float *ln_b, double eps, const float *rope, const int32_t *pos, double *y,
                   uint8_t *code);
void orc_latent_row(int32_t T, int32_t D_qk, int32_t D_rope, const uint16_t *kv_pre, const float *rope,
                    const int32_t *pos, double *out);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 33);
}
/* finite fp8 codes of small integers, and bf16 of values in [-2, 2) */
static uint8_t fp8_small(void) { return orc_encode_fp8_e4m3fn((double)((int)(next() % 9) - 4)); }
static uint16_t bf16_of(float x)
{
    union { float f; uint32_t u; } v = {x};
    return (uint16_t)(v.u >> 16);
}
static uint16_t bf16_small(void) { return bf16_of((float)((int)(next() % 4096) - 2048) / 1024.0f); }
static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p)
        exit(2);
    return p;
}

int main(void)
{
    int bad = 0;
    /* every code of both formats, decoded one by one and in bulk */
    uint8_t c8[256];
    uint16_t *c16 = xmalloc(sizeof(uint16_t) * 65536);
    double *d = xmalloc(sizeof(double) * 65536);
    for (int i = 0; i < 256; ++i)
        c8[i] = (uint8_t)i;
    for (int i = 0; i < 65536; ++i)
        c16[i] = (uint16_t)i;
    orc_decode_fp8(c8, d, 256);
    for (int i = 0; i < 256; ++i)
        bad += !(isnan(d[i]) ? isnan(orc_fp8_e4m3fn_to_double(c8[i])) : d[i] == orc_fp8_e4m3fn_to_double(c8[i]));
    orc_decode_bf16(c16, d, 65536);
    for (int i = 0; i < 65536; i += 257)
        bad += !(isnan(d[i]) || d[i] == orc_bf16_to_double(c16[i]));
    /* the encoder across its range, saturation and specials included */
    const double specials[] = {0.0, -0.0, 1e-12, 448.0, 464.0, 1e9, -1e9, INFINITY, -INFINITY, NAN};
    for (int i = 0; i < 10; ++i)
        (void)orc_encode_fp8_e4m3fn(specials[i]);
    for (int i = -5000; i <= 5000; ++i)
        (void)orc_encode_fp8_e4m3fn(i * 0.0937);

    /* indexer and top-k: 3 queries (one empty) over their own rows */
    enum { T = 3, HI = 4, DI = 32, ROWS = 700, K = 64, LD = 512 };
    int64_t base[T] = {0, 500, 500};
    int32_t n[T] = {500, 0, 200};
    uint8_t *q_idx = xmalloc(T * HI * DI), *k_idx = xmalloc(ROWS * DI);
    float w[T * HI];
    for (int i = 0; i < T * HI * DI; ++i)
        q_idx[i] = fp8_small();
    for (int i = 0; i < ROWS * DI; ++i)
        k_idx[i] = fp8_small();
    for (int i = 0; i < T * HI; ++i)
        w[i] = (float)(1 + next() % 3);
    double *sc = xmalloc(sizeof(double) * T * LD);
    float *scf = xmalloc(sizeof(float) * T * LD);
    for (int i = 0; i < T * LD; ++i)
        sc[i] = -1.0;
    orc_indexer_scores(T, HI, DI, q_idx, w, k_idx, base, n, sc, LD);
    for (int i = 0; i < T * LD; ++i)
        scf[i] = (float)sc[i];
    int32_t idx[T * K];
    orc_topk(T, scf, LD, n, K, idx);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < K; ++j)
            bad += !(idx[t * K + j] >= -1 && idx[t * K + j] < n[t]);

    /* sparse MLA (80/64 shape) over those lists, the sink included */
    enum { H = 4, DQK = 80, DV = 64 };
    uint16_t *q = xmalloc(sizeof(uint16_t) * T * H * DQK), *kv = xmalloc(sizeof(uint16_t) * ROWS * DQK);
    for (int i = 0; i < T * H * DQK; ++i)
        q[i] = bf16_small();
    for (int i = 0; i < ROWS * DQK; ++i)
        kv[i] = bf16_small();
    float sink[H] = {0.5f, -1.0f, 0.0f, 2.0f};
    double *o = xmalloc(sizeof(double) * T * H * DV);
    orc_sparse_mla(T, H, DQK, DV, q, kv, base, idx, K, sink, 1.0 / sqrt((double)DQK), o);
    for (int i = 0; i < T * H * DV; ++i)
        bad += !isfinite(o[i]);

    /* gated output */
    enum { DO = 16 };
    uint16_t *ob = xmalloc(sizeof(uint16_t) * T * H * DV), *wv = xmalloc(sizeof(uint16_t) * H * DO * DV),
             *gate = xmalloc(sizeof(uint16_t) * T * H * DO);
    for (int i = 0; i < T * H * DV; ++i)
        ob[i] = bf16_small();
    for (int i = 0; i < H * DO * DV; ++i)
        wv[i] = bf16_small();
    for (int i = 0; i < T * H * DO; ++i)
        gate[i] = bf16_small();
    double *go = xmalloc(sizeof(double) * T * H * DO);
    orc_gated_output(T, H, DV, DO, ob, wv, gate, go);
    for (int i = 0; i < T * H * DO; ++i)
        bad += !isfinite(go[i]);

    /* cache write: index key (LayerNorm, rotation, fp8 code) and latent row */
    enum { TT = 5, DROPE = 16, NPOS = 40, DQ2 = 80 };
    uint16_t *kp = xmalloc(sizeof(uint16_t) * TT * DI), *kvp = xmalloc(sizeof(uint16_t) * TT * DQ2);
    float lw[DI], lb[DI], rope[NPOS * DROPE];
    int32_t pos[TT] = {0, 1, 17, 38, 39};
    for (int i = 0; i < TT * DI; ++i)
        kp[i] = bf16_small();
    for (int i = 0; i < TT * DQ2; ++i)
        kvp[i] = bf16_small();
    for (int i = 0; i < DI; ++i) {
        lw[i] = 1.0f + 0.01f * i;
        lb[i] = 0.1f;
    }
    for (int p = 0; p < NPOS; ++p)
        for (int i = 0; i < DROPE / 2; ++i) {
            rope[p * DROPE + i] = (float)cos(p * 0.1 * (i + 1));
            rope[p * DROPE + DROPE / 2 + i] = (float)sin(p * 0.1 * (i + 1));
        }
    double *y = xmalloc(sizeof(double) * TT * DI), *lo = xmalloc(sizeof(double) * TT * DQ2);
    uint8_t *code = xmalloc(TT * DI);
    orc_index_key(TT, DI, DROPE, kp, lw, lb, 1e-6, rope, pos, y, code);
    orc_latent_row(TT, DQ2, DROPE, kvp, rope, pos, lo);
    for (int i = 0; i < TT * DQ2; ++i)
        bad += !isfinite(lo[i]);

    free(c16); free(d); free(q_idx); free(k_idx); free(sc); free(scf); free(q); free(kv); free(o);
    free(ob); free(wv); free(gate); free(go); free(kp); free(kvp); free(y); free(lo); free(code);
    printf("%s: %d unexpected value(s)\n", bad ? "FAILED" : "ok", bad);
    return bad ? 1 : 0;
}
