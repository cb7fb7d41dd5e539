/*
 * DSA oracle: plain, slow, obviously correct CPU implementation of the
 * DeepSeek Sparse Attention hot path.  TEST INFRASTRUCTURE ONLY: it is built
 * and called by tests/, by __graft_entry__.smoke() and by the cpu_baseline leg
 * of bench.py, never by the product library.  It shares no code, header,
 * table or constant with the GPU path.
 *
 * Sources (web pages; section named for each function):
 *  - DeepSeek-V3.2-Exp summary page, section "Method": the index score
 *    I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s]) over every earlier key,
 *    H_I heads, FP8; top-k = 2048; MLA in MQA mode, one latent KV row serving
 *    every query head of its token.
 *  - AMD "MI355X GPUs Power DeepSeek-V3.2-Exp" article, section "DeepSeek
 *    Sparse Attention (DSA)": the indexer scores the keys before the query;
 *    2048 keys per query are kept for the main attention.
 *  - createthis gist page, indexer listing: FP8 E4M3 inputs quantized along the
 *    last dimension.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - the query's own position is visible: n_t = min(S, pos_t + 1);
 *  - rows with n_t < k select every visible key and pad with -1;
 *  - equal scores: the lower key index wins; -0.0 equals +0.0;
 *  - MLA: K = all D_qk columns of the latent row, V = its first D_v columns;
 *    softmax scale is a parameter; LSE is natural-log, fp32;
 *  - index entries outside [0, n_t) are skipped, duplicates count with
 *    multiplicity; a row with no valid entry gives out = 0, lse = -inf.
 *
 * Arithmetic: fp32 with a fixed ascending summation order (no fused
 * multiply-add; built with -ffp-contract=off).  Each query row is computed by
 * one thread, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- value formats --------------------------------------------------- */

/* OCP FP8 E4M3 ("fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there are
 * no infinities.  Largest finite value 1.75 * 2^8 = 448. */
static float e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 7;
    float v;
    if (e == 0xF && m == 7)
        return NAN;
    if (e == 0)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -v : v;
}

static float g_e4m3[256];
static int g_e4m3_ready = 0;

static void e4m3_init(void)
{
    if (g_e4m3_ready)
        return;
    for (int c = 0; c < 256; ++c)
        g_e4m3[c] = e4m3_value((uint8_t)c);
    g_e4m3_ready = 1;
}

/* bf16 is the upper half of an IEEE binary32 word. */
static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb; /* round to nearest, ties to even */
    return (uint16_t)(u >> 16);
}

static void set_threads(int32_t nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

static int64_t visible_keys(int64_t pos, int64_t S)
{
    int64_t n = pos + 1;
    return n < S ? n : S;
}

/* ---- exported helpers ------------------------------------------------- */

void oracle_e4m3_table(float *out256)
{
    e4m3_init();
    memcpy(out256, g_e4m3, sizeof g_e4m3);
}

void oracle_bf16_round(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_round(x[i]);
}

/* Copy logical rows 0..n-1 of a paged pool into a contiguous array: logical
 * row r lives at physical row block_table[r / block_size] * block_size +
 * r % block_size.  Returns 0, or 1 if a table entry is negative. */
int oracle_gather_rows(const void *pool, int64_t row_bytes, const int32_t *block_table,
                       int32_t block_size, int64_t n, void *out)
{
    const uint8_t *src = (const uint8_t *)pool;
    uint8_t *dst = (uint8_t *)out;
    for (int64_t r = 0; r < n; ++r) {
        int32_t blk = block_table[r / block_size];
        if (blk < 0)
            return 1;
        int64_t phys = (int64_t)blk * block_size + r % block_size;
        memcpy(dst + r * row_bytes, src + phys * row_bytes, (size_t)row_bytes);
    }
    return 0;
}

/* ---- step 1: lightning indexer ---------------------------------------
 * DeepSeek-V3.2-Exp summary, "Method": for query row t (absolute position
 * pos[t]) and every visible key s < n_t,
 *     I[t,s] = sum_j w[t,j] * max(0, q_I[t,j] . k_I[s]),
 * with the FP8 inputs dequantized first: q_I[t,j,i] = qs[t,j] * dec(q8[t,j,i]),
 * k_I[s,i] = ks[s] * dec(k8[s,i]).  Entries s >= n_t are not written. */
int oracle_indexer(const uint8_t *q8, const float *qs, const float *w, const int64_t *pos,
                   int64_t T, const uint8_t *k8, const float *ks, int64_t S, int32_t H_I,
                   int32_t D_I, float *logits, int64_t ld, int32_t nthreads)
{
    if (T < 0 || S < 0 || H_I <= 0 || D_I <= 0 || ld < S)
        return 1;
    e4m3_init();
    float *kdec = (float *)malloc(sizeof(float) * (size_t)(S > 0 ? S : 1) * (size_t)D_I);
    if (!kdec)
        return 3;
    for (int64_t s = 0; s < S; ++s)
        for (int32_t i = 0; i < D_I; ++i)
            kdec[s * D_I + i] = ks[s] * g_e4m3[k8[s * D_I + i]];
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        float *qdec = (float *)malloc(sizeof(float) * (size_t)H_I * (size_t)D_I);
        if (!qdec) {
            bad = 3;
            continue;
        }
        for (int32_t j = 0; j < H_I; ++j)
            for (int32_t i = 0; i < D_I; ++i)
                qdec[j * D_I + i] = qs[t * H_I + j] * g_e4m3[q8[(t * H_I + j) * D_I + i]];
        int64_t n = visible_keys(pos[t], S);
        for (int64_t s = 0; s < n; ++s) {
            float I = 0.0f;
            for (int32_t j = 0; j < H_I; ++j) {
                float d = 0.0f;
                for (int32_t i = 0; i < D_I; ++i)
                    d += qdec[j * D_I + i] * kdec[s * D_I + i];
                float r = d > 0.0f ? d : 0.0f;
                I += w[t * H_I + j] * r;
            }
            logits[t * ld + s] = I;
        }
        free(qdec);
    }
    free(kdec);
    return bad;
}

/* ---- step 2: top-k selection -----------------------------------------
 * AMD article, "Fine-Grained Token Selection" and the summary's "Method":
 * keep the k highest-scoring visible keys.  Candidates s < n_t are sorted by
 * (score descending, index ascending); the first min(k, n_t) are returned,
 * the rest of the row is -1.  Non-finite scores are rejected (return 2). */
typedef struct {
    float v;
    int32_t i;
} scored_t;

static int by_score_then_index(const void *a, const void *b)
{
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    return (x->i > y->i) - (x->i < y->i);
}

int oracle_topk(const float *logits, int64_t ld, const int64_t *pos, int64_t T, int64_t S,
                int32_t k, int32_t *idx, int32_t nthreads)
{
    if (T < 0 || S < 0 || k <= 0 || ld < S)
        return 1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        int64_t n = visible_keys(pos[t], S);
        scored_t *c = (scored_t *)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
        if (!c) {
            bad = 3;
            continue;
        }
        for (int64_t s = 0; s < n; ++s) {
            float v = logits[t * ld + s];
            if (!isfinite(v))
                bad = 2;
            c[s].v = v == 0.0f ? 0.0f : v; /* -0.0 -> +0.0 */
            c[s].i = (int32_t)s;
        }
        qsort(c, (size_t)n, sizeof(scored_t), by_score_then_index);
        int64_t m = n < k ? n : k;
        for (int64_t r = 0; r < k; ++r)
            idx[t * k + r] = r < m ? c[r].i : -1;
        free(c);
    }
    return bad;
}

/* ---- step 3: sparse MLA forward, MQA mode ----------------------------
 * Summary page, "Method": the main attention reads only the selected latent
 * KV rows, one row shared by all H query heads.  For query row t, head h and
 * the valid entries i of the index list (0 <= idx < n_t):
 *     z_i = sm_scale * (q[t,h,:] . kv[idx_i, :D_qk])
 *     m = max z, e_i = exp(z_i - m), l = sum e_i
 *     out[t,h,d] = (sum_i e_i * kv[idx_i, d]) / l   for d < D_v
 *     lse[t,h] = m + log(l)
 * out_bf16 (optional) is out rounded to bf16. */
int oracle_sparse_mla(const uint16_t *q, const int32_t *idx, const int64_t *pos, int64_t T,
                      int32_t H, int32_t D_qk, int32_t D_v, int32_t k, const uint16_t *kv,
                      int64_t S, float sm_scale, float *out, uint16_t *out_bf16, float *lse,
                      int32_t nthreads)
{
    if (T < 0 || S < 0 || H <= 0 || D_qk <= 0 || D_v <= 0 || D_v > D_qk || k <= 0)
        return 1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        int64_t n = visible_keys(pos[t], S);
        const int32_t *row = idx + t * k;
        float *z = (float *)malloc(sizeof(float) * (size_t)k);
        float *acc = (float *)malloc(sizeof(float) * (size_t)D_v);
        if (!z || !acc) {
            bad = 3;
            free(z);
            free(acc);
            continue;
        }
        for (int32_t h = 0; h < H; ++h) {
            const uint16_t *qh = q + (t * H + h) * (int64_t)D_qk;
            float m = -INFINITY;
            for (int32_t i = 0; i < k; ++i) {
                int32_t s = row[i];
                if (s < 0 || s >= n)
                    continue;
                const uint16_t *kr = kv + (int64_t)s * D_qk;
                float dot = 0.0f;
                for (int32_t d = 0; d < D_qk; ++d)
                    dot += bf16_value(qh[d]) * bf16_value(kr[d]);
                z[i] = sm_scale * dot;
                if (z[i] > m)
                    m = z[i];
            }
            float *o = out + (t * H + h) * (int64_t)D_v;
            if (m == -INFINITY) { /* no valid entry */
                for (int32_t d = 0; d < D_v; ++d)
                    o[d] = 0.0f;
                if (out_bf16)
                    for (int32_t d = 0; d < D_v; ++d)
                        out_bf16[(t * H + h) * (int64_t)D_v + d] = 0;
                lse[t * H + h] = -INFINITY;
                continue;
            }
            float l = 0.0f;
            for (int32_t d = 0; d < D_v; ++d)
                acc[d] = 0.0f;
            for (int32_t i = 0; i < k; ++i) {
                int32_t s = row[i];
                if (s < 0 || s >= n)
                    continue;
                float e = expf(z[i] - m);
                l += e;
                const uint16_t *vr = kv + (int64_t)s * D_qk;
                for (int32_t d = 0; d < D_v; ++d)
                    acc[d] += e * bf16_value(vr[d]);
            }
            for (int32_t d = 0; d < D_v; ++d)
                o[d] = acc[d] / l;
            if (out_bf16)
                for (int32_t d = 0; d < D_v; ++d)
                    out_bf16[(t * H + h) * (int64_t)D_v + d] = bf16_round(o[d]);
            lse[t * H + h] = m + logf(l);
        }
        free(z);
        free(acc);
    }
    return bad;
}

/* ---- NEXT step: FP8 quantization of the indexer inputs and the paged append -------------
 * createthis gist page, indexer listing: the indexer's query and key vectors are cast to
 * FP8 E4M3 along the last dimension with one scale per vector (per-row absmax); the cache
 * then holds the codes and scales of every key, and the latent row of every token, at the
 * token's slot of the paged layout. */

/* Nearest E4M3 code of a finite y with 0 <= y <= 448.  The non-negative finite codes 0x00 ..
 * 0x7E decode to strictly increasing values, so the nearest one is found by bisection over
 * the decoded table; a y exactly halfway between two neighbouring codes takes the one whose
 * code (low mantissa bit) is even, the nearest-even rule of a cast to the format. */
static uint8_t e4m3_encode_abs(float y)
{
    int lo = 0, hi = 0x7E; /* g_e4m3[lo] <= y < g_e4m3[hi] during the search */
    if (y >= g_e4m3[hi])
        return (uint8_t)hi;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_e4m3[mid] <= y)
            lo = mid;
        else
            hi = mid;
    }
    double dl = (double)y - (double)g_e4m3[lo], dh = (double)g_e4m3[hi] - (double)y;
    if (dl < dh)
        return (uint8_t)lo;
    if (dh < dl)
        return (uint8_t)hi;
    return (uint8_t)((lo & 1) ? hi : lo);
}

/* Code of a finite y with |y| <= 448 (the sign bit copied, also for -0). */
static uint8_t e4m3_encode(float y)
{
    return (uint8_t)((signbit(y) ? 0x80 : 0) | e4m3_encode_abs(fabsf(y)));
}

void oracle_e4m3_encode(const float *y, uint8_t *out, int64_t n)
{
    e4m3_init();
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_encode(y[i]);
}

/* One row of D bf16 values: s = amax / 448 (1 for an all-zero row), code_i =
 * e4m3(clamp(x_i / s, -448, 448)), the division and the clamp in fp32. */
static void quantize_row(const uint16_t *x, int32_t D, uint8_t *codes, float *scale)
{
    float amax = 0.0f;
    for (int32_t i = 0; i < D; ++i) {
        float a = fabsf(bf16_value(x[i]));
        if (a > amax)
            amax = a;
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    *scale = s;
    for (int32_t i = 0; i < D; ++i) {
        float v = bf16_value(x[i]) / s;
        if (v > 448.0f)
            v = 448.0f;
        if (v < -448.0f)
            v = -448.0f;
        codes[i] = e4m3_encode(v);
    }
}

void oracle_quantize_rows(const uint16_t *x, int64_t rows, int32_t D, uint8_t *codes, float *scales)
{
    e4m3_init();
    for (int64_t r = 0; r < rows; ++r)
        quantize_row(x + r * D, D, codes + r * D, scales + r);
}

/* Power-of-two variant (createthis gist page, indexer listing: the cast helper's use_ue8m0
 * option, an unsigned exponent-only scale).  Reading: s = 2^p for the smallest p with
 * 2^p >= t = amax / 448 (fp32 division; t = 1 for an all-zero row), p at least -127 so that s fits
 * the format; the scale is stored as its biased exponent p + 127 and the codes are
 * e4m3(clamp(x / s, -448, 448)) as above (the division by a power of two is exact). */
static void quantize_row_ue8m0(const uint16_t *x, int32_t D, uint8_t *codes, uint8_t *exp8, float *scale)
{
    float amax = 0.0f;
    for (int32_t i = 0; i < D; ++i) {
        float a = fabsf(bf16_value(x[i]));
        if (a > amax)
            amax = a;
    }
    float t = amax > 0.0f ? amax / 448.0f : 1.0f;
    int e;
    float m = frexpf(t, &e); /* t = m 2^e, 0.5 <= m < 1 */
    int p = m == 0.5f ? e - 1 : e;
    if (p < -127)
        p = -127;
    float s = ldexpf(1.0f, p);
    *scale = s;
    *exp8 = (uint8_t)(p + 127);
    for (int32_t i = 0; i < D; ++i) {
        float v = bf16_value(x[i]) / s;
        if (v > 448.0f)
            v = 448.0f;
        if (v < -448.0f)
            v = -448.0f;
        codes[i] = e4m3_encode(v);
    }
}

void oracle_quantize_rows_ue8m0(const uint16_t *x, int64_t rows, int32_t D, uint8_t *codes, uint8_t *exps,
                                float *scales)
{
    e4m3_init();
    for (int64_t r = 0; r < rows; ++r)
        quantize_row_ue8m0(x + r * D, D, codes + r * D, exps + r, scales + r);
}

/* Append n tokens to a paged cache: token i (sequence seq[i], position pos[i]) goes to the
 * physical row block_table[seq[i] * max_blocks + pos[i] / bs] * bs + pos[i] % bs of the pools:
 * the quantized indexer key k[i] (codes and scale) and the latent row kv[i] copied as is.
 * Returns the number of tokens whose block id is negative (those are not written). */
int64_t oracle_append_paged(uint8_t *k8_pool, float *ks_pool, uint16_t *kv_pool, int32_t bs,
                            const int32_t *block_table, int64_t max_blocks, const int32_t *seq,
                            const int32_t *pos, int64_t n, int32_t D_I, int32_t D_qk,
                            const uint16_t *k, const uint16_t *kv)
{
    e4m3_init();
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t blk = block_table[(int64_t)seq[i] * max_blocks + pos[i] / bs];
        if (blk < 0) {
            ++bad;
            continue;
        }
        int64_t row = (int64_t)blk * bs + pos[i] % bs;
        quantize_row(k + i * D_I, D_I, k8_pool + row * D_I, ks_pool + row);
        memcpy(kv_pool + row * D_qk, kv + i * D_qk, (size_t)D_qk * sizeof(uint16_t));
    }
    return bad;
}

/* ---- NEXT step: the indexer's training signal (dense warm-up) and its backward ------------
 * DeepSeek-V3.2-Exp summary page, "Method" (continued pre-training): in a dense warm-up stage
 * only the indexer is trained, against a KL-divergence target given by the main attention; in
 * the sparse stage the indexer keeps its own graph.  The pages give no formula.  Reading:
 *  - the target of query row t is the main attention's distribution over its visible keys
 *    s < n_t averaged over the H heads,
 *        p[t,s] = (1/H) sum_h softmax_s( sm_scale * q[t,h,:] . kv[s, :D_qk] ),
 *    the attention of the sparse step taken over every visible key (MQA: K = the whole latent
 *    row);
 *  - the indexer's distribution is pi[t,.] = softmax_s(I[t,s]) over the same keys;
 *  - the row's loss is KL(p || pi) = sum_s p (log p - log pi), with 0 log 0 = 0, and its
 *    gradient with respect to the scores is dI[t,s] = pi[t,s] - p[t,s] (the p sum to one);
 *  - the backward passes the FP8 quantization straight through: the gradients are taken with
 *    respect to the dequantized vectors q_I = qs * dec(q8), k_I = ks * dec(k8) and the weights
 *    w, and ReLU's derivative is 1 for a positive product and 0 otherwise.
 * Arithmetic in double: every input value (bf16, dequantized FP8, fp32) is exact in double. */

/* Loss and score gradient of every query row.  logits [T][ld] (fp32, the row's visible entries
 * s < n_t are read); loss [T]; dlogits [T][ld_d] (entries s >= n_t untouched).  A row with no
 * visible key has loss 0.  Returns 1 on a bad shape, 2 on a non-finite score, 3 on no memory. */
int oracle_indexer_kl(const uint16_t *q, const uint16_t *kv, const int64_t *pos, int64_t T, int64_t S,
                      int32_t H, int32_t D_qk, double sm_scale, const float *logits, int64_t ld,
                      double *loss, double *dlogits, int64_t ld_d, int32_t nthreads)
{
    if (T < 0 || S < 0 || H <= 0 || D_qk <= 0 || ld < S || ld_d < S)
        return 1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        int64_t n = visible_keys(pos[t], S);
        loss[t] = 0.0;
        if (n <= 0)
            continue;
        double *z = (double *)malloc(sizeof(double) * (size_t)n);
        double *p = (double *)calloc((size_t)n, sizeof(double));
        if (!z || !p) {
            bad = 3;
            free(z);
            free(p);
            continue;
        }
        /* target: softmax of every head over the visible keys, averaged over the heads */
        for (int32_t h = 0; h < H; ++h) {
            const uint16_t *qh = q + (t * H + h) * (int64_t)D_qk;
            double m = -INFINITY;
            for (int64_t s = 0; s < n; ++s) {
                const uint16_t *kr = kv + s * D_qk;
                double dot = 0.0;
                for (int32_t d = 0; d < D_qk; ++d)
                    dot += (double)bf16_value(qh[d]) * (double)bf16_value(kr[d]);
                z[s] = sm_scale * dot;
                if (z[s] > m)
                    m = z[s];
            }
            double l = 0.0;
            for (int64_t s = 0; s < n; ++s)
                l += exp(z[s] - m);
            for (int64_t s = 0; s < n; ++s)
                p[s] += exp(z[s] - m) / l / (double)H;
        }
        /* the indexer's log-probabilities over the same keys */
        const float *I = logits + t * ld;
        double mi = -INFINITY;
        int finite = 1;
        for (int64_t s = 0; s < n; ++s) {
            if (!isfinite(I[s]))
                finite = 0;
            else if ((double)I[s] > mi)
                mi = (double)I[s];
        }
        if (!finite) {
            bad = 2;
            free(z);
            free(p);
            continue;
        }
        double li = 0.0;
        for (int64_t s = 0; s < n; ++s)
            li += exp((double)I[s] - mi);
        double lse_i = mi + log(li);
        double acc = 0.0;
        for (int64_t s = 0; s < n; ++s) {
            double log_pi = (double)I[s] - lse_i;
            if (p[s] > 0.0)
                acc += p[s] * (log(p[s]) - log_pi);
            dlogits[t * ld_d + s] = exp(log_pi) - p[s];
        }
        loss[t] = acc;
        free(z);
        free(p);
    }
    return bad;
}

/* Gradients through the index scores I[t,s] = sum_j w[t,j] max(0, z), z = q_I[t,j] . k_I[s],
 * given dlogits [T][ld] = dL/dI on the visible entries (s < n_t; others never read):
 *     dw[t,j]     = sum_s dI[t,s] max(0, z)
 *     dq[t,j,:]   = sum_{s: z > 0} dI[t,s] w[t,j] k_I[s,:]
 *     dk[s,:]     = sum_{t, j: z > 0} dI[t,s] w[t,j] q_I[t,j,:]
 * Outputs dq [T][H_I][D_I], dw [T][H_I], dk [S][D_I] (double).  Returns 1 on a bad shape, 3 on
 * no memory. */
int oracle_indexer_bwd(const uint8_t *q8, const float *qs, const float *w, const int64_t *pos, int64_t T,
                       const uint8_t *k8, const float *ks, int64_t S, int32_t H_I, int32_t D_I,
                       const float *dlogits, int64_t ld, double *dq, double *dw, double *dk, int32_t nthreads)
{
    if (T < 0 || S < 0 || H_I <= 0 || D_I <= 0 || ld < S)
        return 1;
    e4m3_init();
    size_t nk = (size_t)(S > 0 ? S : 1) * (size_t)D_I, nq = (size_t)(T > 0 ? T : 1) * (size_t)H_I * (size_t)D_I;
    double *kd = (double *)malloc(sizeof(double) * nk);
    double *qd = (double *)malloc(sizeof(double) * nq);
    if (!kd || !qd) {
        free(kd);
        free(qd);
        return 3;
    }
    for (int64_t s = 0; s < S; ++s)
        for (int32_t i = 0; i < D_I; ++i)
            kd[s * D_I + i] = (double)ks[s] * (double)g_e4m3[k8[s * D_I + i]];
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < H_I; ++j)
            for (int32_t i = 0; i < D_I; ++i)
                qd[(t * H_I + j) * D_I + i] = (double)qs[t * H_I + j] * (double)g_e4m3[q8[(t * H_I + j) * D_I + i]];
    set_threads(nthreads);
    /* dq and dw: one query row per iteration */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        int64_t n = visible_keys(pos[t], S);
        for (int32_t j = 0; j < H_I; ++j) {
            const double *qv = qd + (t * H_I + j) * D_I;
            double *g = dq + (t * H_I + j) * D_I;
            double gw = 0.0;
            for (int32_t i = 0; i < D_I; ++i)
                g[i] = 0.0;
            for (int64_t s = 0; s < n; ++s) {
                const double *kv_ = kd + s * D_I;
                double z = 0.0;
                for (int32_t i = 0; i < D_I; ++i)
                    z += qv[i] * kv_[i];
                double di = (double)dlogits[t * ld + s];
                if (z > 0.0) {
                    gw += di * z;
                    for (int32_t i = 0; i < D_I; ++i)
                        g[i] += di * (double)w[t * H_I + j] * kv_[i];
                }
            }
            dw[t * H_I + j] = gw;
        }
    }
    /* dk: one key per iteration, over the query rows that see it */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < S; ++s) {
        double *g = dk + s * D_I;
        const double *kv_ = kd + s * D_I;
        for (int32_t i = 0; i < D_I; ++i)
            g[i] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            if (s >= visible_keys(pos[t], S))
                continue;
            double di = (double)dlogits[t * ld + s];
            for (int32_t j = 0; j < H_I; ++j) {
                const double *qv = qd + (t * H_I + j) * D_I;
                double z = 0.0;
                for (int32_t i = 0; i < D_I; ++i)
                    z += qv[i] * kv_[i];
                if (z > 0.0)
                    for (int32_t i = 0; i < D_I; ++i)
                        g[i] += di * (double)w[t * H_I + j] * qv[i];
            }
        }
    }
    free(kd);
    free(qd);
    return 0;
}

/* Sparse stage (summary page, "Method": with top-k on, the indexer keeps its own graph; the
 * pages print no formula).  Reading: the loss is restricted to the entries of each row's index
 * list.  For row t and its valid entries i (0 <= idx[t][i] < n_t; others skipped, a repeated key
 * counts once per entry, as in the sparse attention):
 *     p_i  = (1/H) sum_h exp(z_hi) / sum_j exp(z_hj),  z_hi = sm_scale q[t,h,:] . kv[idx_i, :D_qk]
 *            (the sparse attention's probabilities averaged over the heads),
 *     pi_i = exp(I[t, idx_i]) / sum_j exp(I[t, idx_j]),
 *     loss[t] = sum_i p_i (log p_i - log pi_i),
 *     dlogits[t][s] = sum_{i: idx_i = s} (pi_i - p_i) for s < n_t (0 for keys not listed).
 * A row without valid entries has loss 0 and dlogits 0.  Arithmetic in double.  Returns 1 on a bad
 * shape, 2 on a non-finite listed score, 3 on no memory. */
int oracle_indexer_kl_sparse(const uint16_t *q, const uint16_t *kv, const int64_t *pos, int64_t T, int64_t S,
                             int32_t H, int32_t D_qk, double sm_scale, const int32_t *idx, int32_t k,
                             const float *logits, int64_t ld, double *loss, double *dlogits, int64_t ld_d,
                             int32_t nthreads)
{
    if (T < 0 || S < 0 || H <= 0 || D_qk <= 0 || k <= 0 || ld < S || ld_d < S)
        return 1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        const int32_t *row = idx + t * k;
        int64_t n = visible_keys(pos[t], S);
        loss[t] = 0.0;
        for (int64_t s = 0; s < n; ++s)
            dlogits[t * ld_d + s] = 0.0;
        double *z = (double *)malloc(sizeof(double) * (size_t)k);
        double *p = (double *)calloc((size_t)k, sizeof(double));
        if (!z || !p) {
            bad = 3;
            free(z);
            free(p);
            continue;
        }
        int any = 0;
        for (int32_t i = 0; i < k; ++i)
            if (row[i] >= 0 && row[i] < n)
                any = 1;
        if (!any) {
            free(z);
            free(p);
            continue;
        }
        for (int32_t h = 0; h < H; ++h) {
            const uint16_t *qh = q + (t * H + h) * (int64_t)D_qk;
            double m = -INFINITY;
            for (int32_t i = 0; i < k; ++i) {
                if (row[i] < 0 || row[i] >= n)
                    continue;
                const uint16_t *kr = kv + (int64_t)row[i] * D_qk;
                double dot = 0.0;
                for (int32_t d = 0; d < D_qk; ++d)
                    dot += (double)bf16_value(qh[d]) * (double)bf16_value(kr[d]);
                z[i] = dot * sm_scale;
                if (z[i] > m)
                    m = z[i];
            }
            double l = 0.0;
            for (int32_t i = 0; i < k; ++i)
                if (row[i] >= 0 && row[i] < n)
                    l += exp(z[i] - m);
            for (int32_t i = 0; i < k; ++i)
                if (row[i] >= 0 && row[i] < n)
                    p[i] += exp(z[i] - m) / l / (double)H;
        }
        const float *I = logits + t * ld;
        double mi = -INFINITY;
        int finite = 1;
        for (int32_t i = 0; i < k; ++i) {
            if (row[i] < 0 || row[i] >= n)
                continue;
            if (!isfinite(I[row[i]]))
                finite = 0;
            else if ((double)I[row[i]] > mi)
                mi = (double)I[row[i]];
        }
        if (!finite) {
            bad = 2;
            free(z);
            free(p);
            continue;
        }
        double li = 0.0;
        for (int32_t i = 0; i < k; ++i)
            if (row[i] >= 0 && row[i] < n)
                li += exp((double)I[row[i]] - mi);
        double lse_i = mi + log(li), acc = 0.0;
        for (int32_t i = 0; i < k; ++i) {
            if (row[i] < 0 || row[i] >= n)
                continue;
            double log_pi = (double)I[row[i]] - lse_i;
            if (p[i] > 0.0)
                acc += p[i] * (log(p[i]) - log_pi);
            dlogits[t * ld_d + row[i]] += exp(log_pi) - p[i];
        }
        loss[t] = acc;
        free(z);
        free(p);
    }
    return bad;
}

/* ---- NEXT step: backward of the sparse MLA forward ---------------------------------------------
 * DeepSeek-V3.2-Exp summary page, section "Method": in the sparse training stage the main model
 * trains with top-k selection on, its attention reading only the selected latent rows (AMD article,
 * section "Training Approach", sparse stage).  The forward of oracle_sparse_mla, for query row t,
 * head h and the valid entries i of its list (0 <= idx_i < n_t; each entry its own term):
 *     z_i = sm_scale q . k_i,  p = softmax(z),  out = sum_i p_i v_i   (k_i = kv[idx_i][:D_qk],
 *                                                                       v_i = kv[idx_i][:D_v]).
 * Given g = dL/dout[t][h] (bf16 bits), the chain rule through the softmax gives
 *     dp_i = g . v_i,   D = sum_i p_i dp_i  (= g . out),   ds_i = p_i (dp_i - D),
 *     dq[t][h][:]  = sm_scale sum_i ds_i k_i,
 *     dkv[s][:]   += sm_scale ds_i q[t][h][:]        for every entry i with idx_i = s (all D_qk columns)
 *     dkv[s][:D_v] += p_i g                         (the value columns of the same row).
 * Rows with no valid entry contribute nothing (dq = 0).  Arithmetic in double, the softmax with
 * its row maximum subtracted.  Each row's contributions are summed over its heads per entry, then
 * added to dkv in ascending entry order, rows in ascending order: the result does not depend on the
 * thread count.  dq [T][H][D_qk], dkv [S][D_qk] (every entry written).  Returns 1 on a bad shape, 3
 * on no memory. */
static int mla_bwd_row(const uint16_t *q, const int32_t *row, int64_t n, int32_t H, int32_t D_qk, int32_t D_v,
                       int32_t k, const uint16_t *kv, double sm_scale, const uint16_t *g, double *dq,
                       double *contrib)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)k);
    double *dp = (double *)malloc(sizeof(double) * (size_t)k);
    if (!z || !dp) {
        free(z);
        free(dp);
        return 3;
    }
    for (int64_t e = 0; e < (int64_t)k * D_qk; ++e)
        contrib[e] = 0.0;
    for (int32_t h = 0; h < H; ++h) {
        const uint16_t *qh = q + (int64_t)h * D_qk;
        const uint16_t *gh = g + (int64_t)h * D_v;
        double *dqh = dq + (int64_t)h * D_qk;
        for (int32_t d = 0; d < D_qk; ++d)
            dqh[d] = 0.0;
        double m = -INFINITY;
        for (int32_t i = 0; i < k; ++i) {
            if (row[i] < 0 || row[i] >= n)
                continue;
            const uint16_t *kr = kv + (int64_t)row[i] * D_qk;
            double dot = 0.0;
            for (int32_t d = 0; d < D_qk; ++d)
                dot += (double)bf16_value(qh[d]) * (double)bf16_value(kr[d]);
            const double zi = sm_scale * dot;
            z[i] = zi;
            if (zi > m)
                m = zi;
        }
        if (m == -INFINITY)
            continue;
        double l = 0.0;
        for (int32_t i = 0; i < k; ++i)
            if (row[i] >= 0 && row[i] < n)
                l += exp(z[i] - m);
        double D = 0.0;
        for (int32_t i = 0; i < k; ++i) {
            if (row[i] < 0 || row[i] >= n)
                continue;
            const uint16_t *vr = kv + (int64_t)row[i] * D_qk;
            double dot = 0.0;
            for (int32_t d = 0; d < D_v; ++d)
                dot += (double)bf16_value(gh[d]) * (double)bf16_value(vr[d]);
            dp[i] = dot;
            D += exp(z[i] - m) / l * dot;
        }
        for (int32_t i = 0; i < k; ++i) {
            if (row[i] < 0 || row[i] >= n)
                continue;
            const double p = exp(z[i] - m) / l;
            const double ds = p * (dp[i] - D);
            const uint16_t *kr = kv + (int64_t)row[i] * D_qk;
            double *c = contrib + (int64_t)i * D_qk;
            for (int32_t d = 0; d < D_qk; ++d) {
                dqh[d] += sm_scale * ds * (double)bf16_value(kr[d]);
                c[d] += sm_scale * ds * (double)bf16_value(qh[d]);
            }
            for (int32_t d = 0; d < D_v; ++d)
                c[d] += p * (double)bf16_value(gh[d]);
        }
    }
    free(z);
    free(dp);
    return 0;
}

int oracle_sparse_mla_bwd(const uint16_t *q, const int32_t *idx, const int64_t *pos, int64_t T, int32_t H,
                          int32_t D_qk, int32_t D_v, int32_t k, const uint16_t *kv, int64_t S, double sm_scale,
                          const uint16_t *dout, double *dq, double *dkv, int32_t nthreads)
{
    if (T < 0 || S < 0 || H <= 0 || D_qk <= 0 || D_v <= 0 || D_v > D_qk || k <= 0)
        return 1;
    set_threads(nthreads);
    for (int64_t e = 0; e < S * (int64_t)D_qk; ++e)
        dkv[e] = 0.0;
    int nt = 1;
#ifdef _OPENMP
    nt = omp_get_max_threads();
#endif
    /* rows in batches of nt: contributions in parallel, added to dkv serially in row order */
    double *contrib = (double *)malloc(sizeof(double) * (size_t)nt * (size_t)k * (size_t)D_qk);
    if (!contrib)
        return 3;
    int bad = 0;
    for (int64_t t0 = 0; t0 < T && !bad; t0 += nt) {
        int64_t t1 = t0 + nt < T ? t0 + nt : T;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t t = t0; t < t1; ++t) {
            int rc = mla_bwd_row(q + t * H * (int64_t)D_qk, idx + t * k, visible_keys(pos[t], S), H, D_qk, D_v, k,
                                 kv, sm_scale, dout + t * H * (int64_t)D_v, dq + t * H * (int64_t)D_qk,
                                 contrib + (t - t0) * (int64_t)k * D_qk);
            if (rc)
                bad = rc;
        }
        for (int64_t t = t0; t < t1 && !bad; ++t) {
            const int32_t *row = idx + t * k;
            int64_t n = visible_keys(pos[t], S);
            for (int32_t i = 0; i < k; ++i) {
                if (row[i] < 0 || row[i] >= n)
                    continue;
                const double *c = contrib + ((t - t0) * (int64_t)k + i) * D_qk;
                double *dst = dkv + (int64_t)row[i] * D_qk;
                for (int32_t d = 0; d < D_qk; ++d)
                    dst[d] += c[d];
            }
        }
    }
    free(contrib);
    return bad;
}
