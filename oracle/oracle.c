/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU implementation of the lossless greedy
 * speculative-decoding verify step.  It exists so that tests, the smoke check
 * and the CPU-baseline leg of the benchmark can check the HIP library against
 * something written straight from the method's definition.  Nothing in the
 * product path may link, load or call it.
 *
 * What it computes (per sequence, independently):
 *   - Jina-OCR-v1 release article and the jina-ocr-v1 tweet digest (the
 *     FastMTP paragraph): K draft tokens are checked by one forward pass of the
 *     target; the longest matching prefix is kept, plus one token of the
 *     target's own, and the result is identical to plain greedy decoding.
 *   - "Architecture and acceleration of an end-to-end OCR expert model",
 *     section 6.1: verification is one teacher-forced forward pass that
 *     yields the target's prediction at every draft position; tokens are
 *     accepted left to right up to the first disagreement, where the target's
 *     own token is taken instead.  Section 7 gives the draft / verify / accept
 *     loop this step implements one iteration of.
 *   - Jina-OCR-v1 paper, abstract and section 3 (Table 1 text): the target
 *     decoder is a DeepSeekMoE decoder; the tweet digest gives its shape
 *     (64 routed + 2 shared experts, top-6).
 *
 * The pages give no layer-level formula for the target decoder.  The layer is
 * the plain pre-norm decoder block: RMSNorm, rotary (rotate-half pairing
 * (i, i + D/2), theta^(-2i/D)), causal softmax attention with scale
 * 1/sqrt(D) and query head h reading KV head floor(h * n_kv / n_q), a
 * residual add, RMSNorm, then either a top-k softmax-routed SwiGLU mixture of
 * experts plus always-on shared experts, or a dense SwiGLU, and a residual
 * add.  A final RMSNorm, the LM head and an argmax give the greedy token.
 *
 * Arithmetic is fp64 throughout.  Stored weights are widened exactly from
 * their storage format (fp32, bf16 bit patterns, OCP e4m3fn codes with one
 * fp32 scale per output row, or OCP MXFP4: E2M1 codes with one E8M0 scale per
 * 32-element block of a row).  Two integer decisions are taken after
 * rounding the deciding values to fp32, the precision the GPU kernels decide
 * in: the expert selection (on the softmax probabilities) and the argmax (on
 * the logits).  New keys and values are rounded to the KV-cache storage type
 * before anything reads them, as a cache of that type forces.
 *
 * OpenMP is used only across independent output elements; every element is
 * summed by one thread in ascending index order, so results do not depend on
 * the thread count.
 *
 * KV-cache layout used here (natural order): for sequence b, layer l, KV head
 * h, position p, channel d, the element of both K and V is at
 *   (((b * L + l) * n_kv + h) * capacity + p) * D + d
 * in the cache storage type (fp32, or bf16 bit patterns).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2, OR_MXFP4 = 3 };
enum { OR_FFN_MOE = 0, OR_FFN_DENSE = 1 };

/* per-sequence status bits */
enum { OR_BAD_TOKEN = 1, OR_CAPACITY = 2, OR_NAN_LOGIT = 4 };

typedef struct {
    int n_layers, hidden, n_q, n_kv, head_dim;
    int ffn_kind;
    int n_experts, expert_inter, top_k, n_shared, renorm_topk;
    int dense_inter;
    int vocab, k_draft, capacity;
    double rope_theta, rms_eps;
    int wdtype;    /* storage of every linear weight (OR_F32 / OR_BF16 / OR_FP8) */
    int embdtype;  /* storage of the embedding table (OR_F32 / OR_BF16) */
    int kvdtype;   /* storage of the KV cache (OR_F32 / OR_BF16) */
} or_config;

/* A row-major matrix [rows][cols].  `dtype` is its storage type, or -1 for
 * the config's wdtype.  fp8: `scale` holds one fp32 per row.  MXFP4: `data`
 * holds two E2M1 codes per byte (even column in the low 4 bits), [rows][cols/2],
 * and `scale` points to E8M0 bytes [rows][cols/32], one per 32-column block. */
typedef struct {
    const void* data;
    const float* scale;
    int dtype;
} or_mat;

static int mat_dt(const or_mat* m, int dflt) { return m->dtype >= 0 ? m->dtype : dflt; }

typedef struct {
    const float* attn_norm;   /* [H] */
    or_mat w_qkv;             /* [(n_q + 2 n_kv) D][H]: q rows, then k rows, then v rows */
    or_mat w_o;               /* [H][n_q D] */
    const float* ffn_norm;    /* [H] */
    or_mat w_router;          /* [E][H] */
    or_mat w_gate_up;         /* [E][2I][H]: rows 0..I-1 gate, I..2I-1 up */
    or_mat w_down;            /* [E][H][I] */
    or_mat w_sh_gate_up;      /* [n_shared][2I][H] */
    or_mat w_sh_down;         /* [n_shared][H][I] */
    or_mat w_dense_gate_up;   /* [2 I_d][H] */
    or_mat w_dense_down;      /* [H][I_d] */
} or_layer;

typedef struct {
    const void* embed;        /* [V][H] in embdtype */
    const or_layer* layers;   /* [L] */
    const float* final_norm;  /* [H] */
    or_mat lm_head;           /* [V][H] */
} or_weights;

/* ---------------------------------------------------------------- formats */

double or_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3FN variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals when the exponent field is 0, no
 * infinities, and S.1111.111 as the only NaN pattern (max finite 448). */
double or_e4m3_to_double(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);            /* (m/8) * 2^(1-7) */
    else        v = ldexp((double)(8 + m), e - 10);  /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* OCP Microscaling (MX) formats: E2M1 is 1 sign bit, 2 exponent bits with
 * bias 1 and 1 mantissa bit, a subnormal when the exponent field is 0 (values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; no infinities or NaN).  An
 * MXFP4 block is 32 such elements sharing one E8M0 scale: an unsigned
 * exponent with bias 127, 2^(s - 127), where 0xFF is NaN. */
double or_e2m1_to_double(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

double or_e8m0_to_double(uint8_t s)
{
    return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127);
}

/* Round to the nearest bf16 value (8 significant bits, ties to even), directly
 * from fp64 so that no intermediate rounding can move a tie. */
double or_round_bf16(double x)
{
    int e;
    double m;
    if (x == 0.0 || !isfinite(x)) return x;
    m = frexp(x, &e);                 /* x = m * 2^e, 0.5 <= |m| < 1 */
    if (e < -125)                     /* bf16 subnormal range: spacing 2^-133 */
        return ldexp(nearbyint(ldexp(x, 133)), -133);
    m = nearbyint(ldexp(m, 8));       /* 8-bit significand, ties to even */
    x = ldexp(m, e - 8);
    if (fabs(x) > 3.3895313892515355e38) return x > 0 ? INFINITY : -INFINITY;
    return x;
}

static double load_elem(int dtype, const void* p, size_t i)
{
    switch (dtype) {
    case OR_F32: return (double)((const float*)p)[i];
    case OR_BF16: return or_bf16_to_double(((const uint16_t*)p)[i]);
    default: return or_e4m3_to_double(((const uint8_t*)p)[i]);
    }
}

static void store_elem(int dtype, void* p, size_t i, double x)
{
    if (dtype == OR_F32) {
        ((float*)p)[i] = (float)x;
    } else {
        float f = (float)or_round_bf16(x);   /* exact: already a bf16 value */
        uint32_t u;
        memcpy(&u, &f, 4);
        ((uint16_t*)p)[i] = (uint16_t)(u >> 16);
    }
}

/* ------------------------------------------------------------- primitives */

/* y[n] = sum_k W[row0 + n][k] * x[k] for n in [0, N), W row-major with K
 * columns; fp8 rows are scaled by their per-row scale after the sum; MXFP4
 * elements are the E2M1 value times the block's E8M0 scale. */
void or_matvec(const void* W, const float* scale, int dtype, long row0, int N, int K,
               const double* x, double* y)
{
    long n;
#pragma omp parallel for schedule(static) if ((long)N * K > 65536)
    for (n = 0; n < N; n++) {
        size_t base = (size_t)(row0 + n) * (size_t)K;
        double acc = 0.0;
        int k;
        switch (dtype) {
        case OR_F32: {
            const float* w = (const float*)W + base;
            for (k = 0; k < K; k++) acc += (double)w[k] * x[k];
        } break;
        case OR_BF16: {
            const uint16_t* w = (const uint16_t*)W + base;
            for (k = 0; k < K; k++) acc += or_bf16_to_double(w[k]) * x[k];
        } break;
        case OR_MXFP4: {
            const uint8_t* w = (const uint8_t*)W + base / 2;
            const uint8_t* sb = (const uint8_t*)scale + (size_t)(row0 + n) * (size_t)(K / 32);
            for (k = 0; k < K; k++) {
                uint8_t code = (k & 1) ? (uint8_t)(w[k >> 1] >> 4) : (uint8_t)(w[k >> 1] & 15);
                acc += or_e2m1_to_double(code) * or_e8m0_to_double(sb[k >> 5]) * x[k];
            }
        } break;
        default: {
            const uint8_t* w = (const uint8_t*)W + base;
            double tab[256];
            int c;
            for (c = 0; c < 256; c++) tab[c] = or_e4m3_to_double((uint8_t)c);
            for (k = 0; k < K; k++) acc += tab[w[k]] * x[k];
            acc *= (double)scale[row0 + n];
        } break;
        }
        y[n] = acc;
    }
}

/* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g */
void or_rmsnorm(const double* x, const float* g, int H, double eps, double* y)
{
    double ss = 0.0;
    int i;
    for (i = 0; i < H; i++) ss += x[i] * x[i];
    ss = 1.0 / sqrt(ss / H + eps);
    for (i = 0; i < H; i++) y[i] = x[i] * ss * (double)g[i];
}

/* Rotary embedding of one head vector v[D] at absolute position pos: the pair
 * (v[i], v[i + D/2]) is turned by the angle pos * theta^(-2i/D). */
void or_rope(double* v, int D, long pos, double theta)
{
    int i, half = D / 2;
    for (i = 0; i < half; i++) {
        double ang = (double)pos * pow(theta, -2.0 * i / D);
        double c = cos(ang), s = sin(ang);
        double a = v[i], b = v[i + half];
        v[i] = a * c - b * s;
        v[i + half] = b * c + a * s;
    }
}

/* Softmax attention of one query q[D] over keys/values 0..n_keys-1 of one KV
 * head; K and V point at that head's [capacity][D] slab. */
void or_attend(const double* q, const void* Kc, const void* Vc, int kvdtype, int D,
               long n_keys, double* out, double* scratch /* [n_keys] */)
{
    double m = -INFINITY, den = 0.0, sc = 1.0 / sqrt((double)D);
    long t;
    int d;
    for (t = 0; t < n_keys; t++) {
        double s = 0.0;
        for (d = 0; d < D; d++) s += q[d] * load_elem(kvdtype, Kc, (size_t)t * D + d);
        s *= sc;
        scratch[t] = s;
        if (s > m) m = s;
    }
    for (d = 0; d < D; d++) out[d] = 0.0;
    for (t = 0; t < n_keys; t++) {
        double w = exp(scratch[t] - m);
        den += w;
        for (d = 0; d < D; d++) out[d] += w * load_elem(kvdtype, Vc, (size_t)t * D + d);
    }
    for (d = 0; d < D; d++) out[d] /= den;
}

/* Numerically-shifted softmax of r[n]. */
void or_softmax(const double* r, int n, double* p)
{
    double m = -INFINITY, s = 0.0;
    int i;
    for (i = 0; i < n; i++) if (r[i] > m) m = r[i];
    for (i = 0; i < n; i++) { p[i] = exp(r[i] - m); s += p[i]; }
    for (i = 0; i < n; i++) p[i] /= s;
}

/* The k largest entries of v[n], largest first; equal values go to the lower
 * index first.  The comparison is made on the values rounded to fp32. */
void or_topk(const double* v, int n, int k, int* idx)
{
    int r, i, j;
    for (r = 0; r < k; r++) {
        int best = -1;
        float bv = 0.0f;
        for (i = 0; i < n; i++) {
            int taken = 0;
            for (j = 0; j < r; j++) if (idx[j] == i) taken = 1;
            if (taken) continue;
            if (best < 0 || (float)v[i] > bv) { best = i; bv = (float)v[i]; }
        }
        idx[r] = best;
    }
}

double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU expert: y = W_down (silu(W_gate h) * (W_up h)); `gu` holds 2I rows
 * (gate rows first) starting at row gu_row0, `dn` holds H rows of I columns
 * starting at row dn_row0. */
void or_swiglu(const or_mat* gu, long gu_row0, const or_mat* dn, long dn_row0, int dtype,
               int H, int I, const double* h, double* y, double* tmp /* [3I] */)
{
    double* g = tmp;
    double* u = tmp + I;
    double* a = tmp + 2 * I;
    int i;
    or_matvec(gu->data, gu->scale, mat_dt(gu, dtype), gu_row0, I, H, h, g);
    or_matvec(gu->data, gu->scale, mat_dt(gu, dtype), gu_row0 + I, I, H, h, u);
    for (i = 0; i < I; i++) a[i] = or_silu(g[i]) * u[i];
    or_matvec(dn->data, dn->scale, mat_dt(dn, dtype), dn_row0, H, I, a, y);
}

/* Feed-forward half of a layer on the normalised input h[H]: routed experts
 * (softmax over all E router logits, top-k on the probabilities, gates are
 * the selected probabilities, optionally renormalised to sum 1) in rank
 * order, then the shared experts in index order; or a dense SwiGLU.
 * Test hooks (each optional): `force` [top_k] replaces the top-k choice by
 * the given experts (gates stay this function's own probabilities), `sel`
 * [top_k] receives the experts used, `rlogits` [E] the router logits. */
void or_ffn(const or_config* c, const or_layer* L, const double* h, double* y, const int* force,
            int* sel, double* rlogits)
{
    int H = c->hidden, i, r;
    if (c->ffn_kind == OR_FFN_DENSE) {
        int I = c->dense_inter;
        double* tmp = (double*)malloc(sizeof(double) * 3 * (size_t)I);
        or_swiglu(&L->w_dense_gate_up, 0, &L->w_dense_down, 0, c->wdtype, H, I, h, y, tmp);
        free(tmp);
        return;
    }
    {
        int E = c->n_experts, I = c->expert_inter, k = c->top_k;
        double* logit = (double*)malloc(sizeof(double) * E);
        double* prob = (double*)malloc(sizeof(double) * E);
        double* ye = (double*)malloc(sizeof(double) * H);
        double* tmp = (double*)malloc(sizeof(double) * 3 * (size_t)I);
        int* idx = (int*)malloc(sizeof(int) * k);
        double gsum = 0.0;
        or_matvec(L->w_router.data, L->w_router.scale, mat_dt(&L->w_router, c->wdtype), 0, E, H, h, logit);
        or_softmax(logit, E, prob);
        if (force) for (r = 0; r < k; r++) idx[r] = force[r];
        else or_topk(prob, E, k, idx);
        if (rlogits) for (i = 0; i < E; i++) rlogits[i] = logit[i];
        for (r = 0; r < k; r++) gsum += prob[idx[r]];
        for (i = 0; i < H; i++) y[i] = 0.0;
        for (r = 0; r < k; r++) {
            int e = idx[r];
            double gate = c->renorm_topk ? prob[e] / gsum : prob[e];
            or_swiglu(&L->w_gate_up, (long)e * 2 * I, &L->w_down, (long)e * H, c->wdtype, H, I,
                      h, ye, tmp);
            for (i = 0; i < H; i++) y[i] += gate * ye[i];
        }
        for (r = 0; r < c->n_shared; r++) {
            or_swiglu(&L->w_sh_gate_up, (long)r * 2 * I, &L->w_sh_down, (long)r * H, c->wdtype, H,
                      I, h, ye, tmp);
            for (i = 0; i < H; i++) y[i] += ye[i];
        }
        if (sel) for (r = 0; r < k; r++) sel[r] = idx[r];
        free(logit); free(prob); free(ye); free(tmp); free(idx);
    }
}

/* Greedy token: index of the largest logit (compared in fp32), lowest index
 * on ties.  Returns -1 if any logit is NaN. */
int or_argmax(const double* logits, long V)
{
    long v, best = 0;
    float bv = (float)logits[0];
    for (v = 0; v < V; v++) if (isnan(logits[v])) return -1;
    for (v = 1; v < V; v++) {
        float f = (float)logits[v];
        if (f > bv) { bv = f; best = v; }
    }
    return (int)best;
}

/* Longest-matching-prefix acceptance with a bonus token.  g[0..K] are the
 * target's greedy tokens at the K+1 verified positions (g[j] follows the
 * prefix that ends with token j of the block), d[0..K-1] the drafts.
 * accepted = number of drafts kept (0..K); next = the target's own token at
 * the first disagreement, or after the last draft if all agree. */
void or_accept(int K, const int* g, const int* d, int* accepted, int* next)
{
    int a = 0;
    while (a < K && d[a] == g[a]) a++;
    *accepted = a;
    *next = g[a];
}

/* -------------------------------------------------------- the verify step */

static size_t kv_off(const or_config* c, long b, int l, int h, long pos)
{
    return ((((size_t)b * c->n_layers + l) * c->n_kv + h) * (size_t)c->capacity + pos) *
           (size_t)c->head_dim;
}

/* Test hooks on the expert routing of one verify step (all optional):
 * force [B][L][K+1][top_k] selections to use instead of the top-k choice,
 * sel_out [B][L][K+1][top_k] the selections used, rlogits_out
 * [B][L][K+1][E] the router logits. */
typedef struct {
    const int* force;
    int* sel_out;
    double* rlogits_out;
} or_route_io;

/* Embedding row of token t, widened. */
static void embed_row(const or_config* c, const or_weights* w, int t, double* x)
{
    int i;
    for (i = 0; i < c->hidden; i++) x[i] = load_elem(c->embdtype, w->embed, (size_t)t * c->hidden + i);
}

/* Logits of the final hidden state x[H]: rms(x) . W_lm */
static void lm_logits(const or_config* c, const or_weights* w, const double* x, double* logits)
{
    double* f = (double*)malloc(sizeof(double) * c->hidden);
    or_rmsnorm(x, w->final_norm, c->hidden, c->rms_eps, f);
    or_matvec(w->lm_head.data, w->lm_head.scale, mat_dt(&w->lm_head, c->wdtype), 0, c->vocab,
              c->hidden, f, logits);
    free(f);
}

/*
 * Teacher-forced forward of the n positions tok[0..n-1] of sequence b, placed
 * at cache positions ctx .. ctx+n-1, through all layers.  Within a layer every
 * position's key and value are computed and written to the cache first; then
 * each position attends causally to cache positions 0..its own.  On return
 * x[n][H] holds the residual stream after the last layer; `layer_hidden`
 * (optional, [L][n][H]) receives it after each layer.
 */
static void forward_block(const or_config* c, const or_weights* w, void* kc, void* vc, long b,
                          long ctx, int n, const int* tok, const double* x_in, double* x,
                          double* layer_hidden, const or_route_io* rio)
{
    int H = c->hidden, D = c->head_dim, nq = c->n_q, nkv = c->n_kv;
    int QKV = (nq + 2 * nkv) * D;
    double* h = (double*)malloc(sizeof(double) * H);
    double* qkv = (double*)malloc(sizeof(double) * (size_t)n * QKV);
    double* att = (double*)malloc(sizeof(double) * (size_t)nq * D);
    double* o = (double*)malloc(sizeof(double) * H);
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(ctx + n) * nq);
    int l, j, i, hh;

    if (x_in) memcpy(x, x_in, sizeof(double) * (size_t)n * H);   /* given residual input */
    else for (j = 0; j < n; j++) embed_row(c, w, tok[j], x + (size_t)j * H);

    for (l = 0; l < c->n_layers; l++) {
        const or_layer* L = &w->layers[l];
        /* 1) norm, projections, rotary; every new key/value goes to the cache */
        for (j = 0; j < n; j++) {
            double* q = qkv + (size_t)j * QKV;
            long pos = ctx + j;
            or_rmsnorm(x + (size_t)j * H, L->attn_norm, H, c->rms_eps, h);
            or_matvec(L->w_qkv.data, L->w_qkv.scale, mat_dt(&L->w_qkv, c->wdtype), 0, QKV, H, h, q);
            for (hh = 0; hh < nq + nkv; hh++) or_rope(q + (size_t)hh * D, D, pos, c->rope_theta);
            for (hh = 0; hh < nkv; hh++) {
                const double* kk = q + (size_t)(nq + hh) * D;
                const double* vv = q + (size_t)(nq + nkv + hh) * D;
                size_t off = kv_off(c, b, l, hh, pos);
                for (i = 0; i < D; i++) {
                    store_elem(c->kvdtype, kc, off + i, kk[i]);
                    store_elem(c->kvdtype, vc, off + i, vv[i]);
                }
            }
        }
        /* 2) causal attention, output projection and residual, feed-forward */
        for (j = 0; j < n; j++) {
            const double* q = qkv + (size_t)j * QKV;
            long nk = ctx + j + 1;
            double* xj = x + (size_t)j * H;
#pragma omp parallel for schedule(static)
            for (hh = 0; hh < nq; hh++) {
                int kvh = (int)(((long)hh * nkv) / nq);
                size_t off = kv_off(c, b, l, kvh, 0);
                size_t eb = c->kvdtype == OR_F32 ? 4 : 2;
                or_attend(q + (size_t)hh * D, (const char*)kc + off * eb, (const char*)vc + off * eb,
                          c->kvdtype, D, nk, att + (size_t)hh * D, scratch + (size_t)hh * (ctx + n));
            }
            or_matvec(L->w_o.data, L->w_o.scale, mat_dt(&L->w_o, c->wdtype), 0, H, nq * D, att, o);
            for (i = 0; i < H; i++) xj[i] += o[i];
            or_rmsnorm(xj, L->ffn_norm, H, c->rms_eps, h);
            {
                size_t rs = ((size_t)l * n + j) * (size_t)c->top_k;   /* this (layer, position) */
                or_ffn(c, L, h, o, rio && rio->force ? rio->force + rs : NULL,
                       rio && rio->sel_out ? rio->sel_out + rs : NULL,
                       rio && rio->rlogits_out
                           ? rio->rlogits_out + ((size_t)l * n + j) * (size_t)c->n_experts
                           : NULL);
            }
            for (i = 0; i < H; i++) xj[i] += o[i];
        }
        if (layer_hidden)
            memcpy(layer_hidden + (size_t)l * n * H, x, sizeof(double) * (size_t)n * H);
    }
    free(h); free(qkv); free(att); free(o); free(scratch);
}

/*
 * One verify step for sequences 0..B-1.  For sequence b the block is
 * (committed[b], drafts[b][0..K-1]) at positions ctx_in[b] .. ctx_in[b]+K.
 * Outputs: accepted[b] (0..K), next_tok[b], ctx_out[b] = ctx_in[b] +
 * accepted + 1, status[b] (0 or OR_* bits; on error accepted = next = -1 and
 * ctx_out = ctx_in).  Optional outputs (NULL to skip): target[b][K+1] greedy
 * tokens, logits[b][K+1][V], hidden[b][K+1][H] (residual after the last
 * layer), layer_hidden[b][L][K+1][H], route (routing test hooks).  The caches
 * are updated in place at the K+1 new positions.
 */
void or_verify_step(const or_config* c, const or_weights* w, void* kc, void* vc, int B,
                    const int* committed, const int* drafts, const int* ctx_in, int* ctx_out,
                    int* accepted, int* next_tok, int* status, int* target, double* logits,
                    double* hidden, double* layer_hidden, const or_route_io* route)
{
    int K = c->k_draft, n = K + 1, H = c->hidden;
    long V = c->vocab;
    int b, j;
    for (b = 0; b < B; b++) {
        int* tok = (int*)malloc(sizeof(int) * n);
        int* g = (int*)malloc(sizeof(int) * n);
        double* x = (double*)malloc(sizeof(double) * (size_t)n * H);
        double* lg = (double*)malloc(sizeof(double) * V);
        int st = 0;
        tok[0] = committed[b];
        for (j = 0; j < K; j++) tok[j + 1] = drafts[(size_t)b * K + j];
        for (j = 0; j < n; j++) if (tok[j] < 0 || tok[j] >= V) st |= OR_BAD_TOKEN;
        if (ctx_in[b] < 0 || (long)ctx_in[b] + n > c->capacity) st |= OR_CAPACITY;
        if (st == 0) {
            or_route_io rio = {NULL, NULL, NULL};
            size_t per_b = (size_t)c->n_layers * n;
            if (route && c->ffn_kind == OR_FFN_MOE) {
                if (route->force) rio.force = route->force + (size_t)b * per_b * c->top_k;
                if (route->sel_out) rio.sel_out = route->sel_out + (size_t)b * per_b * c->top_k;
                if (route->rlogits_out)
                    rio.rlogits_out = route->rlogits_out + (size_t)b * per_b * c->n_experts;
            }
            forward_block(c, w, kc, vc, b, ctx_in[b], n, tok, NULL, x,
                          layer_hidden ? layer_hidden + (size_t)b * c->n_layers * n * H : NULL,
                          &rio);
            for (j = 0; j < n; j++) {
                lm_logits(c, w, x + (size_t)j * H, lg);
                g[j] = or_argmax(lg, V);
                if (g[j] < 0) st |= OR_NAN_LOGIT;
                if (logits) memcpy(logits + ((size_t)b * n + j) * V, lg, sizeof(double) * V);
                if (target) target[(size_t)b * n + j] = g[j];
            }
            if (hidden) memcpy(hidden + (size_t)b * n * H, x, sizeof(double) * (size_t)n * H);
        }
        status[b] = st;
        if (st) {
            accepted[b] = -1;
            next_tok[b] = -1;
            ctx_out[b] = ctx_in[b];
        } else {
            or_accept(K, g, drafts + (size_t)b * K, &accepted[b], &next_tok[b]);
            ctx_out[b] = ctx_in[b] + accepted[b] + 1;
        }
        free(tok); free(g); free(x); free(lg);
    }
}

/*
 * Plain autoregressive decode of one token of sequence b: token `tok` at
 * position `pos` (its key/value are written to the cache there); returns the
 * greedy next token (-1 on a NaN logit).  Optional logits[V] and hidden[H].
 */
int or_decode_one(const or_config* c, const or_weights* w, void* kc, void* vc, long b, long pos,
                  int tok, double* logits, double* hidden)
{
    double* x = (double*)malloc(sizeof(double) * c->hidden);
    double* lg = (double*)malloc(sizeof(double) * c->vocab);
    int g;
    forward_block(c, w, kc, vc, b, pos, 1, &tok, NULL, x, NULL, NULL);
    lm_logits(c, w, x, lg);
    g = or_argmax(lg, c->vocab);
    if (logits) memcpy(logits, lg, sizeof(double) * c->vocab);
    if (hidden) memcpy(hidden, x, sizeof(double) * c->hidden);
    free(x); free(lg);
    return g;
}

/*
 * Draft stream of the synthetic workloads: for i = 1..K, if coin[i-1] is set
 * the draft is the target's greedy token after the prefix (committed,
 * d_1..d_{i-1}); otherwise it is rand_tok[i-1].  The prefix is decoded one
 * token at a time with or_decode_one (this writes the cache at positions
 * ctx .. ctx+K-1, which the verify step rewrites with the same values).
 */
void or_make_drafts(const or_config* c, const or_weights* w, void* kc, void* vc, long b, long ctx,
                    int committed, const unsigned char* coin, const int* rand_tok, int* drafts)
{
    int i, prev = committed;
    for (i = 0; i < c->k_draft; i++) {
        int g = or_decode_one(c, w, kc, vc, b, ctx + i, prev, NULL, NULL);
        drafts[i] = coin[i] ? g : rand_tok[i];
        prev = drafts[i];
    }
}

/*
 * The decoder on given residual inputs: rows x_in[n][H] at cache positions
 * ctx .. ctx+n-1 of sequence b, through all layers (keys and values written
 * to the cache), then the final norm: f_out[n][H] (the LM head's input),
 * logits[n][V] (optional) and the greedy token of every row (argmax_out[n],
 * -1 on a NaN logit).
 */
void or_forward_rows(const or_config* c, const or_weights* w, void* kc, void* vc, long b, long ctx,
                     int n, const double* x_in, double* f_out, double* logits, int* argmax_out)
{
    int H = c->hidden, j;
    long V = c->vocab;
    double* x = (double*)malloc(sizeof(double) * (size_t)n * H);
    double* lg = (double*)malloc(sizeof(double) * V);
    forward_block(c, w, kc, vc, b, ctx, n, NULL, x_in, x, NULL, NULL);
    for (j = 0; j < n; j++) {
        double* f = f_out + (size_t)j * H;
        or_rmsnorm(x + (size_t)j * H, w->final_norm, H, c->rms_eps, f);
        or_matvec(w->lm_head.data, w->lm_head.scale, mat_dt(&w->lm_head, c->wdtype), 0, V, H, f, lg);
        argmax_out[j] = or_argmax(lg, V);
        if (logits) memcpy(logits + (size_t)j * V, lg, sizeof(double) * V);
    }
    free(x); free(lg);
}

/*
 * FastMTP drafting (Jina-OCR-v1 paper, section 3.1): one shared dense block
 * B applied recursively for K depths.  With e = embedding, N_e / N_h RMSNorms
 * with gains g_e / g_h, P the [H][2H] projection, N_o and the LM head shared
 * with the target:
 *   a(1) = the target's post-norm state at a position, a(k) = u(k-1) of the
 *   previous depth; z(k) = P [N_e(e(next token)); N_h(a(k))];
 *   u(k) = N_o(B(z(k); pos)); the draft is argmax of W_lm u(k).
 * After a verify step that kept `a` drafts of sequence b (positions ctx ..
 * ctx+a committed, `next_tok` the target's token at ctx+a+1): depth 1 runs
 * the block over rows j = 0..a (state bstate[j], the target's post-norm row
 * of position ctx+j; next token d_{j+1} for j < a, next_tok for j = a) at
 * positions ctx+j, writing the block's cache there, and the draft d'_1 comes
 * from row a; depth k > 1 runs one row at position ctx+a+k-1 with state
 * u(k-1) and token d'_{k-1}.  The block is `w`'s single layer (the LM head,
 * final norm and embedding are the target's, as the paper ties them).
 * Outputs drafts_out[K] and gap_out[K] (each depth's top-2 logit gap over
 * its logit range, in fp32, for choosing a check set).
 */
void or_mtp_draft(const or_config* c, const or_weights* w, const float* g_e, const float* g_h,
                  const or_mat* P, void* kc, void* vc, long b, long ctx, int a, const int* drafts,
                  int next_tok, const double* bstate, int* drafts_out, double* gap_out)
{
    int H = c->hidden, K = c->k_draft, k, j;
    long V = c->vocab;
    int n = a + 1;
    double* cat = (double*)malloc(sizeof(double) * 2 * H);
    double* e = (double*)malloc(sizeof(double) * H);
    double* z = (double*)malloc(sizeof(double) * (size_t)n * H);
    double* f = (double*)malloc(sizeof(double) * (size_t)n * H);
    double* lg = (double*)malloc(sizeof(double) * (size_t)n * V);
    int* am = (int*)malloc(sizeof(int) * n);
    double* u = (double*)malloc(sizeof(double) * H);
    int prev = -1;
    for (k = 1; k <= K; k++) drafts_out[k - 1] = -1;
    for (k = 1; k <= K; k++) {
        if (k > 1 && prev < 0) break;   /* a NaN logit ended the recursion */
        int rows = k == 1 ? n : 1;
        long pos0 = k == 1 ? ctx : ctx + a + k - 1;
        for (j = 0; j < rows; j++) {
            int tok = k == 1 ? (j < a ? drafts[j] : next_tok) : prev;
            const double* st = k == 1 ? bstate + (size_t)j * H : u;
            embed_row(c, w, tok, e);
            or_rmsnorm(e, g_e, H, c->rms_eps, cat);
            or_rmsnorm(st, g_h, H, c->rms_eps, cat + H);
            or_matvec(P->data, P->scale, mat_dt(P, c->wdtype), 0, H, 2 * H, cat, z + (size_t)j * H);
        }
        or_forward_rows(c, w, kc, vc, b, pos0, rows, z, f, lg, am);
        {
            int r = k == 1 ? a : 0;
            const double* l = lg + (size_t)r * V;
            float t1 = -INFINITY, t2 = -INFINITY;
            double lo = l[0], hi = l[0];
            long v;
            for (v = 0; v < V; v++) {
                float fv = (float)l[v];
                if (fv > t1) { t2 = t1; t1 = fv; } else if (fv > t2) t2 = fv;
                if (l[v] < lo) lo = l[v];
                if (l[v] > hi) hi = l[v];
            }
            prev = am[r];
            drafts_out[k - 1] = prev;
            gap_out[k - 1] = hi > lo ? ((double)t1 - (double)t2) / (hi - lo) : 0.0;
            memcpy(u, f + (size_t)r * H, sizeof(double) * H);
        }
    }
    free(cat); free(e); free(z); free(f); free(lg); free(am); free(u);
}

/* Threads the parallel loops use (for reporting). */
int or_num_threads(void) { return omp_get_max_threads(); }
