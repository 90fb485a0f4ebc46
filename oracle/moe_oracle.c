/*
 * moe_oracle.c -- plain, slow CPU oracle of the local MoE forward chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header or table with the HIP
 * library: it has its own number formats, its own rounding and its own loops.
 *
 * What it follows (citations name the page and its section):
 *   - ruDNN User Guide (ruDNN 0.1.5 on docs.rs), section 3 "MoE workflow":
 *     the chain is logits -> softmax/top-k -> compact dispatch -> SwiGLU
 *     experts -> weighted combine.
 *   - same guide, section 4 "Routing contract": FP32 softmax over all E
 *     experts before top-k, ties to the lower expert id, optional
 *     renormalisation of the selected weights, then a cast to the logits
 *     dtype; rows holding NaN, +inf or only -inf keep NaN weights.
 *   - same guide, section 5 "Expert weights and dispatch": x is [T,H], gate
 *     and up are [E,I,H], down is [E,H,I]; dispatch drops no token; a saved
 *     mapping restores token order.
 *   - tiny-llm deep dive 5 (ops.rs), "SiLU" block: silu(z) = z / (1 + exp(-z)) and the SwiGLU FFN
 *     W_down(SiLU(W_gate x) * W_up x); "RMSNorm" block: why sums are kept
 *     in double; "matvec" block: rows are independent, so rows may be
 *     split over threads without locks.
 *
 * Precision: routing runs in binary32 exactly as the contract fixes it
 * (each exp is computed in double and rounded once, the sum is taken
 * sequentially in ascending expert id, p = q / S by IEEE division).  The
 * experts and the combine accumulate in binary64 and round once to the
 * storage dtype.  Build with -ffp-contract=off and without -ffast-math.
 *
 * Parity status: every function here is pinned by the CPU tests in
 * tests/test_oracle.py (closed forms, brute force, library routines,
 * invariants, the printed gather example).  Agreement with the oracle on
 * the large workloads beyond those invariants is, by nature, unpinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes of this file (its own numbering, matched by oracle/__init__.py) */
enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2 };

#define O_INVALID_ROW 0xFFFFFFFFu

/* ------------------------------------------------------------------ */
/* Number formats, written from the IEEE 754 definitions.              */
/* ------------------------------------------------------------------ */

/* Round x to a binary format with p significand bits (hidden bit
 * included), minimum normal exponent emin and maximum exponent emax,
 * rounding to nearest, ties to even.  Subnormals keep the fixed quantum
 * 2^(emin-p+1); values past the largest finite number become +-inf. */
static double round_to_format(double x, int p, int emin, int emax)
{
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e2;
    frexp(fabs(x), &e2);          /* |x| = m * 2^e2, m in [0.5, 1) */
    int lead = e2 - 1;            /* exponent of the leading bit */
    if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, lead - (p - 1));
    double r = nearbyint(x / quantum) * quantum; /* default mode: ties to even */
    double maxfin = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxfin) return copysign(INFINITY, x);
    return r;
}

double oracle_round_f32(double x) { return round_to_format(x, 24, -126, 127); }
double oracle_round_f16(double x) { return round_to_format(x, 11, -14, 15); }
double oracle_round_bf16(double x) { return round_to_format(x, 8, -126, 127); }

static double f16_bits_to_double(uint16_t b)
{
    int sign = b >> 15, ex = (b >> 10) & 31, man = b & 1023;
    double v;
    if (ex == 31) v = man ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)man, -24);
    else v = ldexp((double)(1024 + man), ex - 25);
    return sign ? -v : v;
}

static uint16_t double_to_f16_bits(double x) /* x already representable */
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return sign | 0x7E00;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) return sign | (uint16_t)ldexp(a, 24); /* subnormal */
    int e2;
    frexp(a, &e2);
    int lead = e2 - 1;
    uint16_t man = (uint16_t)(ldexp(a, -lead) * 1024.0 - 1024.0);
    return sign | (uint16_t)((lead + 15) << 10) | man;
}

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static uint16_t double_to_bf16_bits(double x) /* x already representable */
{
    if (isnan(x)) return (uint16_t)((signbit(x) ? 0x8000 : 0) | 0x7FC0);
    float f = (float)x; /* exact: every bf16 value is a binary32 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* element i of a buffer of dtype dt, widened to double (exact) */
static double load_elem(const void* base, int dt, int64_t i)
{
    switch (dt) {
    case O_F32: return (double)((const float*)base)[i];
    case O_F16: return f16_bits_to_double(((const uint16_t*)base)[i]);
    default:    return bf16_bits_to_double(((const uint16_t*)base)[i]);
    }
}

/* store v into element i of a buffer of dtype dt, rounding once (RNE) */
static void store_elem(void* base, int dt, int64_t i, double v)
{
    switch (dt) {
    case O_F32: ((float*)base)[i] = (float)oracle_round_f32(v); break;
    case O_F16: ((uint16_t*)base)[i] = double_to_f16_bits(oracle_round_f16(v)); break;
    default:    ((uint16_t*)base)[i] = double_to_bf16_bits(oracle_round_bf16(v)); break;
    }
}

static int elem_bytes(int dt) { return dt == O_F32 ? 4 : 2; }

/* Exposed so the tests can pin the formats against numpy / torch. */
void oracle_widen(const void* src, int dt, int64_t n, double* dst)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, dt, i);
}

void oracle_narrow(const double* src, int dt, int64_t n, void* dst)
{
    for (int64_t i = 0; i < n; ++i) store_elem(dst, dt, i, src[i]);
}

/* ------------------------------------------------------------------ */
/* A tiny row-parallel loop (rows are independent, as in the matvec     */
/* block of the tiny-llm ops.rs walk-through).                          */
/* ------------------------------------------------------------------ */

typedef void (*row_fn)(void* ctx, int64_t row);

typedef struct {
    row_fn fn;
    void* ctx;
    int64_t begin, end;
} slice_t;

static void* run_slice(void* arg)
{
    slice_t* s = (slice_t*)arg;
    for (int64_t r = s->begin; r < s->end; ++r) s->fn(s->ctx, r);
    return NULL;
}

static void parallel_rows(int64_t n, int nthreads, row_fn fn, void* ctx)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        for (int64_t r = 0; r < n; ++r) fn(ctx, r);
        return;
    }
    pthread_t th[256];
    slice_t sl[256];
    for (int t = 0; t < nthreads; ++t) {
        sl[t].fn = fn;
        sl[t].ctx = ctx;
        sl[t].begin = n * t / nthreads;
        sl[t].end = n * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, run_slice, &sl[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* Routing (ruDNN User Guide, section 4 "Routing contract").            */
/* ------------------------------------------------------------------ */

/* The routing contract's probabilities of one row: the logits widened to
 * binary32, then p_e = exp(l_e - m) / S over all E experts, with m the row
 * maximum (the shift leaves p unchanged in exact arithmetic and keeps exp
 * finite) and S the sum of exp(l_j - m).  Each exp is rounded once to
 * binary32; S is summed in ascending expert id; p_e is one IEEE division.
 * Rows the contract turns into NaN rows need no test of their own: m
 * ignores NaN ("l > m" is false for it), so a NaN logit, a +inf logit
 * (inf - inf) or a row of only -inf (-inf - -inf) puts a NaN into some
 * l_e - m, which reaches S and from there every p_e. */
static void softmax_row_f32(const void* logits, int dt, int64_t row, int64_t E, float* p)
{
    for (int64_t e = 0; e < E; ++e) p[e] = (float)load_elem(logits, dt, row * E + e);
    float m = -INFINITY;
    for (int64_t e = 0; e < E; ++e) m = p[e] > m ? p[e] : m;
    float S = 0.0f;
    for (int64_t e = 0; e < E; ++e) {
        p[e] = (float)exp((double)(p[e] - m)); /* exp(l_e - m), rounded once */
        S += p[e];
    }
    for (int64_t e = 0; e < E; ++e) p[e] = p[e] / S;
}

void oracle_softmax(const void* logits, int dt, int64_t T, int64_t E, float* probs)
{
    for (int64_t t = 0; t < T; ++t) softmax_row_f32(logits, dt, t, E, probs + t * E);
}

typedef struct {
    const void* logits;
    int dt;
    int64_t E;
    int k, renorm;
    uint32_t* idx;
    void* w;
    float* w_f32;
} route_ctx;

static void route_one(void* vctx, int64_t t)
{
    route_ctx* c = (route_ctx*)vctx;
    int64_t E = c->E;
    int k = c->k;
    float* p = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    float* sel = (float*)malloc(sizeof(float) * (size_t)k);
    softmax_row_f32(c->logits, c->dt, t, E, p);
    /* top-k: k rounds, each takes the largest p not yet taken; only a
     * strictly larger p displaces the current pick, so among equal p the
     * lower expert id wins (ties favour lower ids).  In a NaN row no p is
     * larger than another, so the picks are experts 0, 1, ..., k-1. */
    for (int j = 0; j < k; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || p[e] > p[best]) best = e;
        }
        taken[best] = 1;
        c->idx[t * k + j] = (uint32_t)best;
        sel[j] = p[best];
    }
    if (c->renorm) {
        float R = 0.0f;
        for (int j = 0; j < k; ++j) R += sel[j]; /* FP32, slot order */
        for (int j = 0; j < k; ++j) sel[j] = sel[j] / R;
    }
    for (int j = 0; j < k; ++j) {
        if (c->w_f32) c->w_f32[t * k + j] = sel[j];
        store_elem(c->w, c->dt, t * k + j, (double)sel[j]); /* cast to logits dtype */
    }
    free(sel);
    free(taken);
    free(p);
}

/* logits [T,E] (dt), top_k in 1..E.  Writes idx [T,k] (U32), w [T,k] in the
 * logits dtype and, if w_f32 is non-NULL, the FP32 weights before the cast.
 * Returns 0, or -1 on a bad argument. */
int oracle_route(const void* logits, int dt, int64_t T, int64_t E, int k, int renorm,
                 uint32_t* idx, void* w, float* w_f32, int nthreads)
{
    if (T < 0 || E < 1 || k < 1 || k > E) return -1;
    route_ctx c = {logits, dt, E, k, renorm, idx, w, w_f32};
    parallel_rows(T, nthreads, route_one, &c);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Group-limited sigmoid routing (ruDNN user guide, section 10).        */
/* ------------------------------------------------------------------ */

/* sigmoid in binary32: the exact 1/(1+exp(-x)) of the binary32 input,
 * evaluated in double and rounded once. */
static float sigmoid_f32(float x)
{
    return (float)(1.0 / (1.0 + exp(-(double)x)));
}

typedef struct {
    const void* logits;
    int dt;
    const float* bias; /* [E] FP32 or NULL */
    int64_t E;
    int k, groups, selected, top_two, renorm;
    float scale;
    uint32_t* idx;
    void* w;
    float* w_f32;
    float* corr; /* [T,E] corrected scores, or NULL */
} sroute_ctx;

static void sroute_one(void* vctx, int64_t t)
{
    sroute_ctx* c = (sroute_ctx*)vctx;
    const int64_t E = c->E;
    const int k = c->k, G = c->groups, m = c->selected;
    const int64_t gsz = E / G;
    float* s = (float*)malloc(sizeof(float) * (size_t)E);
    float* cs = (float*)malloc(sizeof(float) * (size_t)E);
    float* gscore = (float*)malloc(sizeof(float) * (size_t)G);
    unsigned char* gtaken = (unsigned char*)calloc((size_t)G, 1);
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    float* sel = (float*)malloc(sizeof(float) * (size_t)k);
    int nan_row = 0;
    /* 1. sigmoid scores, and the corrected scores that only steer selection */
    for (int64_t e = 0; e < E; ++e) {
        s[e] = sigmoid_f32((float)load_elem(c->logits, c->dt, t * E + e));
        cs[e] = s[e] + (c->bias ? c->bias[e] : 0.0f);
        if (cs[e] != cs[e]) nan_row = 1;
        if (c->corr) c->corr[t * E + e] = cs[e];
    }
    if (nan_row) {
        /* a NaN score leaves no order: experts 0..k-1 with NaN weights, as
         * the routing contract does for softmax rows */
        for (int j = 0; j < k; ++j) {
            c->idx[t * k + j] = (uint32_t)j;
            if (c->w_f32) c->w_f32[t * k + j] = NAN;
            store_elem(c->w, c->dt, t * k + j, NAN);
        }
        goto done;
    }
    /* 2. group scores over contiguous blocks of E/G experts: the largest
     *    corrected score, or the sum of the two largest */
    for (int g = 0; g < G; ++g) {
        float a = -INFINITY, b = -INFINITY;
        for (int64_t e = g * gsz; e < (g + 1) * gsz; ++e) {
            if (cs[e] > a) {
                b = a;
                a = cs[e];
            } else if (cs[e] > b) {
                b = cs[e];
            }
        }
        gscore[g] = c->top_two ? a + b : a;
    }
    /* 3. the m best groups; a strictly larger score displaces the pick, so
     *    equal scores favour the lower group id */
    for (int r = 0; r < m; ++r) {
        int best = -1;
        for (int g = 0; g < G; ++g) {
            if (gtaken[g]) continue;
            if (best < 0 || gscore[g] > gscore[best]) best = g;
        }
        gtaken[best] = 1;
    }
    /* 4. top-k experts of the chosen groups by corrected score, in slot
     *    order of decreasing score, equal scores favouring the lower id */
    for (int j = 0; j < k; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e] || !gtaken[e / gsz]) continue;
            if (best < 0 || cs[e] > cs[best]) best = e;
        }
        taken[best] = 1;
        c->idx[t * k + j] = (uint32_t)best;
        sel[j] = s[best]; /* the weight uses the uncorrected score */
    }
    /* 5. optional renormalisation over the chosen scores (FP32, slot
     *    order), then the scale, then the cast to the logits dtype */
    if (c->renorm) {
        float R = 0.0f;
        for (int j = 0; j < k; ++j) R += sel[j];
        for (int j = 0; j < k; ++j) sel[j] = sel[j] / R;
    }
    for (int j = 0; j < k; ++j) {
        sel[j] = sel[j] * c->scale;
        if (c->w_f32) c->w_f32[t * k + j] = sel[j];
        store_elem(c->w, c->dt, t * k + j, (double)sel[j]);
    }
done:
    free(sel);
    free(taken);
    free(gtaken);
    free(gscore);
    free(cs);
    free(s);
}

/* logits [T,E] (dt); bias [E] FP32 or NULL; G groups of E/G experts, the
 * best `selected` groups, then top_k experts inside them.  Writes idx [T,k]
 * (U32), w [T,k] in the logits dtype, optionally the FP32 weights before the
 * cast and the corrected scores [T,E].  Returns 0, or -1 when the options
 * break the section's limits. */
int oracle_route_sigmoid_grouped(const void* logits, int dt, const float* bias, int64_t T, int64_t E,
                                 int k, int groups, int selected, int top_two, int renorm, float scale,
                                 uint32_t* idx, void* w, float* w_f32, float* corr, int nthreads)
{
    if (T < 0 || E < 1 || E > 1024 || groups < 1 || groups > 128 || E % groups) return -1;
    if (selected < 1 || selected > groups) return -1;
    if (k < 1 || k > 64 || (int64_t)k > (int64_t)selected * (E / groups)) return -1;
    if (top_two && E / groups < 2) return -1;
    if (!(scale > 0.0f) || scale == INFINITY) return -1;
    sroute_ctx c = {logits, dt, bias, E, k, groups, selected, top_two, renorm, scale, idx, w, w_f32, corr};
    parallel_rows(T, nthreads, sroute_one, &c);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dispatch (ruDNN User Guide, section 5): drop-free, grouped by expert. */
/* ------------------------------------------------------------------ */

/* Canonical order inside an expert: slots by (token, slot) ascending.
 * The contract leaves the order inside an expert open; this is one valid
 * order.  A slot whose expert id is >= E is not copied and its row_of_slot
 * is 0xFFFFFFFF.  offsets is [E+1]: rows of expert e are
 * [offsets[e], offsets[e+1]). */
int oracle_dispatch(const uint32_t* idx, int64_t T, int k, int64_t E,
                    const void* x, int64_t H, int dt,
                    uint32_t* offsets, uint32_t* row_of_slot, uint32_t* token_of_row,
                    void* dispatched)
{
    if (T < 0 || E < 1 || k < 1 || H < 0) return -1;
    int64_t N = T * (int64_t)k;
    uint32_t* cursor = (uint32_t*)calloc((size_t)E + 1, sizeof(uint32_t));
    for (int64_t s = 0; s < N; ++s)
        if (idx[s] < (uint64_t)E) cursor[idx[s]] += 1; /* counts */
    uint32_t run = 0;
    for (int64_t e = 0; e < E; ++e) { /* exclusive prefix sum, ascending e */
        uint32_t n = cursor[e];
        offsets[e] = run;
        cursor[e] = run;
        run += n;
    }
    offsets[E] = run;
    size_t rowb = (size_t)H * (size_t)elem_bytes(dt);
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t s = t * k + j;
            uint32_t e = idx[s];
            if (e >= (uint64_t)E) {
                row_of_slot[s] = O_INVALID_ROW;
                continue;
            }
            uint32_t r = cursor[e]++;
            row_of_slot[s] = r;
            token_of_row[r] = (uint32_t)t;
            memcpy((char*)dispatched + (size_t)r * rowb, (const char*)x + (size_t)t * rowb, rowb);
        }
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------ */
/* SwiGLU experts (ruDNN User Guide, section 5; tiny-llm ops.rs, SiLU). */
/* ------------------------------------------------------------------ */

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

typedef struct {
    const void* const* gate; /* E pointers, each [I,H] of dtype dt */
    const void* const* up;   /* E pointers, each [I,H] */
    const void* const* down; /* E pointers, each [H,I] */
    int dt;
    const void* rows; /* [N,H] dispatched rows */
    const uint32_t* offsets;
    int64_t E, H, I;
    void* out;   /* [N,H] */
    void* h_out; /* optional [N,I]: the stored activation */
    int* bad;
} experts_ctx;

static int64_t expert_of_row(const uint32_t* offsets, int64_t E, int64_t r)
{
    for (int64_t e = 0; e < E; ++e)
        if ((uint64_t)r < offsets[e + 1]) return e;
    return -1;
}

static void expert_row(void* vctx, int64_t r)
{
    experts_ctx* c = (experts_ctx*)vctx;
    int64_t e = expert_of_row(c->offsets, c->E, r);
    int64_t H = c->H, I = c->I;
    if (e < 0 || !c->gate[e] || !c->up[e] || !c->down[e]) {
        *c->bad = 1;
        return;
    }
    double* x = (double*)malloc(sizeof(double) * (size_t)H);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    for (int64_t c2 = 0; c2 < H; ++c2) x[c2] = load_elem(c->rows, c->dt, r * H + c2);
    for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t c2 = 0; c2 < H; ++c2) {
            g += x[c2] * load_elem(c->gate[e], c->dt, i * H + c2);
            u += x[c2] * load_elem(c->up[e], c->dt, i * H + c2);
        }
        double a = oracle_silu(g) * u;
        /* h is stored in the weight dtype before the down projection */
        switch (c->dt) {
        case O_F32: h[i] = oracle_round_f32(a); break;
        case O_F16: h[i] = oracle_round_f16(a); break;
        default:    h[i] = oracle_round_bf16(a); break;
        }
        if (c->h_out) store_elem(c->h_out, c->dt, r * I + i, h[i]);
    }
    for (int64_t c2 = 0; c2 < H; ++c2) {
        double y = 0.0;
        for (int64_t i = 0; i < I; ++i) y += h[i] * load_elem(c->down[e], c->dt, c2 * I + i);
        store_elem(c->out, c->dt, r * H + c2, y);
    }
    free(h);
    free(x);
}

/* rows [N,H] grouped by offsets [E+1]; per-expert weight pointers (NULL for
 * an expert that owns no row is fine).  out [N,H]; h_out [N,I] or NULL.
 * Returns 0, or -1 if a row's expert has no weights. */
int oracle_experts(const void* const* gate, const void* const* up, const void* const* down, int dt,
                   const void* rows, const uint32_t* offsets, int64_t E, int64_t H, int64_t I,
                   void* out, void* h_out, int nthreads)
{
    if (E < 1 || H < 1 || I < 1) return -1;
    int bad = 0;
    experts_ctx c = {gate, up, down, dt, rows, offsets, E, H, I, out, h_out, &bad};
    parallel_rows((int64_t)offsets[E], nthreads, expert_row, &c);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Combine (ruDNN User Guide, sections 5 and 6): restore token order    */
/* through the saved mapping and merge with the routing weights.        */
/* ------------------------------------------------------------------ */

typedef struct {
    const void* Y;
    int dt;
    const uint32_t* row_of_slot;
    const void* w;
    int wdt;
    int k;
    int64_t H;
    void* out;
} combine_ctx;

static void combine_one(void* vctx, int64_t t)
{
    combine_ctx* c = (combine_ctx*)vctx;
    int k = c->k;
    int64_t H = c->H;
    int invalid = 0;
    for (int j = 0; j < k; ++j)
        if (c->row_of_slot[t * k + j] == O_INVALID_ROW) invalid = 1;
    for (int64_t col = 0; col < H; ++col) {
        double acc = 0.0;
        if (invalid) {
            acc = NAN;
        } else {
            for (int j = 0; j < k; ++j) { /* fixed slot order */
                double wj = load_elem(c->w, c->wdt, t * k + j); /* stored, cast weight */
                double y = load_elem(c->Y, c->dt, (int64_t)c->row_of_slot[t * k + j] * H + col);
                acc += wj * y;
            }
        }
        store_elem(c->out, c->dt, t * H + col, acc);
    }
}

int oracle_combine(const void* Y, int dt, const uint32_t* row_of_slot, const void* w, int wdt,
                   int64_t T, int k, int64_t H, void* out, int nthreads)
{
    if (T < 0 || k < 1 || H < 0) return -1;
    combine_ctx c = {Y, dt, row_of_slot, w, wdt, k, H, out};
    parallel_rows(T, nthreads, combine_one, &c);
    return 0;
}

/* ------------------------------------------------------------------ */
/* First-order MoE training (RUDA ruDNN library guide, section 12).     */
/* ------------------------------------------------------------------ */

/* Router weights of a fixed selection.  scoring 0: softmax over all E (the
 * routing contract's FP32 softmax); 1: sigmoid of the selected logits.  The
 * selected scores q_j (gathered: a repeated index is gathered twice) are
 * divided by their FP32 sum in slot order when renorm is set, then
 * multiplied by scale.  An index outside [0, E) makes the token's row NaN. */
typedef struct {
    const void* logits;
    int dt;
    const int64_t* idx;
    const float* gw; /* [T,k] FP32 incoming gradient, backward only */
    int64_t E;
    int k, scoring, renorm;
    float scale;
    float* w;        /* [T,k] FP32 weights, forward only */
    void* dl;        /* [T,E] gradient in the logits dtype, backward only */
} rweights_ctx;

static int row_indices_valid(const int64_t* idx, int k, int64_t E)
{
    for (int j = 0; j < k; ++j)
        if (idx[j] < 0 || idx[j] >= E) return 0;
    return 1;
}

static void router_scores(const rweights_ctx* c, int64_t t, float* p)
{
    if (c->scoring == 0) {
        softmax_row_f32(c->logits, c->dt, t, c->E, p);
    } else {
        for (int64_t e = 0; e < c->E; ++e) p[e] = sigmoid_f32((float)load_elem(c->logits, c->dt, t * c->E + e));
    }
}

static void rweights_one(void* vctx, int64_t t)
{
    rweights_ctx* c = (rweights_ctx*)vctx;
    const int k = c->k;
    const int64_t* idx = c->idx + t * k;
    if (!row_indices_valid(idx, k, c->E)) {
        for (int j = 0; j < k; ++j) c->w[t * k + j] = NAN;
        return;
    }
    float* p = (float*)malloc(sizeof(float) * (size_t)c->E);
    router_scores(c, t, p);
    float S = 0.0f;
    for (int j = 0; j < k; ++j) S += p[idx[j]];
    for (int j = 0; j < k; ++j) {
        float q = p[idx[j]];
        if (c->renorm) q = q / S;
        c->w[t * k + j] = q * c->scale;
    }
    free(p);
}

/* d loss / d logits from d loss / d weights, for the fixed selection: only
 * the continuous weights are differentiated, not the choice.  Evaluated in
 * double from the binary32 scores, rounded once to the logits dtype. */
static void rbackward_one(void* vctx, int64_t t)
{
    rweights_ctx* c = (rweights_ctx*)vctx;
    const int k = c->k;
    const int64_t E = c->E;
    const int64_t* idx = c->idx + t * k;
    if (!row_indices_valid(idx, k, E)) {
        for (int64_t e = 0; e < E; ++e) store_elem(c->dl, c->dt, t * E + e, NAN);
        return;
    }
    float* p = (float*)malloc(sizeof(float) * (size_t)E);
    double* dscore = (double*)calloc((size_t)E, sizeof(double));
    router_scores(c, t, p);
    double S = 0.0, dot = 0.0;
    for (int j = 0; j < k; ++j) {
        S += p[idx[j]];
        dot += (double)c->gw[t * k + j] * p[idx[j]];
    }
    for (int j = 0; j < k; ++j) {
        double g = (double)c->gw[t * k + j];
        /* w_j = scale q_j / S (renorm) or scale q_j */
        double dq = c->renorm ? c->scale * (g / S - dot / (S * S)) : c->scale * g;
        dscore[idx[j]] += dq; /* gather: repeated indices add up */
    }
    if (c->scoring == 0) {
        /* softmax Jacobian: dl_e = p_e (ds_e - sum_f p_f ds_f) */
        double m = 0.0;
        for (int64_t e = 0; e < E; ++e) m += (double)p[e] * dscore[e];
        for (int64_t e = 0; e < E; ++e) store_elem(c->dl, c->dt, t * E + e, (double)p[e] * (dscore[e] - m));
    } else {
        for (int64_t e = 0; e < E; ++e) {
            double s = p[e];
            store_elem(c->dl, c->dt, t * E + e, dscore[e] * s * (1.0 - s));
        }
    }
    free(dscore);
    free(p);
}

int oracle_router_weights(const void* logits, int dt, const int64_t* idx, int64_t T, int64_t E, int k,
                          int scoring, int renorm, float scale, float* w, int nthreads)
{
    if (T < 0 || E < 1 || k < 1 || k > 64 || k > E || (scoring != 0 && scoring != 1)) return -1;
    if (!(scale > 0.0f) || isinf(scale)) return -1; /* a finite, positive scale */
    rweights_ctx c = {logits, dt, idx, NULL, E, k, scoring, renorm, scale, w, NULL};
    parallel_rows(T, nthreads, rweights_one, &c);
    return 0;
}

int oracle_router_backward(const void* logits, int dt, const int64_t* idx, const float* gw, int64_t T,
                           int64_t E, int k, int scoring, int renorm, float scale, void* dl, int nthreads)
{
    if (T < 0 || E < 1 || k < 1 || k > 64 || k > E || (scoring != 0 && scoring != 1)) return -1;
    if (!(scale > 0.0f) || isinf(scale)) return -1;
    rweights_ctx c = {logits, dt, idx, gw, E, k, scoring, renorm, scale, NULL, dl};
    parallel_rows(T, nthreads, rbackward_one, &c);
    return 0;
}

/* combine backward: for out[t] = sum_j w_j Y[row_j]:
 *   dY[row_j] = w_j g_t (rounded to the expert dtype), dw_j = <Y[row_j], g_t>
 * (double, rounded to FP32).  A token with a slot outside [0, N) -- NaN in
 * the forward -- gets NaN weight gradients; its valid rows still get w g. */
typedef struct {
    const void* Y;
    int dt;
    const uint32_t* ros;
    const void* w;
    int wdt;
    const void* gout;
    int k;
    int64_t H, N;
    void* dY;
    float* dw;
} cback_ctx;

static void cback_one(void* vctx, int64_t t)
{
    cback_ctx* c = (cback_ctx*)vctx;
    const int k = c->k;
    const int64_t H = c->H;
    int invalid = 0;
    for (int j = 0; j < k; ++j)
        if ((int64_t)c->ros[t * k + j] >= c->N) invalid = 1;
    for (int j = 0; j < k; ++j) {
        const int64_t row = c->ros[t * k + j];
        double dot = 0.0;
        if (row < c->N) {
            const double wj = load_elem(c->w, c->wdt, t * k + j);
            for (int64_t col = 0; col < H; ++col) {
                const double g = load_elem(c->gout, c->dt, t * H + col);
                store_elem(c->dY, c->dt, row * H + col, wj * g);
                dot += load_elem(c->Y, c->dt, row * H + col) * g;
            }
        }
        c->dw[t * k + j] = invalid ? NAN : (float)dot;
    }
}

int oracle_combine_backward(const void* Y, int dt, const uint32_t* ros, const void* w, int wdt, const void* gout,
                            int64_t T, int k, int64_t H, int64_t N, void* dY, float* dw, int nthreads)
{
    if (T < 0 || k < 1 || H < 0 || N < 0) return -1;
    cback_ctx c = {Y, dt, ros, w, wdt, gout, k, H, N, dY, dw};
    parallel_rows(T, nthreads, cback_one, &c);
    return 0;
}

/* dispatch backward: dx[t] = sum_j dinput[row_j] (double, slot order,
 * rounded once); the routing weights are not applied again.  A token with a
 * slot outside [0, N) gets a NaN row. */
typedef struct {
    const void* din;
    int dt;
    const uint32_t* ros;
    int k;
    int64_t H, N;
    void* dx;
} dback_ctx;

static void dback_one(void* vctx, int64_t t)
{
    dback_ctx* c = (dback_ctx*)vctx;
    int invalid = 0;
    for (int j = 0; j < c->k; ++j)
        if ((int64_t)c->ros[t * c->k + j] >= c->N) invalid = 1;
    for (int64_t col = 0; col < c->H; ++col) {
        double acc = 0.0;
        if (invalid) {
            acc = NAN;
        } else {
            for (int j = 0; j < c->k; ++j) acc += load_elem(c->din, c->dt, (int64_t)c->ros[t * c->k + j] * c->H + col);
        }
        store_elem(c->dx, c->dt, t * c->H + col, acc);
    }
}

int oracle_dispatch_backward(const void* din, int dt, const uint32_t* ros, int64_t T, int k, int64_t H, int64_t N,
                             void* dx, int nthreads)
{
    if (T < 0 || k < 1 || H < 0 || N < 0) return -1;
    dback_ctx c = {din, dt, ros, k, H, N, dx};
    parallel_rows(T, nthreads, dback_one, &c);
    return 0;
}

/* Expert training forward and backward.  For row r of expert e:
 *   g = gate_e x, u = up_e x            (the saved pre-activations, FP32)
 *   h = silu(g) u  in the weight dtype  (as in the inference forward)
 *   y = down_e h
 * backward from dy:
 *   dh = down_e^T dy
 *   du = dh silu(g),  dg = dh u silu'(g),  silu'(g) = s (1 + g (1 - s)),
 *        s = 1/(1+exp(-g)); both rounded to the weight dtype
 *   dx = gate_e^T dg + up_e^T du        (rounded to the weight dtype)
 *   dgate_e += dg x^T, dup_e += du x^T, ddown_e += dy h^T   (FP32)
 * Sums in double, each result rounded once. */
static double round_dt(double v, int dt)
{
    switch (dt) {
    case O_F32: return oracle_round_f32(v);
    case O_F16: return oracle_round_f16(v);
    default: return oracle_round_bf16(v);
    }
}

typedef struct {
    const void* const* gate;
    const void* const* up;
    const void* const* down;
    int dt;
    const void* rows;
    const uint32_t* offsets;
    int64_t E, H, I;
    void* out;   /* [N,H] */
    void* h;     /* [N,I] weight dtype */
    float* g;    /* [N,I] */
    float* u;    /* [N,I] */
    int* bad;
} tfwd_ctx;

static void tfwd_row(void* vctx, int64_t r)
{
    tfwd_ctx* c = (tfwd_ctx*)vctx;
    const int64_t e = expert_of_row(c->offsets, c->E, r);
    const int64_t H = c->H, I = c->I;
    if (e < 0 || !c->gate[e] || !c->up[e] || !c->down[e]) {
        *c->bad = 1;
        return;
    }
    double* x = (double*)malloc(sizeof(double) * (size_t)H);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    for (int64_t j = 0; j < H; ++j) x[j] = load_elem(c->rows, c->dt, r * H + j);
    for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            g += x[j] * load_elem(c->gate[e], c->dt, i * H + j);
            u += x[j] * load_elem(c->up[e], c->dt, i * H + j);
        }
        c->g[r * I + i] = (float)g;
        c->u[r * I + i] = (float)u;
        h[i] = round_dt(oracle_silu(g) * u, c->dt);
        store_elem(c->h, c->dt, r * I + i, h[i]);
    }
    for (int64_t j = 0; j < H; ++j) {
        double y = 0.0;
        for (int64_t i = 0; i < I; ++i) y += h[i] * load_elem(c->down[e], c->dt, j * I + i);
        store_elem(c->out, c->dt, r * H + j, y);
    }
    free(h);
    free(x);
}

int oracle_experts_train_forward(const void* const* gate, const void* const* up, const void* const* down, int dt,
                                 const void* rows, const uint32_t* offsets, int64_t E, int64_t H, int64_t I,
                                 void* out, void* h, float* g, float* u, int nthreads)
{
    if (E < 1 || H < 1 || I < 1) return -1;
    int bad = 0;
    tfwd_ctx c = {gate, up, down, dt, rows, offsets, E, H, I, out, h, g, u, &bad};
    parallel_rows((int64_t)offsets[E], nthreads, tfwd_row, &c);
    return bad ? -1 : 0;
}

typedef struct {
    const void* const* gate;
    const void* const* up;
    const void* const* down;
    int dt;
    const void* rows;
    const uint32_t* offsets;
    int64_t E, H, I;
    const float* g;
    const float* u;
    const void* dy;   /* [N,H] */
    void* dx;         /* [N,H] */
    double* dg;       /* [N,I] scratch: the rounded dg */
    double* du;       /* [N,I] scratch */
    int* bad;
} tbwd_ctx;

static void tbwd_row(void* vctx, int64_t r)
{
    tbwd_ctx* c = (tbwd_ctx*)vctx;
    const int64_t e = expert_of_row(c->offsets, c->E, r);
    const int64_t H = c->H, I = c->I;
    if (e < 0 || !c->gate[e] || !c->up[e] || !c->down[e]) {
        *c->bad = 1;
        return;
    }
    for (int64_t i = 0; i < I; ++i) {
        double dh = 0.0;
        for (int64_t j = 0; j < H; ++j)
            dh += load_elem(c->dy, c->dt, r * H + j) * load_elem(c->down[e], c->dt, j * I + i);
        const double g = c->g[r * I + i], u = c->u[r * I + i];
        const double s = 1.0 / (1.0 + exp(-g));
        c->du[r * I + i] = round_dt(dh * g * s, c->dt);
        c->dg[r * I + i] = round_dt(dh * u * s * (1.0 + g * (1.0 - s)), c->dt);
    }
    for (int64_t j = 0; j < H; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i)
            acc += c->dg[r * I + i] * load_elem(c->gate[e], c->dt, i * H + j) +
                   c->du[r * I + i] * load_elem(c->up[e], c->dt, i * H + j);
        store_elem(c->dx, c->dt, r * H + j, acc);
    }
}

typedef struct {
    tbwd_ctx* b;
    const void* h;
    float* dgate; /* [E,I,H] */
    float* dup;
    float* ddown; /* [E,H,I] */
} twgrad_ctx;

/* one expert's weight gradients, summed over its rows in ascending order */
static void twgrad_expert(void* vctx, int64_t e)
{
    twgrad_ctx* c = (twgrad_ctx*)vctx;
    const tbwd_ctx* b = c->b;
    const int64_t H = b->H, I = b->I;
    const int64_t r0 = b->offsets[e], r1 = b->offsets[e + 1] > r0 ? b->offsets[e + 1] : r0;
    for (int64_t i = 0; i < I; ++i) {
        for (int64_t j = 0; j < H; ++j) {
            double sg = 0.0, su = 0.0;
            for (int64_t r = r0; r < r1; ++r) {
                const double x = load_elem(b->rows, b->dt, r * H + j);
                sg += b->dg[r * I + i] * x;
                su += b->du[r * I + i] * x;
            }
            c->dgate[(e * I + i) * H + j] = (float)sg;
            c->dup[(e * I + i) * H + j] = (float)su;
        }
    }
    for (int64_t j = 0; j < H; ++j) {
        for (int64_t i = 0; i < I; ++i) {
            double sd = 0.0;
            for (int64_t r = r0; r < r1; ++r)
                sd += load_elem(b->dy, b->dt, r * H + j) * load_elem(c->h, b->dt, r * I + i);
            c->ddown[(e * H + j) * I + i] = (float)sd;
        }
    }
}

/* dgu_out: NULL, or [N,2I] doubles that receive the rounded dg | du. */
int oracle_experts_backward(const void* const* gate, const void* const* up, const void* const* down, int dt,
                            const void* rows, const uint32_t* offsets, int64_t E, int64_t H, int64_t I,
                            const float* g, const float* u, const void* h, const void* dy, void* dx,
                            float* dgate, float* dup, float* ddown, double* dgu_out, int nthreads)
{
    if (E < 1 || H < 1 || I < 1) return -1;
    const int64_t N = offsets[E];
    int bad = 0;
    double* dg = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N * I : 1));
    double* du = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N * I : 1));
    tbwd_ctx b = {gate, up, down, dt, rows, offsets, E, H, I, g, u, dy, dx, dg, du, &bad};
    parallel_rows(N, nthreads, tbwd_row, &b);
    if (!bad) {
        twgrad_ctx w = {&b, h, dgate, dup, ddown};
        parallel_rows(E, nthreads, twgrad_expert, &w);
    }
    if (!bad && dgu_out) {
        for (int64_t r = 0; r < N; ++r)
            for (int64_t i = 0; i < I; ++i) {
                dgu_out[r * 2 * I + i] = dg[r * I + i];
                dgu_out[r * 2 * I + I + i] = du[r * I + i];
            }
    }
    free(du);
    free(dg);
    return bad ? -1 : 0;
}
