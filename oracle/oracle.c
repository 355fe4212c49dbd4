/*
 * oracle.c -- plain, slow fp64 CPU reference of the HypeNet RNN mixer (Lightning Attention).
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists so that tests, the smoke check and the
 * benchmark's CPU-baseline leg can check the GPU library against an independent definition.
 * The GPU library never includes, links, loads or calls anything in this directory, and this
 * file uses nothing from the GPU library.
 *
 * What it follows (all from "Hybrid Linear Attention Done Right: Efficient Distillation and
 * Effective Architectures for Extremely Long Contexts", arXiv 2601.22156):
 *   - Appendix A, Eq. 18 (RNN layer):  q = Norm(x W_q), k = Norm(x W_k), v = x W_v,
 *     q~ = RoPE_t(q), k~ = RoPE_t(k) / sqrt(d_h), S_t = S_{t-1} gamma + k~^T v,
 *     o_t = q~ S_t, y_t = Norm(o_t) (.) sigmoid(x W_z)   (the W_o product is outside the mixer).
 *   - Appendix A, Eq. 15 text: Norm is RMSNorm.
 *   - Appendix A, Eq. 19: the per-head forget gate gamma_h (here an input, lambda[h]).
 *   - Section 5.2, Eq. 12 (QK-normalization) and Eq. 14 (normalised, gated output).
 * The inputs are the projections x W_q, x W_k, x W_v and the gate logits x W_z, one d-vector per
 * (batch, token, head), laid out [B][T][H][d].
 *
 * Readings where the pages leave a step open (each is also listed with the design notes):
 *   - RMSNorm(x) = x / sqrt(mean(x^2) + eps) (.) w, over the d entries of one head.
 *   - RoPE uses half-split pairs (i, i + d/2) with inv_freq_i = base^(-2i/d) and the whole
 *     head dimension rotated; positions are 0-based absolute positions p = pos0 + t.
 *   - The state is S[a][c] with a indexing the key dimension and c the value dimension,
 *     S_t = lambda S_{t-1} + k~^T v (update first), then o = q~ S_t (token t sees itself).
 *   - 0^0 := 1, so lambda = 0 gives o_t = (q~_t . k~_t) v_t.
 *
 * Three evaluation orders are provided.  They are written separately and are compared with each
 * other and with closed forms by the tests:
 *   oracle_prefill_slices : the token-by-token recurrence (the definition).
 *   oracle_chunked_slices : the chunkwise form (intra-chunk decayed scores, inter-chunk carry).
 *   oracle_decode_step    : one recurrence step per (b, h) at an arbitrary position.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* ---- element access ---------------------------------------------------------------------- */

/* Widen one stored element to fp64.  bf16 is the upper half of an IEEE fp32 word, so the
 * widening is exact. */
static double load_elem(const void* base, int dtype, size_t i) {
    if (dtype == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[i];
}

/* ---- the per-vector steps ---------------------------------------------------------------- */

/* RMSNorm over n entries: out_i = x_i / sqrt(mean(x^2) + eps) * w_i  (w == NULL means ones). */
void oracle_rmsnorm(const double* x, const double* w, int n, double eps, double* out) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i) out[i] = x[i] * inv * (w ? w[i] : 1.0);
}

/* Rotary embedding at absolute position pos: the pair (x_i, x_{i+n/2}) is rotated by the angle
 * pos * base^(-2i/n), for i = 0 .. n/2-1. */
void oracle_rope(const double* x, int n, double pos, double base, double* out) {
    int half = n / 2;
    for (int i = 0; i < half; ++i) {
        double theta = pos * pow(base, -2.0 * i / n);
        double c = cos(theta), s = sin(theta);
        double x1 = x[i], x2 = x[i + half];
        out[i] = x1 * c - x2 * s;
        out[i + half] = x2 * c + x1 * s;
    }
}

double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* ---- shared argument block --------------------------------------------------------------- */

typedef struct {
    const void *q, *k, *v, *g;
    int dtype;
    const float *qw, *kw, *ow; /* [H][d] or shared [d] (stride 0); ow may be NULL */
    int w_stride;              /* elements between heads in qw/kw/ow: d, or 0 for shared */
    const double* lambda;      /* [H] */
    double rope_base, eps;
    int64_t pos0;
    const float* state_in; /* [B][H][d][d] or NULL (zeros) */
    int B, T, H, d;
    int chunk; /* chunked form only */
    const int *b_idx, *h_idx;
    int n_slices;
    double *y_out, *o_out, *s_out; /* [n][T][d], [n][T][d] (or NULL), [n][d][d] (or NULL) */
} PrefillArgs;

/* Prologue of one token: RMSNorm + RoPE of q and k, key scaled by 1/sqrt(d); v and g widened. */
static void token_prologue(const PrefillArgs* a, int b, int h, int t, double* qt, double* kt,
                           double* vt, double* gt, double* tmp, double* wq, double* wk) {
    int d = a->d;
    size_t row = (((size_t)b * a->T + t) * a->H + h) * (size_t)d;
    for (int i = 0; i < d; ++i) tmp[i] = load_elem(a->q, a->dtype, row + i);
    oracle_rmsnorm(tmp, wq, d, a->eps, tmp);
    oracle_rope(tmp, d, (double)(a->pos0 + t), a->rope_base, qt);
    for (int i = 0; i < d; ++i) tmp[i] = load_elem(a->k, a->dtype, row + i);
    oracle_rmsnorm(tmp, wk, d, a->eps, tmp);
    oracle_rope(tmp, d, (double)(a->pos0 + t), a->rope_base, kt);
    double ks = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) kt[i] *= ks;
    for (int i = 0; i < d; ++i) vt[i] = load_elem(a->v, a->dtype, row + i);
    for (int i = 0; i < d; ++i) gt[i] = load_elem(a->g, a->dtype, row + i);
}

static void head_weights(const PrefillArgs* a, int h, double* wq, double* wk, double* wo) {
    size_t off = (size_t)h * a->w_stride;
    for (int i = 0; i < a->d; ++i) {
        wq[i] = a->qw[off + i];
        wk[i] = a->kw[off + i];
        wo[i] = a->ow ? a->ow[off + i] : 1.0;
    }
}

/* Output epilogue: y = RMSNorm(o) * w_o * sigmoid(g). */
static void token_epilogue(int d, double eps, const double* o, const double* g, const double* wo,
                           double* y) {
    oracle_rmsnorm(o, wo, d, eps, y);
    for (int i = 0; i < d; ++i) y[i] *= oracle_sigmoid(g[i]);
}

/* ---- the recurrence (the definition) ----------------------------------------------------- */

static void recurrence_slice(const PrefillArgs* a, int slot) {
    int b = a->b_idx[slot], h = a->h_idx[slot], d = a->d, T = a->T;
    double lam = a->lambda[h];
    double* S = calloc((size_t)d * d, sizeof(double));
    double* buf = malloc(sizeof(double) * 10 * (size_t)d);
    double *qt = buf, *kt = buf + d, *vt = buf + 2 * d, *gt = buf + 3 * d, *tmp = buf + 4 * d;
    double *o = buf + 5 * d, *wq = buf + 6 * d, *wk = buf + 7 * d, *wo = buf + 8 * d;
    double* y = buf + 9 * d;
    head_weights(a, h, wq, wk, wo);
    if (a->state_in) {
        const float* s0 = a->state_in + ((size_t)b * a->H + h) * (size_t)d * d;
        for (size_t i = 0; i < (size_t)d * d; ++i) S[i] = s0[i];
    }
    for (int t = 0; t < T; ++t) {
        token_prologue(a, b, h, t, qt, kt, vt, gt, tmp, wq, wk);
        /* update: S <- lambda S + k~^T v */
        for (int r = 0; r < d; ++r)
            for (int c = 0; c < d; ++c) S[(size_t)r * d + c] = lam * S[(size_t)r * d + c] + kt[r] * vt[c];
        /* query: o = q~ S */
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int r = 0; r < d; ++r) acc += qt[r] * S[(size_t)r * d + c];
            o[c] = acc;
        }
        token_epilogue(d, a->eps, o, gt, wo, y);
        size_t out = ((size_t)slot * T + t) * (size_t)d;
        for (int c = 0; c < d; ++c) a->y_out[out + c] = y[c];
        if (a->o_out)
            for (int c = 0; c < d; ++c) a->o_out[out + c] = o[c];
    }
    if (a->s_out) memcpy(a->s_out + (size_t)slot * d * d, S, sizeof(double) * (size_t)d * d);
    free(buf);
    free(S);
}

/* ---- the chunkwise form ------------------------------------------------------------------ */

/* Chunk of n tokens starting at t0, entering with state S (state after token t0-1):
 *   o_i = lambda^(i+1) q~_i S + sum_{j<=i} lambda^(i-j) (q~_i . k~_j) v_j
 *   S  <- lambda^n S + sum_j lambda^(n-1-j) k~_j^T v_j
 * pow(0, 0) is 1 in C, which is the 0^0 := 1 reading. */
static void chunked_slice(const PrefillArgs* a, int slot) {
    int b = a->b_idx[slot], h = a->h_idx[slot], d = a->d, T = a->T, C = a->chunk;
    double lam = a->lambda[h];
    double* S = calloc((size_t)d * d, sizeof(double));
    double* Q = malloc(sizeof(double) * (size_t)C * d);
    double* K = malloc(sizeof(double) * (size_t)C * d);
    double* V = malloc(sizeof(double) * (size_t)C * d);
    double* G = malloc(sizeof(double) * (size_t)C * d);
    double* buf = malloc(sizeof(double) * 6 * (size_t)d);
    double *tmp = buf, *o = buf + d, *wq = buf + 2 * d, *wk = buf + 3 * d, *wo = buf + 4 * d;
    double* y = buf + 5 * d;
    head_weights(a, h, wq, wk, wo);
    if (a->state_in) {
        const float* s0 = a->state_in + ((size_t)b * a->H + h) * (size_t)d * d;
        for (size_t i = 0; i < (size_t)d * d; ++i) S[i] = s0[i];
    }
    for (int t0 = 0; t0 < T; t0 += C) {
        int n = (T - t0 < C) ? T - t0 : C;
        for (int i = 0; i < n; ++i)
            token_prologue(a, b, h, t0 + i, Q + (size_t)i * d, K + (size_t)i * d, V + (size_t)i * d,
                           G + (size_t)i * d, tmp, wq, wk);
        for (int i = 0; i < n; ++i) {
            const double* qi = Q + (size_t)i * d;
            double carry = pow(lam, i + 1);
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int r = 0; r < d; ++r) acc += qi[r] * S[(size_t)r * d + c];
                o[c] = carry * acc;
            }
            for (int j = 0; j <= i; ++j) {
                const double* kj = K + (size_t)j * d;
                double score = 0.0;
                for (int r = 0; r < d; ++r) score += qi[r] * kj[r];
                score *= pow(lam, i - j);
                for (int c = 0; c < d; ++c) o[c] += score * V[(size_t)j * d + c];
            }
            token_epilogue(d, a->eps, o, G + (size_t)i * d, wo, y);
            size_t out = ((size_t)slot * T + t0 + i) * (size_t)d;
            for (int c = 0; c < d; ++c) a->y_out[out + c] = y[c];
            if (a->o_out)
                for (int c = 0; c < d; ++c) a->o_out[out + c] = o[c];
        }
        double decay_all = pow(lam, n);
        for (size_t e = 0; e < (size_t)d * d; ++e) S[e] *= decay_all;
        for (int j = 0; j < n; ++j) {
            double w = pow(lam, n - 1 - j);
            for (int r = 0; r < d; ++r)
                for (int c = 0; c < d; ++c)
                    S[(size_t)r * d + c] += w * K[(size_t)j * d + r] * V[(size_t)j * d + c];
        }
    }
    if (a->s_out) memcpy(a->s_out + (size_t)slot * d * d, S, sizeof(double) * (size_t)d * d);
    free(buf);
    free(G);
    free(V);
    free(K);
    free(Q);
    free(S);
}

/* ---- thread pool over independent (b, h) slices ------------------------------------------ */

typedef struct {
    const PrefillArgs* a;
    void (*fn)(const PrefillArgs*, int);
    int first, step;
} Worker;

static void* worker_main(void* p) {
    Worker* w = (Worker*)p;
    for (int s = w->first; s < w->a->n_slices; s += w->step) w->fn(w->a, s);
    return NULL;
}

static int run_slices(const PrefillArgs* a, void (*fn)(const PrefillArgs*, int), int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > a->n_slices) nthreads = a->n_slices;
    pthread_t* th = malloc(sizeof(pthread_t) * (size_t)nthreads);
    Worker* ws = malloc(sizeof(Worker) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        ws[i].a = a;
        ws[i].fn = fn;
        ws[i].first = i;
        ws[i].step = nthreads;
        if (pthread_create(&th[i], NULL, worker_main, &ws[i]) != 0) break;
        ++started;
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    int ok = (started == nthreads);
    if (!ok) /* finish the unstarted strides serially */
        for (int i = started; i < nthreads; ++i) worker_main(&ws[i]);
    free(ws);
    free(th);
    return nthreads;
}

static int check_common(int B, int T, int H, int d, int dtype, int n, const int* b_idx,
                        const int* h_idx) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || (d & 1) || n <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    for (int i = 0; i < n; ++i)
        if (b_idx[i] < 0 || b_idx[i] >= B || h_idx[i] < 0 || h_idx[i] >= H) return -1;
    return 0;
}

/* Token-by-token recurrence for the listed (b, h) slices.  Returns the number of threads used,
 * or -1 on a bad argument. */
int oracle_prefill_slices(const void* q, const void* k, const void* v, const void* g, int dtype,
                          const float* qw, const float* kw, const float* ow, int w_stride,
                          const double* lambda, double rope_base, double eps, int64_t pos0,
                          const float* state_in, int B, int T, int H, int d, const int* b_idx,
                          const int* h_idx, int n_slices, double* y_out, double* o_out,
                          double* s_out, int nthreads) {
    if (check_common(B, T, H, d, dtype, n_slices, b_idx, h_idx)) return -1;
    PrefillArgs a = {q, k, v, g, dtype, qw, kw, ow, w_stride, lambda, rope_base, eps, pos0,
                     state_in, B, T, H, d, 0, b_idx, h_idx, n_slices, y_out, o_out, s_out};
    return run_slices(&a, recurrence_slice, nthreads);
}

/* Chunkwise form with chunk length `chunk` (any value >= 1), same outputs as above. */
int oracle_chunked_slices(const void* q, const void* k, const void* v, const void* g, int dtype,
                          const float* qw, const float* kw, const float* ow, int w_stride,
                          const double* lambda, double rope_base, double eps, int64_t pos0,
                          const float* state_in, int B, int T, int H, int d, int chunk,
                          const int* b_idx, const int* h_idx, int n_slices, double* y_out,
                          double* o_out, double* s_out, int nthreads) {
    if (check_common(B, T, H, d, dtype, n_slices, b_idx, h_idx) || chunk < 1) return -1;
    PrefillArgs a = {q, k, v, g, dtype, qw, kw, ow, w_stride, lambda, rope_base, eps, pos0,
                     state_in, B, T, H, d, chunk, b_idx, h_idx, n_slices, y_out, o_out, s_out};
    return run_slices(&a, chunked_slice, nthreads);
}

/* ---- one decode step --------------------------------------------------------------------- */

typedef struct {
    const void *q, *k, *v, *g;
    int dtype;
    const float *qw, *kw, *ow;
    int w_stride;
    const double* lambda;
    double rope_base, eps;
    const int64_t* positions; /* [B] */
    const float* state_in;    /* [B][H][d][d] */
    int B, H, d;
    double *y_out, *o_out, *s_out; /* [B][H][d], [B][H][d] or NULL, [B][H][d][d] */
} DecodeArgs;

static void decode_one(const DecodeArgs* a, int b, int h) {
    int d = a->d;
    /* A decode step is the recurrence run for one token at position positions[b]: reuse the
     * prefill prologue with T = 1 and pos0 = positions[b]. */
    PrefillArgs pa = {a->q, a->k, a->v, a->g, a->dtype, a->qw, a->kw, a->ow, a->w_stride,
                      a->lambda, a->rope_base, a->eps, a->positions[b], NULL, a->B, 1, a->H, d,
                      0, NULL, NULL, 0, NULL, NULL, NULL};
    double lam = a->lambda[h];
    double* buf = malloc(sizeof(double) * 10 * (size_t)d);
    double *qt = buf, *kt = buf + d, *vt = buf + 2 * d, *gt = buf + 3 * d, *tmp = buf + 4 * d;
    double *o = buf + 5 * d, *wq = buf + 6 * d, *wk = buf + 7 * d, *wo = buf + 8 * d;
    double* y = buf + 9 * d;
    head_weights(&pa, h, wq, wk, wo);
    token_prologue(&pa, b, h, 0, qt, kt, vt, gt, tmp, wq, wk);
    size_t sb = ((size_t)b * a->H + h) * (size_t)d * d;
    double* S = a->s_out + sb;
    for (int r = 0; r < d; ++r)
        for (int c = 0; c < d; ++c)
            S[(size_t)r * d + c] = lam * (double)a->state_in[sb + (size_t)r * d + c] + kt[r] * vt[c];
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int r = 0; r < d; ++r) acc += qt[r] * S[(size_t)r * d + c];
        o[c] = acc;
    }
    token_epilogue(d, a->eps, o, gt, wo, y);
    size_t ob = ((size_t)b * a->H + h) * (size_t)d;
    for (int c = 0; c < d; ++c) a->y_out[ob + c] = y[c];
    if (a->o_out)
        for (int c = 0; c < d; ++c) a->o_out[ob + c] = o[c];
    free(buf);
}

typedef struct {
    const DecodeArgs* a;
    int first, step;
} DecodeWorker;

static void* decode_worker(void* p) {
    DecodeWorker* w = (DecodeWorker*)p;
    int n = w->a->B * w->a->H;
    for (int s = w->first; s < n; s += w->step) decode_one(w->a, s / w->a->H, s % w->a->H);
    return NULL;
}

/* One recurrence step for every (b, h) at position positions[b].  The q/k/v/g layout is
 * [B][H][d]; the incoming state is fp32 [B][H][d][d]; outputs are fp64. */
int oracle_decode_step(const void* q, const void* k, const void* v, const void* g, int dtype,
                       const float* qw, const float* kw, const float* ow, int w_stride,
                       const double* lambda, double rope_base, double eps,
                       const int64_t* positions, const float* state_in, int B, int H, int d,
                       double* y_out, double* o_out, double* s_out, int nthreads) {
    if (B <= 0 || H <= 0 || d <= 0 || (d & 1)) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    DecodeArgs a = {q, k, v, g, dtype, qw, kw, ow, w_stride, lambda, rope_base, eps,
                    positions, state_in, B, H, d, y_out, o_out, s_out};
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B * H) nthreads = B * H;
    pthread_t* th = malloc(sizeof(pthread_t) * (size_t)nthreads);
    DecodeWorker* ws = malloc(sizeof(DecodeWorker) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        ws[i].a = &a;
        ws[i].first = i;
        ws[i].step = nthreads;
        if (pthread_create(&th[i], NULL, decode_worker, &ws[i]) != 0) break;
        ++started;
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    for (int i = started; i < nthreads; ++i) decode_worker(&ws[i]);
    free(ws);
    free(th);
    return nthreads;
}
