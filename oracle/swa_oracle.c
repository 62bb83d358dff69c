/*
 * fp64 CPU oracle for causal sliding-window softmax attention with attention
 * sinks.  TEST INFRASTRUCTURE ONLY: this file is built into liboracle.so and
 * is called by the tests, by the smoke check and by the CPU-baseline leg of
 * the benchmark.  The product library never links it, and it shares no code
 * with the HIP path.
 *
 * What it computes, per query row, follows the pages directly:
 *
 *  - Key set.  Query t sees the first s tokens (the attention sinks) plus its
 *    r most recent tokens including itself, each key once:
 *        U(t) = { i <= t : i < s  or  i >= t - r + 1 }.
 *    Sources: "带 Sink 的滑动窗口注意力" section of the hyper.ai summary of
 *    arXiv 2608.28444 (the SWA sum over i = max(1, t-w+1) .. t, and the
 *    always-visible first s = 4 tokens next to the window); the
 *    eq:attn-fixed-streaming cache composition (sinks KV[0:k] plus recent
 *    KV[t-m:t]) on the t6page "滑窗与固定稀疏" page.
 *    With a dilation delta >= 1 the window keeps r keys but takes every
 *    delta-th position, t, t - delta, ..., t - (r-1) delta (the glossary
 *    entry on dilated SWA and the Longformer section of that page: attended
 *    positions skip delta - 1 tokens, same count, wider reach); the sinks
 *    are unchanged and a key in both sets counts once.  delta = 1 is U(t).
 *
 *    With task-bound global tokens (a sorted list G of positions; the
 *    Longformer section and the glossary entry on global tokens of that
 *    page: a few tokens visible to the whole sequence, and seeing all of it),
 *    in causal form: a row t in G attends every key <= t; any other row
 *    attends U(t) plus the global positions g <= t, each key once.
 *
 *  - Scores and normalisation.  x_i = (q_t . k_i) / sqrt(d) (here: times the
 *    caller's scale), then softmax over U(t) and the weighted sum of values:
 *    eq:attn-fixed-softmax-sink on the t6page page, eq.(1) of section 2.1 of
 *    the Blurry Window Attention page (arXiv 2606.09862).  The largest score
 *    is subtracted before exp only to keep fp64 in range; it cancels exactly.
 *
 *  - RoPE re-positioning (only when rope_base > 0).  The keys of U(t), taken
 *    in temporal order, sit at cache positions 0 .. |U(t)|-1 and the query at
 *    the position of its own key, |U(t)|-1; keys are stored before rotation
 *    and rotated at those positions for every query (the StreamingLLM
 *    paragraph after eq:attn-fixed-streaming on the t6page page).  The
 *    rotation pairs dimension j with j + d/2 and turns the pair by angle
 *    p * base^(-2j/d): the pages do not fix the pairing; this is the Llama
 *    convention, the model family those pages evaluate.
 *
 * All arithmetic is fp64; inputs are the float32 values the device receives.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

/* Whether position t is in the sorted list G (ng entries). */
static int is_global(int64_t t, const int64_t* G, int64_t ng) {
    for (int64_t j = 0; j < ng; ++j)
        if (G[j] == t) return 1;
    return 0;
}

/* Number of keys in U(t) and the list itself, in increasing (temporal)
 * order: the sinks, then (with global tokens) the global positions between
 * the sinks and the window, then the window.  A global row takes 0 .. t.
 * Global tokens are defined for the plain window (dil = 1). */
static int64_t key_set(int64_t t, int64_t s, int64_t r, int64_t dil, const int64_t* G, int64_t ng, int64_t* keys) {
    int64_t n = 0;
    if (ng > 0 && is_global(t, G, ng)) {
        for (int64_t j = 0; j <= t; ++j) keys[n++] = j;
        return n;
    }
    int64_t ns = s < t + 1 ? s : t + 1;
    for (int64_t j = 0; j < ns; ++j) keys[n++] = j;
    /* global positions >= s and before the window (those in the window or
       among the sinks are already in the set) */
    int64_t win_lo = t - r + 1 > s ? t - r + 1 : s;
    for (int64_t j = 0; j < ng; ++j)
        if (G[j] >= s && G[j] < win_lo && G[j] <= t) keys[n++] = G[j];
    /* window positions t - dil*m, m = r-1 .. 0 (increasing), those >= s */
    for (int64_t m = r - 1; m >= 0; --m) {
        int64_t i = t - dil * m;
        if (i >= s && i >= 0) keys[n++] = i;
    }
    return n;
}

/* G must be strictly increasing, positions >= 0. */
static int globals_ok(const int64_t* G, int64_t ng) {
    if (ng < 0 || (ng > 0 && !G)) return 0;
    for (int64_t j = 0; j < ng; ++j)
        if (G[j] < 0 || (j > 0 && G[j] <= G[j - 1])) return 0;
    return 1;
}

/* Rotation angles.  Position p turns pair j by p * theta_j with
 * theta_j = base^(-2j/d).  cos/sin are tabulated for the positions a call can
 * use (0 .. s+r-1); each entry is computed exactly as the formula states. */
typedef struct { int64_t npos, half; double* c; double* s; } rope_table;

static int rope_table_init(rope_table* T, int64_t npos, int64_t d, double base) {
    T->npos = npos; T->half = d / 2;
    T->c = (double*)malloc(sizeof(double) * (size_t)(npos * T->half));
    T->s = (double*)malloc(sizeof(double) * (size_t)(npos * T->half));
    if (!T->c || !T->s) { free(T->c); free(T->s); T->c = T->s = NULL; return ORACLE_ENOMEM; }
    for (int64_t j = 0; j < T->half; ++j) {
        double theta = pow(base, -2.0 * (double)j / (double)d);
        for (int64_t p = 0; p < npos; ++p) {
            T->c[p * T->half + j] = cos((double)p * theta);
            T->s[p * T->half + j] = sin((double)p * theta);
        }
    }
    return ORACLE_OK;
}

static void rope_table_free(rope_table* T) { free(T->c); free(T->s); T->c = T->s = NULL; }

/* Rotate x (length d) to position p: pair (j, j + d/2). */
static void rope_rotate(const rope_table* T, const double* x, double* y, int64_t p) {
    int64_t h = T->half;
    const double* c = T->c + p * h;
    const double* sn = T->s + p * h;
    for (int64_t j = 0; j < h; ++j) {
        double x0 = x[j], x1 = x[j + h];
        y[j] = x0 * c[j] - x1 * sn[j];
        y[j + h] = x0 * sn[j] + x1 * c[j];
    }
}

/*
 * Attention rows of a prefill (or of any token history).
 *   q:  [B, Hq, Lq, d] float32, row i of q is the token at position qpos0 + i
 *   k, v: [B, Hkv, Lk, d] float32, row p is the token at position p
 *   rows: nrows triples (b, h, i); out: [nrows, d] fp64;
 *   nkeys (may be NULL): |U(t)| per row.
 * Requires qpos0 + i < Lk for every requested row, Hq % Hkv == 0, r >= 1,
 * s >= 0, d even when rope_base > 0.  The q-head h reads kv-head
 * h / (Hq / Hkv).
 */
int swa_oracle_rows(const float* q, const float* k, const float* v,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                    int64_t s, int64_t r, double scale, double rope_base, int64_t qpos0,
                    int64_t nrows, const int64_t* rows, double* out, int64_t* nkeys, int64_t dil,
                    const int64_t* G, int64_t ng) {
    if (!q || !k || !v || !rows || !out) return ORACLE_EINVAL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || d < 1 || r < 1 || s < 0 || qpos0 < 0 || dil < 1)
        return ORACLE_EINVAL;
    if (rope_base > 0 && (d % 2)) return ORACLE_EINVAL;
    if (!globals_ok(G, ng) || (ng > 0 && (rope_base > 0 || dil != 1))) return ORACLE_EINVAL;
    for (int64_t n = 0; n < nrows; ++n) {
        int64_t b = rows[3 * n], h = rows[3 * n + 1], i = rows[3 * n + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Lq || qpos0 + i >= Lk) return ORACLE_EINVAL;
    }
    int64_t group = Hq / Hkv;
    int64_t maxkeys = s + r + ng;
    if (ng > 0 && maxkeys < Lk) maxkeys = Lk;   /* a global row takes 0 .. t */
    int failed = 0;
    rope_table T = {0, 0, NULL, NULL};
    if (rope_base > 0 && rope_table_init(&T, maxkeys, d, rope_base) != ORACLE_OK) return ORACLE_ENOMEM;

#pragma omp parallel
    {
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)maxkeys);
        double* x = (double*)malloc(sizeof(double) * (size_t)maxkeys);
        double* qd = (double*)malloc(sizeof(double) * (size_t)d);
        double* qr = (double*)malloc(sizeof(double) * (size_t)d);
        double* kd = (double*)malloc(sizeof(double) * (size_t)d);
        double* kr = (double*)malloc(sizeof(double) * (size_t)d);
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        if (!keys || !x || !qd || !qr || !kd || !kr || !acc) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t n = 0; n < nrows; ++n) {
                int64_t b = rows[3 * n], h = rows[3 * n + 1], i = rows[3 * n + 2];
                int64_t kvh = h / group;
                int64_t t = qpos0 + i;
                const float* qrow = q + ((b * Hq + h) * Lq + i) * d;
                const float* kbase = k + (b * Hkv + kvh) * Lk * d;
                const float* vbase = v + (b * Hkv + kvh) * Lk * d;

                int64_t nk = key_set(t, s, r, dil, G, ng, keys);
                if (nkeys) nkeys[n] = nk;

                for (int64_t e = 0; e < d; ++e) qd[e] = (double)qrow[e];
                if (rope_base > 0) rope_rotate(&T, qd, qr, nk - 1);
                else memcpy(qr, qd, sizeof(double) * (size_t)d);

                double m = -INFINITY;
                for (int64_t j = 0; j < nk; ++j) {
                    const float* krow = kbase + keys[j] * d;
                    for (int64_t e = 0; e < d; ++e) kd[e] = (double)krow[e];
                    const double* kk = kd;
                    if (rope_base > 0) {
                        rope_rotate(&T, kd, kr, j);
                        kk = kr;
                    }
                    double dot = 0.0;
                    for (int64_t e = 0; e < d; ++e) dot += qr[e] * kk[e];
                    x[j] = dot * scale;
                    if (x[j] > m) m = x[j];
                }
                double l = 0.0;
                for (int64_t e = 0; e < d; ++e) acc[e] = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    double w = exp(x[j] - m);
                    l += w;
                    const float* vrow = vbase + keys[j] * d;
                    for (int64_t e = 0; e < d; ++e) acc[e] += w * (double)vrow[e];
                }
                double* o = out + n * d;
                for (int64_t e = 0; e < d; ++e) o[e] = acc[e] / l;
            }
        }
        free(keys); free(x); free(qd); free(qr); free(kd); free(kr); free(acc);
    }
    rope_table_free(&T);
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Softmax attention of one query over an explicit list of n key/value rows
 * (the decode step over the valid slots of a rolling cache).  Softmax over a
 * set does not depend on the order of its members, so the rows may be given
 * in slot order.  q: [d], kv rows: [n, d] float32, out: [d] fp64.
 */
int swa_oracle_attend_set(const float* q, const float* keys, const float* vals, int64_t n, int64_t d,
                          double scale, double* out) {
    if (!q || !keys || !vals || !out || n < 1 || d < 1) return ORACLE_EINVAL;
    double* x = (double*)malloc(sizeof(double) * (size_t)n);
    if (!x) return ORACLE_ENOMEM;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int64_t e = 0; e < d; ++e) dot += (double)q[e] * (double)keys[j * d + e];
        x[j] = dot * scale;
        if (x[j] > m) m = x[j];
    }
    double l = 0.0;
    for (int64_t e = 0; e < d; ++e) out[e] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(x[j] - m);
        l += w;
        for (int64_t e = 0; e < d; ++e) out[e] += w * (double)vals[j * d + e];
    }
    for (int64_t e = 0; e < d; ++e) out[e] /= l;
    free(x);
    return ORACLE_OK;
}

/* The rotation alone, exposed so tests can pin it to closed forms.  One
 * position, so the angles are formed directly (the same cos(p * theta_j) and
 * sin(p * theta_j) a table entry holds), for positions of any size. */
int swa_oracle_rope(const double* x, double* y, int64_t d, int64_t pos, double base) {
    if (!x || !y || d < 2 || (d % 2) || !(base > 0) || pos < 0) return ORACLE_EINVAL;
    int64_t h = d / 2;
    for (int64_t j = 0; j < h; ++j) {
        double theta = pow(base, -2.0 * (double)j / (double)d);
        double c = cos((double)pos * theta), sn = sin((double)pos * theta);
        double x0 = x[j], x1 = x[j + h];
        y[j] = x0 * c - x1 * sn;
        y[j + h] = x0 * sn + x1 * c;
    }
    return ORACLE_OK;
}

/* |U(t)| and the key list, exposed for the key-set pins; keys must hold
 * s + r + ng entries, or t + 1 if that is more. */
int64_t swa_oracle_key_set(int64_t t, int64_t s, int64_t r, int64_t dil, const int64_t* G, int64_t ng, int64_t* keys) {
    if (t < 0 || s < 0 || r < 1 || dil < 1 || !keys || !globals_ok(G, ng) || (ng > 0 && dil != 1))
        return ORACLE_EINVAL;
    return key_set(t, s, r, dil, G, ng, keys);
}

/* Threads the parallel loops use (the CPU-baseline leg reports it). */
int swa_oracle_threads(void) { return omp_get_max_threads(); }
