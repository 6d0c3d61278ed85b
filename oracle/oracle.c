/*
 * ORACLE -- test infrastructure only. Plain, slow, double-precision CPU
 * attention used to check the HIP library. Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the library never calls it and
 * shares no code with it.
 *
 * What it computes is the plain definition of exact softmax attention
 * ("Attention" glossary page, section on Query/Key/Value: each query is dotted
 * with every key, the scores are normalised by a softmax, and the values are
 * averaged with those weights; the Tree Attention explainer, section 2, stresses
 * that the tree method is exact, not an approximation, so the oracle is that
 * definition written out). The softmax subtracts the row maximum before
 * exponentiating, the stability step the Grayskull explainer names in its
 * section 3. Everything is evaluated in double precision from the exact values
 * the GPU reads (fp32, bf16 bit patterns, or fp8-e4m3 codes times their fp32
 * per-head scale), decoded here from the format definitions.
 *
 * Readings where the pages are silent (all pages give no formula):
 *  - score scale sigma is an argument (1/sqrt(d) by default in the callers);
 *  - grouped KV heads: query head h reads KV head floor(h / (Hq/Hkv));
 *  - causal mask is aligned bottom-right: with n keys and Lq queries, query i
 *    sits at absolute position n - Lq + i and sees keys j <= n - Lq + i;
 *  - a row that sees no key returns O = 0 and lse = -inf.
 *
 * The partial / merge / combine / energy functions restate the Tree Attention
 * explainer's section 3 (attention written as the gradient of a scalar energy
 * function, evaluated by an associative reduction along the sequence axis):
 *  partial over a key set J: (o = sum_J e^{s_j - m} v_j, m = max_J s_j,
 *                             l = sum_J e^{s_j - m});
 *  merge(a, b): m = max(m_a, m_b), o = e^{m_a-m} o_a + e^{m_b-m} o_b,
 *               l = e^{m_a-m} l_a + e^{m_b-m} l_b; identity (0, -inf, 0);
 *  finalise: O = o / l, lse = m + ln l;
 *  energy F(zeta) = ln sum_J exp(s_j + zeta . v_j), so F(0) = lse and the
 *  gradient of F at 0 is O.
 *
 * The backward pass (oracle_backward) differentiates the same definition: for
 * a loss with gradient dO on the outputs, with z_ij = sigma q_i . k_j and P the
 * softmax of each row over its visible keys,
 *  dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   D_i = sum_j P_ij dP_ij,
 *  dz_ij = P_ij (dP_ij - D_i),   dQ_i = sigma sum_j dz_ij k_j,
 *  dK_j = sigma sum_i dz_ij q_i   (sums over every query head sharing the KV
 *  head). It is pinned against finite differences of the forward.
 *
 * A cache kept in two precisions (the ThriftAttention page: its introduction
 * gives each token or head a precision, its Physical AI Stack section keeps
 * the first and last tenth of the tokens in bf16) is, for one query, plain
 * attention over the union of the two key sets at their real values: the
 * Python side decodes both spans with oracle_decode_elems, multiplies the fp8
 * span by its scale in double, concatenates them, and calls oracle_attention
 * with OR_F64 keys and values. The low-precision span may also be FP4 (the
 * page names a 4-bit float with a 2-bit exponent): stored as OCP MX FP4, whose
 * elements are E2M1 codes and whose every 32 consecutive elements of a row
 * share a power-of-two E8M0 scale (OCP Microscaling Formats (MX) v1.0); it is
 * decoded exactly by oracle_mxfp4_decode.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_E4M3 2
#define OR_F64 3 /* already-decoded values, e.g. the union of two cache spans */

/* bf16: the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, 4);
    return (double)f;
}

/* OCP FP8 E4M3 (e4m3fn): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * exponent field 0: subnormal, value m/8 * 2^(1-7); exponent 15 with mantissa 7
 * is NaN (there is no infinity); otherwise (1 + m/8) * 2^(e-7). */
double oracle_e4m3_to_f64(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, 1 - 7);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* E2M1 (the MX FP4 element): 1 sign, 2 exponent (bias 1), 1 mantissa bit.
 * Exponent field 0: subnormal, value m * 2^-1; otherwise (1 + m/2) * 2^(e-1).
 * No infinities or NaN. */
double oracle_e2m1_to_f64(uint8_t code) {
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double v = e ? ldexp(1.0 + (double)m / 2.0, e - 1) : ldexp((double)m, -1);
    return s ? -v : v;
}

/* E8M0 (the MX shared scale): 2^(E - 127); E = 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t e) {
    if (e == 255) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* Real values of `rows` rows of d MX FP4 elements: codes [rows][d/2] (element
 * 2i in the low nibble of byte i, element 2i + 1 in the high nibble), scales
 * [rows][d/32] (one per 32 consecutive elements); dst [rows][d]. */
void oracle_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int d, double* dst) {
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < d; ++c) {
            const uint8_t byte = codes[r * (d / 2) + c / 2];
            const uint8_t code = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
            dst[r * d + c] = oracle_e2m1_to_f64(code) * oracle_e8m0_to_f64(scales[r * (d / 32) + c / 32]);
        }
}

typedef struct {
    const void* q;
    int q_dtype;
    const void* k;
    const void* v;
    int kv_dtype;
    const float* k_scale;
    const float* v_scale;
    const int32_t* kv_lens;
    int B, Hq, Hkv, Lq, Lcap, d;
    double scale;
    int causal;
    /* pi-Attention mask (pi_mask != 0): window, period, prior (see below) */
    int pi_mask;
    int window, period;
    const float* alpha;
} problem;

static double elem(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
    case OR_E4M3: return oracle_e4m3_to_f64(((const uint8_t*)base)[idx]);
    case OR_F64: return ((const double*)base)[idx];
    default: return NAN;
    }
}

/* The real values of n stored elements (no scale applied). */
void oracle_decode_elems(const void* src, int dtype, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = elem(src, dtype, i);
}

/* Decoded key or value row j of (b, g), multiplied by its fp8 scale if any. */
static void load_kv_row(const problem* p, const void* base, const float* scales, int b, int g, int64_t j,
                        double* dst) {
    int64_t off = (((int64_t)b * p->Hkv + g) * p->Lcap + j) * p->d;
    double sc = scales ? (double)scales[(int64_t)b * p->Hkv + g] : 1.0;
    for (int c = 0; c < p->d; ++c) dst[c] = elem(base, p->kv_dtype, off + c) * sc;
}

static int64_t seq_len(const problem* p, int b) {
    int64_t n = p->kv_lens ? (int64_t)p->kv_lens[b] : (int64_t)p->Lcap;
    if (n < 0) n = 0;
    if (n > p->Lcap) n = p->Lcap;
    return n;
}

/* Keys visible to query i of sequence b: [0, hi). */
static int64_t visible_end(const problem* p, int b, int i) {
    int64_t n = seq_len(p, b);
    if (!p->causal) return n;
    int64_t hi = n - p->Lq + i + 1;
    if (hi < 0) hi = 0;
    if (hi > n) hi = n;
    return hi;
}

static void load_q_row(const problem* p, int b, int h, int i, double* dst) {
    int64_t off = (((int64_t)b * p->Hq + h) * p->Lq + i) * p->d;
    for (int c = 0; c < p->d; ++c) dst[c] = elem(p->q, p->q_dtype, off + c);
}

static double score(const problem* p, const double* q, const double* krow) {
    double acc = 0.0;
    for (int c = 0; c < p->d; ++c) acc += q[c] * krow[c];
    return p->scale * acc;
}

/* One output row by the definition: scores, max, weights, weighted mean. */
static void attend_row(const problem* p, int b, int h, int i, double* s, double* tmp, double* qd, double* out,
                       double* lse) {
    int g = h / (p->Hq / p->Hkv);
    int64_t hi = visible_end(p, b, i);
    for (int c = 0; c < p->d; ++c) out[c] = 0.0;
    if (hi <= 0) {
        *lse = -INFINITY;
        return;
    }
    load_q_row(p, b, h, i, qd);
    double mx = -INFINITY;
    for (int64_t j = 0; j < hi; ++j) {
        load_kv_row(p, p->k, p->k_scale, b, g, j, tmp);
        s[j] = score(p, qd, tmp);
        if (s[j] > mx) mx = s[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < hi; ++j) {
        double w = exp(s[j] - mx);
        z += w;
        load_kv_row(p, p->v, p->v_scale, b, g, j, tmp);
        for (int c = 0; c < p->d; ++c) out[c] += w * tmp[c];
    }
    for (int c = 0; c < p->d; ++c) out[c] /= z;
    *lse = mx + log(z);
}

/*
 * pi-Attention's key set and log-prior for row (b, h, i) (the pi-Attention
 * explainer, method section A: a ring-local neighbourhood of k tokens on either
 * side, skip links to tokens a whole number of periods pi away -- past only
 * when causal -- and an adaptive gate alpha that enters the one softmax as a
 * log-prior). The query sits at pos = n - Lq + i. Key j is
 *   local  if |pos - j| <= window (and j <= pos when causal),
 *   skip   if not local, period > 0, (pos - j) is a multiple of period
 *          (and j < pos when causal),
 *   absent otherwise.
 * With alpha (clamped to [0, 1], one per row [B, Hq, Lq]) the logits of local
 * keys get + ln(alpha) and those of skip keys + ln(1 - alpha); without it no
 * prior is added. Returns 0 (absent), 1 (local) or 2 (skip).
 */
static int pi_class(const problem* p, int64_t pos, int64_t j) {
    int64_t dist = pos - j;
    if (p->causal && dist < 0) return 0;
    if ((dist < 0 ? -dist : dist) <= p->window) return 1;
    if (p->period > 0 && dist % p->period == 0) return 2;
    return 0;
}

static void attend_row_pi(const problem* p, int b, int h, int i, double* s, double* tmp, double* qd, double* out,
                          double* lse) {
    int g = h / (p->Hq / p->Hkv);
    int64_t n = seq_len(p, b), pos = n - p->Lq + i;
    double bias_local = 0.0, bias_skip = 0.0;
    if (p->alpha) {
        double a = (double)p->alpha[((int64_t)b * p->Hq + h) * p->Lq + i];
        if (!(a >= 0.0)) a = 0.0; /* NaN or negative */
        if (a > 1.0) a = 1.0;
        bias_local = log(a);
        bias_skip = log(1.0 - a);
    }
    for (int c = 0; c < p->d; ++c) out[c] = 0.0;
    load_q_row(p, b, h, i, qd);
    double mx = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        int cls = pi_class(p, pos, j);
        if (!cls) {
            s[j] = -INFINITY;
            continue;
        }
        load_kv_row(p, p->k, p->k_scale, b, g, j, tmp);
        s[j] = score(p, qd, tmp) + (cls == 1 ? bias_local : bias_skip);
        if (s[j] > mx) mx = s[j];
    }
    if (mx == -INFINITY) { /* no key, or every key weighted zero by the prior */
        *lse = -INFINITY;
        return;
    }
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        if (s[j] == -INFINITY) continue;
        double w = exp(s[j] - mx);
        z += w;
        load_kv_row(p, p->v, p->v_scale, b, g, j, tmp);
        for (int c = 0; c < p->d; ++c) out[c] += w * tmp[c];
    }
    for (int c = 0; c < p->d; ++c) out[c] /= z;
    *lse = mx + log(z);
}

typedef struct {
    const problem* p;
    const int64_t* rows;
    int64_t nrows;
    int tid, nthreads;
    double* out;
    double* lse;
} row_job;

static void* row_worker(void* arg) {
    row_job* j = (row_job*)arg;
    const problem* p = j->p;
    double* s = (double*)malloc(sizeof(double) * (size_t)(p->Lcap > 0 ? p->Lcap : 1));
    double* tmp = (double*)malloc(sizeof(double) * (size_t)p->d);
    double* qd = (double*)malloc(sizeof(double) * (size_t)p->d);
    for (int64_t r = j->tid; r < j->nrows; r += j->nthreads) {
        int64_t flat = j->rows ? j->rows[r] : r;
        int i = (int)(flat % p->Lq);
        int h = (int)((flat / p->Lq) % p->Hq);
        int b = (int)(flat / ((int64_t)p->Lq * p->Hq));
        if (p->pi_mask) attend_row_pi(p, b, h, i, s, tmp, qd, j->out + r * p->d, j->lse + r);
        else attend_row(p, b, h, i, s, tmp, qd, j->out + r * p->d, j->lse + r);
    }
    free(s);
    free(tmp);
    free(qd);
    return NULL;
}

static int check_problem(const problem* p) {
    if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Lq <= 0 || p->Lcap < 0 || p->d <= 0) return 1;
    if (p->Hq % p->Hkv) return 1;
    if (p->kv_dtype == OR_E4M3 && (!p->k_scale || !p->v_scale)) return 1;
    return 0;
}

static int run_rows(const problem* pp, const int64_t* rows, int64_t nrows, double* out, double* lse, int nthreads);

/*
 * Exact attention for the listed rows (flat row id r = (b*Hq + h)*Lq + i), or for
 * every row when rows == NULL. Layouts are contiguous: q [B,Hq,Lq,d],
 * k/v [B,Hkv,Lcap,d], fp8 scales [B*Hkv], kv_lens [B] (NULL = all Lcap).
 * out [nrows, d] and lse [nrows] are double. Returns 0, or 1 on a bad argument.
 */
int oracle_attention(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                     const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv,
                     int Lq, int Lcap, int d, double scale, int causal, const int64_t* rows, int64_t nrows,
                     double* out, double* lse, int nthreads) {
    problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, kv_lens, B, Hq, Hkv, Lq, Lcap, d, scale, causal};
    return run_rows(&p, rows, nrows, out, lse, nthreads);
}

/*
 * pi-Attention (see pi_class above) for the listed rows, or every row when
 * rows == NULL; arguments as oracle_attention plus window >= 0, period >= 0
 * (0: no skip links) and alpha (float [B, Hq, Lq] or NULL).
 */
int oracle_pi_attention(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                        const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv,
                        int Lq, int Lcap, int d, double scale, int causal, int window, int period,
                        const float* alpha, const int64_t* rows, int64_t nrows, double* out, double* lse,
                        int nthreads) {
    problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, kv_lens, B, Hq, Hkv, Lq, Lcap, d, scale, causal,
                 1, window, period, alpha};
    if (window < 0 || period < 0) return 1;
    return run_rows(&p, rows, nrows, out, lse, nthreads);
}

static int run_rows(const problem* pp, const int64_t* rows, int64_t nrows, double* out, double* lse, int nthreads) {
    problem p = *pp;
    if (check_problem(&p)) return 1;
    if (!rows) nrows = (int64_t)p.B * p.Hq * p.Lq;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
    pthread_t th[256];
    row_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (row_job){&p, rows, nrows, t, nthreads, out, lse};
        pthread_create(&th[t], NULL, row_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

typedef struct {
    const problem* p;
    const void* dout;
    int g0, ng; /* the (b, g) groups this thread owns: flat ids g0, g0 + ng, ... */
    double *dq, *dk, *dv;
} bwd_job;

static void* bwd_worker(void* arg) {
    bwd_job* j = (bwd_job*)arg;
    const problem* p = j->p;
    const int G = p->Hq / p->Hkv, d = p->d;
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* dod = (double*)malloc(sizeof(double) * (size_t)d);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
    double* P = (double*)malloc(sizeof(double) * (size_t)(p->Lcap > 0 ? p->Lcap : 1));
    double* dP = (double*)malloc(sizeof(double) * (size_t)(p->Lcap > 0 ? p->Lcap : 1));
    for (int flat = j->g0; flat < p->B * p->Hkv; flat += j->ng) {
        const int b = flat / p->Hkv, g = flat % p->Hkv;
        for (int h = g * G; h < (g + 1) * G; ++h) {
            for (int i = 0; i < p->Lq; ++i) {
                const int64_t hi = visible_end(p, b, i);
                double* dqi = j->dq + (((int64_t)b * p->Hq + h) * p->Lq + i) * d;
                for (int c = 0; c < d; ++c) dqi[c] = 0.0;
                if (hi <= 0) continue;
                load_q_row(p, b, h, i, qd);
                const int64_t off = (((int64_t)b * p->Hq + h) * p->Lq + i) * d;
                for (int c = 0; c < d; ++c) dod[c] = elem(j->dout, p->q_dtype, off + c);
                /* P: the softmax of the row, by the definition */
                double mx = -INFINITY;
                for (int64_t jj = 0; jj < hi; ++jj) {
                    load_kv_row(p, p->k, p->k_scale, b, g, jj, tmp);
                    P[jj] = score(p, qd, tmp);
                    if (P[jj] > mx) mx = P[jj];
                }
                double z = 0.0;
                for (int64_t jj = 0; jj < hi; ++jj) {
                    P[jj] = exp(P[jj] - mx);
                    z += P[jj];
                }
                double D = 0.0;
                for (int64_t jj = 0; jj < hi; ++jj) {
                    P[jj] /= z;
                    load_kv_row(p, p->v, p->v_scale, b, g, jj, tmp);
                    double acc = 0.0;
                    for (int c = 0; c < d; ++c) acc += dod[c] * tmp[c];
                    dP[jj] = acc;
                    D += P[jj] * acc;
                }
                for (int64_t jj = 0; jj < hi; ++jj) {
                    const double dz = P[jj] * (dP[jj] - D);
                    double* dkj = j->dk + (((int64_t)b * p->Hkv + g) * p->Lcap + jj) * d;
                    double* dvj = j->dv + (((int64_t)b * p->Hkv + g) * p->Lcap + jj) * d;
                    load_kv_row(p, p->k, p->k_scale, b, g, jj, tmp);
                    for (int c = 0; c < d; ++c) {
                        dqi[c] += p->scale * dz * tmp[c];
                        dkj[c] += p->scale * dz * qd[c];
                        dvj[c] += P[jj] * dod[c];
                    }
                }
            }
        }
    }
    free(qd);
    free(dod);
    free(tmp);
    free(P);
    free(dP);
    return NULL;
}

/*
 * Gradients of exact attention: given dout [B,Hq,Lq,d] (the q dtype), writes
 * dq [B,Hq,Lq,d], dk and dv [B,Hkv,Lcap,d] (double, zero for keys no query
 * sees). Arguments otherwise as oracle_attention. Returns 0, or 1 on a bad
 * argument.
 */
int oracle_backward(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, const float* k_scale,
                    const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int Lq, int Lcap, int d,
                    double scale, int causal, const void* dout, double* dq, double* dk, double* dv, int nthreads) {
    problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, kv_lens, B, Hq, Hkv, Lq, Lcap, d, scale, causal};
    if (check_problem(&p) || !dout) return 1;
    const int64_t nkv = (int64_t)B * Hkv * Lcap * d;
    for (int64_t x = 0; x < nkv; ++x) dk[x] = dv[x] = 0.0;
    const int groups = B * Hkv;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > groups) nthreads = groups;
    pthread_t th[256];
    bwd_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (bwd_job){&p, dout, t, nthreads, dq, dk, dv};
        pthread_create(&th[t], NULL, bwd_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/*
 * The same gradients for chosen rows and keys only, for problems too large for
 * oracle_backward: dq of the listed query rows and dk, dv of the listed keys,
 * each by the formulas above. A key's gradients sum over every query row of
 * its KV head's query heads that sees it, so for each (b, g) that owns a
 * listed key the softmax statistics of all those rows come first: the row
 * maximum M_i, Z_i = sum_j exp(s_ij - M_i) and D_i = sum_j P_ij dP_ij over
 * the row's visible keys. Then P_ij = exp(s_ij - M_i) / Z_i and
 * dz_ij = P_ij (dP_ij - D_i) as before.
 */
typedef struct {
    const problem* p;
    const void* dout;
    const int64_t* items; /* query rows or keys, flat ids */
    int64_t n;
    int tid, nthreads;
    /* key mode: the (b, g) being processed and its decoded operands */
    int b, g;
    const double *kd, *vd, *qg, *dog, *M, *Z, *D;
    double *out0, *out1;
} sub_job;

static double dot(const double* a, const double* b, int d) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += a[c] * b[c];
    return acc;
}

/* dq of listed rows (b*Hq + h)*Lq + i: one row at a time, by the definition. */
static void* sub_dq_worker(void* arg) {
    sub_job* j = (sub_job*)arg;
    const problem* p = j->p;
    const int d = p->d;
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* dod = (double*)malloc(sizeof(double) * (size_t)d);
    double* kr = (double*)malloc(sizeof(double) * (size_t)d);
    double* vr = (double*)malloc(sizeof(double) * (size_t)d);
    double* P = (double*)malloc(sizeof(double) * (size_t)(p->Lcap > 0 ? p->Lcap : 1));
    double* dP = (double*)malloc(sizeof(double) * (size_t)(p->Lcap > 0 ? p->Lcap : 1));
    for (int64_t r = j->tid; r < j->n; r += j->nthreads) {
        const int64_t flat = j->items[r];
        const int i = (int)(flat % p->Lq), h = (int)((flat / p->Lq) % p->Hq);
        const int b = (int)(flat / ((int64_t)p->Lq * p->Hq)), g = h / (p->Hq / p->Hkv);
        double* dqi = j->out0 + r * d;
        for (int c = 0; c < d; ++c) dqi[c] = 0.0;
        const int64_t hi = visible_end(p, b, i);
        if (hi <= 0) continue;
        load_q_row(p, b, h, i, qd);
        for (int c = 0; c < d; ++c) dod[c] = elem(j->dout, p->q_dtype, flat * d + c);
        double mx = -INFINITY;
        for (int64_t jj = 0; jj < hi; ++jj) {
            load_kv_row(p, p->k, p->k_scale, b, g, jj, kr);
            P[jj] = score(p, qd, kr);
            if (P[jj] > mx) mx = P[jj];
        }
        double z = 0.0;
        for (int64_t jj = 0; jj < hi; ++jj) {
            P[jj] = exp(P[jj] - mx);
            z += P[jj];
        }
        double D = 0.0;
        for (int64_t jj = 0; jj < hi; ++jj) {
            P[jj] /= z;
            load_kv_row(p, p->v, p->v_scale, b, g, jj, vr);
            dP[jj] = dot(dod, vr, d);
            D += P[jj] * dP[jj];
        }
        for (int64_t jj = 0; jj < hi; ++jj) {
            const double dz = P[jj] * (dP[jj] - D);
            load_kv_row(p, p->k, p->k_scale, b, g, jj, kr);
            for (int c = 0; c < d; ++c) dqi[c] += p->scale * dz * kr[c];
        }
    }
    free(qd);
    free(dod);
    free(kr);
    free(vr);
    free(P);
    free(dP);
    return NULL;
}

/* Statistics M, Z, D of the rows of (b, g): row index hl*Lq + i for the
 * group's local query head hl. */
static void* sub_stats_worker(void* arg) {
    sub_job* j = (sub_job*)arg;
    const problem* p = j->p;
    const int d = p->d, G = p->Hq / p->Hkv;
    double* s = (double*)malloc(sizeof(double) * (size_t)(p->Lcap > 0 ? p->Lcap : 1));
    double* M = (double*)j->M;
    double* Z = (double*)j->Z;
    double* D = (double*)j->D;
    for (int64_t r = j->tid; r < (int64_t)G * p->Lq; r += j->nthreads) {
        const int i = (int)(r % p->Lq);
        const double* qd = j->qg + r * d;
        const double* dod = j->dog + r * d;
        const int64_t hi = visible_end(p, j->b, i);
        double mx = -INFINITY;
        for (int64_t jj = 0; jj < hi; ++jj) {
            s[jj] = p->scale * dot(qd, j->kd + jj * d, d);
            if (s[jj] > mx) mx = s[jj];
        }
        double z = 0.0;
        for (int64_t jj = 0; jj < hi; ++jj) z += exp(s[jj] - mx);
        double dd = 0.0;
        for (int64_t jj = 0; jj < hi; ++jj) dd += exp(s[jj] - mx) / z * dot(dod, j->vd + jj * d, d);
        M[r] = mx;
        Z[r] = z;
        D[r] = dd;
    }
    free(s);
    return NULL;
}

/* dk, dv of the listed keys that belong to (b, g). */
static void* sub_key_worker(void* arg) {
    sub_job* j = (sub_job*)arg;
    const problem* p = j->p;
    const int d = p->d, G = p->Hq / p->Hkv;
    int64_t mine = 0;
    for (int64_t r = 0; r < j->n; ++r) {
        const int64_t flat = j->items[r];
        const int64_t jj = flat % p->Lcap;
        if (flat / p->Lcap != (int64_t)j->b * p->Hkv + j->g) continue;
        if (mine++ % j->nthreads != j->tid) continue;
        double* dkj = j->out0 + r * d;
        double* dvj = j->out1 + r * d;
        for (int c = 0; c < d; ++c) dkj[c] = dvj[c] = 0.0;
        const double* kr = j->kd + jj * d;
        const double* vr = j->vd + jj * d;
        for (int hl = 0; hl < G; ++hl) {
            for (int i = 0; i < p->Lq; ++i) {
                if (jj >= visible_end(p, j->b, i)) continue;
                const int64_t row = (int64_t)hl * p->Lq + i;
                const double* qd = j->qg + row * d;
                const double* dod = j->dog + row * d;
                const double P = exp(p->scale * dot(qd, kr, d) - j->M[row]) / j->Z[row];
                const double dz = P * (dot(dod, vr, d) - j->D[row]);
                for (int c = 0; c < d; ++c) {
                    dkj[c] += p->scale * dz * qd[c];
                    dvj[c] += P * dod[c];
                }
            }
        }
    }
    return NULL;
}

static void run_sub(void* (*fn)(void*), sub_job* proto, int nthreads) {
    pthread_t th[256];
    sub_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].tid = t;
        jobs[t].nthreads = nthreads;
        pthread_create(&th[t], NULL, fn, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/*
 * Arguments as oracle_backward, plus: q_rows [nq] flat query rows
 * (b*Hq + h)*Lq + i with dq [nq, d]; keys [nk] flat keys (b*Hkv + g)*Lcap + j
 * with dk, dv [nk, d] (zero for a key no query sees). Returns 0, or 1 on a
 * bad argument (including an id out of range).
 */
int oracle_backward_subset(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                           const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B, int Hq,
                           int Hkv, int Lq, int Lcap, int d, double scale, int causal, const void* dout,
                           const int64_t* q_rows, int64_t nq, const int64_t* keys, int64_t nk, double* dq,
                           double* dk, double* dv, int nthreads) {
    problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, kv_lens, B, Hq, Hkv, Lq, Lcap, d, scale, causal};
    if (check_problem(&p) || !dout || nq < 0 || nk < 0) return 1;
    for (int64_t r = 0; r < nq; ++r)
        if (q_rows[r] < 0 || q_rows[r] >= (int64_t)B * Hq * Lq) return 1;
    for (int64_t r = 0; r < nk; ++r)
        if (keys[r] < 0 || keys[r] >= (int64_t)B * Hkv * Lcap) return 1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    sub_job job;
    memset(&job, 0, sizeof(job));
    job.p = &p;
    job.dout = dout;
    if (nq > 0) {
        job.items = q_rows;
        job.n = nq;
        job.out0 = dq;
        run_sub(sub_dq_worker, &job, nthreads);
    }
    if (nk == 0) return 0;
    const int G = Hq / Hkv;
    double* kd = (double*)malloc(sizeof(double) * (size_t)Lcap * d + 8);
    double* vd = (double*)malloc(sizeof(double) * (size_t)Lcap * d + 8);
    double* qg = (double*)malloc(sizeof(double) * (size_t)G * Lq * d);
    double* dog = (double*)malloc(sizeof(double) * (size_t)G * Lq * d);
    double* M = (double*)malloc(sizeof(double) * (size_t)G * Lq);
    double* Z = (double*)malloc(sizeof(double) * (size_t)G * Lq);
    double* D = (double*)malloc(sizeof(double) * (size_t)G * Lq);
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            int used = 0;
            for (int64_t r = 0; r < nk && !used; ++r) used = keys[r] / Lcap == (int64_t)b * Hkv + g;
            if (!used) continue;
            for (int64_t jj = 0; jj < Lcap; ++jj) {
                load_kv_row(&p, k, k_scale, b, g, jj, kd + jj * d);
                load_kv_row(&p, v, v_scale, b, g, jj, vd + jj * d);
            }
            for (int hl = 0; hl < G; ++hl)
                for (int i = 0; i < Lq; ++i) {
                    const int64_t row = (int64_t)hl * Lq + i;
                    const int64_t off = (((int64_t)b * Hq + g * G + hl) * Lq + i) * d;
                    load_q_row(&p, b, g * G + hl, i, qg + row * d);
                    for (int c = 0; c < d; ++c) dog[row * d + c] = elem(dout, q_dtype, off + c);
                }
            job.b = b;
            job.g = g;
            job.kd = kd;
            job.vd = vd;
            job.qg = qg;
            job.dog = dog;
            job.M = M;
            job.Z = Z;
            job.D = D;
            run_sub(sub_stats_worker, &job, nthreads);
            job.items = keys;
            job.n = nk;
            job.out0 = dk;
            job.out1 = dv;
            run_sub(sub_key_worker, &job, nthreads);
        }
    }
    free(kd);
    free(vd);
    free(qg);
    free(dog);
    free(M);
    free(Z);
    free(D);
    return 0;
}

/* Partial (o, m, l) of row (b, h, i) over keys [j0, j1) intersected with the
 * keys the row may see. An empty set gives the identity (0, -inf, 0). */
int oracle_partial(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, const float* k_scale,
                   const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int Lq, int Lcap, int d,
                   double scale, int causal, int b, int h, int i, int64_t j0, int64_t j1, double* o, double* m,
                   double* l) {
    problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, kv_lens, B, Hq, Hkv, Lq, Lcap, d, scale, causal};
    if (check_problem(&p)) return 1;
    int g = h / (Hq / Hkv);
    int64_t hi = visible_end(&p, b, i);
    if (j1 > hi) j1 = hi;
    if (j0 < 0) j0 = 0;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    *m = -INFINITY;
    *l = 0.0;
    if (j1 <= j0) return 0;
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
    double* s = (double*)malloc(sizeof(double) * (size_t)(j1 - j0));
    load_q_row(&p, b, h, i, qd);
    double mx = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        load_kv_row(&p, k, k_scale, b, g, j, tmp);
        s[j - j0] = score(&p, qd, tmp);
        if (s[j - j0] > mx) mx = s[j - j0];
    }
    double z = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        double w = exp(s[j - j0] - mx);
        z += w;
        load_kv_row(&p, v, v_scale, b, g, j, tmp);
        for (int c = 0; c < d; ++c) o[c] += w * tmp[c];
    }
    *m = mx;
    *l = z;
    free(qd);
    free(tmp);
    free(s);
    return 0;
}

/* Associative merge of two partials (the reduction step of the tree). */
void oracle_merge(const double* oa, double ma, double la, const double* ob, double mb, double lb, int d, double* o,
                  double* m, double* l) {
    double mm = ma > mb ? ma : mb;
    if (mm == -INFINITY) {
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        *m = -INFINITY;
        *l = 0.0;
        return;
    }
    double a = exp(ma - mm), bb = exp(mb - mm);
    for (int c = 0; c < d; ++c) o[c] = a * oa[c] + bb * ob[c];
    *m = mm;
    *l = a * la + bb * lb;
}

void oracle_finalize(const double* o, double m, double l, int d, double* out, double* lse) {
    if (l <= 0.0 || m == -INFINITY) {
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    for (int c = 0; c < d; ++c) out[c] = o[c] / l;
    *lse = m + log(l);
}

/*
 * Combine S fp32 partials per row into the normalised output, by the plain
 * definition of the merged result: m = max_s m_s, w_s = e^{m_s - m},
 * O = sum_s w_s o_s / sum_s w_s l_s, lse = m + ln sum_s w_s l_s.
 * o_part [R,S,d], m_part/l_part [R,S]; count [R] (NULL = S) limits the partials
 * read per row. out [R,d], lse [R] double.
 */
int oracle_combine(const float* o_part, const float* m_part, const float* l_part, int R, int S, int d,
                   const int32_t* count, double* out, double* lse) {
    if (R < 0 || S < 0 || d <= 0) return 1;
    for (int64_t r = 0; r < R; ++r) {
        int n = count ? count[r] : S;
        if (n > S) n = S;
        double mx = -INFINITY;
        for (int s = 0; s < n; ++s) {
            double ms = (double)m_part[r * S + s];
            if (ms > mx) mx = ms;
        }
        double* o = out + r * d;
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (int s = 0; s < n; ++s) {
            double ms = (double)m_part[r * S + s];
            if (ms == -INFINITY) continue;
            double w = exp(ms - mx);
            z += w * (double)l_part[r * S + s];
            for (int c = 0; c < d; ++c) o[c] += w * (double)o_part[((int64_t)r * S + s) * d + c];
        }
        if (z <= 0.0) {
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        for (int c = 0; c < d; ++c) o[c] /= z;
        lse[r] = mx + log(z);
    }
    return 0;
}

/* Energy of row (b, h, i) at zeta: F = ln sum_{visible j} exp(s_j + zeta . v_j). */
double oracle_energy(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, const float* k_scale,
                     const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int Lq, int Lcap, int d,
                     double scale, int causal, int b, int h, int i, const double* zeta) {
    problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, kv_lens, B, Hq, Hkv, Lq, Lcap, d, scale, causal};
    if (check_problem(&p)) return NAN;
    int g = h / (Hq / Hkv);
    int64_t hi = visible_end(&p, b, i);
    if (hi <= 0) return -INFINITY;
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
    double* e = (double*)malloc(sizeof(double) * (size_t)hi);
    load_q_row(&p, b, h, i, qd);
    double mx = -INFINITY;
    for (int64_t j = 0; j < hi; ++j) {
        load_kv_row(&p, k, k_scale, b, g, j, tmp);
        double sj = score(&p, qd, tmp);
        load_kv_row(&p, v, v_scale, b, g, j, tmp);
        double zv = 0.0;
        for (int c = 0; c < d; ++c) zv += zeta[c] * tmp[c];
        e[j] = sj + zv;
        if (e[j] > mx) mx = e[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < hi; ++j) z += exp(e[j] - mx);
    free(qd);
    free(tmp);
    free(e);
    return mx + log(z);
}
