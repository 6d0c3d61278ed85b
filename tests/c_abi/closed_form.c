/*
 * A plain C99 caller of libattn.so: device memory from the HIP runtime, every
 * call through include/attn.h, results checked against closed forms that
 * need no reference implementation:
 *
 *  - all keys zero: every visible key scores 0, so the softmax weights are
 *    uniform and O is the mean of the visible values, lse = ln(count) (the
 *    softmax of equal scores, glossary page "Attention", Query/Key/Value
 *    section);
 *  - one visible key: O is that key's value exactly;
 *  - no visible key: O = 0, lse = -inf;
 *  - partials whose o is (weight) * w: the log-sum-exp merge returns w for any
 *    weights, and lse = M + ln(sum e^(m_s - M) l_s) (the reduction along the
 *    sequence axis, Tree Attention explainer, section 3).
 *
 * The values are multiples of 1/8 in [-1, 1], exact in fp32 and bf16, so
 * with unit weights every sum the kernels form is exact and only the final
 * division (and the bf16 rounding of the output) can differ from the
 * closed form. Also checked: argument errors return their codes before any
 * launch, and two identical calls give bit-identical results.
 *
 * Exit status 0 when every check passes; each check prints one line.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attn.h"

static int g_fail = 0;

#define HIP_OK(x)                                                                     \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

static void check(int ok, const char* what) {
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) g_fail = 1;
}

static uint16_t to_bf16(float x) { /* exact for the values used here */
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

static float val(int b, int g, int j, int c) { return (float)((j * 7 + c * 3 + g * 11 + b * 5) % 17 - 8) / 8.0f; }

static void* dev_copy(const void* host, size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    if (bytes) HIP_OK(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
    return p;
}

static attn_tensor view(void* data, int dtype, int H, int L, int d) {
    attn_tensor t;
    t.data = data;
    t.dtype = dtype;
    t.stride_s = d;
    t.stride_h = (int64_t)L * d;
    t.stride_b = (int64_t)H * L * d;
    return t;
}

/* Decode with all-zero keys over ragged lengths {L, 1234, 1, 0}: O = mean of
 * the first L_b values, lse = ln(L_b); L_b = 1 gives the first value exactly,
 * L_b = 0 gives O = 0 and lse = -inf. */
static void decode_uniform(int bf16, int num_splits) {
    const int B = 4, Hq = 8, Hkv = 2, G = Hq / Hkv, d = 128, L = 3000;
    const int32_t lens[4] = {L, 1234, 1, 0};
    const size_t nq = (size_t)B * Hq * d, nkv = (size_t)B * Hkv * L * d;
    const size_t esz = bf16 ? 2 : 4;
    void* hq = malloc(nq * esz);
    void* hk = calloc(nkv, esz);
    void* hv = malloc(nkv * esz);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h)
            for (int c = 0; c < d; ++c) {
                const float x = (float)((b * 3 + h * 5 + c) % 9 - 4) / 4.0f;
                const size_t i = ((size_t)b * Hq + h) * d + c;
                if (bf16) ((uint16_t*)hq)[i] = to_bf16(x);
                else ((float*)hq)[i] = x;
            }
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g)
            for (int j = 0; j < L; ++j)
                for (int c = 0; c < d; ++c) {
                    const size_t i = (((size_t)b * Hkv + g) * L + j) * d + c;
                    if (bf16) ((uint16_t*)hv)[i] = to_bf16(val(b, g, j, c));
                    else ((float*)hv)[i] = val(b, g, j, c);
                }
    const int dt = bf16 ? ATTN_BF16 : ATTN_F32;
    void *dq = dev_copy(hq, nq * esz), *dk = dev_copy(hk, nkv * esz), *dv = dev_copy(hv, nkv * esz);
    void* dlens = dev_copy(lens, sizeof(lens));
    void* dout = NULL;
    float* dlse = NULL;
    HIP_OK(hipMalloc(&dout, nq * esz));
    HIP_OK(hipMalloc((void**)&dlse, (size_t)B * Hq * 4));
    int S = num_splits ? num_splits : attn_decode_auto_splits(B, Hkv, L, dt, 1);
    const size_t ws_bytes = attn_decode_workspace_size(B, Hq, d, S);
    void* ws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    check(attn_decode_workspace_init(ws, ws_bytes, NULL) == ATTN_OK, "workspace init");
    attn_tensor tq = view(dq, dt, Hq, 1, d), tk = view(dk, dt, Hkv, L, d), tv = view(dv, dt, Hkv, L, d);
    attn_tensor to = view(dout, dt, Hq, 1, d);
    attn_status st = attn_decode(&tq, &tk, &tv, NULL, NULL, (const int32_t*)dlens, B, Hq, Hkv, d, L, 0.0f, 1,
                                 num_splits, &to, dlse, ws, ws_bytes, NULL);
    HIP_OK(hipDeviceSynchronize());
    char what[160];
    snprintf(what, sizeof what, "attn_decode %s splits %d returns ATTN_OK (%s)", bf16 ? "bf16" : "fp32", num_splits,
             attn_status_string(st));
    check(st == ATTN_OK, what);
    void* ho = malloc(nq * esz);
    float* hl = (float*)malloc((size_t)B * Hq * 4);
    HIP_OK(hipMemcpy(ho, dout, nq * esz, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, dlse, (size_t)B * Hq * 4, hipMemcpyDeviceToHost));
    double worst = 0.0, worst_lse = 0.0;
    int special_ok = 1;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G, n = lens[b];
            const float l = hl[b * Hq + h];
            if (n == 0) special_ok &= isinf(l) && l < 0;
            else worst_lse = fmax(worst_lse, fabs((double)l - log((double)n)));
            for (int c = 0; c < d; ++c) {
                double ref = 0.0;
                for (int j = 0; j < n; ++j) ref += val(b, g, j, c);
                if (n) ref /= n;
                const size_t i = ((size_t)b * Hq + h) * d + c;
                const double got = bf16 ? from_bf16(((uint16_t*)ho)[i]) : ((float*)ho)[i];
                if (n <= 1) special_ok &= got == ref; /* one key: its value exactly; none: 0 */
                const double tol = bf16 ? ldexp(fabs(ref), -8) + 1e-6 : 1e-6;
                worst = fmax(worst, fabs(got - ref) / tol);
            }
        }
    snprintf(what, sizeof what, "%s decode, uniform weights: max error / tolerance %.3f, lse error %.2g", bf16 ? "bf16" : "fp32",
             worst, worst_lse);
    check(worst <= 1.0 && worst_lse <= 1e-5, what);
    check(special_ok, "one visible key gives its value exactly; no visible key gives O = 0, lse = -inf");
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(dlens));
    HIP_OK(hipFree(dout));
    HIP_OK(hipFree(dlse));
    HIP_OK(hipFree(ws));
    free(hq);
    free(hk);
    free(hv);
    free(ho);
    free(hl);
}

/* Causal prefill (bf16, MFMA path) with all-zero keys: row i sees keys 0..i,
 * so O_i is the mean of the first i + 1 values and lse_i = ln(i + 1);
 * without the mask (Lq < Lkv) every row sees all Lkv keys. */
static void prefill_uniform(int causal) {
    const int B = 1, Hq = 4, Hkv = 1, d = 128, Lkv = 300, Lq = causal ? 300 : 100;
    const size_t nq = (size_t)B * Hq * Lq * d, nkv = (size_t)B * Hkv * Lkv * d;
    uint16_t* hq = (uint16_t*)malloc(nq * 2);
    uint16_t* hk = (uint16_t*)calloc(nkv, 2);
    uint16_t* hv = (uint16_t*)malloc(nkv * 2);
    for (size_t i = 0; i < nq; ++i) hq[i] = to_bf16((float)((int)(i % 9) - 4) / 4.0f);
    for (int j = 0; j < Lkv; ++j)
        for (int c = 0; c < d; ++c) hv[(size_t)j * d + c] = to_bf16(val(0, 0, j, c));
    void *dq = dev_copy(hq, nq * 2), *dk = dev_copy(hk, nkv * 2), *dv = dev_copy(hv, nkv * 2);
    void* dout = NULL;
    float* dlse = NULL;
    HIP_OK(hipMalloc(&dout, nq * 2));
    HIP_OK(hipMalloc((void**)&dlse, (size_t)B * Hq * Lq * 4));
    attn_tensor tq = view(dq, ATTN_BF16, Hq, Lq, d), tk = view(dk, ATTN_BF16, Hkv, Lkv, d);
    attn_tensor tv = view(dv, ATTN_BF16, Hkv, Lkv, d), to = view(dout, ATTN_BF16, Hq, Lq, d);
    attn_status st = attn_prefill(&tq, &tk, &tv, B, Hq, Hkv, d, Lq, Lkv, 0.0f, causal, &to, dlse, NULL);
    HIP_OK(hipDeviceSynchronize());
    check(st == ATTN_OK, causal ? "attn_prefill causal returns ATTN_OK" : "attn_prefill full returns ATTN_OK");
    uint16_t* ho = (uint16_t*)malloc(nq * 2);
    float* hl = (float*)malloc((size_t)B * Hq * Lq * 4);
    HIP_OK(hipMemcpy(ho, dout, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, dlse, (size_t)B * Hq * Lq * 4, hipMemcpyDeviceToHost));
    double worst = 0.0, worst_lse = 0.0;
    for (int h = 0; h < Hq; ++h)
        for (int i = 0; i < Lq; ++i) {
            const int n = causal ? i + 1 : Lkv;
            worst_lse = fmax(worst_lse, fabs((double)hl[h * Lq + i] - log((double)n)));
            for (int c = 0; c < d; ++c) {
                double ref = 0.0;
                for (int j = 0; j < n; ++j) ref += val(0, 0, j, c);
                ref /= n;
                const double got = from_bf16(ho[((size_t)h * Lq + i) * d + c]);
                worst = fmax(worst, fabs(got - ref) / (ldexp(fabs(ref), -8) + 1e-6));
            }
        }
    char what[160];
    snprintf(what, sizeof what, "bf16 %s prefill, uniform weights: max error / tolerance %.3f, lse error %.2g",
             causal ? "causal" : "full", worst, worst_lse);
    check(worst <= 1.0 && worst_lse <= 1e-5, what);
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(dout));
    HIP_OK(hipFree(dlse));
    free(hq);
    free(hk);
    free(hv);
    free(ho);
    free(hl);
}

/* Merge of partials (o_s, m_s, l_s) with o_s = l_s * w: the result is w for
 * any maxima, and lse = M + ln(sum_s e^(m_s - M) l_s). Row 2 holds only
 * identity partials (o = 0, m = -inf, l = 0): O = 0, lse = -inf. */
static void combine_closed_form(void) {
    const int R = 3, S = 5, d = 128;
    float* o = (float*)malloc((size_t)R * S * d * 4);
    float m[15], l[15];
    for (int r = 0; r < R; ++r)
        for (int s = 0; s < S; ++s) {
            const int i = r * S + s;
            m[i] = r == 2 ? -INFINITY : (float)(s - 2) * (r ? 3.0f : 0.5f);
            l[i] = r == 2 ? 0.0f : (float)(s + 1);
            for (int c = 0; c < d; ++c) o[(size_t)i * d + c] = l[i] * (float)(c - 64) / 64.0f;
        }
    void *dov = dev_copy(o, (size_t)R * S * d * 4), *dm = dev_copy(m, sizeof(m)), *dl = dev_copy(l, sizeof(l));
    void* dout = NULL;
    float* dlse = NULL;
    HIP_OK(hipMalloc(&dout, (size_t)R * d * 4));
    HIP_OK(hipMalloc((void**)&dlse, (size_t)R * 4));
    attn_tensor to;
    to.data = dout;
    to.dtype = ATTN_F32;
    to.stride_b = 0;
    to.stride_h = 0;
    to.stride_s = d;
    attn_status st = attn_combine_partials((const float*)dov, (const float*)dm, (const float*)dl, R, S, d, &to, dlse,
                                           NULL);
    HIP_OK(hipDeviceSynchronize());
    check(st == ATTN_OK, "attn_combine_partials returns ATTN_OK");
    float* ho = (float*)malloc((size_t)R * d * 4);
    float hl[3];
    HIP_OK(hipMemcpy(ho, dout, (size_t)R * d * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, dlse, sizeof(hl), hipMemcpyDeviceToHost));
    double worst = 0.0, worst_lse = 0.0;
    int empty_ok = 1;
    for (int r = 0; r < R; ++r) {
        if (r == 2) {
            empty_ok &= isinf(hl[r]) && hl[r] < 0;
            for (int c = 0; c < d; ++c) empty_ok &= ho[r * d + c] == 0.0f;
            continue;
        }
        double M = -INFINITY, z = 0.0;
        for (int s = 0; s < S; ++s) M = fmax(M, m[r * S + s]);
        for (int s = 0; s < S; ++s) z += exp((double)m[r * S + s] - M) * l[r * S + s];
        worst_lse = fmax(worst_lse, fabs((double)hl[r] - (M + log(z))));
        for (int c = 0; c < d; ++c) worst = fmax(worst, fabs((double)ho[r * d + c] - (c - 64) / 64.0));
    }
    char what[160];
    snprintf(what, sizeof what, "merge of scaled partials returns w: max error %.2g, lse error %.2g", worst, worst_lse);
    check(worst <= 1e-6 && worst_lse <= 1e-5, what);
    check(empty_ok, "a row of identity partials gives O = 0, lse = -inf");
    HIP_OK(hipFree(dov));
    HIP_OK(hipFree(dm));
    HIP_OK(hipFree(dl));
    HIP_OK(hipFree(dout));
    HIP_OK(hipFree(dlse));
    free(o);
    free(ho);
}

/* Bad arguments return their codes (and a message) without launching;
 * two identical calls on nonzero keys give bit-identical outputs. */
static void errors_and_repeats(void) {
    const int B = 1, Hq = 8, Hkv = 2, d = 128, L = 5000, S = 16;
    const size_t nq = (size_t)B * Hq * d, nkv = (size_t)B * Hkv * L * d;
    uint16_t* hq = (uint16_t*)malloc(nq * 2);
    uint16_t* hk = (uint16_t*)malloc(nkv * 2);
    for (size_t i = 0; i < nq; ++i) hq[i] = to_bf16((float)((int)(i % 9) - 4) / 4.0f);
    for (size_t i = 0; i < nkv; ++i) hk[i] = to_bf16((float)((int)((i * 2654435761u) % 17) - 8) / 8.0f);
    void *dq = dev_copy(hq, nq * 2), *dk = dev_copy(hk, nkv * 2);
    void *o1 = NULL, *o2 = NULL, *ws = NULL;
    HIP_OK(hipMalloc(&o1, nq * 2));
    HIP_OK(hipMalloc(&o2, nq * 2));
    const size_t ws_bytes = attn_decode_workspace_size(B, Hq, d, S);
    HIP_OK(hipMalloc(&ws, ws_bytes));
    check(attn_decode_workspace_init(ws, ws_bytes, NULL) == ATTN_OK, "workspace init");
    attn_tensor tq = view(dq, ATTN_BF16, Hq, 1, d), tk = view(dk, ATTN_BF16, Hkv, L, d);
    attn_tensor t1 = view(o1, ATTN_BF16, Hq, 1, d), t2 = view(o2, ATTN_BF16, Hq, 1, d);
    attn_status st = attn_decode(&tq, &tk, &tk, NULL, NULL, NULL, B, 6, 4, d, L, 0.0f, 0, S, &t1, NULL, ws, ws_bytes,
                                 NULL);
    check(st == ATTN_ERR_INVALID_ARG && strlen(attn_last_error()) > 0,
          "Hq not a multiple of Hkv: ATTN_ERR_INVALID_ARG with a message");
    st = attn_decode(&tq, &tk, &tk, NULL, NULL, NULL, B, Hq, Hkv, d, L, 0.0f, 0, S, &t1, NULL, ws, 64, NULL);
    check(st == ATTN_ERR_WORKSPACE, "workspace too small: ATTN_ERR_WORKSPACE");
    st = attn_decode(&tq, &tk, &tk, NULL, NULL, NULL, B, Hq, Hkv, 96, L, 0.0f, 0, S, &t1, NULL, ws, ws_bytes, NULL);
    check(st == ATTN_ERR_UNSUPPORTED || st == ATTN_ERR_INVALID_ARG, "head dim 96: rejected");
    check(attn_status_string(ATTN_OK) != NULL && attn_status_string(ATTN_ERR_HIP) != NULL, "status strings");
    attn_status s1 = attn_decode(&tq, &tk, &tk, NULL, NULL, NULL, B, Hq, Hkv, d, L, 0.0f, 0, S, &t1, NULL, ws,
                                 ws_bytes, NULL);
    attn_status s2 = attn_decode(&tq, &tk, &tk, NULL, NULL, NULL, B, Hq, Hkv, d, L, 0.0f, 0, S, &t2, NULL, ws,
                                 ws_bytes, NULL);
    HIP_OK(hipDeviceSynchronize());
    uint16_t* h1 = (uint16_t*)malloc(nq * 2);
    uint16_t* h2 = (uint16_t*)malloc(nq * 2);
    HIP_OK(hipMemcpy(h1, o1, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h2, o2, nq * 2, hipMemcpyDeviceToHost));
    check(s1 == ATTN_OK && s2 == ATTN_OK && memcmp(h1, h2, nq * 2) == 0, "two identical calls: bit-identical outputs");
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(o1));
    HIP_OK(hipFree(o2));
    HIP_OK(hipFree(ws));
    free(hq);
    free(hk);
    free(h1);
    free(h2);
}

int main(void) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        printf("no GPU\n");
        return 3;
    }
    decode_uniform(0, 4);
    decode_uniform(1, 0);
    decode_uniform(1, 7);
    decode_uniform(1, 64);
    prefill_uniform(1);
    prefill_uniform(0);
    combine_closed_form();
    errors_and_repeats();
    printf(g_fail ? "FAILED\n" : "all checks passed\n");
    return g_fail;
}
