// C-ABI front end of libattn.so: argument validation (host only, before any
// HIP call), the split plan, workspace layout and kernel dispatch. The
// operations and their sources are described in include/attn.h.
#include "attn.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

attn_status fail(attn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

constexpr int kChunkQuantum = 64;  // split chunks are a multiple of this many keys
constexpr int kPrecBf16 = 0, kPrecFp8 = 1, kPrecFp4 = 2;  // span precisions of launch_decode_mfma_two
// Split-plan cost per key of an fp8 and of an MX fp4 span, against 2 for
// bf16 (bytes per element), measured on the two-span decodes at 128K keys,
// 20 % bf16, 8 KV heads. fp8: 22 + 42 splits 56.1-56.2 us, 20 + 44 56.5-56.8,
// 18 + 46 58.6-58.7, 16 + 48 61.1-61.5. fp4 (two boxes, the current body):
// 19 + 45 41.2-41.5 us, 20 + 44 41.6-41.8, 18 + 46 42.6-42.7, 21 + 43
// 43.0-43.2, 22 + 42 43.8, 24 + 40 45.2. The three-precision decode (20 %
// bf16, 20 % fp8, 60 % fp4) takes the same weights: 20 + 10 + 34 45.7-45.8 us,
// 22 + 10 + 32 46.3-46.5, 20 + 9 + 35 48.7; 1.1 plans 20 + 44 and 20 + 10 +
// 34 (1.15 and up would give the three spans 20 + 9 + 35).
// Both bodies run scores and P.V on the MFMA; an fp8 key has twice the bytes
// of an fp4 key, an fp4 key more conversion work per byte.
constexpr double kFp8Cost = 0.95;
constexpr double kFp4Cost = 1.1;
constexpr float kLog2e = 1.44269504088896340736f;

int elem_size(int dt) {
    switch (dt) {
    case ATTN_F32: return 4;
    case ATTN_BF16: return 2;
    case ATTN_FP8_E4M3: return 1;
    case ATTN_MXFP4: return 1;  // a byte of two codes
    case ATTN_E8M0: return 1;
    default: return 0;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks a [*, *, *, d] operand: data present, known dtype, 16-byte aligned
// base and 16-byte multiples for the strides the kernels step with.
attn_status check_tensor(const attn_tensor* t, const char* name, bool need_row_alignment) {
    if (!t) return fail(ATTN_ERR_INVALID_ARG, "%s: null tensor", name);
    if (!t->data) return fail(ATTN_ERR_INVALID_ARG, "%s: null data pointer", name);
    const int es = elem_size(t->dtype);
    if (!es) return fail(ATTN_ERR_INVALID_ARG, "%s: unknown dtype %d", name, t->dtype);
    if (t->stride_b < 0 || t->stride_h < 0 || t->stride_s < 0)
        return fail(ATTN_ERR_INVALID_ARG, "%s: negative stride", name);
    if (need_row_alignment) {
        if (!aligned16(t->data)) return fail(ATTN_ERR_INVALID_ARG, "%s: data must be 16-byte aligned", name);
        if ((t->stride_b * es) % 16 || (t->stride_h * es) % 16 || (t->stride_s * es) % 16)
            return fail(ATTN_ERR_INVALID_ARG, "%s: strides must be multiples of 16 bytes", name);
    }
    return ATTN_OK;
}

int device_cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split plan shared by attn_decode and its size queries.
struct Plan {
    int chunk;  // keys per split, a multiple of kChunkQuantum
    int S;      // splits actually launched
};

Plan plan_splits(int L_cap, int requested) {
    Plan pl;
    pl.chunk = (int)(ceil_div(ceil_div(L_cap, requested), kChunkQuantum) * kChunkQuantum);
    pl.S = (int)ceil_div(L_cap, pl.chunk);
    return pl;
}

size_t partial_bytes(int64_t rows, int64_t S, int64_t d) { return (size_t)(rows * S * (d + 2) * 4); }

}  // namespace

extern "C" {

const char* attn_status_string(attn_status status) {
    switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_UNKNOWN_STATUS";
    }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_decode_auto_splits(int B, int Hkv, int L_cap, int kv_dtype, int ragged) {
    if (B <= 0 || Hkv <= 0 || L_cap <= 0 || !elem_size(kv_dtype)) return 0;
    const int cus = device_cu_count();
    if (cus <= 0) return 0;
    int64_t S;
    if (ragged) {
        // Lengths are only known on the device: cut every sequence into chunks
        // of 1216 keys (twice that for fp8, the same bytes) so that short and
        // long sequences balance across many workgroups. Not a power of two:
        // with 1024-key chunks every split starts on a 256 KiB boundary and a
        // batch of 16 x 8 heads of 4K-64K keys ran 6 % slower (330 us against
        // 309 us).
        const int64_t chunk = kv_dtype == ATTN_FP8_E4M3 ? 2432 : 1216;
        S = ceil_div(L_cap, chunk);
    } else {
        // Equal chunks, all workgroups resident at once and the same number
        // on every compute unit: 2 per CU for 16-bit caches, 4 for fp8 (a
        // quarter of the bytes per load, more waves to keep the bytes in
        // flight). With one per CU the merge would be fused into the decode
        // kernel, whose agent-scope release per workgroup costs more than the
        // second kernel (128K keys: 32 splits fused 91.3 us, 64 splits and the
        // merge kernel 86.3 us).
        const int64_t per_cu = kv_dtype == ATTN_FP8_E4M3 ? 4 : 2;
        S = (per_cu * cus) / ((int64_t)B * Hkv);
    }
    const int64_t max_s = ceil_div(L_cap, 256);  // no split shorter than 256 keys
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    return (int)S;
}

size_t attn_decode_workspace_size(int B, int Hq, int d, int num_splits) {
    if (B <= 0 || Hq <= 0 || d <= 0 || num_splits <= 0) return 0;
    return attn::kCounterBytes + partial_bytes((int64_t)B * Hq, num_splits, d) +
           partial_bytes((int64_t)B * Hq, attn::kMaxTicketBlocks, d);
}

attn_status attn_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = 0;
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is null");
    if (workspace_bytes < attn::kCounterBytes)
        return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes, need at least %zu", workspace_bytes, attn::kCounterBytes);
    if (!aligned16(workspace)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    hipError_t e = attn::launch_zero(workspace, attn::kCounterBytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "workspace init: %s", hipGetErrorString(e));
    return ATTN_OK;
}

int attn_decode_plan(int L_cap, int num_splits, int* chunk) {
    if (L_cap <= 0 || num_splits <= 0) return 0;
    const Plan pl = plan_splits(L_cap, num_splits);
    if (chunk) *chunk = pl.chunk;
    return pl.S;
}

}  // extern "C"

namespace {

// Validation and the first level (partials) shared by attn_decode and
// attn_decode_partials. On success *pl holds the split plan used.
struct FusedOut {
    uint32_t* counters;
    const attn_tensor* out;
    float* lse;
    float* blk_o;
    float* blk_m;
    float* blk_l;
    size_t clear_bytes;  // > 0: zero this many bytes of counters before a fused launch
};

// Splits per first-level ticket block of the fused merge: one level up to 32
// splits, else blocks of about sqrt(S) splits (at most kMaxTicketBlocks).
int ticket_block_for(int S) {
    int tb = S;
    if (tb > 32) {
        tb = 1;
        while (tb * tb < S) ++tb;
        while ((S + tb - 1) / tb > attn::kMaxTicketBlocks) ++tb;
    }
    return tb;
}

int requested_splits(int B, int Hkv, int L_cap, const attn_tensor* k, const int32_t* kv_lens, int num_splits) {
    if (num_splits > 0) return num_splits;
    if (B <= 0 || Hkv <= 0 || L_cap <= 0 || !k) return 0;
    return attn_decode_auto_splits(B, Hkv, L_cap, k->dtype, kv_lens != nullptr);
}

attn_status decode_level1(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, const float* k_scale,
                          const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int d, int L_cap,
                          float softmax_scale, int num_splits, const attn_tensor* out, float* o_part,
                          float* m_part, float* l_part, size_t part_bytes, Plan* pl, hipStream_t stream,
                          const FusedOut* fused, bool* used_fused) {
    *used_fused = false;
    attn_status st;
    if ((st = check_tensor(q, "q", true)) || (st = check_tensor(k, "k", true)) || (st = check_tensor(v, "v", true)))
        return st;
    if (out && (st = check_tensor(out, "out", false))) return st;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || L_cap <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d L_cap=%d)", B, Hq, Hkv, d,
                    L_cap);
    if (B > 65535 || Hkv > 65535) return fail(ATTN_ERR_INVALID_ARG, "B and Hkv must be <= 65535");
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    const int G = Hq / Hkv;
    if (num_splits < 0) return fail(ATTN_ERR_INVALID_ARG, "num_splits must be >= 0");
    if (isnan(softmax_scale) || isinf(softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale not finite");
    if (k->dtype != v->dtype) return fail(ATTN_ERR_INVALID_ARG, "k and v dtypes differ");
    if (out && out->dtype != q->dtype) return fail(ATTN_ERR_INVALID_ARG, "out dtype must equal q dtype");
    const bool fp8 = k->dtype == ATTN_FP8_E4M3;
    if (q->dtype == ATTN_F32 && k->dtype != ATTN_F32) return fail(ATTN_ERR_UNSUPPORTED, "fp32 q needs fp32 k/v");
    if (q->dtype == ATTN_BF16 && k->dtype == ATTN_F32) return fail(ATTN_ERR_UNSUPPORTED, "bf16 q with fp32 k/v");
    if (q->dtype != ATTN_F32 && q->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "q must be fp32 or bf16");
    // MX fp4 codes and E8M0 scales have their own entry point (attn_decode_mixed_fp4)
    if (k->dtype != ATTN_F32 && k->dtype != ATTN_BF16 && !fp8)
        return fail(ATTN_ERR_UNSUPPORTED, "k/v must be fp32, bf16 or fp8 e4m3 (dtype %d)", k->dtype);
    if (fp8 && (!k_scale || !v_scale)) return fail(ATTN_ERR_INVALID_ARG, "fp8 k/v need k_scale and v_scale");
    if (!fp8 && (k_scale || v_scale)) return fail(ATTN_ERR_INVALID_ARG, "scales are only for fp8 k/v");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(ATTN_ERR_UNSUPPORTED, "Hq/Hkv = %d (supported: 1, 2, 4, 8)", G);

    const int requested = requested_splits(B, Hkv, L_cap, k, kv_lens, num_splits);
    if (requested <= 0) return fail(ATTN_ERR_HIP, "could not query the device for the split plan");
    *pl = plan_splits(L_cap, requested);
    const int64_t rows = (int64_t)B * Hq;
    if (!o_part || !m_part || !l_part) return fail(ATTN_ERR_WORKSPACE, "workspace (partials) is null");
    if (!aligned16(o_part)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (part_bytes != (size_t)-1 && part_bytes < partial_bytes(rows, pl->S, d))
        return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes, need %zu for %d splits", part_bytes,
                    partial_bytes(rows, pl->S, d), pl->S);

    const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
    attn::DecodeParams p;
    p.q = q->data;
    p.q_sb = q->stride_b;
    p.q_sh = q->stride_h;
    p.k = k->data;
    p.k_sb = k->stride_b;
    p.k_sh = k->stride_h;
    p.k_ss = k->stride_s;
    p.v = v->data;
    p.v_sb = v->stride_b;
    p.v_sh = v->stride_h;
    p.v_ss = v->stride_s;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.kv_lens = kv_lens;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.d = d;
    p.L_cap = L_cap;
    p.chunk = pl->chunk;
    p.S = pl->S;
    p.scale_log2 = sc * kLog2e;
    p.o_part = o_part;
    p.m_part = m_part;
    p.l_part = l_part;
    p.counters = nullptr;
    p.ticket_block = 1;
    p.blk_o = p.blk_m = p.blk_l = nullptr;
    p.S0 = 0;
    p.sp0 = p.sp1 = attn::KvSpan{};
    p.alpha = nullptr;
    p.out = nullptr;
    p.out_sb = p.out_sh = 0;
    p.lse = nullptr;

    hipError_t e;
    const bool mfma = q->dtype == ATTN_BF16;  // every supported d (64, 128) and G (1, 2, 4, 8)
    // the MFMA path reads 32-key tiles addressed by 32-bit byte offsets
    if (mfma) {
        const int64_t esz = fp8 ? 1 : 2, lim = int64_t(1) << 26;
        if (k->stride_s < 0 || v->stride_s < 0 || k->stride_s * esz >= lim || v->stride_s * esz >= lim)
            return fail(ATTN_ERR_INVALID_ARG, "k/v row strides must be below 2^26 bytes on the grouped-query path");
    }
    // Fuse the merge into the decode kernel when the launch has at most one
    // workgroup per compute unit. Timed back to back, the fused tail (publish,
    // ticket, merge by the last workgroup) costs about what a second kernel
    // does; with one workgroup per CU the two were even at 128K keys, with two
    // the second kernel won (64 splits: 88.5 against 86.8 us).
    const int cus = device_cu_count();
    const int64_t wgs = (int64_t)B * Hkv * pl->S;
    if (mfma && G == 4 && d == 128 && fused && (int64_t)B * Hkv <= attn::kMaxCounterGroups && pl->S <= attn::kMaxFusedSplits &&
        cus > 0 && wgs <= cus) {
        p.counters = fused->counters;
        p.ticket_block = ticket_block_for(pl->S);
        p.blk_o = fused->blk_o;
        p.blk_m = fused->blk_m;
        p.blk_l = fused->blk_l;
        p.out = fused->out->data;
        p.out_sb = fused->out->stride_b;
        p.out_sh = fused->out->stride_h;
        p.lse = fused->lse;
        *used_fused = true;
        if (fused->clear_bytes) {
            e = attn::launch_zero(fused->counters, fused->clear_bytes, stream);
            if (e != hipSuccess) return fail(ATTN_ERR_HIP, "clearing the merge counters: %s", hipGetErrorString(e));
        }
    }
    if (mfma) e = attn::launch_decode_mfma(p, fp8 ? attn::DT_FP8 : attn::DT_BF16, G, stream);
    else e = attn::launch_decode_valu(p, q->dtype, k->dtype, G, stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}


// Automatic split plan of a launch over n spans (n <= 3): two resident
// workgroups per compute unit in all, shared in proportion to keys * cost,
// every split at least 256 keys long. Stores each span's splits (after
// planning) in S[i] and returns their sum, 0 on failure.
int span_splits(int B, int Hkv, int n, const int* L, const double* cost, int* S) {
    const int cus = device_cu_count();
    int64_t keys = 0;
    double W = 0.0;
    int last = -1;  // the last span with keys takes what the others leave
    for (int i = 0; i < n; ++i) {
        keys += L[i];
        W += cost[i] * L[i];
        if (L[i]) last = i;
    }
    if (cus <= 0 || keys <= 0) return 0;
    int64_t T = (2LL * cus) / ((int64_t)B * Hkv);
    if (T < n) T = n;
    int64_t r[3] = {0, 0, 0}, given = 0;
    for (int i = 0; i < n; ++i) {
        if (!L[i] || i == last) continue;
        r[i] = (int64_t)llround((double)T * cost[i] * L[i] / W);
        given += r[i];
    }
    r[last] = T - given;
    int total = 0;
    for (int i = 0; i < n; ++i) {
        S[i] = 0;
        if (!L[i]) continue;
        const int64_t max_s = ceil_div(L[i], 256);
        const int64_t ri = r[i] < 1 ? 1 : (r[i] > max_s ? max_s : r[i]);
        S[i] = plan_splits(L[i], (int)ri).S;
        total += S[i];
    }
    return total;
}

int two_span_splits(int B, int Hkv, int L0, double cost0, int L1, double cost1, int* s0, int* s1) {
    const int L[2] = {L0, L1};
    const double c[2] = {cost0, cost1};
    int S[2];
    const int total = span_splits(B, Hkv, 2, L, c, S);
    if (total <= 0) return 0;
    if (s0) *s0 = S[0];
    if (s1) *s1 = S[1];
    return total;
}

// Most keys each pi-Attention span can hold for a decode query at position
// L_cap - 1: the window's window + 1 keys, and the skip keys below the window.
struct PiCaps {
    int window, skip;
};
PiCaps pi_caps(int L_cap, int window, int period) {
    PiCaps c;
    c.window = (int)((int64_t)window + 1 < (int64_t)L_cap ? window + 1 : L_cap);
    const int64_t last = (int64_t)L_cap - 2 - window;  // highest row a skip key can take
    c.skip = (period > 0 && last >= 0) ? (int)(last / period + 1) : 0;
    return c;
}

// A span over a [B, Hkv, L_cap, d] cache; lens_per_head: lens is [B, Hkv]
// rather than [B].
attn::KvSpan span_of(const attn_tensor* k, const attn_tensor* v, const int32_t* lens, int lens_per_head_hkv,
                     int L_cap, int chunk) {
    attn::KvSpan sp{};
    if (L_cap && k && v) {
        sp.k = k->data;
        sp.k_sb = k->stride_b;
        sp.k_sh = k->stride_h;
        sp.k_ss = k->stride_s;
        sp.v = v->data;
        sp.v_sb = v->stride_b;
        sp.v_sh = v->stride_h;
        sp.v_ss = v->stride_s;
    }
    sp.kv_lens = lens;
    sp.lens_sb = lens_per_head_hkv ? lens_per_head_hkv : 1;
    sp.lens_sh = lens_per_head_hkv ? 1 : 0;
    sp.L_cap = L_cap;
    sp.chunk = chunk;
    sp.geom = attn::kGeomAll;
    sp.period = 1;
    return sp;
}

// Query heads per KV head the MFMA decode kernels take.
bool mfma_head_ratio(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

// Spans are read in 32-key tiles addressed by 32-bit byte offsets from the
// tile's first row: the distance between the rows a span visits (the row
// stride in bytes, times the period of a skip span) must stay below 2^26
// bytes, so that 32 of them fit.
bool tile32_strides_ok(const attn::KvSpan& sp, int prec) {
    if (sp.L_cap == 0) return true;
    const int64_t lim = int64_t(1) << 26;
    const int64_t mul = (sp.geom == attn::kGeomSkip ? sp.period : 1) * (prec == kPrecBf16 ? 2 : 1);
    int64_t st[4] = {sp.k_ss, sp.v_ss, 0, 0};
    if (prec == kPrecFp4) {
        st[2] = sp.ksc_ss;
        st[3] = sp.vsc_ss;
    }
    for (int64_t x : st)
        if (x < 0 || x * mul >= lim) return false;
    return true;
}

attn::DecodeParams two_span_params(const attn_tensor* q, int B, int Hq, int Hkv, int d, float softmax_scale,
                                   const float* k_scale, const float* v_scale) {
    const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
    attn::DecodeParams p{};
    p.q = q->data;
    p.q_sb = q->stride_b;
    p.q_sh = q->stride_h;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.d = d;
    p.scale_log2 = sc * kLog2e;
    p.ticket_block = 1;
    return p;
}

// Workspace layout (that of attn_decode with S splits), the fused-merge
// decision, the launch (two spans, or three when prec2 >= 0), and the
// separate merge when not fused.
attn_status two_span_launch(attn::DecodeParams& p, int S, int prec0, int prec1, attn_tensor* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t hs, int prec2 = -1) {
    const int B = p.B, Hq = p.Hq, Hkv = p.Hkv, d = p.d;
    if (!tile32_strides_ok(p.sp0, prec0) || !tile32_strides_ok(p.sp1, prec1) ||
        (prec2 >= 0 && !tile32_strides_ok(p.sp2, prec2)))
        return fail(ATTN_ERR_INVALID_ARG,
                    "the bytes between the rows a span visits (row stride x skip period) must be below 2^26");
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is null");
    if (!aligned16(workspace)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    const int64_t rows = (int64_t)B * Hq;
    const size_t need = attn_decode_workspace_size(B, Hq, d, S);
    if (workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes, need %zu for %d splits", workspace_bytes, need, S);
    uint32_t* counters = static_cast<uint32_t*>(workspace);
    float* o_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + attn::kCounterBytes);
    float* m_part = o_part + rows * S * d;
    float* l_part = m_part + rows * S;
    float* blk_o = l_part + rows * S;
    float* blk_m = blk_o + rows * attn::kMaxTicketBlocks * d;
    float* blk_l = blk_m + rows * attn::kMaxTicketBlocks;
    p.S = S;
    p.o_part = o_part;
    p.m_part = m_part;
    p.l_part = l_part;

    const int cus = device_cu_count();
    const int64_t wgs = (int64_t)B * Hkv * S;
    // the same rule as the one-span decode (pi decode, 200 workgroups: fused
    // 12.8 us, two kernels 13.5 us; two-precision, 512: fused 65 us, two
    // kernels 64 us)
    const bool fused = Hq == 4 * Hkv && d == 128 && (int64_t)B * Hkv <= attn::kMaxCounterGroups && S <= attn::kMaxFusedSplits &&
                       cus > 0 && wgs <= cus;
    if (fused) {
        p.counters = counters;
        p.ticket_block = ticket_block_for(S);
        p.blk_o = blk_o;
        p.blk_m = blk_m;
        p.blk_l = blk_l;
        p.out = out->data;
        p.out_sb = out->stride_b;
        p.out_sh = out->stride_h;
        p.lse = lse;
    }
    hipError_t e = prec2 < 0 ? attn::launch_decode_mfma_two(p, prec0, prec1, hs)
                             : attn::launch_decode_mfma_three(p, prec0, prec1, prec2, hs);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    if (fused) return ATTN_OK;

    // every split publishes a partial (the identity when empty): merge all S
    attn::CombineParams cp;
    cp.o_part = o_part;
    cp.m_part = m_part;
    cp.l_part = l_part;
    cp.R = (int)rows;
    cp.S = S;
    cp.d = d;
    cp.Hq = Hq;
    cp.kv_lens = nullptr;
    cp.chunk = 1;
    cp.L_cap = 0;
    cp.out = out->data;
    cp.out_dtype = out->dtype;
    cp.out_sb = out->stride_b;
    cp.out_sh = out->stride_h;
    cp.lse = lse;
    e = attn::launch_combine(cp, hs);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// general: also accept what the vector-ALU prefill takes (fp32 with d = 64 or
// 128, bf16 with d = 64); otherwise only the MFMA kernel's bf16, d = 128.
attn_status check_prefill(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, const attn_tensor* out,
                          int B, int Hq, int Hkv, int d, int Lq, int Lkv, float softmax_scale, int causal,
                          bool general = false) {
    attn_status st;
    if ((st = check_tensor(q, "q", true)) || (st = check_tensor(k, "k", true)) || (st = check_tensor(v, "v", true)) ||
        (st = check_tensor(out, "out", true)))
        return st;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Lq <= 0 || Lkv <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive");
    if (B > 65535 || Hq > 65535) return fail(ATTN_ERR_INVALID_ARG, "B and Hq must be <= 65535");
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (causal && Lq > Lkv) return fail(ATTN_ERR_INVALID_ARG, "causal with Lq (%d) > Lkv (%d)", Lq, Lkv);
    if (isnan(softmax_scale) || isinf(softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale not finite");
    const bool same = q->dtype == k->dtype && q->dtype == v->dtype && q->dtype == out->dtype;
    const bool mfma = same && q->dtype == ATTN_BF16 && (d == 128 || d == 64);
    const bool valu = same && q->dtype == ATTN_F32 && (d == 64 || d == 128);
    if (!mfma && !(general && valu)) {
        if (general) return fail(ATTN_ERR_UNSUPPORTED, "prefill takes bf16 with d = 64 or 128, or fp32 with d = 64 or 128 "
                                                       "(q, k, v and out of one dtype; got d = %d)", d);
        return fail(ATTN_ERR_UNSUPPORTED, "this entry point takes bf16 q/k/v/out with d = 64 or 128 (got d = %d)", d);
    }
    // K/V tiles (64 rows) and Q blocks (32 rows) are read through 32-bit buffer offsets
    if (q->stride_s >= (1 << 24) || k->stride_s >= (1 << 24) || v->stride_s >= (1 << 24))
        return fail(ATTN_ERR_UNSUPPORTED, "prefill q/k/v row stride must be below 2^24 elements");
    return ATTN_OK;
}

attn::PrefillParams prefill_params(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                   const attn_tensor* out, float* lse, int B, int Hq, int Hkv, int d, int Lq, int Lkv,
                                   float softmax_scale, int causal) {
    const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
    attn::PrefillParams p;
    p.q = q->data;
    p.q_sb = q->stride_b;
    p.q_sh = q->stride_h;
    p.q_ss = q->stride_s;
    p.k = k->data;
    p.k_sb = k->stride_b;
    p.k_sh = k->stride_h;
    p.k_ss = k->stride_s;
    p.v = v->data;
    p.v_sb = v->stride_b;
    p.v_sh = v->stride_h;
    p.v_ss = v->stride_s;
    p.out = out->data;
    p.o_sb = out->stride_b;
    p.o_sh = out->stride_h;
    p.o_ss = out->stride_s;
    p.lse = lse;
    p.lse_sb = (int64_t)Hq * Lq;
    p.lse_sh = Lq;
    p.lse_ss = 1;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.d = d;
    p.Lq = Lq;
    p.Lkv = Lkv;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = sc * kLog2e;
    p.band = 0;
    p.diag = Lkv - Lq;
    p.window = -1;
    p.merge = 0;
    p.lse_w = nullptr;
    p.alpha = nullptr;
    return p;
}

}  // namespace

extern "C" {

attn_status attn_decode(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, const float* k_scale,
                        const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int d, int L_cap,
                        float softmax_scale, int causal, int num_splits, attn_tensor* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = 0;
    return attn::decode_impl(q, k, v, k_scale, v_scale, kv_lens, B, Hq, Hkv, d, L_cap, softmax_scale, causal,
                             num_splits, out, lse, workspace, workspace_bytes, 0, stream);
}

}  // extern "C"

namespace attn {

void set_last_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}

attn_status decode_impl(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, const float* k_scale,
                        const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int d, int L_cap,
                        float softmax_scale, int causal, int num_splits, attn_tensor* out, float* lse,
                        void* workspace, size_t workspace_bytes, size_t clear_counter_bytes, void* stream) {
    (void)causal;  // one query aligned bottom-right sees every valid key
    if (!out) return fail(ATTN_ERR_INVALID_ARG, "out: null tensor");
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is null");
    if (!aligned16(workspace)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (workspace_bytes < attn::kCounterBytes)
        return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes, need more than %zu", workspace_bytes,
                    attn::kCounterBytes);
    // Layout: [merge counters | o_part | m_part | l_part]; the partial arrays
    // depend on the split plan, which is a pure function of the arguments.
    const int requested = requested_splits(B, Hkv, L_cap, k, kv_lens, num_splits);
    const int S_layout = (requested > 0 && L_cap > 0) ? plan_splits(L_cap, requested).S : 1;
    const int64_t rows = (int64_t)(B > 0 ? B : 0) * (Hq > 0 ? Hq : 0);
    uint32_t* counters = static_cast<uint32_t*>(workspace);
    float* o_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + attn::kCounterBytes);
    float* m_part = o_part + rows * S_layout * (d > 0 ? d : 0);
    float* l_part = m_part + rows * S_layout;
    float* blk_o = l_part + rows * S_layout;
    float* blk_m = blk_o + rows * attn::kMaxTicketBlocks * (d > 0 ? d : 0);
    float* blk_l = blk_m + rows * attn::kMaxTicketBlocks;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    Plan pl{0, 0};
    const FusedOut fo{counters, out, lse, blk_o, blk_m, blk_l, clear_counter_bytes};
    bool fused = false;
    const size_t fixed = attn::kCounterBytes + partial_bytes(rows, attn::kMaxTicketBlocks, d > 0 ? d : 0);
    if (workspace_bytes < fixed)
        return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes, need more than %zu", workspace_bytes, fixed);
    attn_status st = decode_level1(q, k, v, k_scale, v_scale, kv_lens, B, Hq, Hkv, d, L_cap, softmax_scale,
                                   num_splits, out, o_part, m_part, l_part, workspace_bytes - fixed, &pl, hs, &fo,
                                   &fused);
    if (st != ATTN_OK || fused) return st;

    attn::CombineParams cp;
    cp.o_part = o_part;
    cp.m_part = m_part;
    cp.l_part = l_part;
    cp.R = (int)rows;
    cp.S = pl.S;
    cp.d = d;
    cp.Hq = Hq;
    cp.kv_lens = kv_lens;
    cp.chunk = pl.chunk;
    cp.L_cap = L_cap;
    cp.out = out->data;
    cp.out_dtype = out->dtype;
    cp.out_sb = out->stride_b;
    cp.out_sh = out->stride_h;
    cp.lse = lse;
    hipError_t e = attn::launch_combine(cp, hs);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}

}  // namespace attn

extern "C" {

attn_status attn_decode_partials(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                 const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B, int Hq,
                                 int Hkv, int d, int L_cap, float softmax_scale, int causal, int num_splits,
                                 float* o_part, float* m_part, float* l_part, int* splits_used, void* stream) {
    (void)causal;
    g_last_error[0] = 0;
    Plan pl{0, 0};
    bool fused = false;
    attn_status st = decode_level1(q, k, v, k_scale, v_scale, kv_lens, B, Hq, Hkv, d, L_cap, softmax_scale,
                                   num_splits, nullptr, o_part, m_part, l_part, (size_t)-1, &pl,
                                   static_cast<hipStream_t>(stream), nullptr, &fused);
    if (st == ATTN_OK && splits_used) *splits_used = pl.S;
    return st;
}

attn_status attn_combine_partials(const float* o_part, const float* m_part, const float* l_part, int R, int S,
                                  int d, attn_tensor* out, float* lse, void* stream) {
    g_last_error[0] = 0;
    if (!o_part || !m_part || !l_part) return fail(ATTN_ERR_INVALID_ARG, "null partial pointer");
    attn_status st;
    if ((st = check_tensor(out, "out", false))) return st;
    if (R <= 0 || S <= 0 || d <= 0) return fail(ATTN_ERR_INVALID_ARG, "R, S and d must be positive");
    if (out->dtype != ATTN_F32 && out->dtype != ATTN_BF16)
        return fail(ATTN_ERR_UNSUPPORTED, "out must be fp32 or bf16");
    attn::CombineParams cp;
    cp.o_part = o_part;
    cp.m_part = m_part;
    cp.l_part = l_part;
    cp.R = R;
    cp.S = S;
    cp.d = d;
    cp.Hq = 1;
    cp.kv_lens = nullptr;
    cp.chunk = 1;
    cp.L_cap = 0;
    cp.out = out->data;
    cp.out_dtype = out->dtype;
    cp.out_sb = out->stride_s;  // row r = "batch" r with Hq = 1
    cp.out_sh = 0;
    cp.lse = lse;
    hipError_t e = attn::launch_combine(cp, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}

int attn_decode_mixed_splits(int B, int Hkv, int L_hi_cap, int L_lo_cap, int* splits_hi, int* splits_lo) {
    if (B <= 0 || Hkv <= 0 || L_hi_cap < 0 || L_lo_cap < 0 || L_hi_cap + L_lo_cap <= 0) return 0;
    // cost per key: 2 for bf16, kFp8Cost for fp8
    return two_span_splits(B, Hkv, L_hi_cap, 2.0, L_lo_cap, kFp8Cost, splits_hi, splits_lo);
}

attn_status attn_decode_mixed(const attn_tensor* q, const attn_tensor* k_hi, const attn_tensor* v_hi,
                              const int32_t* hi_lens, int L_hi_cap, const attn_tensor* k_lo,
                              const attn_tensor* v_lo, const float* k_scale, const float* v_scale,
                              const int32_t* lo_lens, int L_lo_cap, int B, int Hq, int Hkv, int d,
                              float softmax_scale, int num_splits_hi, int num_splits_lo, attn_tensor* out,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = 0;
    attn_status st;
    if ((st = check_tensor(q, "q", true)) || (st = check_tensor(out, "out", false))) return st;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d)", B, Hq, Hkv, d);
    if (L_hi_cap < 0 || L_lo_cap < 0 || L_hi_cap + L_lo_cap <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "span capacities must be >= 0 and not both 0 (%d, %d)", L_hi_cap,
                    L_lo_cap);
    if (B > 65535 || Hkv > 65535) return fail(ATTN_ERR_INVALID_ARG, "B and Hkv must be <= 65535");
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (num_splits_hi < 0 || num_splits_lo < 0) return fail(ATTN_ERR_INVALID_ARG, "split counts must be >= 0");
    if (isnan(softmax_scale) || isinf(softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale not finite");
    if (L_hi_cap) {
        if ((st = check_tensor(k_hi, "k_hi", true)) || (st = check_tensor(v_hi, "v_hi", true))) return st;
        if (k_hi->dtype != ATTN_BF16 || v_hi->dtype != ATTN_BF16)
            return fail(ATTN_ERR_UNSUPPORTED, "the high-precision span must be bf16");
    }
    if (L_lo_cap) {
        if ((st = check_tensor(k_lo, "k_lo", true)) || (st = check_tensor(v_lo, "v_lo", true))) return st;
        if (k_lo->dtype != ATTN_FP8_E4M3 || v_lo->dtype != ATTN_FP8_E4M3)
            return fail(ATTN_ERR_UNSUPPORTED, "the low-precision span must be fp8 e4m3");
        if (!k_scale || !v_scale) return fail(ATTN_ERR_INVALID_ARG, "the fp8 span needs k_scale and v_scale");
    }
    if (q->dtype != ATTN_BF16 || out->dtype != ATTN_BF16)
        return fail(ATTN_ERR_UNSUPPORTED, "mixed decode takes bf16 q and out");
    if ((d != 64 && d != 128) || !mfma_head_ratio(Hq / Hkv))
        return fail(ATTN_ERR_UNSUPPORTED, "mixed decode supports d in {64, 128} and Hq/Hkv in {1, 2, 4, 8} (got %d, %d)",
                    d, Hq / Hkv);

    int auto_hi = 0, auto_lo = 0;
    if ((!num_splits_hi && L_hi_cap) || (!num_splits_lo && L_lo_cap)) {
        if (attn_decode_mixed_splits(B, Hkv, L_hi_cap, L_lo_cap, &auto_hi, &auto_lo) <= 0)
            return fail(ATTN_ERR_HIP, "could not query the device for the split plan");
    }
    const Plan ph = L_hi_cap ? plan_splits(L_hi_cap, num_splits_hi ? num_splits_hi : auto_hi) : Plan{kChunkQuantum, 0};
    const Plan plo = L_lo_cap ? plan_splits(L_lo_cap, num_splits_lo ? num_splits_lo : auto_lo) : Plan{kChunkQuantum, 0};

    attn::DecodeParams p = two_span_params(q, B, Hq, Hkv, d, softmax_scale, k_scale, v_scale);
    p.S0 = ph.S;
    p.sp0 = span_of(k_hi, v_hi, hi_lens, Hkv, L_hi_cap, ph.chunk);
    p.sp1 = span_of(k_lo, v_lo, lo_lens, Hkv, L_lo_cap, plo.chunk);
    return two_span_launch(p, ph.S + plo.S, kPrecBf16, kPrecFp8, out, lse, workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream));
}

int attn_decode_mixed_fp4_splits(int B, int Hkv, int L_hi_cap, int L_lo_cap, int* splits_hi, int* splits_lo) {
    if (B <= 0 || Hkv <= 0 || L_hi_cap < 0 || L_lo_cap < 0 || L_hi_cap + L_lo_cap <= 0) return 0;
    return two_span_splits(B, Hkv, L_hi_cap, 2.0, L_lo_cap, kFp4Cost, splits_hi, splits_lo);
}

// An E8M0 scale array [B, Hkv, L, d/32] read as one 4-byte word per row.
attn_status check_scales(const attn_tensor* t, const char* name) {
    if (!t) return fail(ATTN_ERR_INVALID_ARG, "%s: null tensor", name);
    if (!t->data) return fail(ATTN_ERR_INVALID_ARG, "%s: null data pointer", name);
    if (t->dtype != ATTN_E8M0) return fail(ATTN_ERR_INVALID_ARG, "%s: dtype must be ATTN_E8M0", name);
    if (t->stride_b < 0 || t->stride_h < 0 || t->stride_s < 0)
        return fail(ATTN_ERR_INVALID_ARG, "%s: negative stride", name);
    if ((reinterpret_cast<uintptr_t>(t->data) & 3u) || t->stride_b % 4 || t->stride_h % 4 || t->stride_s % 4)
        return fail(ATTN_ERR_INVALID_ARG, "%s: data and strides must be multiples of 4 bytes", name);
    return ATTN_OK;
}

attn_status attn_decode_mixed_fp4(const attn_tensor* q, const attn_tensor* k_hi, const attn_tensor* v_hi,
                                  const int32_t* hi_lens, int L_hi_cap, const attn_tensor* k_lo,
                                  const attn_tensor* v_lo, const attn_tensor* k_lo_scale,
                                  const attn_tensor* v_lo_scale, const int32_t* lo_lens, int L_lo_cap, int B, int Hq,
                                  int Hkv, int d, float softmax_scale, int num_splits_hi, int num_splits_lo,
                                  attn_tensor* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    g_last_error[0] = 0;
    attn_status st;
    if ((st = check_tensor(q, "q", true)) || (st = check_tensor(out, "out", false))) return st;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d)", B, Hq, Hkv, d);
    if (L_hi_cap < 0 || L_lo_cap < 0 || L_hi_cap + L_lo_cap <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "span capacities must be >= 0 and not both 0 (%d, %d)", L_hi_cap,
                    L_lo_cap);
    if (B > 65535 || Hkv > 65535) return fail(ATTN_ERR_INVALID_ARG, "B and Hkv must be <= 65535");
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (num_splits_hi < 0 || num_splits_lo < 0) return fail(ATTN_ERR_INVALID_ARG, "split counts must be >= 0");
    if (isnan(softmax_scale) || isinf(softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale not finite");
    if (L_hi_cap) {
        if ((st = check_tensor(k_hi, "k_hi", true)) || (st = check_tensor(v_hi, "v_hi", true))) return st;
        if (k_hi->dtype != ATTN_BF16 || v_hi->dtype != ATTN_BF16)
            return fail(ATTN_ERR_UNSUPPORTED, "the high-precision span must be bf16");
    }
    if (L_lo_cap) {
        if ((st = check_tensor(k_lo, "k_lo", true)) || (st = check_tensor(v_lo, "v_lo", true))) return st;
        if (k_lo->dtype != ATTN_MXFP4 || v_lo->dtype != ATTN_MXFP4)
            return fail(ATTN_ERR_UNSUPPORTED, "the low-precision span must be ATTN_MXFP4");
        if ((st = check_scales(k_lo_scale, "k_lo_scale")) || (st = check_scales(v_lo_scale, "v_lo_scale")))
            return st;
        // the kernel steps through a 32-row tile with 32-bit offsets
        const int64_t lim = int64_t(1) << 26;
        if (k_lo->stride_s >= lim || v_lo->stride_s >= lim || k_lo_scale->stride_s >= lim ||
            v_lo_scale->stride_s >= lim)
            return fail(ATTN_ERR_INVALID_ARG, "fp4 span row strides must be below 64 MiB");
    }
    if (q->dtype != ATTN_BF16 || out->dtype != ATTN_BF16)
        return fail(ATTN_ERR_UNSUPPORTED, "mixed decode takes bf16 q and out");
    if (d != 128 || !mfma_head_ratio(Hq / Hkv))
        return fail(ATTN_ERR_UNSUPPORTED, "mixed decode supports d = 128 and Hq/Hkv in {1, 2, 4, 8} (got %d, %d)", d,
                    Hq / Hkv);

    int auto_hi = 0, auto_lo = 0;
    if ((!num_splits_hi && L_hi_cap) || (!num_splits_lo && L_lo_cap)) {
        if (attn_decode_mixed_fp4_splits(B, Hkv, L_hi_cap, L_lo_cap, &auto_hi, &auto_lo) <= 0)
            return fail(ATTN_ERR_HIP, "could not query the device for the split plan");
    }
    const Plan ph = L_hi_cap ? plan_splits(L_hi_cap, num_splits_hi ? num_splits_hi : auto_hi) : Plan{kChunkQuantum, 0};
    const Plan plo = L_lo_cap ? plan_splits(L_lo_cap, num_splits_lo ? num_splits_lo : auto_lo) : Plan{kChunkQuantum, 0};

    attn::DecodeParams p = two_span_params(q, B, Hq, Hkv, d, softmax_scale, nullptr, nullptr);
    p.S0 = ph.S;
    p.sp0 = span_of(k_hi, v_hi, hi_lens, Hkv, L_hi_cap, ph.chunk);
    p.sp1 = span_of(k_lo, v_lo, lo_lens, Hkv, L_lo_cap, plo.chunk);  // strides of byte tensors: bytes
    if (L_lo_cap) {
        p.sp1.k_sc = k_lo_scale->data;
        p.sp1.ksc_sb = k_lo_scale->stride_b;
        p.sp1.ksc_sh = k_lo_scale->stride_h;
        p.sp1.ksc_ss = k_lo_scale->stride_s;
        p.sp1.v_sc = v_lo_scale->data;
        p.sp1.vsc_sb = v_lo_scale->stride_b;
        p.sp1.vsc_sh = v_lo_scale->stride_h;
        p.sp1.vsc_ss = v_lo_scale->stride_s;
    }
    return two_span_launch(p, ph.S + plo.S, kPrecBf16, kPrecFp4, out, lse, workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream));
}

int attn_decode_mixed3_splits(int B, int Hkv, int L_hi_cap, int L_mid_cap, int L_lo_cap, int* splits_hi,
                              int* splits_mid, int* splits_lo) {
    if (B <= 0 || Hkv <= 0 || L_hi_cap < 0 || L_mid_cap < 0 || L_lo_cap < 0 ||
        (int64_t)L_hi_cap + L_mid_cap + L_lo_cap <= 0)
        return 0;
    // the costs per key of the two-span plans: bf16 2, fp8 and fp4 (see
    // kFp8Cost and kFp4Cost)
    const int L[3] = {L_hi_cap, L_mid_cap, L_lo_cap};
    const double c[3] = {2.0, kFp8Cost, kFp4Cost};
    int S[3];
    const int total = span_splits(B, Hkv, 3, L, c, S);
    if (total <= 0) return 0;
    if (splits_hi) *splits_hi = S[0];
    if (splits_mid) *splits_mid = S[1];
    if (splits_lo) *splits_lo = S[2];
    return total;
}

attn_status attn_decode_mixed3(const attn_tensor* q, const attn_tensor* k_hi, const attn_tensor* v_hi,
                               const int32_t* hi_lens, int L_hi_cap, const attn_tensor* k_mid,
                               const attn_tensor* v_mid, const float* k_mid_scale, const float* v_mid_scale,
                               const int32_t* mid_lens, int L_mid_cap, const attn_tensor* k_lo,
                               const attn_tensor* v_lo, const attn_tensor* k_lo_scale, const attn_tensor* v_lo_scale,
                               const int32_t* lo_lens, int L_lo_cap, int B, int Hq, int Hkv, int d,
                               float softmax_scale, int num_splits_hi, int num_splits_mid, int num_splits_lo,
                               attn_tensor* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = 0;
    attn_status st;
    if ((st = check_tensor(q, "q", true)) || (st = check_tensor(out, "out", false))) return st;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d)", B, Hq, Hkv, d);
    if (L_hi_cap < 0 || L_mid_cap < 0 || L_lo_cap < 0 || (int64_t)L_hi_cap + L_mid_cap + L_lo_cap <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "span capacities must be >= 0 and not all 0 (%d, %d, %d)", L_hi_cap,
                    L_mid_cap, L_lo_cap);
    if (B > 65535 || Hkv > 65535) return fail(ATTN_ERR_INVALID_ARG, "B and Hkv must be <= 65535");
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (num_splits_hi < 0 || num_splits_mid < 0 || num_splits_lo < 0)
        return fail(ATTN_ERR_INVALID_ARG, "split counts must be >= 0");
    if (isnan(softmax_scale) || isinf(softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale not finite");
    if (L_hi_cap) {
        if ((st = check_tensor(k_hi, "k_hi", true)) || (st = check_tensor(v_hi, "v_hi", true))) return st;
        if (k_hi->dtype != ATTN_BF16 || v_hi->dtype != ATTN_BF16)
            return fail(ATTN_ERR_UNSUPPORTED, "the high-precision span must be bf16");
    }
    if (L_mid_cap) {
        if ((st = check_tensor(k_mid, "k_mid", true)) || (st = check_tensor(v_mid, "v_mid", true))) return st;
        if (k_mid->dtype != ATTN_FP8_E4M3 || v_mid->dtype != ATTN_FP8_E4M3)
            return fail(ATTN_ERR_UNSUPPORTED, "the middle span must be fp8 e4m3");
        if (!k_mid_scale || !v_mid_scale) return fail(ATTN_ERR_INVALID_ARG, "the fp8 span needs its scales");
    }
    if (L_lo_cap) {
        if ((st = check_tensor(k_lo, "k_lo", true)) || (st = check_tensor(v_lo, "v_lo", true))) return st;
        if (k_lo->dtype != ATTN_MXFP4 || v_lo->dtype != ATTN_MXFP4)
            return fail(ATTN_ERR_UNSUPPORTED, "the low-precision span must be ATTN_MXFP4");
        if ((st = check_scales(k_lo_scale, "k_lo_scale")) || (st = check_scales(v_lo_scale, "v_lo_scale")))
            return st;
        const int64_t lim = int64_t(1) << 26;  // 32-row fp4 tiles with 32-bit offsets
        if (k_lo->stride_s >= lim || v_lo->stride_s >= lim || k_lo_scale->stride_s >= lim ||
            v_lo_scale->stride_s >= lim)
            return fail(ATTN_ERR_INVALID_ARG, "fp4 span row strides must be below 64 MiB");
    }
    if (q->dtype != ATTN_BF16 || out->dtype != ATTN_BF16)
        return fail(ATTN_ERR_UNSUPPORTED, "mixed decode takes bf16 q and out");
    if (d != 128 || !mfma_head_ratio(Hq / Hkv))
        return fail(ATTN_ERR_UNSUPPORTED, "mixed decode supports d = 128 and Hq/Hkv in {1, 2, 4, 8} (got %d, %d)", d,
                    Hq / Hkv);

    int a[3] = {0, 0, 0};
    if ((!num_splits_hi && L_hi_cap) || (!num_splits_mid && L_mid_cap) || (!num_splits_lo && L_lo_cap)) {
        if (attn_decode_mixed3_splits(B, Hkv, L_hi_cap, L_mid_cap, L_lo_cap, &a[0], &a[1], &a[2]) <= 0)
            return fail(ATTN_ERR_HIP, "could not query the device for the split plan");
    }
    const Plan ph = L_hi_cap ? plan_splits(L_hi_cap, num_splits_hi ? num_splits_hi : a[0]) : Plan{kChunkQuantum, 0};
    const Plan pm = L_mid_cap ? plan_splits(L_mid_cap, num_splits_mid ? num_splits_mid : a[1]) : Plan{kChunkQuantum, 0};
    const Plan pl = L_lo_cap ? plan_splits(L_lo_cap, num_splits_lo ? num_splits_lo : a[2]) : Plan{kChunkQuantum, 0};

    attn::DecodeParams p = two_span_params(q, B, Hq, Hkv, d, softmax_scale, k_mid_scale, v_mid_scale);
    p.S0 = ph.S;
    p.S1 = ph.S + pm.S;
    p.sp0 = span_of(k_hi, v_hi, hi_lens, Hkv, L_hi_cap, ph.chunk);
    p.sp1 = span_of(k_mid, v_mid, mid_lens, Hkv, L_mid_cap, pm.chunk);
    p.sp2 = span_of(k_lo, v_lo, lo_lens, Hkv, L_lo_cap, pl.chunk);  // strides of byte tensors: bytes
    if (L_lo_cap) {
        p.sp2.k_sc = k_lo_scale->data;
        p.sp2.ksc_sb = k_lo_scale->stride_b;
        p.sp2.ksc_sh = k_lo_scale->stride_h;
        p.sp2.ksc_ss = k_lo_scale->stride_s;
        p.sp2.v_sc = v_lo_scale->data;
        p.sp2.vsc_sb = v_lo_scale->stride_b;
        p.sp2.vsc_sh = v_lo_scale->stride_h;
        p.sp2.vsc_ss = v_lo_scale->stride_s;
    }
    return two_span_launch(p, ph.S + pm.S + pl.S, kPrecBf16, kPrecFp8, out, lse, workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream), kPrecFp4);
}

int attn_decode_pi_splits(int B, int Hkv, int L_cap, int window, int period, int kv_dtype, int* splits_window,
                          int* splits_skip) {
    if (B <= 0 || Hkv <= 0 || L_cap <= 0 || window < 0 || period < 0 || !elem_size(kv_dtype)) return 0;
    if (window > L_cap) window = L_cap;  // a window past the cache is the whole cache
    const PiCaps c = pi_caps(L_cap, window, period);
    // both spans hold the same dtype: split in proportion to their keys
    return two_span_splits(B, Hkv, c.window, 1.0, c.skip, 1.0, splits_window, splits_skip);
}

attn_status attn_decode_pi(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, const float* k_scale,
                           const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int d, int L_cap,
                           float softmax_scale, int window, int period, const float* alpha,
                           int num_splits_window, int num_splits_skip, attn_tensor* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = 0;
    attn_status st;
    if ((st = check_tensor(q, "q", true)) || (st = check_tensor(k, "k", true)) || (st = check_tensor(v, "v", true)) ||
        (st = check_tensor(out, "out", false)))
        return st;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || L_cap <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d L_cap=%d)", B, Hq, Hkv, d,
                    L_cap);
    if (B > 65535 || Hkv > 65535) return fail(ATTN_ERR_INVALID_ARG, "B and Hkv must be <= 65535");
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (window < 0 || period < 0) return fail(ATTN_ERR_INVALID_ARG, "window and period must be >= 0");
    if (num_splits_window < 0 || num_splits_skip < 0) return fail(ATTN_ERR_INVALID_ARG, "split counts must be >= 0");
    if (isnan(softmax_scale) || isinf(softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale not finite");
    if (k->dtype != v->dtype) return fail(ATTN_ERR_INVALID_ARG, "k and v dtypes differ");
    const bool fp8 = k->dtype == ATTN_FP8_E4M3;
    if (fp8 && (!k_scale || !v_scale)) return fail(ATTN_ERR_INVALID_ARG, "fp8 k/v need k_scale and v_scale");
    if (!fp8 && (k_scale || v_scale)) return fail(ATTN_ERR_INVALID_ARG, "scales are only for fp8 k/v");
    if (q->dtype != ATTN_BF16 || out->dtype != ATTN_BF16 || (k->dtype != ATTN_BF16 && !fp8))
        return fail(ATTN_ERR_UNSUPPORTED, "pi decode takes bf16 q and out, bf16 or fp8 k/v");
    if ((d != 64 && d != 128) || !mfma_head_ratio(Hq / Hkv))
        return fail(ATTN_ERR_UNSUPPORTED, "pi decode supports d in {64, 128} and Hq/Hkv in {1, 2, 4, 8} (got %d, %d)", d,
                    Hq / Hkv);
    if (window > L_cap) window = L_cap;  // same keys; keeps window arithmetic in range

    const PiCaps c = pi_caps(L_cap, window, period);
    int auto_w = 0, auto_s = 0;
    if (!num_splits_window || (!num_splits_skip && c.skip)) {
        if (attn_decode_pi_splits(B, Hkv, L_cap, window, period, k->dtype, &auto_w, &auto_s) <= 0)
            return fail(ATTN_ERR_HIP, "could not query the device for the split plan");
    }
    const Plan pw = plan_splits(c.window, num_splits_window ? num_splits_window : auto_w);
    const Plan ps = c.skip ? plan_splits(c.skip, num_splits_skip ? num_splits_skip : auto_s) : Plan{kChunkQuantum, 0};

    attn::DecodeParams p = two_span_params(q, B, Hq, Hkv, d, softmax_scale, k_scale, v_scale);
    p.S0 = pw.S;
    p.sp0 = span_of(k, v, kv_lens, 0, L_cap, pw.chunk);
    p.sp0.geom = attn::kGeomWindow;
    p.sp0.window = window;
    p.sp1 = span_of(k, v, kv_lens, 0, L_cap, ps.chunk);
    p.sp1.geom = attn::kGeomSkip;
    p.sp1.window = window;
    p.sp1.period = period > 0 ? period : 1;
    p.alpha = alpha;
    if (alpha) {
        p.sp0.prior = 1;  // ln(alpha) on the window's logits
        p.sp1.prior = 2;  // ln(1 - alpha) on the skip keys' logits
    }
    return two_span_launch(p, pw.S + ps.S, fp8 ? kPrecFp8 : kPrecBf16, fp8 ? kPrecFp8 : kPrecBf16, out, lse,
                           workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream));
}

attn_status attn_prefill(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, int B, int Hq, int Hkv,
                         int d, int Lq, int Lkv, float softmax_scale, int causal, attn_tensor* out, float* lse,
                         void* stream) {
    g_last_error[0] = 0;
    attn_status st = check_prefill(q, k, v, out, B, Hq, Hkv, d, Lq, Lkv, softmax_scale, causal, true);
    if (st != ATTN_OK) return st;
    attn::PrefillParams p = prefill_params(q, k, v, out, lse, B, Hq, Hkv, d, Lq, Lkv, softmax_scale, causal);
    hipError_t e;
    if (q->dtype == ATTN_BF16) e = attn::launch_prefill(p, static_cast<hipStream_t>(stream));
    else e = attn::launch_prefill_valu(p, attn::DT_F32, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}

size_t attn_prefill_pi_workspace_size(int B, int Hq, int L, int d) {
    if (B <= 0 || Hq <= 0 || L <= 0 || d <= 0) return 0;
    return round_up((size_t)B * Hq * L * 4, 256);  // the window part's lse
}

attn_status attn_prefill_pi(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, int B, int Hq, int Hkv,
                            int d, int L, float softmax_scale, int causal, int window, int period, const float* alpha,
                            attn_tensor* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = 0;
    attn_status st = check_prefill(q, k, v, out, B, Hq, Hkv, d, L, L, softmax_scale, 1);
    if (st != ATTN_OK) return st;
    if (window < 0 || period < 0) return fail(ATTN_ERR_INVALID_ARG, "window and period must be >= 0");
    if (window > L) window = L;  // same keys; keeps window arithmetic in range
    if (!causal && 2LL * window > 0x7fffffff) return fail(ATTN_ERR_UNSUPPORTED, "two-sided window too long");
    if (period > 0 && ((int64_t)period * q->stride_s >= (1 << 24) || (int64_t)period * k->stride_s >= (1 << 24) ||
                       (int64_t)period * v->stride_s >= (1 << 24)))
        return fail(ATTN_ERR_UNSUPPORTED, "period * q/k/v row stride must be below 2^24 elements");
    const size_t need = attn_prefill_pi_workspace_size(B, Hq, L, d);
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is null");
    if (!aligned16(workspace)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
    float* lse_w = static_cast<float*>(workspace);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // some query has a key farther than the window (below it, or on either side)
    const bool has_skip = period > 0 && L > window + 1;

    // 1. the window: keys [i - window, i] of query i (two-sided: [i - window,
    // i + window], a band of 2 window + 1 keys ending at position i + window).
    // With skip keys to come, its lse goes to the workspace and the skip
    // launches merge; without, it applies the prior itself.
    attn::PrefillParams pw = prefill_params(q, k, v, out, has_skip ? lse_w : lse, B, Hq, Hkv, d, L, L, softmax_scale, 1);
    pw.band = 1;
    pw.diag = causal ? 0 : window;
    pw.window = causal ? window : 2 * window;
    pw.merge = (!has_skip && alpha) ? 2 : 0;
    pw.alpha = alpha;
    hipError_t e = attn::launch_prefill(pw, hs);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    if (!has_skip) return ATTN_OK;

    // 2. the skip keys: for each residue class r of the positions mod period,
    // queries r, r + period, ... against keys r, r + period, ...; query m of
    // the class sees keys m' <= m - delta (positions more than window below)
    // and, two-sided, keys m' >= m + delta (more than window above). Classes
    // are the batch of banded launches over strided views; the first L %
    // period classes have one row more than the others. Each row's epilogue
    // merges its skip part with what `out` already holds: the window part
    // (merge 1), or, for the keys above, the window and the keys below
    // (merge 3; the keys below then leave their merged lse in the workspace).
    const int delta = window / period + 1;
    const int n = L / period, rem = L % period;
    for (int b = 0; b < B; ++b) {
        for (int part = 0; part < 2; ++part) {
            const int r0 = part ? rem : 0;
            const int ncls = part ? period - rem : rem;
            const int nrows = part ? n : n + 1;
            if (ncls <= 0 || nrows <= 0) continue;
            attn::PrefillParams ps = pw;
            ps.q = static_cast<const uint16_t*>(q->data) + b * q->stride_b + r0 * q->stride_s;
            ps.q_sb = q->stride_s;
            ps.q_ss = (int64_t)period * q->stride_s;
            ps.k = static_cast<const uint16_t*>(k->data) + b * k->stride_b + r0 * k->stride_s;
            ps.k_sb = k->stride_s;
            ps.k_ss = (int64_t)period * k->stride_s;
            ps.v = static_cast<const uint16_t*>(v->data) + b * v->stride_b + r0 * v->stride_s;
            ps.v_sb = v->stride_s;
            ps.v_ss = (int64_t)period * v->stride_s;
            ps.out = static_cast<uint16_t*>(out->data) + b * out->stride_b + r0 * out->stride_s;
            ps.o_sb = out->stride_s;
            ps.o_ss = (int64_t)period * out->stride_s;
            // lse, lse_w and alpha are [B, Hq, L] contiguous: the same class view
            const int64_t base = (int64_t)b * Hq * L + r0;
            float* lse_final = lse ? lse + base : nullptr;
            ps.lse_w = lse_w + base;
            ps.alpha = alpha ? alpha + base : nullptr;
            ps.lse_sb = 1;
            ps.lse_sh = L;
            ps.lse_ss = period;
            ps.B = ncls;
            ps.Lq = ps.Lkv = nrows;
            // keys below: [0, m - delta]
            const bool above = !causal && delta <= nrows - 1;  // some row has keys above
            ps.lse = above ? lse_w + base : lse_final;
            ps.diag = -delta;
            ps.window = -1;
            ps.merge = 1;
            e = attn::launch_prefill(ps, hs);
            if (e != hipSuccess) return fail(ATTN_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
            if (!above) continue;
            // keys above: [m + delta, nrows - 1], a band ending at position m + nrows
            ps.lse = lse_final;
            ps.diag = nrows;
            ps.window = nrows - delta;
            ps.merge = 3;
            e = attn::launch_prefill(ps, hs);
            if (e != hipSuccess) return fail(ATTN_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
        }
    }
    return ATTN_OK;
}

size_t attn_prefill_backward_workspace_size(int B, int Hq, int Lq) {
    if (B <= 0 || Hq <= 0 || Lq <= 0) return 0;
    return round_up((size_t)B * Hq * Lq * 4, 256);
}

attn_status attn_prefill_backward(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                  const attn_tensor* out, const float* lse, const attn_tensor* dout, int B, int Hq,
                                  int Hkv, int d, int Lq, int Lkv, float softmax_scale, int causal, attn_tensor* dq,
                                  attn_tensor* dk, attn_tensor* dv, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    g_last_error[0] = 0;
    attn_status st;
    if ((st = check_prefill(q, k, v, out, B, Hq, Hkv, d, Lq, Lkv, softmax_scale, causal))) return st;
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "the backward takes d = 128 (got d = %d)", d);
    if ((st = check_tensor(dout, "dout", true)) || (st = check_tensor(dq, "dq", false)) ||
        (st = check_tensor(dk, "dk", false)) || (st = check_tensor(dv, "dv", false)))
        return st;
    if (!lse) return fail(ATTN_ERR_INVALID_ARG, "lse (from the forward pass) is required");
    if ((Lq + 63) / 64 > 65535 || (Lkv + 63) / 64 > 65535)
        return fail(ATTN_ERR_UNSUPPORTED, "backward supports up to 65535 blocks of 64 positions");
    if (dout->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "dout must be bf16");
    if (dq->dtype != dk->dtype || dq->dtype != dv->dtype || (dq->dtype != ATTN_BF16 && dq->dtype != ATTN_F32))
        return fail(ATTN_ERR_UNSUPPORTED, "dq, dk and dv must all be bf16 or all fp32");
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is null");
    if (!aligned16(workspace)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    const size_t need = attn_prefill_backward_workspace_size(B, Hq, Lq);
    if (workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
    const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
    attn::BackwardParams p;
    p.q = q->data;
    p.q_sb = q->stride_b;
    p.q_sh = q->stride_h;
    p.q_ss = q->stride_s;
    p.k = k->data;
    p.k_sb = k->stride_b;
    p.k_sh = k->stride_h;
    p.k_ss = k->stride_s;
    p.v = v->data;
    p.v_sb = v->stride_b;
    p.v_sh = v->stride_h;
    p.v_ss = v->stride_s;
    p.o = out->data;
    p.o_sb = out->stride_b;
    p.o_sh = out->stride_h;
    p.o_ss = out->stride_s;
    p.dout = dout->data;
    p.do_sb = dout->stride_b;
    p.do_sh = dout->stride_h;
    p.do_ss = dout->stride_s;
    p.lse = lse;
    p.delta = static_cast<float*>(workspace);
    p.dq = dq->data;
    p.dq_sb = dq->stride_b;
    p.dq_sh = dq->stride_h;
    p.dq_ss = dq->stride_s;
    p.dk = dk->data;
    p.dk_sb = dk->stride_b;
    p.dk_sh = dk->stride_h;
    p.dk_ss = dk->stride_s;
    p.dv = dv->data;
    p.dv_sb = dv->stride_b;
    p.dv_sh = dv->stride_h;
    p.dv_ss = dv->stride_s;
    p.grad_dtype = dq->dtype == ATTN_BF16 ? attn::DT_BF16 : attn::DT_F32;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.d = d;
    p.Lq = Lq;
    p.Lkv = Lkv;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = sc * kLog2e;
    hipError_t e = attn::launch_backward(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}

}  // extern "C"
