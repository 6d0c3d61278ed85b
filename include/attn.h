/*
 * attn.h -- C ABI of libattn.so: exact scaled-dot-product softmax attention on
 * AMD Instinct MI355X (gfx950).
 *
 *   O = softmax(sigma * Q K^T + mask) V,  sigma = 1/sqrt(d) unless given.
 *
 * What is computed, and where the pages define it:
 *  - Attention itself: every query is dotted with every key, the scores are
 *    normalised by a softmax and used to average the values (glossary page
 *    "Attention", section on Query/Key/Value). The result is exact, not an
 *    approximation (explainer of "Tree Attention: Topology-aware Decoding for
 *    Long-Context Attention on GPU Clusters", section 2).
 *  - Decode splits the key/value sequence into chunks; each chunk yields a
 *    partial result that a reduction along the sequence axis merges into the
 *    exact answer (same Tree Attention explainer, sections 1 and 3). On one GPU
 *    the chunks are workgroups and the reduction is a two-level tree: LDS inside
 *    a workgroup, then global memory across workgroups.
 *  - Score scaling and softmax are fused with the matrix products so that the
 *    score matrix never travels to DRAM ("Attention in SRAM on Tenstorrent
 *    Grayskull" explainer, sections 1 and 3), and the softmax subtracts the
 *    running maximum for stability (same explainer, section 3).
 *  - Decode reads a KV cache (glossary page, section on memory bandwidth and
 *    VRAM) and is bound by memory bandwidth (same section); prefill is the
 *    O(n^2) compute-bound case (glossary page, section on Self-Attention and
 *    Transformers).
 *
 * Conventions (readings where the pages are silent):
 *  - Tensors are [batch, heads, sequence, head_dim]. Strides are in ELEMENTS and
 *    the last dimension is contiguous. Head dimension d is 64 or 128.
 *  - Grouped KV heads: query head h reads KV head h / (Hq / Hkv).
 *  - Causal masking is aligned bottom-right: with Lkv keys and Lq queries, query
 *    i sits at position Lkv - Lq + i and sees keys 0 .. Lkv - Lq + i. For a
 *    single decode query this means "all keys of the sequence".
 *  - Partials use natural-log units: m = max scaled score, l = sum exp(s - m),
 *    o = sum exp(s - m) v (unnormalised). The identity is (o=0, m=-inf, l=0).
 *    A normalised (O, lse) pair is the partial (O, lse, 1).
 *  - lse (log-sum-exp of the scaled scores, natural log) is fp32; a row that
 *    sees no key gets O = 0 and lse = -inf.
 *  - fp8 is OCP E4M3 (bias 7, max 448, no infinity); the real value is
 *    code * scale with one fp32 scale per (batch, KV head), separately for K
 *    and V.
 *
 * Ownership and errors:
 *  - Every data pointer is device memory owned by the caller. The library
 *    allocates nothing and keeps no state between calls; it is thread-safe.
 *    The one exception is attn_decode_noalloc, whose scratch is a fixed
 *    array the library holds on each GPU (calls on one GPU share it).
 *  - Arguments are validated on the host before any launch; a bad argument
 *    returns an error code and launches nothing. Launches are asynchronous on
 *    `stream` (a hipStream_t; NULL = the null stream). A launch failure returns
 *    ATTN_ERR_HIP. attn_last_error() gives a message for the calling thread's
 *    most recent failure.
 *  - Determinism: same inputs, same num_splits, same device => bit-identical
 *    outputs. No floating-point atomics are used.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_API __attribute__((visibility("default")))

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shapes */
    ATTN_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for */
    ATTN_ERR_WORKSPACE = 3,   /* workspace missing or too small */
    ATTN_ERR_HIP = 4          /* the HIP runtime reported an error */
} attn_status;

typedef enum attn_dtype {
    ATTN_F32 = 0,
    ATTN_BF16 = 1,
    ATTN_FP8_E4M3 = 2,
    /* OCP MX fp4 elements (E2M1: sign, 2-bit exponent with bias 1, 1-bit
     * mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte, the
     * first of a pair in the low nibble. A tensor of this dtype is a tensor of
     * those bytes: [batch, heads, seq, d/2], strides in bytes. */
    ATTN_MXFP4 = 3,
    /* OCP MX E8M0 shared scales, one byte per 32 consecutive elements of a
     * row: the byte e stands for 2^(e - 127) (255: NaN). [batch, heads, seq,
     * d/32], strides in bytes. */
    ATTN_E8M0 = 4
} attn_dtype;

/* A strided 4-D view [batch, heads, sequence, d]; strides in elements. */
typedef struct attn_tensor {
    void* data;
    int32_t dtype; /* attn_dtype */
    int64_t stride_b, stride_h, stride_s;
} attn_tensor;

/* Human-readable name of a status code (static string). */
ATTN_API const char* attn_status_string(attn_status status);

/* Message describing the calling thread's most recent failed call ("" if none). */
ATTN_API const char* attn_last_error(void);

/*
 * Split count that attn_decode uses when num_splits == 0: a pure function of
 * the shapes, the KV storage type, whether per-sequence lengths are given
 * (ragged != 0) and the compute-unit count of the current device. Returns
 * >= 1, or 0 on a bad argument or when the device cannot be queried.
 */
ATTN_API int attn_decode_auto_splits(int B, int Hkv, int L_cap, int kv_dtype, int ragged);

/*
 * Bytes of device workspace attn_decode needs for `num_splits` splits (>= 1):
 * a fixed 4 MiB block of merge counters, the fp32 partials o [B*Hq, S, d],
 * m [B*Hq, S], l [B*Hq, S], and the same three arrays for 16 merge blocks
 * (the first level of the fused merge). 0 on a bad argument.
 */
ATTN_API size_t attn_decode_workspace_size(int B, int Hq, int d, int num_splits);

/*
 * Prepares a decode workspace for its first use: zeroes its counter block
 * with a small kernel on `stream` (asynchronous; no memset, so the call may be
 * captured in a graph). The workspace must be 16-byte aligned. A workspace
 * must be prepared once, after it
 * is allocated; every attn_decode call leaves the counters zero again, so
 * calls may reuse it with any shapes. Calls that share one workspace must be
 * ordered (the same stream, or synchronised): overlapping calls race.
 */
ATTN_API attn_status attn_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split plan of attn_decode / attn_decode_partials for a capacity of L_cap keys
 * and `num_splits` requested splits (>= 1): chunk = roundup(ceil(L_cap /
 * num_splits), 64) keys per split; returns the number of splits actually used,
 * S = ceil(L_cap / chunk) <= num_splits (the partials' row stride), and stores
 * chunk in *chunk if it is not NULL. 0 on a bad argument.
 */
ATTN_API int attn_decode_plan(int L_cap, int num_splits, int* chunk);

/*
 * Single-query decode over a KV cache (one new token per sequence): the
 * memory-bound generation step the glossary page "Attention" describes in its
 * sections on the KV cache and memory bandwidth, computed as the Tree
 * Attention explainer's sequence-axis reduction (sections 1 and 3): the cache
 * is cut into chunks (workgroups), each chunk's partial (o, m, l) is merged by
 * log-sum-exp into the exact softmax result (section 2: exact, not an
 * approximation), with the max subtracted before every exponential
 * (Grayskull explainer, section 3).
 *
 * q        [B, Hq, 1, d]      ATTN_F32 or ATTN_BF16
 * k, v     [B, Hkv, L_cap, d] same dtype as q, or ATTN_FP8_E4M3 with bf16 q
 * k_scale, v_scale  device float [B*Hkv] (index b*Hkv + g); required for fp8,
 *          must be NULL otherwise
 * kv_lens  device int32 [B]: valid keys per sequence (values are clamped to
 *          [0, L_cap]); NULL means every sequence has L_cap keys
 * softmax_scale  <= 0 selects 1/sqrt(d)
 * causal   accepted for either value; with one query aligned bottom-right the
 *          query sees every valid key, so it does not change the result
 * num_splits  0 = attn_decode_auto_splits(..., kv_lens != NULL); otherwise
 *          >= 1. The sequence is
 *          cut into chunks of roundup(ceil(L_cap/num_splits), 64) keys; a
 *          sequence of L_b keys uses ceil(L_b/chunk) of them.
 * out      [B, Hq, 1, d] same dtype as q (bf16 output is rounded to nearest even)
 * lse      device float [B*Hq] or NULL
 * workspace  device memory of at least attn_decode_workspace_size(B, Hq, d, S)
 *          bytes for the split count S in use, 16-byte aligned, prepared once
 *          by attn_decode_workspace_init. The partials are merged by a second
 *          kernel, except on the MFMA path when the launch has at most one
 *          workgroup per compute unit (B * Hkv * S <= CUs): then the last
 *          workgroup of each (sequence, KV head) merges them in the same kernel.
 *
 * q, k and v need 16-byte aligned data and strides that are multiples of 16
 * bytes. Supported: d in {64, 128}; Hq % Hkv == 0 with Hq/Hkv in {1, 2, 4, 8}.
 * bf16 q with bf16 or fp8 KV (d 64 or 128, every supported Hq/Hkv) runs on
 * MFMA; fp32 runs on the vector ALUs. On the MFMA path rows are
 * read 32 at a time with 32-bit byte offsets, so k/v row strides must be
 * below 2^26 bytes (else ATTN_ERR_INVALID_ARG). The merge is fused into the
 * decode kernel only for Hq/Hkv == 4 and d == 128.
 */
ATTN_API attn_status attn_decode(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                 const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B,
                                 int Hq, int Hkv, int d, int L_cap, float softmax_scale, int causal,
                                 int num_splits, attn_tensor* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * attn_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc. Arguments,
 * results, split plan and kernels are those of attn_decode, without the
 * workspace: the merge counters and split partials live in a fixed array of
 * 32 MiB (33,554,432 bytes) of device memory that the library holds on each
 * GPU it runs on until the process ends. The call allocates nothing (no
 * hipMalloc or allocating library routine).
 *
 * Limit: attn_decode_workspace_size(B, Hq, d, S) for the split count S in use
 * must not exceed 32 MiB (e.g. 32 query rows with up to 1024 splits, or 512
 * rows with 54); larger requests return ATTN_ERR_WORKSPACE before any launch.
 * The array keeps the previous call's contents; a call that takes the fused
 * merge first clears the counters it uses with a small kernel on `stream`.
 * All calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other threads, without ordering between them) race and give wrong
 * results. Errors otherwise as attn_decode.
 */
ATTN_API attn_status attn_decode_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                         const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B,
                                         int Hq, int Hkv, int d, int L_cap, float softmax_scale, int causal,
                                         int num_splits, attn_tensor* out, float* lse, void* stream);

/*
 * The first level of attn_decode on its own: the per-chunk partials, merged
 * inside each workgroup but not across chunks -- what one device contributes
 * before the cross-device reduction of the Tree Attention explainer (sections
 * 1 and 3). Arguments as for attn_decode, except the outputs:
 *   o_part [B*Hq, S, d], m_part [B*Hq, S], l_part [B*Hq, S]: contiguous device
 *   fp32, row r = b*Hq + h, S = attn_decode_plan(L_cap, num_splits, NULL)
 *   (num_splits = 0 selects attn_decode_auto_splits()). No workspace and no
 *   counters are involved. Splits past the end of
 *   a shorter sequence hold the identity (0, -inf, 0). *splits_used (host
 *   pointer, may be NULL) receives S.
 * attn_combine_partials(o_part, m_part, l_part, B*Hq, S, d, ...) on the result
 * gives exactly the output of attn_decode.
 */
ATTN_API attn_status attn_decode_partials(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                          const float* k_scale, const float* v_scale, const int32_t* kv_lens,
                                          int B, int Hq, int Hkv, int d, int L_cap, float softmax_scale,
                                          int causal, int num_splits, float* o_part, float* m_part,
                                          float* l_part, int* splits_used, void* stream);

/*
 * Selective mixed-precision decode: one decode over a KV cache kept in two
 * precisions, bf16 for the keys that are sensitive to quantisation and fp8
 * for the rest (the ThriftAttention page: its introduction assigns each head
 * or token a precision by its sensitivity and keeps the first and last tokens
 * of the sequence in high precision; the COMPUTE and ORCHESTRATE layers of its
 * Physical AI Stack section switch precisions inside one kernel and name the
 * first and last 10 % of the tokens). The softmax over all keys is a sum over
 * keys, so the order in which keys are stored does not change O: the cache of
 * each (sequence, KV head) is two key sets, and the result is exact attention
 * over their union, with the fp8 keys and values taken at code * scale. The
 * split partials of both spans go through one log-sum-exp merge (Tree
 * Attention explainer, section 3).
 *
 * q        [B, Hq, 1, d] bf16, d in {64, 128}, Hq/Hkv in {1, 2, 4, 8}
 * k_hi, v_hi  [B, Hkv, L_hi_cap, d] bf16: the high-precision span (may be NULL
 *          when L_hi_cap = 0)
 * hi_lens  device int32 [B, Hkv] (index b*Hkv + g): valid keys of the bf16 span
 *          per (sequence, KV head), clamped to [0, L_hi_cap]; NULL = L_hi_cap
 * k_lo, v_lo  [B, Hkv, L_lo_cap, d] ATTN_FP8_E4M3: the low-precision span (may
 *          be NULL when L_lo_cap = 0)
 * Every span's row strides must be below 2^26 bytes (rows are read 32 at a
 * time with 32-bit byte offsets); else ATTN_ERR_INVALID_ARG.
 * k_scale, v_scale  device float [B*Hkv]: the fp8 span's scales
 * lo_lens  device int32 [B, Hkv]: valid keys of the fp8 span, as hi_lens
 * L_hi_cap, L_lo_cap  >= 0, not both 0
 * num_splits_hi, num_splits_lo  requested splits of each span (planned as by
 *          attn_decode_plan); 0 takes that span's value from
 *          attn_decode_mixed_splits(). S = S_hi + S_lo splits in all.
 * out      [B, Hq, 1, d] bf16; lse device float [B*Hq] or NULL
 * workspace  attn_decode_workspace_size(B, Hq, d, S) bytes, 16-byte aligned,
 *          prepared by attn_decode_workspace_init (shared with attn_decode).
 *
 * A (sequence, KV head) with no valid key in either span gets O = 0 and lse =
 * -inf. Errors as for attn_decode; a dtype or shape outside the above returns
 * ATTN_ERR_UNSUPPORTED.
 */
ATTN_API attn_status attn_decode_mixed(const attn_tensor* q, const attn_tensor* k_hi, const attn_tensor* v_hi,
                                       const int32_t* hi_lens, int L_hi_cap, const attn_tensor* k_lo,
                                       const attn_tensor* v_lo, const float* k_scale, const float* v_scale,
                                       const int32_t* lo_lens, int L_lo_cap, int B, int Hq, int Hkv, int d,
                                       float softmax_scale, int num_splits_hi, int num_splits_lo,
                                       attn_tensor* out, float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * The same decode with the low-precision span held in OCP MX fp4, the page's
 * FP4 on this hardware (the ThriftAttention page keeps most tokens in FP4 and
 * the first and last tenth in high precision): a key or value row of d = 128
 * elements is 64 bytes of E2M1 codes plus 4 E8M0 scale bytes, one per 32
 * elements (OCP Microscaling Formats (MX) v1.0). The result is exact attention
 * over the union of the bf16 keys and the fp4 keys at code * 2^(scale - 127).
 *
 * k_lo, v_lo  [B, Hkv, L_lo_cap, d/2] ATTN_MXFP4 (16-byte aligned data and
 *          strides)
 * k_lo_scale, v_lo_scale  [B, Hkv, L_lo_cap, d/32] ATTN_E8M0, the scales of
 *          k_lo and v_lo (4-byte aligned data, strides multiples of 4 bytes)
 * Everything else as attn_decode_mixed; the split plan is that of
 * attn_decode_mixed_fp4_splits(). An fp4 span with 0 keys (L_lo_cap = 0)
 * makes this the bf16 decode.
 *
 * Range: codes are widened to fp32 with the block scale applied, then to bf16
 * for the products. Scale bytes 1 .. 252 give exact values for every code; a
 * value past the fp32 range (|code| * 2^(e - 127) >= 2^128: bytes 253 and 254
 * with the larger codes) becomes +-inf, and byte 0 (2^-127) gives fp32
 * subnormals, which the products may flush to zero. Byte 255 is NaN and makes
 * the outputs it reaches NaN, as in the definition.
 */
ATTN_API attn_status attn_decode_mixed_fp4(const attn_tensor* q, const attn_tensor* k_hi, const attn_tensor* v_hi,
                                           const int32_t* hi_lens, int L_hi_cap, const attn_tensor* k_lo,
                                           const attn_tensor* v_lo, const attn_tensor* k_lo_scale,
                                           const attn_tensor* v_lo_scale, const int32_t* lo_lens, int L_lo_cap,
                                           int B, int Hq, int Hkv, int d, float softmax_scale, int num_splits_hi,
                                           int num_splits_lo, attn_tensor* out, float* lse, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * Automatic split plan of attn_decode_mixed_fp4: as attn_decode_mixed_splits,
 * with a cost per key of 2 for bf16 and 1.1 for fp4 (measured: an fp4 key
 * costs about half a bf16 key, its widening making up for most of its fewer
 * bytes). Returns S_hi + S_lo, 0 on a bad argument or a failed device query.
 */
ATTN_API int attn_decode_mixed_fp4_splits(int B, int Hkv, int L_hi_cap, int L_lo_cap, int* splits_hi,
                                          int* splits_lo);

/*
 * Selective mixed-precision decode over a cache kept in all three precisions
 * the ThriftAttention page names (its Physical AI Stack section: BF16, FP8
 * and FP4 switched inside one kernel; the COMPUTE layer): per (sequence, KV
 * head) a bf16 span, an fp8-e4m3 span and an MX fp4 span, each with its own
 * length, in one launch (each workgroup streams one span in one precision)
 * and one log-sum-exp merge (Tree Attention explainer, section 3). The
 * result is exact attention over the union of the three key sets at their
 * real values (fp8 code * scale, fp4 code * 2^(scale - 127)).
 *
 * k_hi, v_hi, hi_lens, L_hi_cap: the bf16 span, as in attn_decode_mixed.
 * k_mid, v_mid [B, Hkv, L_mid_cap, d] ATTN_FP8_E4M3 with k_mid_scale,
 *          v_mid_scale device float [B*Hkv], mid_lens device int32 [B, Hkv]
 *          (or NULL = L_mid_cap): the fp8 span. Every span's row strides
 *          must be below 2^26 bytes.
 * k_lo, v_lo, k_lo_scale, v_lo_scale, lo_lens, L_lo_cap: the MX fp4 span, as
 *          in attn_decode_mixed_fp4.
 * A span with capacity 0 may come without tensors; not all three may be 0.
 * num_splits_*: requested splits per span, 0 = the value of
 *          attn_decode_mixed3_splits(). S = S_hi + S_mid + S_lo splits, and
 *          the workspace is attn_decode_workspace_size(B, Hq, d, S) bytes,
 *          prepared by attn_decode_workspace_init.
 * q, out, lse, softmax_scale, B, Hq, Hkv, d, stream and errors as
 * attn_decode_mixed (bf16 q and out, Hq/Hkv in {1, 2, 4, 8}), with d = 128.
 */
ATTN_API attn_status attn_decode_mixed3(const attn_tensor* q, const attn_tensor* k_hi, const attn_tensor* v_hi,
                                        const int32_t* hi_lens, int L_hi_cap, const attn_tensor* k_mid,
                                        const attn_tensor* v_mid, const float* k_mid_scale, const float* v_mid_scale,
                                        const int32_t* mid_lens, int L_mid_cap, const attn_tensor* k_lo,
                                        const attn_tensor* v_lo, const attn_tensor* k_lo_scale,
                                        const attn_tensor* v_lo_scale, const int32_t* lo_lens, int L_lo_cap, int B,
                                        int Hq, int Hkv, int d, float softmax_scale, int num_splits_hi,
                                        int num_splits_mid, int num_splits_lo, attn_tensor* out, float* lse,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Automatic split plan of attn_decode_mixed3: about two workgroups per compute
 * unit in all, shared among the three spans in proportion to keys times the
 * cost per key of the two-precision plans (2 bf16, 0.95 fp8, 1.1 fp4), no
 * split shorter than 256 keys. Stores each span's splits (host pointers, may
 * be NULL) and returns their sum; 0 on a bad argument or a failed device query.
 */
ATTN_API int attn_decode_mixed3_splits(int B, int Hkv, int L_hi_cap, int L_mid_cap, int L_lo_cap, int* splits_hi,
                                       int* splits_mid, int* splits_lo);

/*
 * Automatic split plan of attn_decode_mixed: about two workgroups per compute
 * unit of the current device in all, shared between the spans in proportion
 * to 2 * L_hi_cap and 0.95 * L_lo_cap (a measured cost per key: an fp8
 * workgroup streams its bytes more slowly than a bf16 one), no split shorter
 * than 256 keys. Stores the splits each span
 * will use (after planning) in *splits_hi and *splits_lo (host pointers, may
 * be NULL) and returns their sum; 0 on a bad argument or a failed device
 * query.
 */
ATTN_API int attn_decode_mixed_splits(int B, int Hkv, int L_hi_cap, int L_lo_cap, int* splits_hi, int* splits_lo);

/*
 * pi-Attention decode: the query of each sequence (at position i = L_b - 1)
 * attends to a structured subset of its keys inside one softmax (the
 * pi-Attention explainer, method section A):
 *  - the ring-local window: keys j with i - window <= j <= i;
 *  - the periodic skip keys: keys below the window that lie a whole number of
 *    periods from i, j = i - m * period (m >= 1), read as a strided gather;
 *  - the adaptive fusion gate as a log-prior: with alpha (clamped to [0, 1])
 *    the window's logits get + ln(alpha) and the skip keys' + ln(1 - alpha).
 * The window and the skip keys are the two spans of one launch; their split
 * partials carry the prior in their max and go through one log-sum-exp merge
 * (Tree Attention explainer, section 3), so the result is exact attention over
 * the union with those priors.
 *
 * q, k, v, k_scale, v_scale, kv_lens ([B] per sequence), softmax_scale, out,
 * lse, workspace: as attn_decode, with bf16 q/out, bf16 or fp8 k/v, d in
 * {64, 128} and Hq/Hkv in {1, 2, 4, 8}.
 * window   >= 0 keys before the query (the query's own key is always local)
 * period   >= 1, or 0 for no skip keys; period times the row stride in bytes
 *          must be below 2^26 (the skip keys are read 32 rows at a time with
 *          32-bit byte offsets), else ATTN_ERR_INVALID_ARG
 * alpha    device float [B*Hq] (row b*Hq + h) or NULL (no prior: plain
 *          attention over the union)
 * num_splits_window, num_splits_skip  requested splits per span; 0 takes the
 *          value of attn_decode_pi_splits(). S = S_window + S_skip splits, and
 *          the workspace is attn_decode_workspace_size(B, Hq, d, S) bytes.
 * A row whose keys all carry weight zero (alpha = 0 with no skip key) gets O =
 * 0 and lse = -inf.
 */
ATTN_API attn_status attn_decode_pi(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                    const float* k_scale, const float* v_scale, const int32_t* kv_lens, int B,
                                    int Hq, int Hkv, int d, int L_cap, float softmax_scale, int window, int period,
                                    const float* alpha, int num_splits_window, int num_splits_skip,
                                    attn_tensor* out, float* lse, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * Automatic split plan of attn_decode_pi for a cache of capacity L_cap: the
 * window holds at most min(window + 1, L_cap) keys and the skip keys at most
 * floor((L_cap - 2 - window) / period) + 1; about two workgroups per compute
 * unit in all, shared in proportion to those counts, no split shorter than 256
 * keys. Stores each span's splits (host pointers, may be NULL) and returns
 * their sum; 0 on a bad argument or a failed device query.
 */
ATTN_API int attn_decode_pi_splits(int B, int Hkv, int L_cap, int window, int period, int kv_dtype,
                                   int* splits_window, int* splits_skip);

/*
 * Prefill: attention of Lq queries over Lkv keys (causal or not), the O(n^2)
 * compute-bound case (glossary page "Attention", section on Self-Attention
 * and Transformers; causal = past keys only, the pi-Attention explainer's
 * method section), with matmul, scaling and softmax fused on chip as the
 * Grayskull explainer's sections 1 and 3 describe, so the
 * Lq x Lkv score matrix never reaches memory.
 *
 * q [B, Hq, Lq, d], k and v [B, Hkv, Lkv, d], out [B, Hq, Lq, d]: one dtype,
 * 16-byte aligned data and strides.
 * lse: device float [B, Hq, Lq] (contiguous) or NULL.
 * causal with Lq > Lkv is rejected (queries with no visible key).
 * bf16 with d == 64 or 128 runs on MFMA; fp32 with d == 64 or 128 runs on a
 * slower vector-ALU kernel (one wave per query row). Other combinations give
 * ATTN_ERR_UNSUPPORTED, as do q, k or v row strides (stride_s) of 2^24
 * elements or more. Hq % Hkv == 0.
 */
ATTN_API attn_status attn_prefill(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, int B,
                                  int Hq, int Hkv, int d, int Lq, int Lkv, float softmax_scale, int causal,
                                  attn_tensor* out, float* lse, void* stream);

/*
 * pi-Attention prefill (Lq = Lkv = L): query i attends to its ring-local
 * window and to its periodic skip keys in one softmax, with the gate alpha as
 * a log-prior: + ln(alpha) on the window's logits, + ln(1 - alpha) on the
 * skip keys' (the pi-Attention explainer, method section A; the oracle's
 * masked definition).
 *  causal != 0: the window is keys i - window .. i and the skip keys are
 *          i - m * period below the window (m >= 1);
 *  causal == 0 (two-sided, for tasks that also look ahead): the window is
 *          keys i - window .. i + window and the skip keys are i +- m * period
 *          outside it.
 * Computed as banded prefills: the window (two-sided: a band of 2 window + 1
 * keys), then, for each residue class of the positions modulo `period`, the
 * class's queries against the class's keys as strided views (the strided
 * gather the page names): the keys below, and two-sided also the keys above,
 * each launch's epilogue merging its part into the row by log-sum-exp (Tree
 * Attention explainer, section 3).
 *
 * q, k, v, out, lse, softmax_scale: as attn_prefill (bf16, d = 64 or 128), with
 * Lq = Lkv = L.
 * window   >= 0; period >= 1, or 0 for no skip keys. period * q/k/v row stride
 *          must be below 2^24 elements.
 * alpha    device float [B, Hq, L] contiguous (clamped to [0, 1]) or NULL (no
 *          prior).
 * workspace  attn_prefill_pi_workspace_size(B, Hq, L, d) bytes of device
 *          memory, 16-byte aligned, no preparation needed (the lse of the
 *          parts merged so far).
 * The parts pass through `out` in bf16 before the merge. A row whose keys all
 * carry weight zero (alpha = 0 with no skip key) gets O = 0 and lse = -inf.
 */
ATTN_API attn_status attn_prefill_pi(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, int B,
                                     int Hq, int Hkv, int d, int L, float softmax_scale, int causal, int window,
                                     int period, const float* alpha, attn_tensor* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Workspace bytes of attn_prefill_pi (0 on a bad argument). */
ATTN_API size_t attn_prefill_pi_workspace_size(int B, int Hq, int L, int d);

/*
 * Backward pass of attn_prefill: the gradients of a loss with respect to q, k
 * and v, given its gradient dout with respect to the output. Attention is the
 * gradient of a scalar energy function (Tree Attention explainer, section 3);
 * this differentiates the same definition once more. With logits z = sigma q.k,
 * P the softmax of each row over its visible keys and D_i = dout_i . out_i:
 *   dv_j = sum_i P_ij dout_i,   dz_ij = P_ij (dout_i . v_j - D_i),
 *   dq_i = sigma sum_j dz_ij k_j,   dk_j = sigma sum_i dz_ij q_i,
 * dk and dv summing over the query heads that share a KV head. P is
 * recomputed from `lse`; no L x L matrix is stored.
 *
 * q, k, v, softmax_scale, causal, B, Hq, Hkv, d, Lq, Lkv: as passed to
 * attn_prefill (bf16, d = 128). out and lse: what attn_prefill returned for
 * them (lse [B, Hq, Lq] contiguous, required). dout: bf16 like out.
 * dq [B, Hq, Lq, d], dk and dv [B, Hkv, Lkv, d]: all bf16 or all fp32,
 * written entirely (zero for keys no query sees); strided views allowed.
 * workspace: attn_prefill_backward_workspace_size(B, Hq, Lq) bytes of device
 * memory, 16-byte aligned, no preparation needed.
 * Deterministic: no atomics. P and dz enter the products as bf16.
 */
ATTN_API attn_status attn_prefill_backward(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                           const attn_tensor* out, const float* lse, const attn_tensor* dout, int B,
                                           int Hq, int Hkv, int d, int Lq, int Lkv, float softmax_scale, int causal,
                                           attn_tensor* dq, attn_tensor* dk, attn_tensor* dv, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Workspace bytes of attn_prefill_backward (0 on a bad argument). */
ATTN_API size_t attn_prefill_backward_workspace_size(int B, int Hq, int Lq);

/*
 * Merge S partials per row into the exact normalised result (the reduction
 * step of the Tree Attention explainer, section 3, on one device): with
 * m = max_s m_s and w_s = exp(m_s - m), O = sum_s w_s o_s / sum_s w_s l_s and
 * lse = m + ln sum_s w_s l_s, summed in an order fixed by R, S and d (each
 * lane group a strided running merge, then the groups of a wave by a
 * butterfly, then the waves in order).
 *
 * o_part [R, S, d], m_part [R, S], l_part [R, S]: contiguous device fp32.
 * out: row r of d elements at out->data + r * out->stride_s (F32 or BF16);
 * stride_b and stride_h are ignored. lse: device float [R] or NULL.
 * Rows whose partials are all the identity get O = 0 and lse = -inf.
 */
ATTN_API attn_status attn_combine_partials(const float* o_part, const float* m_part, const float* l_part, int R,
                                           int S, int d, attn_tensor* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
