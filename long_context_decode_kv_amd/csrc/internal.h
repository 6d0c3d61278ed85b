// Internal interfaces between the C-ABI front end (api.cpp) and the HIP
// kernels. Nothing here is exported from libattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

// One span of a KV cache: [B, Hkv, L_cap, d] K and V with element strides,
// valid lengths L_b = kv_lens[b*lens_sb + g*lens_sh] (or nullptr: all L_cap).
// The keys a span visits follow from L_b and `geom`, and are cut into splits
// of `chunk` keys:
//   kGeomAll:    rows [0, L_b);
//   kGeomWindow: for a query at position i = L_b - 1, rows [max(0, i - window), i];
//   kGeomSkip:   rows below i - window that are a whole number of periods from
//                i, in increasing order r, r + period, ... (r = i mod period).
// `prior` selects the log-prior added to the span's logits per query head:
// 0 none, 1 ln(alpha), 2 ln(1 - alpha), alpha from DecodeParams::alpha.
enum { kGeomAll = 0, kGeomWindow = 1, kGeomSkip = 2 };
struct KvSpan {
    const void* k;
    int64_t k_sb, k_sh, k_ss;
    const void* v;
    int64_t v_sb, v_sh, v_ss;
    const int32_t* kv_lens;
    int lens_sb, lens_sh;
    int L_cap;
    int chunk;
    int geom, window, period;
    int prior;
    // MX fp4 spans only (k and its strides above are then in bytes): the E8M0
    // block scales, 4 bytes per row (d = 128), strides in bytes
    const void* k_sc;
    int64_t ksc_sb, ksc_sh, ksc_ss;
    const void* v_sc;
    int64_t vsc_sb, vsc_sh, vsc_ss;
};

// One split-KV decode launch: grid (S, Hkv, B); workgroup (s, g, b) owns keys
// [s*chunk, min((s+1)*chunk, L_b)) of KV head g of sequence b and writes one
// partial (o, m, l) for each of the G query heads of that group.
struct DecodeParams {
    const void* q;
    int64_t q_sb, q_sh;
    const void* k;
    int64_t k_sb, k_sh, k_ss;
    const void* v;
    int64_t v_sb, v_sh, v_ss;
    const float* k_scale;  // fp8 only, [B*Hkv]
    const float* v_scale;  // fp8 only, [B*Hkv]
    const int32_t* kv_lens;  // [B] or nullptr
    int B, Hq, Hkv, d, L_cap;
    int chunk;         // keys per split (multiple of 64)
    int S;             // splits in the grid; row stride of the partial arrays
    float scale_log2;  // softmax scale * log2(e): scores are kept in base-2 units
    float* o_part;     // [B*Hq, S, d]
    float* m_part;     // [B*Hq, S], natural-log units
    float* l_part;     // [B*Hq, S]
    // Fused level 2 (decode_mfma only): when `counters` is set, the last
    // workgroup of each (b, g) to finish merges that group's partials and
    // writes the normalised output itself.
    uint32_t* counters;  // ticket lines (see kCounterBytes), zero on entry, left zero on exit
    int ticket_block;    // splits per first-level ticket block
    float* blk_o;        // block partials [B*Hq, kMaxTicketBlocks, d]
    float* blk_m;        // [B*Hq, kMaxTicketBlocks]
    float* blk_l;        // [B*Hq, kMaxTicketBlocks]
    void* out;           // [B, Hq, 1, d] bf16
    int64_t out_sb, out_sh;
    float* lse;          // [B*Hq] or nullptr
    // Two-span launches (launch_decode_mfma_two; k, v, kv_lens, L_cap and
    // chunk above are then unused): splits [0, S0) read span sp0, splits
    // [S0, S) span sp1; every split publishes a partial and all S partials of
    // a row are merged.
    int S0;
    KvSpan sp0, sp1;
    const float* alpha;  // [B*Hq] gate of the spans' log-priors, or nullptr
    // Three-span launches (launch_decode_mfma_three): splits [S0, S1) read
    // sp1 and splits [S1, S) span sp2.
    int S1;
    KvSpan sp2;
};

// Bytes at the start of a decode workspace reserved for the fused-merge
// tickets. Each (batch, KV head) group owns 1 + kMaxTicketBlocks counters:
// one per block of splits and one for the group; each counter sits alone in a
// 256-byte line (tickets on one address are served one after another, so the
// two levels keep that queue short).
constexpr size_t kCounterBytes = 4 << 20;
constexpr int kCounterStride = 64;  // uint32 per counter line
constexpr int kMaxTicketBlocks = 16;
constexpr int kMaxCounterGroups = (int)(kCounterBytes / (4 * kCounterStride * (1 + kMaxTicketBlocks)));
// Largest split count whose merge is fused into the decode kernel.
constexpr int kMaxFusedSplits = 256;

// Sets the calling thread's attn_last_error() message.
void set_last_error(const char* fmt, ...);
// attn_decode on a given workspace; clear_counter_bytes > 0 zeroes that many
// bytes of the counter block first when the launch takes the fused merge.
attn_status decode_impl(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, const float* k_scale,
                        const float* v_scale, const int32_t* kv_lens, int B, int Hq, int Hkv, int d, int L_cap,
                        float softmax_scale, int causal, int num_splits, attn_tensor* out, float* lse,
                        void* workspace, size_t workspace_bytes, size_t clear_counter_bytes, void* stream);

// Level-2 merge: one output row per (b, h) from its partials.
struct CombineParams {
    const float* o_part;
    const float* m_part;
    const float* l_part;
    int R, S, d;
    int Hq;  // row r = b*Hq + h
    // Partials to read per row: ceil(clamp(kv_lens[b], 0, L_cap) / chunk) when
    // kv_lens is set, otherwise S.
    const int32_t* kv_lens;
    int chunk, L_cap;
    void* out;
    int out_dtype;
    int64_t out_sb, out_sh;
    float* lse;  // [R] or nullptr
};

struct PrefillParams {
    const void* q;
    int64_t q_sb, q_sh, q_ss;
    const void* k;
    int64_t k_sb, k_sh, k_ss;
    const void* v;
    int64_t v_sb, v_sh, v_ss;
    void* out;
    int64_t o_sb, o_sh, o_ss;
    float* lse;  // element (b, h, i) at b*lse_sb + h*lse_sh + i*lse_ss, or nullptr
    int64_t lse_sb, lse_sh, lse_ss;
    int B, Hq, Hkv, d, Lq, Lkv;
    int causal;
    float scale_log2;
    // Banded variant (band != 0): query i sits at position i + diag and sees
    // keys [position - window, position] (window < 0: no lower bound).
    int band, diag, window;
    // Banded epilogue for pi-Attention (lse_w and alpha use the lse strides):
    // merge 0: plain; 1: this launch computes the skip part of its rows and
    // merges it with the window part already in `out` (its lse in lse_w),
    // the parts weighted by the priors ln(alpha) and ln(1 - alpha);
    // 2: the window part alone, shifted by ln(alpha); 3: as 1, but the part in
    // `out` / lse_w already carries its priors (the window and the other
    // skip keys of a two-sided row), so only ln(1 - alpha) is added here.
    int merge;
    const float* lse_w;
    const float* alpha;  // or nullptr: no prior
};

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int G, hipStream_t stream);
// Two-span decode: fp8_0 / fp8_1 give the KV dtype of sp0 / sp1 (bf16 or fp8).
// Span precisions: 0 bf16, 1 fp8-e4m3, 2 MX fp4.
hipError_t launch_decode_mfma_two(const DecodeParams& p, int prec0, int prec1, hipStream_t stream);
// Three spans in one launch: bf16, fp8-e4m3 and MX fp4 (precisions 0, 1, 2).
hipError_t launch_decode_mfma_three(const DecodeParams& p, int prec0, int prec1, int prec2, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, int q_dtype, int kv_dtype, int G, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
// Zeroes `bytes` (a multiple of 16) at 16-byte aligned device address `p`.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
// Vector-ALU prefill: fp32 with d = 64 or 128, bf16 with d = 64 (dtype DT_F32 or DT_BF16).
hipError_t launch_prefill_valu(const PrefillParams& p, int dtype, hipStream_t stream);

// Backward pass of (causal or full) attention, bf16 inputs, d = 128.
struct BackwardParams {
    const void* q;
    int64_t q_sb, q_sh, q_ss;
    const void* k;
    int64_t k_sb, k_sh, k_ss;
    const void* v;
    int64_t v_sb, v_sh, v_ss;
    const void* o;  // the forward output
    int64_t o_sb, o_sh, o_ss;
    const void* dout;
    int64_t do_sb, do_sh, do_ss;
    const float* lse;  // [B, Hq, Lq] contiguous, from the forward
    float* delta;      // [B, Hq, Lq] workspace: rowsum(dO * O)
    void* dq;
    int64_t dq_sb, dq_sh, dq_ss;
    void* dk;
    int64_t dk_sb, dk_sh, dk_ss;
    void* dv;
    int64_t dv_sb, dv_sh, dv_ss;
    int grad_dtype;  // DT_BF16 or DT_F32 for dq, dk, dv
    int B, Hq, Hkv, d, Lq, Lkv;
    int causal;
    float scale_log2;
};
hipError_t launch_backward(const BackwardParams& p, hipStream_t stream);


}  // namespace attn
