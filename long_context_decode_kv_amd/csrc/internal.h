// Internal interfaces between the C-ABI front end (api.cpp) and the HIP
// kernels. Nothing here is exported from libattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

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
};

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
    float* lse;  // [B, Hq, Lq] or nullptr
    int B, Hq, Hkv, d, Lq, Lkv;
    int causal;
    float scale_log2;
};

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, int q_dtype, int kv_dtype, int G, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

}  // namespace attn
