// Split-KV decode on the vector ALUs for fp32 inputs (the MFMA kernel takes
// bf16 queries; the template is written over the element types, and only the
// fp32 instances are launched). Same work split and partial format as decode_mfma.hip: workgroup
// (s, g, b) owns one chunk of keys of KV head g and emits one partial
// (o, m, l) per query head of the group (explainer of "Tree Attention:
// Topology-aware Decoding for Long-Context Attention on GPU Clusters",
// section 3, done across workgroups of one GPU).
//
// Lane layout: each key row is read by D/8 consecutive lanes, 8 elements each
// (a "slot" of lanes per key), so a wave covers 64/(D/8) keys per step. The
// dot product is reduced across the slot with butterfly shuffles; each slot
// keeps its own running (m, l, o) with the max-subtracted online softmax (the
// stability step of the "Attention in SRAM on Tenstorrent Grayskull"
// explainer, section 3). Slots, then waves, are merged at the end.
#include "internal.h"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight consecutive elements of a row, widened to fp32.
template <int DT>
__device__ __forceinline__ void load8(const char* row, int elem0, float (&x)[8]) {
    if constexpr (DT == DT_F32) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(row + 4 * elem0);
        const f32x4 b = *reinterpret_cast<const f32x4*>(row + 4 * elem0 + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    } else if constexpr (DT == DT_BF16) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(row + 2 * elem0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __builtin_bit_cast(float, a[e] << 16);
            x[2 * e + 1] = __builtin_bit_cast(float, a[e] & 0xffff0000u);
        }
    } else {
        const u32x2 a = *reinterpret_cast<const u32x2*>(row + elem0);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(a[e], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(a[e], true);
            x[4 * e + 0] = lo[0];
            x[4 * e + 1] = lo[1];
            x[4 * e + 2] = hi[0];
            x[4 * e + 3] = hi[1];
        }
    }
}

template <int QDT, int KVDT, int D, int G>
__global__ __launch_bounds__(256) void decode_valu(DecodeParams p) {
    constexpr int LPT = D / 8;     // lanes per key row
    constexpr int TPW = 64 / LPT;  // keys per wave step
    constexpr int qsz = QDT == DT_F32 ? 4 : 2;
    constexpr int kvsz = KVDT == DT_F32 ? 4 : (KVDT == DT_BF16 ? 2 : 1);

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int slot = lane / LPT, part = lane % LPT;
    int L_b = p.L_cap;
    if (p.kv_lens) L_b = min(max(p.kv_lens[b], 0), p.L_cap);
    const int t_begin = s * p.chunk;
    const int t_end = min(t_begin + p.chunk, L_b);
    if (t_begin >= t_end) {
        // A split past the end of a shorter sequence: the identity partial.
        for (int i = tid; i < G * D; i += 256) {
            const int64_t row = (int64_t)b * p.Hq + g * G + i / D;
            p.o_part[(row * p.S + s) * D + i % D] = 0.f;
            if (i % D == 0) {
                p.m_part[row * p.S + s] = kNegInf;
                p.l_part[row * p.S + s] = 0.f;
            }
        }
        return;
    }

    float scale2 = p.scale_log2;
    float vsc = 1.0f;
    if constexpr (KVDT == DT_FP8) {
        scale2 *= p.k_scale[b * p.Hkv + g];
        vsc = p.v_scale[b * p.Hkv + g];
    }
    // This lane's 8 query elements of each head, pre-multiplied by the scale.
    float q[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const char* qrow = static_cast<const char*>(p.q) + (b * p.q_sb + (int64_t)(g * G + h) * p.q_sh) * qsz;
        load8<QDT>(qrow, 8 * part, q[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[h][e] *= scale2;
    }
    const char* kbase = static_cast<const char*>(p.k) + (b * p.k_sb + g * p.k_sh) * kvsz;
    const char* vbase = static_cast<const char*>(p.v) + (b * p.v_sb + g * p.v_sh) * kvsz;

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    for (int tile = t_begin + w * TPW; tile < t_end; tile += kWaves * TPW) {
        const int tok = tile + slot;
        const bool valid = tok < t_end;
        const int row = min(tok, t_end - 1);
        float kf[8], vf[8];
        load8<KVDT>(kbase + (int64_t)row * p.k_ss * kvsz, 8 * part, kf);
        load8<KVDT>(vbase + (int64_t)row * p.v_ss * kvsz, 8 * part, vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(q[h][e], kf[e], dot);
#pragma unroll
            for (int off = 1; off < LPT; off <<= 1) dot += __shfl_xor(dot, off);
            const float sc = valid ? dot : kNegInf;
            const float m_new = fmaxf(m[h], sc);
            const float alpha = (m[h] == kNegInf) ? (m_new == kNegInf ? 1.f : 0.f) : fast_exp2(m[h] - m_new);
            const float pw = (sc == kNegInf) ? 0.f : fast_exp2(sc - m_new);
            m[h] = m_new;
            l[h] = l[h] * alpha + pw;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pw, vf[e], o[h][e] * alpha);
        }
    }

    // Merge the slots of this wave (butterfly over the slot bits of the lane id).
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float M = m[h];
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float f = (m[h] == kNegInf) ? 0.f : fast_exp2(m[h] - M);
        float lw = l[h] * f;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[h][e] * f;
#pragma unroll
            for (int off = LPT; off < 64; off <<= 1) x += __shfl_xor(x, off);
            o[h][e] = x;
        }
        m[h] = M;
        l[h] = lw;
    }

    // Merge the waves in LDS.
    __shared__ float lds_o[kWaves][G][D];
    __shared__ float lds_m[kWaves][G];
    __shared__ float lds_l[kWaves][G];
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) lds_o[w][h][8 * part + e] = o[h][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            lds_m[w][h] = m[h];
            lds_l[w][h] = l[h];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int h = idx / D, c = idx % D;
        float mw[kWaves], fw[kWaves], Mx = kNegInf;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            mw[i] = lds_m[i][h];
            Mx = fmaxf(Mx, mw[i]);
        }
#pragma unroll
        for (int i = 0; i < kWaves; ++i) fw[i] = (mw[i] == kNegInf) ? 0.f : fast_exp2(mw[i] - Mx);
        const float v = (fw[0] * lds_o[0][h][c] + fw[1] * lds_o[1][h][c]) +
                        (fw[2] * lds_o[2][h][c] + fw[3] * lds_o[3][h][c]);
        const int64_t row = (int64_t)b * p.Hq + g * G + h;
        p.o_part[(row * p.S + s) * D + c] = v * vsc;
        if (c == 0) {
            p.m_part[row * p.S + s] = Mx * kLn2;
            p.l_part[row * p.S + s] =
                (fw[0] * lds_l[0][h] + fw[1] * lds_l[1][h]) + (fw[2] * lds_l[2][h] + fw[3] * lds_l[3][h]);
        }
    }
}

template <int QDT, int KVDT, int D>
hipError_t launch_g(const DecodeParams& p, int G, hipStream_t stream) {
    dim3 grid(p.S, p.Hkv, p.B);
    switch (G) {
    case 1: hipLaunchKernelGGL((decode_valu<QDT, KVDT, D, 1>), grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_valu<QDT, KVDT, D, 2>), grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_valu<QDT, KVDT, D, 4>), grid, dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_valu<QDT, KVDT, D, 8>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int QDT, int KVDT>
hipError_t launch_d(const DecodeParams& p, int G, hipStream_t stream) {
    if (p.d == 64) return launch_g<QDT, KVDT, 64>(p, G, stream);
    if (p.d == 128) return launch_g<QDT, KVDT, 128>(p, G, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, int q_dtype, int kv_dtype, int G, hipStream_t stream) {
    // bf16 queries run on the MFMA decode (decode_mfma.hip)
    if (q_dtype == DT_F32 && kv_dtype == DT_F32) return launch_d<DT_F32, DT_F32>(p, G, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
