// Prefill on the vector ALUs: the general (slow) path for what the MFMA
// kernel does not take -- fp32 inputs (head dim 64 or 128). Same operation as prefill.hip (every query dotted with the keys
// it may see, a max-subtracted softmax, the weighted mean of the values:
// glossary page "Attention", section on Query/Key/Value; the stability step of
// the "Attention in SRAM on Tenstorrent Grayskull" explainer, section 3), the
// same bottom-right causal alignment and the same (out, lse) outputs.
//
// One wave per query row, lanes over the head dim (D/64 elements each). Keys
// are taken one at a time: the dot product is reduced across the wave with
// butterfly shuffles and folded into a running (max, sum, accumulator).
#include "internal.h"

namespace attn {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
    return (float)x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_valu_kernel(PrefillParams p) {
    constexpr int E = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int h = blockIdx.y, b = blockIdx.z;
    if (i >= p.Lq) return;  // whole waves leave together
    const int g = h / (p.Hq / p.Hkv);
    const T* qrow = static_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)i * p.q_ss;
    const T* kbase = static_cast<const T*>(p.k) + b * p.k_sb + g * p.k_sh;
    const T* vbase = static_cast<const T*>(p.v) + b * p.v_sb + g * p.v_sh;
    float q[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        q[e] = to_f32(qrow[lane + 64 * e]);
        acc[e] = 0.f;
    }
    // keys 0 .. hi - 1 are visible (bottom-right causal alignment)
    const int hi = p.causal ? min(p.Lkv, max(0, p.Lkv - p.Lq + i + 1)) : p.Lkv;
    float m = kNegInf, l = 0.f;
    for (int j = 0; j < hi; ++j) {
        const T* krow = kbase + (int64_t)j * p.k_ss;
        const T* vrow = vbase + (int64_t)j * p.v_ss;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) part = fmaf(q[e], to_f32(krow[lane + 64 * e]), part);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        const float s = part * p.scale_log2;  // base-2 units
        const float m_new = fmaxf(m, s);
        const float alpha = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
        const float w = __builtin_amdgcn_exp2f(s - m_new);
        l = fmaf(l, alpha, w);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(acc[e], alpha, w * to_f32(vrow[lane + 64 * e]));
        m = m_new;
    }
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    T* orow = static_cast<T*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_ss;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[lane + 64 * e] = (T)(acc[e] * inv);
    if (p.lse && lane == 0)
        p.lse[b * p.lse_sb + h * p.lse_sh + (int64_t)i * p.lse_ss] = empty ? kNegInf : m * kLn2 + logf(l);
}

}  // namespace

hipError_t launch_prefill_valu(const PrefillParams& p, int dtype, hipStream_t stream) {
    const dim3 grid((p.Lq + 3) / 4, p.Hq, p.B);
    if (dtype == DT_F32 && p.d == 128)
        hipLaunchKernelGGL((prefill_valu_kernel<float, 128>), grid, dim3(256), 0, stream, p);
    else if (dtype == DT_F32 && p.d == 64)
        hipLaunchKernelGGL((prefill_valu_kernel<float, 64>), grid, dim3(256), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
