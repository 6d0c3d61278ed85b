// Level-2 merge of split-KV partials: the global step of the two-level
// log-sum-exp tree (the reduction along the sequence axis of the explainer of
// "Tree Attention: Topology-aware Decoding for Long-Context Attention on GPU
// Clusters", section 3; "exact, not approximate", its section 2).
//
// For a row with partials (o_s, m_s, l_s), s < n:
//   m = max_s m_s,  w_s = exp(m_s - m),
//   O = sum_s w_s o_s / sum_s w_s l_s,  lse = m + ln sum_s w_s l_s.
// Workgroup (r, 32-dim block): 8 lane groups of 32 threads each take every 8th
// partial in order; the 8 group sums are then added as a fixed balanced tree,
// so the result is deterministic for a given n.
#include "internal.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(256) void combine_partials_kernel(CombineParams p) {
    const int r = blockIdx.x;
    const int c0 = blockIdx.y * 32;
    const int tid = threadIdx.x;
    const int b = r / p.Hq, h = r % p.Hq;
    int n = p.S;
    if (p.kv_lens) {
        const int len = min(max(p.kv_lens[b], 0), p.L_cap);
        n = min((len + p.chunk - 1) / p.chunk, p.S);
    }
    const float* m_row = p.m_part + (int64_t)r * p.S;
    const float* l_row = p.l_part + (int64_t)r * p.S;

    __shared__ float red[256];
    float mx = kNegInf;
    for (int s = tid; s < n; s += 256) mx = fmaxf(mx, m_row[s]);
    red[tid] = mx;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();

    const int grp = tid >> 5, c = c0 + (tid & 31);
    const int cc = min(c, p.d - 1);  // lanes past d read a valid column and discard it
    const float* o_col = p.o_part + (int64_t)r * p.S * p.d + cc;
    float ao = 0.f, al = 0.f;
    auto step = [&](float ms, float ls, float os) {
        const float wgt = (ms == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((ms - mx) * kLog2e);
        al = fmaf(wgt, ls, al);
        ao = fmaf(wgt, os, ao);
    };
    if (mx != kNegInf) {
        // the group's partials s = grp, grp + 8, ... in order; loads for eight
        // of them are issued before their terms are added (the adds keep the
        // same order, so the result does not depend on the unrolling)
        int s = grp;
        for (; s + 56 < n; s += 64) {
            float ms[8], ls[8], os[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ms[i] = m_row[s + 8 * i];
                ls[i] = l_row[s + 8 * i];
                os[i] = o_col[(int64_t)(s + 8 * i) * p.d];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) step(ms[i], ls[i], os[i]);
        }
        for (; s < n; s += 8) step(m_row[s], l_row[s], o_col[(int64_t)s * p.d]);
    }
    __shared__ float red_o[8][32];
    __shared__ float red_l[8];
    red_o[grp][tid & 31] = ao;
    if ((tid & 31) == 0) red_l[grp] = al;
    __syncthreads();
    if (grp == 0 && c < p.d) {
        const int j = tid & 31;
        const float so = ((red_o[0][j] + red_o[1][j]) + (red_o[2][j] + red_o[3][j])) +
                         ((red_o[4][j] + red_o[5][j]) + (red_o[6][j] + red_o[7][j]));
        const float sl = ((red_l[0] + red_l[1]) + (red_l[2] + red_l[3])) + ((red_l[4] + red_l[5]) + (red_l[6] + red_l[7]));
        const bool empty = (mx == kNegInf) || !(sl > 0.f);
        const float val = empty ? 0.f : so / sl;
        const int64_t off = b * p.out_sb + h * p.out_sh + c;
        if (p.out_dtype == DT_BF16) static_cast<uint16_t*>(p.out)[off] = f32_to_bf16_rne(val);
        else static_cast<float*>(p.out)[off] = val;
        if (p.lse && blockIdx.y == 0 && j == 0) p.lse[r] = empty ? kNegInf : mx + logf(sl);
    }
}

}  // namespace

// Zero-fill of `n16` 16-byte words (a kernel rather than a memset, so that
// the clear is an ordinary kernel node when a caller captures the stream).
__global__ __launch_bounds__(256) void zero16_kernel(uint4* p, size_t n16) {
    for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
    if (bytes % 16 || reinterpret_cast<uintptr_t>(p) % 16) return hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const size_t blocks = (n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024;
    hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<uint4*>(p), n16);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
    dim3 grid(p.R, (p.d + 31) / 32);
    hipLaunchKernelGGL(combine_partials_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace attn
