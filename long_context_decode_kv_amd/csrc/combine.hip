// Level-2 merge of split-KV partials: the global step of the two-level
// log-sum-exp tree (the reduction along the sequence axis of the explainer of
// "Tree Attention: Topology-aware Decoding for Long-Context Attention on GPU
// Clusters", section 3; the merge is exact, as its section 2 stresses).
//
// For a row with partials (o_s, m_s, l_s), s < n:
//   m = max_s m_s,  w_s = exp(m_s - m),
//   O = sum_s w_s o_s / sum_s w_s l_s,  lse = m + ln sum_s w_s l_s.
// Workgroup (r, column block) with W = 4..16 waves. Each wave is cut into
// 64/LP lane groups of LP lanes, and each lane group -- a "slot" -- takes
// every (number of slots)-th partial in order, eight at a time, over 2*LP
// columns (two per lane), keeping its own running (max, sum, accumulator), so
// that all loads of a batch -- and those of the next batch, issued before the
// current one is added -- are in flight at once: a row of up to 128 partials
// costs one memory round trip. LP = 64 normally; launches with few rows and
// many partials use LP = 32, 16 or 8, i.e. narrower column blocks and more
// workgroups. The slots of a wave are merged by a butterfly over its lane
// groups, then the waves in LDS, each in a fixed order, so the result is
// deterministic for a given n and launch shape (which depends on R, S, d).
#include "internal.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBatch = 8;      // partials per slot per batch
constexpr int kMaxWaves = 16;  // waves per workgroup

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One batch of a slot's partials: s = s0 + NS*i, i < kBatch (clamped to
// n - 1; the clamped copies are not added).
struct Batch {
    float m[kBatch], l[kBatch];
    f32x2 o[kBatch];
};

template <int LP>
__global__ __launch_bounds__(64 * kMaxWaves) void combine_partials_kernel(CombineParams p) {
    constexpr int G = 64 / LP;  // slots per wave
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int W = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane % LP;
    const int slot = w * G + lane / LP, NS = W * G;
    const int b = r / p.Hq, h = r % p.Hq;
    int n = p.S;
    if (p.kv_lens) {
        const int len = min(max(p.kv_lens[b], 0), p.L_cap);
        n = min((len + p.chunk - 1) / p.chunk, p.S);
    }
    // this lane's two columns; lanes past d read valid columns and discard them
    const int c0 = blockIdx.y * 2 * LP + 2 * li;
    const bool even = (p.d & 1) == 0;  // then (row * S + s) * d + c0 is even: 8-byte loads
    const int64_t cv = min(c0, p.d - 2);
    const int64_t cc0 = min(c0, p.d - 1), cc1 = min(c0 + 1, p.d - 1);
    const float* m_row = p.m_part + (int64_t)r * p.S;
    const float* l_row = p.l_part + (int64_t)r * p.S;
    const float* o_row = p.o_part + (int64_t)r * p.S * p.d;

    auto load = [&](Batch& t, int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int64_t s = min(s0 + NS * i, n - 1);
            t.m[i] = m_row[s];
            t.l[i] = l_row[s];
            if (even) {
                t.o[i] = *reinterpret_cast<const f32x2*>(o_row + s * p.d + cv);
            } else {
                t.o[i][0] = o_row[s * p.d + cc0];
                t.o[i][1] = o_row[s * p.d + cc1];
            }
        }
    };
    float M = kNegInf, L = 0.f, a0 = 0.f, a1 = 0.f;
    auto add = [&](const Batch& t, int s0) __attribute__((always_inline)) {
        float bm = M;
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (s0 + NS * i < n) bm = fmaxf(bm, t.m[i]);
        if (bm > M) {  // the running max moves: rescale what is summed so far
            const float f = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((M - bm) * kLog2e);
            L *= f;
            a0 *= f;
            a1 *= f;
            M = bm;
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const bool use = s0 + NS * i < n && t.m[i] != kNegInf;
            const float wgt = use ? __builtin_amdgcn_exp2f((t.m[i] - M) * kLog2e) : 0.f;
            L = fmaf(wgt, t.l[i], L);
            a0 = fmaf(wgt, t.o[i][0], a0);
            a1 = fmaf(wgt, t.o[i][1], a1);
        }
    };
    if (slot < n) {
        Batch cur, nxt;
        int s0 = slot;
        load(cur, s0);
        while (true) {
            const int s1 = s0 + NS * kBatch;
            const bool more = s1 < n;
            if (more) load(nxt, s1);
            add(cur, s0);
            if (!more) break;
            cur = nxt;
            s0 = s1;
        }
    }
    // The G slots of a wave hold the same columns: merge them in registers,
    // a butterfly over the lane groups (both partners compute the same sum,
    // so every lane ends with the wave's result, in a fixed order).
#pragma unroll
    for (int off = LP; off < 64; off <<= 1) {
        const float Mo = __shfl_xor(M, off), Lo = __shfl_xor(L, off);
        const float o0 = __shfl_xor(a0, off), o1 = __shfl_xor(a1, off);
        const float Mn = fmaxf(M, Mo);
        const float f = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
        const float fo = (Mo == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((Mo - Mn) * kLog2e);
        L = f * L + fo * Lo;
        a0 = f * a0 + fo * o0;
        a1 = f * a1 + fo * o1;
        M = Mn;
    }
    // wave-major: wave k's columns at [k * 2LP, (k + 1) * 2LP)
    __shared__ float sm_m[kMaxWaves], sm_l[kMaxWaves];
    __shared__ float sm_o[kMaxWaves * 128];
    if (lane < LP) {
        sm_o[w * 2 * LP + 2 * li] = a0;
        sm_o[w * 2 * LP + 2 * li + 1] = a1;
        if (li == 0) {
            sm_m[w] = M;
            sm_l[w] = L;
        }
    }
    __syncthreads();
    if (tid < LP) {  // wave 0, lane group 0: the row's 2*LP columns
        float mx = kNegInf;
        for (int k = 0; k < W; ++k) mx = fmaxf(mx, sm_m[k]);
        float so0 = 0.f, so1 = 0.f, sl = 0.f;
        if (mx != kNegInf)
            for (int k = 0; k < W; ++k) {
                const float mk = sm_m[k];
                const float f = (mk == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((mk - mx) * kLog2e);
                sl = fmaf(f, sm_l[k], sl);
                so0 = fmaf(f, sm_o[k * 2 * LP + 2 * li], so0);
                so1 = fmaf(f, sm_o[k * 2 * LP + 2 * li + 1], so1);
            }
        const bool empty = (mx == kNegInf) || !(sl > 0.f);
        const float inv = empty ? 0.f : 1.f / sl;
        const int64_t off = b * p.out_sb + h * p.out_sh;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = c0 + e;
            if (c < p.d) {
                const float val = (e ? so1 : so0) * inv;
                if (p.out_dtype == DT_BF16) static_cast<uint16_t*>(p.out)[off + c] = f32_to_bf16_rne(val);
                else static_cast<float*>(p.out)[off + c] = val;
            }
        }
        if (p.lse && blockIdx.y == 0 && tid == 0) p.lse[r] = empty ? kNegInf : mx + logf(sl);
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
    // Lanes per partial: 64 unless that leaves fewer than 256 workgroups for a
    // deep merge (more than 64 partials per row); then narrower column blocks.
    int lp = 64;
    while (lp > 8 && p.S > 64 && (int64_t)p.R * ((p.d + 2 * lp - 1) / (2 * lp)) < 256) lp >>= 1;
    // enough waves (4 to 16) that each slot takes one batch where it can
    const int need = (p.S + kBatch * (64 / lp) - 1) / (kBatch * (64 / lp));
    const int waves = need < 4 ? 4 : (need > kMaxWaves ? kMaxWaves : need);
    const dim3 grid(p.R, (p.d + 2 * lp - 1) / (2 * lp)), block(64 * waves);
    if (lp == 64) hipLaunchKernelGGL(combine_partials_kernel<64>, grid, block, 0, stream, p);
    else if (lp == 32) hipLaunchKernelGGL(combine_partials_kernel<32>, grid, block, 0, stream, p);
    else if (lp == 16) hipLaunchKernelGGL(combine_partials_kernel<16>, grid, block, 0, stream, p);
    else hipLaunchKernelGGL(combine_partials_kernel<8>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace attn
