// Fused prefill attention for gfx950 (bf16, head dim 128, causal or not).
//
// The score matrix never leaves the chip: per tile of keys, scores, scaling,
// the max-subtracted softmax and the product with V all happen in registers
// and LDS (the fused matmul + scale + softmax of the "Attention in SRAM on
// Tenstorrent Grayskull" explainer, sections 1 and 3; the on-chip tiling the
// glossary page "Attention" credits to FlashAttention in its hardware section).
//
// Workgroup: 4 waves x 32 query rows = 128 consecutive query positions of one
// query head. Each wave keeps, per query row, a running max m and sum l and an
// fp32 output accumulator, and walks 64-key tiles staged in LDS by the whole
// workgroup (double buffered, one barrier per tile).
//
// Both products are computed transposed so that one query row lives in one
// lane and the softmax needs no cross-lane reduction except one swap:
//   S^T (32 keys x 32 rows) = K Q^T      v_mfma_f32_32x32x16_bf16, 8 steps over d
//   O^T (32 dims x 32 rows) += V^T P^T   same instruction, 16 keys per step
// Lane l holds query row (l & 31) and 16 of the 32 keys of each key block; the
// K rows are fed to the MFMA in a permuted order (bits 2 and 3 of the row
// index swapped) so that those 16 keys come as two runs of 8 consecutive keys,
// which makes P^T usable directly as the B operand of the second product and
// lets V^T be read from LDS with one 16-byte load per operand. V is transposed
// once, while being copied into LDS.
//
// Causal masking (bottom-right aligned: query i sees keys <= Lkv - Lq + i) is
// applied only on tiles that cross the diagonal; tiles past it are skipped.
// Workgroups are issued heaviest (latest) query block first, and the query
// heads that share a KV head are sent to the same XCD so that their K/V tiles
// are shared in that XCD's L2.
#include "internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kM = 128;        // query rows per workgroup
constexpr int kN = 64;         // keys per tile
constexpr int kD = 128;        // head dim
constexpr int kKStride = 136;  // bf16 per K row in LDS (272 B: conflict-free operand reads)
constexpr int kVStride = 72;   // bf16 per V^T row in LDS (144 B)
constexpr int kKBuf = kN * kKStride;
constexpr int kVBuf = kD * kVStride;
constexpr float kHeadroom = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    // round to nearest even (finite inputs)
    uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
    ua += 0x7fffu + ((ua >> 16) & 1u);
    ub += 0x7fffu + ((ub >> 16) & 1u);
    return (ua >> 16) | (ub & 0xffff0000u);
}

// Key-row order fed to the MFMA: swap bits 2 and 3 of the row index.
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Key offset (within a 32-key block) of accumulator register j of a lane in
// half hb, given the permuted row order.
__device__ __forceinline__ int key_of(int j, int hb) { return j < 8 ? 8 * hb + j : 16 + 8 * hb + (j - 8); }

struct Staged {
    u32x4 k[4];  // key 16i + tid/16, dims 8*(tid%16) .. +7
    u32x4 v[4];  // key 4*(tid/16) + i, dims 8*(tid%16) .. +7
};

__device__ __forceinline__ void load_tile(Staged& st, const char* kbase, const char* vbase, int64_t kss, int64_t vss,
                                          int key0, int klast, int tid) {
    const int c = tid & 15, r = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = min(key0 + 16 * i + r, klast);
        st.k[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * kss + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = min(key0 + 4 * r + i, klast);
        st.v[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * vss + 16 * c);
    }
}

__device__ __forceinline__ void store_tile(const Staged& st, uint16_t* kl, uint16_t* vl, int tid) {
    const int c = tid & 15, r = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(kl + (16 * i + r) * kKStride + 8 * c) = st.k[i];
    // transpose: dims 8c..8c+7 of keys 4r..4r+3 -> V^T rows 8c+e, columns 4r..4r+3
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        u32x2 lo, hi;
        lo[0] = (st.v[0][m] & 0xffffu) | (st.v[1][m] << 16);
        lo[1] = (st.v[2][m] & 0xffffu) | (st.v[3][m] << 16);
        hi[0] = (st.v[0][m] >> 16) | (st.v[1][m] & 0xffff0000u);
        hi[1] = (st.v[2][m] >> 16) | (st.v[3][m] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(vl + (8 * c + 2 * m) * kVStride + 4 * r) = lo;
        *reinterpret_cast<u32x2*>(vl + (8 * c + 2 * m + 1) * kVStride + 4 * r) = hi;
    }
}

__global__ __launch_bounds__(256, 2) void prefill_fwd_d128(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (kKBuf + kVBuf)];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int hb = lane >> 5, row = lane & 31;
    const int G = p.Hq / p.Hkv;
    const int nqb = (p.Lq + kM - 1) / kM;

    // Workgroup -> (query block, batch, head). Query-head groups sharing a KV
    // head go to one XCD (workgroup ids are dealt to the 8 XCDs round robin),
    // heaviest query blocks first.
    const int id = blockIdx.x;
    const int ngroups = nqb * p.B * p.Hkv;
    int grp, hg;
    if (ngroups % 8 == 0) {
        const int xcd = id & 7, slot = id >> 3;
        grp = (slot / G) * 8 + xcd;
        hg = slot % G;
    } else {
        grp = id / G;
        hg = id % G;
    }
    const int qb = nqb - 1 - grp / (p.B * p.Hkv);
    const int bg = grp % (p.B * p.Hkv);
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int h = g * G + hg;

    const int off = p.Lkv - p.Lq;  // bottom-right alignment
    const int p0 = qb * kM;
    const int q0 = p0 + 32 * w;     // first query row of this wave
    const int kv_limit = p.causal ? min(p.Lkv, p0 + kM + off) : p.Lkv;
    const int ntiles = (kv_limit + kN - 1) / kN;
    const int wave_last_key = p.causal ? min(p.Lkv - 1, q0 + 31 + off) : p.Lkv - 1;

    const char* kbase = static_cast<const char*>(p.k) + (b * p.k_sb + g * p.k_sh) * 2;
    const char* vbase = static_cast<const char*>(p.v) + (b * p.v_sb + g * p.v_sh) * 2;
    const int64_t kss = p.k_ss * 2, vss = p.v_ss * 2;

    // Q^T operand: column `row` is query q0 + row; k-slots are dims 16ks + 8hb + e.
    bf16x8 qop[8];
    {
        const int qr = min(q0 + row, p.Lq - 1);
        const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)qr * p.q_ss;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qop[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * hb);
    }
    const float c2 = p.scale_log2;
    const int qabs = q0 + row + off;  // absolute position of this lane's query row
    const int prow = perm_row(row);

    f32x16 oacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    Staged st;
    load_tile(st, kbase, vbase, kss, vss, 0, p.Lkv - 1, tid);
    store_tile(st, lds, lds + kKBuf, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        uint16_t* kl = lds + (t & 1) * (kKBuf + kVBuf);
        uint16_t* vl = kl + kKBuf;
        const bool more = t + 1 < ntiles;
        if (more) load_tile(st, kbase, vbase, kss, vss, (t + 1) * kN, p.Lkv - 1, tid);

        const int key0 = t * kN;
        if (key0 <= wave_last_key) {
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8*>(kl + (32 * kb + prow) * kKStride + 16 * ks + 8 * hb);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], sacc[kb], 0, 0, 0);
                }
            }
            // mask keys past the diagonal or past the end
            const bool edge = (key0 + kN > p.Lkv) || (p.causal && key0 + kN - 1 > q0 + off);
            if (edge) {
                const int lim = p.causal ? min(qabs, p.Lkv - 1) : p.Lkv - 1;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (key0 + 32 * kb + key_of(j, hb) > lim) sacc[kb][j] = kNegInf;
            }
            float mt = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[kb][j]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float mts = mt * c2;
            if (__builtin_amdgcn_ballot_w64(mts > m_run + kHeadroom) != 0) {
                const float m_new = fmaxf(m_run, mts);
                const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 16; ++j) oacc[i][j] *= alpha;
            }
            bf16x8 pb[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float pr[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    pr[j] = fast_exp2(fmaf(sacc[kb][j], c2, -m_run));
                    l_run += pr[j];
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    u32x4 pk;
#pragma unroll
                    for (int e = 0; e < 4; ++e) pk[e] = pack_bf16(pr[8 * half + 2 * e], pr[8 * half + 2 * e + 1]);
                    pb[kb][half] = __builtin_bit_cast(bf16x8, pk);
                }
            }
#pragma unroll
            for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vl + (32 * dblk + row) * kVStride + 32 * kb +
                                                                          16 * half + 8 * hb);
                        oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][half], oacc[dblk], 0, 0, 0);
                    }
        }
        if (more) {
            uint16_t* nk = lds + ((t + 1) & 1) * (kKBuf + kVBuf);
            store_tile(st, nk, nk + kKBuf, tid);
        }
        __syncthreads();
    }

    // epilogue: O = acc / l, lse = m ln2 + ln l
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const int qr = q0 + row;
    if (qr < p.Lq) {
        const float inv = 1.0f / l_tot;
        uint16_t* orow = static_cast<uint16_t*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)qr * p.o_ss;
#pragma unroll
        for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * dblk + 8 * jj + 4 * hb;
                u32x2 pk;
                pk[0] = pack_bf16(oacc[dblk][4 * jj] * inv, oacc[dblk][4 * jj + 1] * inv);
                pk[1] = pack_bf16(oacc[dblk][4 * jj + 2] * inv, oacc[dblk][4 * jj + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + d0) = pk;
            }
        if (p.lse && hb == 0) p.lse[((int64_t)b * p.Hq + h) * p.Lq + qr] = m_run * kLn2 + logf(l_tot);
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    if (p.d != kD) return hipErrorInvalidValue;
    const int nqb = (p.Lq + kM - 1) / kM;
    const int64_t wgs = (int64_t)nqb * p.B * p.Hq;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_fwd_d128, dim3((unsigned)wgs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace attn
