// Fused prefill attention for gfx950 (bf16, head dim 128, causal or not).
//
// The score matrix never leaves the chip: per tile of keys, scores, scaling,
// the max-subtracted softmax and the product with V all happen in registers
// and LDS (the fused matmul + scale + softmax of the "Attention in SRAM on
// Tenstorrent Grayskull" explainer, sections 1 and 3; the on-chip tiling the
// glossary page "Attention" credits to FlashAttention in its hardware section).
//
// Workgroup: 8 waves x 32 query rows. The waves are the query heads that share
// one KV head (up to 4 of them) times consecutive 32-position blocks, so every
// K/V tile staged in LDS serves all eight waves (and each KV byte is read from
// L2 once per 256 query rows). Each wave keeps, per query row, a running max m
// and sum l and an fp32 output accumulator, and walks 64-key tiles (double
// buffered in LDS, loads two tiles ahead, one barrier per tile). Waves 0-3
// stage V, waves 4-7 stage K.
//
// Both products are computed transposed so that one query row lives in one
// lane and the softmax needs no cross-lane reduction except one lane-pair exchange:
//   S^T (32 keys x 32 rows) = K Q^T      v_mfma_f32_32x32x16_bf16, 8 steps over d
//   O^T (32 dims x 32 rows) += V^T P^T   same instruction, 16 keys per step
// Lane l holds query row (l & 31) and 16 of the 32 keys of each key block; the
// K rows are fed to the MFMA in a permuted order (bits 2 and 3 of the row
// index swapped) so that those 16 keys come as two runs of 8 consecutive keys,
// which makes P^T usable directly as the B operand of the second product and
// lets V^T be read from LDS with one 16-byte load per operand.
//
// LDS layout: K tile [64 keys][128 dims] with rows padded to 272 bytes and
// each key stored at the permuted row position it is read from, and V^T tile
// [128 dims][64 keys] with rows padded to 144 bytes. Every MFMA-operand read is
// then a per-lane base plus a constant offset, and every 8 lanes of a 16-byte
// read or write touch 8 distinct 16-byte bank groups (no bank conflicts). V is
// transposed 8x8 in registers before it is written.
//
// Causal masking (bottom-right aligned: query i sees keys <= Lkv - Lq + i) is
// applied only on tiles that cross the diagonal; tiles past it are skipped.
// Workgroups are issued heaviest (latest) query block first.
#include "internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 32;        // query rows per wave
constexpr int kWaves = 8;        // waves per workgroup
constexpr int kN = 64;           // keys per tile
constexpr int kD = 128;          // head dim
constexpr int kKStride = 136;    // bf16 per K row in LDS (272 bytes)
constexpr int kVStride = 72;     // bf16 per V^T row in LDS (144 bytes)
constexpr int kKElems = kN * kKStride;
constexpr int kVElems = kD * kVStride;
constexpr float kHeadroom = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> packed bf16 pair (hardware round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Reductions over the lane pair (l, l ^ 32), which hold the two halves of
// one query row's keys.
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 32); }

// Key-row order fed to the MFMA: swap bits 2 and 3 of the row index.
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Key offset (within a 32-key block) of accumulator register j of a lane in
// half hb, given the permuted row order.
__device__ __forceinline__ int key_of(int j, int hb) { return j < 8 ? 8 * hb + j : 16 + 8 * hb + (j - 8); }

// Per-thread share of one tile (512 threads): threads 0-255 load 4 keys x 8
// dims of V (16 consecutive lanes read 16 different keys, so the transposed
// 8-byte writes below hit 16 different bank pairs); threads 256-511 load four
// 16-byte pieces of K (16 lanes per 256-byte row).
struct Staged {
    u32x4 x[4];
};

__device__ __forceinline__ void load_tile(Staged& st, const char* kbase, const char* vbase, int64_t kss, int64_t vss,
                                          int key0, int klast, int tid) {
    if (tid < 256) {
        const int u = tid & 15, c = tid >> 4;  // keys 4u.., dims 8c..
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = min(key0 + 4 * u + i, klast);
            st.x[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * vss + 16 * c);
        }
    } else {
        const int t = tid - 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = min(key0 + 16 * i + (t >> 4), klast);
            st.x[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * kss + 16 * (t & 15));
        }
    }
}

__device__ __forceinline__ void store_tile(const Staged& st, uint16_t* kl, uint16_t* vl, int tid) {
    if (tid < 256) {
        const int u = tid & 15, c = tid >> 4;
        // 4x8 transpose: dims 8c+e of keys 4u..4u+3 -> V^T row 8c+e, columns 4u..4u+3
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x2 o;
            o[0] = __builtin_amdgcn_perm(st.x[1][e >> 1], st.x[0][e >> 1], sel);
            o[1] = __builtin_amdgcn_perm(st.x[3][e >> 1], st.x[2][e >> 1], sel);
            *reinterpret_cast<u32x2*>(vl + (8 * c + e) * kVStride + 4 * u) = o;
        }
    } else {
        const int t = tid - 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 16 * i + (t >> 4);  // stored at its permuted row position
            const int pos = (key & ~31) | perm_row(key & 31);
            *reinterpret_cast<u32x4*>(kl + pos * kKStride + 8 * (t & 15)) = st.x[i];
        }
    }
}

__global__ __launch_bounds__(512, 2) void prefill_fwd_d128(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKElems];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kVElems];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int hb = lane >> 5, row = lane & 31;
    const int G = p.Hq / p.Hkv;
    const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);  // query heads per workgroup
    const int PW = kWaves / HW;                                // 32-position blocks per workgroup
    const int span = kRows * PW;                               // positions per workgroup
    const int nqb = (p.Lq + span - 1) / span;
    const int hgroups = G / HW;

    // Workgroup -> (position block, batch, KV head, head group), heaviest first.
    const int id = blockIdx.x;
    const int per_qb = p.B * p.Hkv * hgroups;
    const int qb = nqb - 1 - id / per_qb;
    const int rem = id % per_qb;
    const int hgi = rem % hgroups;
    const int bg = rem / hgroups;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int h = g * G + hgi * HW + (w % HW);

    const int off = p.Lkv - p.Lq;  // bottom-right alignment
    const int p0 = qb * span;
    const int q0 = p0 + kRows * (w / HW);  // first query row of this wave
    const int kv_limit = p.causal ? min(p.Lkv, p0 + span + off) : p.Lkv;
    const int ntiles = (kv_limit + kN - 1) / kN;
    const int wave_last_key = p.causal ? min(p.Lkv - 1, q0 + kRows - 1 + off) : p.Lkv - 1;

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

    f32x16 oacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    // Tiles are staged through two register sets: tile t+2 is requested while
    // tile t is computed and tile t+1 (requested one iteration earlier) is
    // written to LDS.
    Staged st0, st1;
    load_tile(st0, kbase, vbase, kss, vss, 0, p.Lkv - 1, tid);
    if (ntiles > 1) load_tile(st1, kbase, vbase, kss, vss, kN, p.Lkv - 1, tid);
    store_tile(st0, lds_k[0], lds_v[0], tid);
    __syncthreads();

    // One tile: `ld` receives tile t+2 from global memory, `nx` (tile t+1,
    // requested an iteration earlier) is written to LDS.
    auto tile_step = [&](int t, Staged& ld, const Staged& nx) {
            const uint16_t* kl = lds_k[t & 1] + row * kKStride + 8 * hb;   // + 32kb*kKStride + 16ks
            const uint16_t* vl = lds_v[t & 1] + row * kVStride + 8 * hb;   // + 32dblk*kVStride + 32kb + 16half
            const bool more = t + 1 < ntiles;
            if (t + 2 < ntiles) load_tile(ld, kbase, vbase, kss, vss, (t + 2) * kN, p.Lkv - 1, tid);

            const int key0 = t * kN;
            if (key0 <= wave_last_key) {
                // All 16 K operands of the tile are read before the first MFMA, so
                // LDS latency is paid once per tile, not once per MFMA.
                bf16x8 ka[2][8];
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                    for (int ks = 0; ks < 8; ++ks)
                        ka[kb][ks] = *reinterpret_cast<const bf16x8*>(kl + 32 * kb * kKStride + 16 * ks);
                __builtin_amdgcn_sched_barrier(0);
                f32x16 sacc[2];
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
    #pragma unroll
                    for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
    #pragma unroll
                    for (int ks = 0; ks < 8; ++ks)
                        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][ks], qop[ks], sacc[kb], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                // V operands of key block 0, in flight during the softmax
                bf16x8 va[8];
    #pragma unroll
                for (int i = 0; i < 8; ++i)
                    va[i] = *reinterpret_cast<const bf16x8*>(vl + 32 * (i >> 1) * kVStride + 16 * (i & 1));
                __builtin_amdgcn_sched_barrier(0);
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
                // Lazy running max: the exponentials use m_run as long as no score
                // of the lane exceeds it by the headroom; only then (wave vote) the
                // row max over the lane pair is taken and the accumulators rescaled.
                float lm = kNegInf;
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                    for (int j = 0; j < 16; j += 2) lm = fmaxf(lm, fmaxf(sacc[kb][j], sacc[kb][j + 1]));
                if (__builtin_amdgcn_ballot_w64(lm * c2 > m_run + kHeadroom) != 0) {
                    const float m_new = fmaxf(m_run, pair_max(lm) * c2);
                    const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
                    m_run = m_new;
                    l_run *= alpha;
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
    #pragma unroll
                        for (int j = 0; j < 16; ++j) oacc[i][j] *= alpha;
                }
                const float nm = -m_run;
                // key block 0: exponentials, bf16 weights
                u32x4 pk[2][2];
                float lsum = 0.f;
    #pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float pr[8];
    #pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(fmaf(sacc[0][8 * half + e], c2, nm));
                    lsum += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    #pragma unroll
                    for (int e = 0; e < 4; ++e) pk[0][half][e] = pack_bf16(pr[2 * e], pr[2 * e + 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // P.V of key block 0 (8 MFMAs); between them, the V operands of key
                // block 1 are requested and its exponentials computed (two scores
                // per MFMA), so the matrix core and the vector ALU overlap
                bf16x8 vb[8];
                float ls1 = 0.f;
    #pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int dblk = i >> 1, half = i & 1;
                    oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], __builtin_bit_cast(bf16x8, pk[0][half]),
                                                                         oacc[dblk], 0, 0, 0);
                    vb[i] = *reinterpret_cast<const bf16x8*>(vl + 32 * dblk * kVStride + 32 + 16 * half);
                    const float p0 = fast_exp2(fmaf(sacc[1][2 * i], c2, nm));
                    const float p1 = fast_exp2(fmaf(sacc[1][2 * i + 1], c2, nm));
                    ls1 += p0 + p1;
                    pk[1][i >> 2][i & 3] = pack_bf16(p0, p1);
                    __builtin_amdgcn_sched_barrier(0);
                }
                l_run += lsum + ls1;
                // P.V of key block 1
    #pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int dblk = i >> 1, half = i & 1;
                    oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i], __builtin_bit_cast(bf16x8, pk[1][half]),
                                                                         oacc[dblk], 0, 0, 0);
                }
            }
            if (more) store_tile(nx, lds_k[(t + 1) & 1], lds_v[(t + 1) & 1], tid);
            __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        tile_step(t, st0, st1);
        if (t + 1 < ntiles) tile_step(t + 1, st1, st0);
    }

    // epilogue: O = acc / l, lse = m ln2 + ln l
    const float l_tot = pair_sum(l_run);
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
    const int G = p.Hq / p.Hkv;
    const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
    const int span = kRows * (kWaves / HW);
    const int64_t nqb = (p.Lq + span - 1) / span;
    const int64_t wgs = nqb * p.B * p.Hkv * (G / HW);
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_fwd_d128, dim3((unsigned)wgs), dim3(64 * kWaves), 0, stream, p);
    return hipGetLastError();
}

}  // namespace attn
