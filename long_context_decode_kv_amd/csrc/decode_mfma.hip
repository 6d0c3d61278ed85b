// Split-KV grouped-query decode for gfx950: one query token, four query heads
// per KV head, head dim 128, KV cache in bf16 or OCP fp8-e4m3.
//
// Work split (the single-GPU form of the sequence-axis tree reduction in the
// explainer of "Tree Attention: Topology-aware Decoding for Long-Context
// Attention on GPU Clusters", section 3): workgroup (s, g, b) owns one chunk of
// keys of KV head g of sequence b and emits one partial (o, m, l) per query
// head. The four waves of the workgroup interleave 16-key tiles of the chunk;
// inside a wave, each group of 16 lanes keeps its own running partial, so the
// hot loop needs no cross-lane reduction at all. The partials are merged in
// registers (lane groups), then in LDS (waves) -- the level-1 tree. The
// level-2 tree across workgroups runs either here (the last workgroup of each
// (sequence, KV head) to finish merges its group's partials, see FUSED) or in
// combine.hip.
//
// Per 16-key tile and wave:
//  * scores: S^T = K Q^T on one v_mfma_f32_16x16x32_bf16 chain (4 steps over
//    d=128). A = 16 key rows, B = Q^T with the four query heads repeated in the
//    16 columns, so lane l receives the scores of head (l & 3) for keys
//    4*(l>>4) .. 4*(l>>4)+3 of the tile. MFMA is used only because this product
//    is a dense contraction; 75% of its columns are repeats, which costs
//    nothing that matters at 4 flop/byte.
//  * softmax: scores stay in base-2 units (scale folded with log2 e). The
//    running maximum moves only when a score exceeds it by 8 (2^8 headroom
//    in fp32), so rescaling the accumulators is rare; the result is the same
//    exact quantity, normalised with the same maximum in o and l. The
//    stability step is the max subtraction the Grayskull explainer names in
//    section 3.
//  * P.V on the vector ALUs: lane l holds V for the same four keys at dims
//    8*(l&15) .. +7, fetches the four heads' weights of each key from its quad
//    with DPP broadcasts, and accumulates 4 heads x 8 dims in fp32.
// K and V are both read as whole rows per load instruction with non-temporal
// loads (K then goes through a small wave-private LDS stage into the MFMA
// operand layout); every valid key is read from HBM exactly once, and the next
// tile's loads are issued before the current tile is computed.
#include "internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kTile = 16;          // keys per wave per step
constexpr float kHeadroom = 8.0f;  // base-2 units a score may exceed the running max by
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

// Value of lane (l & ~3) + H, for every lane l (DPP quad_perm broadcast).
template <int H>
__device__ __forceinline__ float quad_bcast(float x) {
    constexpr int ctrl = H | (H << 2) | (H << 4) | (H << 6);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Storage precision of a span of the cache: bf16; OCP fp8-e4m3 with one fp32
// scale per (sequence, KV head); OCP MX fp4 (E2M1 codes, two per byte with
// the first in the low nibble, and one E8M0 power-of-two scale per 32
// consecutive elements of a row, in a separate array of 4 bytes per row).
constexpr int kBf16 = 0, kFp8 = 1, kFp4 = 2;

template <int P>
struct Tile;
template <>
struct Tile<kBf16> {
    u32x4 k[4];  // key row 4i + (lane>>4), bytes 16*(lane & 15) .. +15 (coalesced rows)
    u32x4 v[4];  // key 4*(lane>>4) + u: 8 bf16 at dims 8*(lane & 15)
};
template <>
struct Tile<kFp8> {
    u32x4 k[2];  // key row 8i + (lane>>3), bytes 16*(lane & 7) .. +15 (coalesced rows)
    u32x2 v[4];  // key 4*(lane>>4) + u: 8 fp8 at dims 8*(lane & 15)
};
template <>
struct Tile<kFp4> {
    u32x4 k;         // key row lane>>2, bytes 16*(lane & 3) .. +15: the 32 codes of block lane & 3
    uint32_t ks;     // the four block scales of key row lane & 15 (byte i: block i)
    uint32_t v[4];   // key 4*(lane>>4) + u: 8 codes at dims 8*(lane & 15)
    uint32_t vs[4];  // the four block scales of that key
};

// Rows of an MX fp4 span's scale arrays (unused for the other precisions).
struct ScaleRows {
    const char* k;
    const char* v;
    int64_t kss, vss;  // bytes between rows
};

// E8M0 byte (low 8 bits of e) -> 2^(e - 127) as a float (255: NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    e &= 255u;
    const uint32_t bits = e == 0u ? 0x00400000u : (e == 255u ? 0x7fc00000u : e << 23);
    return __builtin_bit_cast(float, bits);
}

// Streaming loads: every byte of the cache is read once, so they are marked
// non-temporal; each load instruction of a wave covers whole 128/256-byte rows.
template <typename T>
__device__ __forceinline__ T ld_stream(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// Loads one 16-key tile; key indices past `tlast` are clamped to it, so every
// address stays inside the cache and the clamped keys are masked later.
template <int P>
__device__ __forceinline__ void load_tile(Tile<P>& t, const char* kbase, const char* vbase, int64_t kss,
                                          int64_t vss, const ScaleRows& sc, int tok0, int tlast, int lane) {
    if constexpr (P == kFp4) {
        // the tile's first row in wide arithmetic (uniform), the lanes' rows
        // as 32-bit offsets from it (a span's row strides are far below 2^27)
        const int last = tlast - tok0;
        const char* kt = kbase + (int64_t)tok0 * kss;
        const char* vt = vbase + (int64_t)tok0 * vss;
        const char* kst = sc.k + (int64_t)tok0 * sc.kss;
        const char* vst = sc.v + (int64_t)tok0 * sc.vss;
        const int ik = (int)kss, iv = (int)vss, iks = (int)sc.kss, ivs = (int)sc.vss;
        t.k = ld_stream<u32x4>(kt + min(lane >> 2, last) * ik + 16 * (lane & 3));
        t.ks = ld_stream<uint32_t>(kst + min(lane & 15, last) * iks);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rv = min(4 * (lane >> 4) + u, last);
            t.v[u] = ld_stream<uint32_t>(vt + rv * iv + 4 * (lane & 15));
            t.vs[u] = ld_stream<uint32_t>(vst + rv * ivs);
        }
    } else {
        if constexpr (P == kBf16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rk = min(tok0 + 4 * i + (lane >> 4), tlast);
                t.k[i] = ld_stream<u32x4>(kbase + (int64_t)rk * kss + 16 * (lane & 15));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rk = min(tok0 + 8 * i + (lane >> 3), tlast);
                t.k[i] = ld_stream<u32x4>(kbase + (int64_t)rk * kss + 16 * (lane & 7));
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rv = min(tok0 + 4 * (lane >> 4) + u, tlast);
            const char* vrow = vbase + (int64_t)rv * vss;
            if constexpr (P == kBf16) t.v[u] = ld_stream<u32x4>(vrow + 2 * 8 * (lane & 15));
            else t.v[u] = ld_stream<u32x2>(vrow + 8 * (lane & 15));
        }
    }
}

// The K tile passes through a wave-private LDS stage to change from row-major
// lanes to the MFMA operand layout (lane = key row, 16 bytes of dims). 16-byte
// chunks are XOR-swizzled by row so both the row writes and the column reads
// touch every bank once per 16 lanes. (fp4: four 16-byte chunks per row, chunk
// c of row r at c ^ (r >> 2); the operand reads are 4-byte words, word g of
// chunk i for row r, which then cover all 64 banks.)
template <int P>
__device__ __forceinline__ int kstage_index(int row, int chunk) {
    if constexpr (P == kBf16) return row * 16 + (chunk ^ (row & 15));
    else if constexpr (P == kFp8) return row * 8 + (chunk ^ ((row >> 1) & 7));
    else return row * 4 + (chunk ^ (row >> 2));
}

template <int P>
__device__ __forceinline__ void stage_k(const Tile<P>& t, u32x4* ks, int lane) {
    if constexpr (P == kBf16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ks[kstage_index<kBf16>(4 * i + (lane >> 4), lane & 15)] = t.k[i];
    } else if constexpr (P == kFp8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) ks[kstage_index<kFp8>(8 * i + (lane >> 3), lane & 7)] = t.k[i];
    } else {
        ks[kstage_index<kFp4>(lane >> 2, lane & 3)] = t.k;
    }
}

// Eight MX fp4 codes (a dword, first code in the low nibble) times 2^scale ->
// eight floats (exact).
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, float sc, float (&f)[8]) {
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
    const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
    const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
    f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

// Four OCP e4m3 codes of a dword pair -> eight bf16 (exact widening).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int P>
__device__ __forceinline__ void v_to_f32(const Tile<P>& t, int u, int lane, float (&vf)[8]) {
    if constexpr (P == kFp4) {
        // dims 8*(lane & 15) .. +7 lie in block (lane & 15) >> 2
        fp4x8_to_f32(t.v[u], e8m0_to_f32(t.vs[u] >> (8 * ((lane & 15) >> 2))), vf);
    } else if constexpr (P == kBf16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vf[2 * e] = bf16_lo(t.v[u][e]);
            vf[2 * e + 1] = bf16_hi(t.v[u][e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(t.v[u][e], false);
            f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(t.v[u][e], true);
            vf[4 * e + 0] = a[0];
            vf[4 * e + 1] = a[1];
            vf[4 * e + 2] = b[0];
            vf[4 * e + 3] = b[1];
        }
    }
}

template <int P>
__device__ __forceinline__ void compute_tile(const Tile<P>& t, u32x4* ks, const bf16x8 (&qop)[4], float scale2,
                                             int tok0, int tend, int lane, float& m_run, float& l_run,
                                             float (&o)[4][8]) {
    stage_k<P>(t, ks, lane);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int row = lane & 15;
    if constexpr (P == kFp4) {
        // MFMA step i is block i (dims 32i .. 32i + 31): this lane's eight
        // codes, dims 32i + 8*(lane >> 4) .., widened with the block's scale
        const uint32_t* ks32 = reinterpret_cast<const uint32_t*>(ks);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float f[8];
            fp4x8_to_f32(ks32[4 * kstage_index<kFp4>(row, i) + (lane >> 4)], e8m0_to_f32(t.ks >> (8 * i)), f);
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (__bf16)f[e];  // exact: two significant bits
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[i], acc, 0, 0, 0);
        }
    } else if constexpr (P == kBf16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 a = ks[kstage_index<false>(row, 4 * i + (lane >> 4))];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qop[i], acc, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 a = ks[kstage_index<true>(row, 4 * h + (lane >> 4))];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(a[0], a[1]), qop[2 * h], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(a[2], a[3]), qop[2 * h + 1], acc, 0, 0,
                                                          0);
        }
    }
    const int kb = tok0 + 4 * (lane >> 4);
    float s[4];
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        s[r] = (kb + r < tend) ? acc[r] * scale2 : kNegInf;
        tmax = fmaxf(tmax, s[r]);
    }
    const bool need = tmax > m_run + kHeadroom;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
        const float a[4] = {quad_bcast<0>(alpha), quad_bcast<1>(alpha), quad_bcast<2>(alpha), quad_bcast<3>(alpha)};
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= a[h];
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = (s[r] == kNegInf) ? 0.f : fast_exp2(s[r] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float pb[4] = {quad_bcast<0>(p[u]), quad_bcast<1>(p[u]), quad_bcast<2>(p[u]), quad_bcast<3>(p[u])};
        float vf[8];
        v_to_f32<P>(t, u, lane, vf);
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pb[h], vf[e], o[h][e]);
    }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Agent-scope relaxed atomics: on this GPU they are performed at the
// device-wide coherence point (past the per-XCD L2), so values written by a
// workgroup on one XCD are read back fresh by a workgroup on another.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent2(float* p, f32x2 v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 ld_agent2(const float* p) {
    return __builtin_bit_cast(
        f32x2, __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT));
}

// Merge n <= kMergeMax partials of the four heads of one KV group, in
// the fixed order j = 0, 1, ...: partial j of head h has o at
// o + (h*rs + j)*128, m at m[h*rs + j], l at l[h*rs + j] (natural-log units).
// Leaves the unnormalised sums in part[h][c] and (max, sum) in red[h].
constexpr int kMergeMax = 32;  // partials one merge4 call takes
struct MergeLds {
    float w[4][kMergeMax];
    float red[4][2];
    float part[2][4][128];
};

// Every load is issued before any is used (the o values do not depend on the
// weights), so the merge waits for one round trip to the other workgroups'
// writes; the weights of head h are computed by wave h, one partial per lane.
__device__ __forceinline__ void merge4(const float* o, const float* m, const float* l, int64_t rs, int n, int tid,
                                       MergeLds& sm) {
    const int lane = tid & 63, h = tid >> 6;
    // thread = (half, head, 4 columns); half k takes j = k, k+2, ... (wave-uniform)
    const int half = tid >> 7, idx = tid & 127, hh = idx >> 5, c4 = (idx & 31) * 4;
    const float* ob = o + hh * rs * 128 + c4;
    f32x2 v[kMergeMax / 2][2];
#pragma unroll
    for (int u = 0; u < kMergeMax / 2; ++u) {
        const int j = half + 2 * u;
        if (j < n) {
            v[u][0] = ld_agent2(ob + (int64_t)j * 128);
            v[u][1] = ld_agent2(ob + (int64_t)j * 128 + 2);
        }
    }
    float mj = kNegInf, lj = 0.f;
    if (lane < n) {  // n <= kMergeMax < 64
        mj = ld_agent(m + h * rs + lane);
        lj = ld_agent(l + h * rs + lane);
    }
    // butterflies: every lane ends with the same, order-fixed result
    float M = mj;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float wgt = (mj == kNegInf) ? 0.f : fast_exp2((mj - M) * kLog2e);
    float L = wgt * lj;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (lane < kMergeMax) sm.w[h][lane] = wgt;
    if (lane == 0) {
        sm.red[h][0] = M;
        sm.red[h][1] = L;
    }
    __syncthreads();
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kMergeMax / 2; ++u) {
        const int j = half + 2 * u;
        if (j < n) {
            const float wv = sm.w[hh][j];
            acc[0] = fmaf(wv, v[u][0][0], acc[0]);
            acc[1] = fmaf(wv, v[u][0][1], acc[1]);
            acc[2] = fmaf(wv, v[u][1][0], acc[2]);
            acc[3] = fmaf(wv, v[u][1][1], acc[3]);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.part[half][hh][c4 + e] = acc[e];
    __syncthreads();
}

// Level 2, fused: a tree over the splits of each (b, g) group. Every
// workgroup publishes its partial (agent-scope stores, waited for), then takes
// a ticket in its block of `ticket_block` splits; the last of a block merges
// the block into a block partial and, if there are several blocks, takes a
// ticket on the group; the last block merges the block partials into O and
// lse. Counters are reset by their last user. The tree shape is a function of
// n and the plan only, so results are deterministic.
__device__ __forceinline__ void merge_group_if_last(const DecodeParams& p, int b, int g, int n, int tid) {
    __shared__ int role;  // 0: done, 1: merged its block, not last; 2: final merger
    __shared__ MergeLds sm;
    // n: the splits of this sequence that publish a partial
    const int s = blockIdx.x, k = p.ticket_block;
    const int nb = (n + k - 1) / k, bi = s / k;
    const int in_block = min(k, n - bi * k);
    uint32_t* line = p.counters + (int64_t)(b * p.Hkv + g) * (1 + kMaxTicketBlocks) * kCounterStride;
    const int64_t row0 = (int64_t)b * p.Hq + g * 4;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
    __syncthreads();
    if (tid == 0) {
        uint32_t* blk = line + (1 + bi) * kCounterStride;
        const uint32_t o1 = __hip_atomic_fetch_add(blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        role = (o1 == (uint32_t)(in_block - 1)) ? 1 : 0;
        if (role) __hip_atomic_store(blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!role) return;
    const int lane = tid & 63, h = tid >> 6;
    // level 2a: this block's splits
    merge4(p.o_part + (row0 * p.S + bi * k) * 128, p.m_part + row0 * p.S + bi * k, p.l_part + row0 * p.S + bi * k,
           p.S, in_block, tid, sm);
    if (nb > 1) {
        // publish the block partial, then take a ticket on the group
        float* bo = p.blk_o + (row0 * kMaxTicketBlocks + bi) * 128;
        const int c = lane * 2;
        f32x2 v;
        v[0] = sm.part[0][h][c] + sm.part[1][h][c];
        v[1] = sm.part[0][h][c + 1] + sm.part[1][h][c + 1];
        st_agent2(bo + (int64_t)h * kMaxTicketBlocks * 128 + c, v);
        if (lane == 0) {
            st_agent(p.blk_m + (row0 + h) * kMaxTicketBlocks + bi, sm.red[h][0]);
            st_agent(p.blk_l + (row0 + h) * kMaxTicketBlocks + bi, sm.red[h][1]);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const uint32_t o2 = __hip_atomic_fetch_add(line, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            role = (o2 == (uint32_t)(nb - 1)) ? 2 : 0;
            if (role) __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!role) return;
        // level 2b: the block partials
        merge4(p.blk_o + row0 * kMaxTicketBlocks * 128, p.blk_m + row0 * kMaxTicketBlocks,
               p.blk_l + row0 * kMaxTicketBlocks, kMaxTicketBlocks, nb, tid, sm);
    }
    const int c = lane * 2;
    const float Mh = sm.red[h][0], Lh = sm.red[h][1];
    const bool empty = !(Lh > 0.f);
    const float inv = empty ? 0.f : 1.0f / Lh;
    uint16_t* orow = static_cast<uint16_t*>(p.out) + b * p.out_sb + (int64_t)(g * 4 + h) * p.out_sh;
    orow[c] = f32_to_bf16_rne((sm.part[0][h][c] + sm.part[1][h][c]) * inv);
    orow[c + 1] = f32_to_bf16_rne((sm.part[0][h][c + 1] + sm.part[1][h][c + 1]) * inv);
    if (p.lse && lane == 0) p.lse[row0 + h] = empty ? kNegInf : Mh + logf(Lh);
}

// LDS of one decode workgroup: the per-wave K staging buffers and the
// cross-wave merge (level 1b).
struct DecodeLds {
    u32x4 kstage[kWaves][256];
    float o[kWaves][4][128];
    float m[kWaves][4];
    float l[kWaves][4];
};

// One workgroup: split s of span `sp`, publishing partial s_out of its rows.
// TWO (two-span launches): the span's key geometry and log-prior apply; every
// split of the launch publishes a partial (an empty one the identity) and
// takes part in the fused merge, which covers all p.S of them.
template <int P, bool FUSED, bool TWO>
__device__ __forceinline__ void decode_wg(const DecodeParams& p, const KvSpan& sp, int s, int s_out,
                                          DecodeLds& lds) {
    constexpr bool FP8 = P == kFp8;
    const int g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile rows and bases in scalar registers
    int L_b = sp.L_cap;
    if (sp.kv_lens) L_b = min(max(sp.kv_lens[b * sp.lens_sb + g * sp.lens_sh], 0), sp.L_cap);
    // keys visited: rows row0 + t * rmul for t in [0, n_keys)
    int n_keys = L_b, row0 = 0, rmul = 1;
    if constexpr (TWO) {
        const int i = L_b - 1;  // the query's position
        if (sp.geom == kGeomWindow) {
            row0 = max(0, i - sp.window);
            n_keys = L_b - row0;
        } else if (sp.geom == kGeomSkip) {
            const int last = i - sp.window - 1;  // the highest row a skip key may take
            const int r = i >= 0 ? i % sp.period : 0;
            n_keys = last >= r ? (last - r) / sp.period + 1 : 0;
            row0 = r;
            rmul = sp.period;
        }
    }
    const int t_begin = s * sp.chunk;
    const int t_end = min(t_begin + sp.chunk, n_keys);
    const int n_merge = TWO ? p.S : (L_b + sp.chunk - 1) / sp.chunk;
    if (t_begin >= t_end) {
        // A split past the end of a shorter sequence: the identity partial.
        for (int i = tid; i < 4 * 128; i += 256) {
            const int64_t row = (int64_t)b * p.Hq + g * 4 + i / 128;
            if constexpr (FUSED && TWO) {
                st_agent(p.o_part + (row * p.S + s_out) * 128 + i % 128, 0.f);
                if (i % 128 == 0) {
                    st_agent(p.m_part + row * p.S + s_out, kNegInf);
                    st_agent(p.l_part + row * p.S + s_out, 0.f);
                }
            } else {
                p.o_part[(row * p.S + s_out) * 128 + i % 128] = 0.f;
                if (i % 128 == 0) {
                    p.m_part[row * p.S + s_out] = kNegInf;
                    p.l_part[row * p.S + s_out] = 0.f;
                }
            }
        }
        if constexpr (FUSED && TWO) merge_group_if_last(p, b, g, n_merge, tid);
        if (FUSED && !TWO && L_b == 0 && s == 0) {
            // an empty sequence: O = 0, lse = -inf (no workgroup of it merges)
            for (int i = tid; i < 4 * 128; i += 256) {
                uint16_t* orow = static_cast<uint16_t*>(p.out) + b * p.out_sb + (int64_t)(g * 4 + i / 128) * p.out_sh;
                orow[i % 128] = 0;
                if (p.lse && i % 128 == 0) p.lse[(int64_t)b * p.Hq + g * 4 + i / 128] = kNegInf;
            }
        }
        return;
    }
    const int ntiles = (t_end - t_begin + kTile - 1) / kTile;

    constexpr int esz = P == kBf16 ? 2 : 1;  // bytes per stride unit (fp4 spans carry byte strides)
    const char* kbase = static_cast<const char*>(sp.k) + (b * sp.k_sb + g * sp.k_sh + row0 * sp.k_ss) * esz;
    const char* vbase = static_cast<const char*>(sp.v) + (b * sp.v_sb + g * sp.v_sh + row0 * sp.v_ss) * esz;
    const int64_t kss = sp.k_ss * esz * rmul, vss = sp.v_ss * esz * rmul;
    ScaleRows sc{nullptr, nullptr, 0, 0};
    if constexpr (P == kFp4) {
        sc.k = static_cast<const char*>(sp.k_sc) + b * sp.ksc_sb + g * sp.ksc_sh + row0 * sp.ksc_ss;
        sc.v = static_cast<const char*>(sp.v_sc) + b * sp.vsc_sb + g * sp.vsc_sh + row0 * sp.vsc_ss;
        sc.kss = sp.ksc_ss * rmul;
        sc.vss = sp.vsc_ss * rmul;
    }

    // Q^T operand: column (lane & 15) is query head 4g + (lane & 3); its k-slots
    // follow the same dim order as the K operand.
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.q_sb + (int64_t)(g * 4 + (lane & 3)) * p.q_sh;
    bf16x8 qop[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dim = FP8 ? 64 * (i >> 1) + 16 * (lane >> 4) + 8 * (i & 1) : 32 * i + 8 * (lane >> 4);
        qop[i] = *reinterpret_cast<const bf16x8*>(qrow + dim);
    }
    float scale2 = p.scale_log2;
    float vsc = 1.0f;
    if constexpr (FP8) {
        scale2 *= p.k_scale[b * p.Hkv + g];
        vsc = p.v_scale[b * p.Hkv + g];
    }

    float m_run = kNegInf, l_run = 0.f;
    float o[4][8];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;

    // Tile buffers used in turn: the next tile is in flight while the current
    // one is computed -- the next two for MX fp4, whose 16-key tiles hold a
    // quarter of a bf16 tile's bytes.
    u32x4* ks = lds.kstage[w];
    int k = w;
    if (P == kFp4 && k < ntiles) {
        Tile<P> ta, tb, tc;
        load_tile<P>(ta, kbase, vbase, kss, vss, sc, t_begin + kTile * k, t_end - 1, lane);
        if (k + kWaves < ntiles)
            load_tile<P>(tb, kbase, vbase, kss, vss, sc, t_begin + kTile * (k + kWaves), t_end - 1, lane);
        // ahead <- tile k + 2 kWaves; compute cur (tile k); false when done
        auto step = [&](Tile<P>& cur, Tile<P>& ahead) __attribute__((always_inline)) {
            if (k + 2 * kWaves < ntiles)
                load_tile<P>(ahead, kbase, vbase, kss, vss, sc, t_begin + kTile * (k + 2 * kWaves), t_end - 1, lane);
            compute_tile<P>(cur, ks, qop, scale2, t_begin + kTile * k, t_end, lane, m_run, l_run, o);
            k += kWaves;
            return k < ntiles;
        };
        while (step(ta, tc) && step(tb, ta) && step(tc, tb)) {
        }
    } else if (k < ntiles) {
        Tile<P> ta, tb;
        load_tile<P>(ta, kbase, vbase, kss, vss, sc, t_begin + kTile * k, t_end - 1, lane);
        while (true) {
            const bool more_b = k + kWaves < ntiles;
            if (more_b) load_tile<P>(tb, kbase, vbase, kss, vss, sc, t_begin + kTile * (k + kWaves), t_end - 1, lane);
            compute_tile<P>(ta, ks, qop, scale2, t_begin + kTile * k, t_end, lane, m_run, l_run, o);
            if (!more_b) break;
            k += kWaves;
            const bool more_a = k + kWaves < ntiles;
            if (more_a) load_tile<P>(ta, kbase, vbase, kss, vss, sc, t_begin + kTile * (k + kWaves), t_end - 1, lane);
            compute_tile<P>(tb, ks, qop, scale2, t_begin + kTile * k, t_end, lane, m_run, l_run, o);
            if (!more_a) break;
            k += kWaves;
        }
    }

    // Level 1a: merge the four lane groups (keys 4*(lane>>4)..) of this wave.
    float M = fmaxf(m_run, __shfl_xor(m_run, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - M);
    float lw = l_run * f;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    {
        const float fh[4] = {quad_bcast<0>(f), quad_bcast<1>(f), quad_bcast<2>(f), quad_bcast<3>(f)};
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = o[h][e] * fh[h];
                x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                o[h][e] = x;
            }
    }

    // Level 1b: merge the four waves in LDS.
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) lds.o[w][h][8 * lane + e] = o[h][e];
    }
    if (lane < 4) {
        lds.m[w][lane] = M;
        lds.l[w][lane] = lw;
    }
    __syncthreads();

    const int h = tid >> 6;
    const int c = (tid & 63) * 2;
    float mw[kWaves], fw[kWaves];
    float Mx = kNegInf;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        mw[i] = lds.m[i][h];
        Mx = fmaxf(Mx, mw[i]);
    }
#pragma unroll
    for (int i = 0; i < kWaves; ++i) fw[i] = (mw[i] == kNegInf) ? 0.f : fast_exp2(mw[i] - Mx);
    const float L = (fw[0] * lds.l[0][h] + fw[1] * lds.l[1][h]) + (fw[2] * lds.l[2][h] + fw[3] * lds.l[3][h]);
    f32x2 out;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
        const float v = (fw[0] * lds.o[0][h][c + cc] + fw[1] * lds.o[1][h][c + cc]) +
                        (fw[2] * lds.o[2][h][c + cc] + fw[3] * lds.o[3][h][c + cc]);
        out[cc] = v * vsc;
    }
    const int64_t row = (int64_t)b * p.Hq + g * 4 + h;
    float m_out = Mx * kLn2;
    if constexpr (TWO) {
        // the span's log-prior shifts its partial's max (natural-log units)
        if (sp.prior && p.alpha) {
            const float a = fminf(fmaxf(p.alpha[row], 0.f), 1.f);
            m_out += logf(sp.prior == 1 ? a : 1.f - a);
        }
    }
    if constexpr (FUSED) {
        st_agent2(p.o_part + (row * p.S + s_out) * 128 + c, out);
        if ((tid & 63) == 0) {
            st_agent(p.m_part + row * p.S + s_out, m_out);
            st_agent(p.l_part + row * p.S + s_out, L);
        }
        merge_group_if_last(p, b, g, n_merge, tid);
    } else {
        *reinterpret_cast<f32x2*>(p.o_part + (row * p.S + s_out) * 128 + c) = out;
        if ((tid & 63) == 0) {
            p.m_part[row * p.S + s_out] = m_out;
            p.l_part[row * p.S + s_out] = L;
        }
    }
}

__device__ __forceinline__ KvSpan main_span(const DecodeParams& p) {
    return KvSpan{p.k,       p.k_sb, p.k_sh,  p.k_ss,    p.v, p.v_sb, p.v_sh, p.v_ss, p.kv_lens,
                  1,         0,      p.L_cap, p.chunk,   kGeomAll, 0, 1, 0};
}

template <bool FP8, bool FUSED>
__global__ __launch_bounds__(256) void decode_gqa4_d128(DecodeParams p) {
    __shared__ DecodeLds lds;
    decode_wg<FP8 ? kFp8 : kBf16, FUSED, false>(p, main_span(p), blockIdx.x, blockIdx.x, lds);
}

// Two spans in one launch (a two-precision cache, or pi-Attention's window
// and skip keys): splits [0, S0) stream span sp0, the others span sp1; one
// merge over all splits.
template <int P0, int P1, bool FUSED>
__global__ __launch_bounds__(256) void decode_gqa4_d128_two(DecodeParams p) {
    __shared__ DecodeLds lds;  // one copy for both branches
    const int s = blockIdx.x;
    if (s < p.S0) decode_wg<P0, FUSED, true>(p, p.sp0, s, s, lds);
    else decode_wg<P1, FUSED, true>(p, p.sp1, s - p.S0, s, lds);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, hipStream_t stream) {
    dim3 grid(p.S, p.Hkv, p.B);
    const bool fused = p.counters != nullptr;
    if (kv_dtype == DT_FP8) {
        if (fused) hipLaunchKernelGGL((decode_gqa4_d128<true, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((decode_gqa4_d128<true, false>), grid, dim3(256), 0, stream, p);
    } else {
        if (fused) hipLaunchKernelGGL((decode_gqa4_d128<false, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((decode_gqa4_d128<false, false>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_decode_mfma_two(const DecodeParams& p, int prec0, int prec1, hipStream_t stream) {
    dim3 grid(p.S, p.Hkv, p.B);
    const bool f = p.counters != nullptr;
#define ATTN_TWO(P0, P1)                                                                                  \
    if (prec0 == P0 && prec1 == P1) {                                                                     \
        if (f) hipLaunchKernelGGL((decode_gqa4_d128_two<P0, P1, true>), grid, dim3(256), 0, stream, p);  \
        else hipLaunchKernelGGL((decode_gqa4_d128_two<P0, P1, false>), grid, dim3(256), 0, stream, p);   \
        return hipGetLastError();                                                                         \
    }
    ATTN_TWO(kBf16, kFp8)
    ATTN_TWO(kBf16, kBf16)
    ATTN_TWO(kFp8, kFp8)
    ATTN_TWO(kBf16, kFp4)
#undef ATTN_TWO
    return hipErrorInvalidValue;  // no kernel for this pair of precisions
}

}  // namespace attn
