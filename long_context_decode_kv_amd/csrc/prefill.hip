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
// and sum l and an fp32 output accumulator, and walks 64-key tiles.
//
// The eight waves form two groups (waves 0-3 and 4-7, one of each on every
// SIMD) that run the same per-tile sequence -- scores (MFMA), softmax (vector
// ALU, mostly exponentials), P.V (MFMA) -- half a tile apart, separated by
// workgroup barriers, so that one wave of each SIMD feeds the matrix core
// while the other computes exponentials (details at the loop). K and V tiles
// pass through registers into a three-tile LDS ring: group 0 stages V^T,
// group 1 stages K, each through buffer loads whose out-of-range rows read as
// zero.
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
// LDS layout (per slot): K tile [64 keys][128 dims] with rows padded to 272 bytes and
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

#include <type_traits>

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

// Word 3 of a raw buffer resource (32-bit data format, no swizzle): loads at
// or past the resource's byte size return zero.
constexpr int kRsrcWord3 = 0x00020000;

// Buffer resource over `rows` rows of `row_bytes` bytes starting at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int rows, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, rows * row_bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS: three K tiles, then three V^T tiles (byte offsets).
constexpr int kKBytes = kKElems * 2;
constexpr int kVBytes = kVElems * 2;
constexpr int kVBase = 3 * kKBytes;
constexpr int kLdsBytes = 3 * (kKBytes + kVBytes);

// Moves a byte offset into a ring of three slots of `size` bytes from the
// slot `slot` (0..2) to the next one.
__device__ __forceinline__ uint32_t next_slot(uint32_t off, int slot, int size) {
    return off + (slot == 2 ? -2 * size : size);
}

__global__ __launch_bounds__(512, 1) void prefill_fwd_d128(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = w >> 2;  // wave group: 0 = waves 0-3, 1 = waves 4-7 (one of each per SIMD)
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
    const int kss = (int)(p.k_ss * 2), vss = (int)(p.v_ss * 2);  // row strides in bytes

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

    // ---- staging. Group 0 stages V^T, group 1 stages K; each of the 256
    // threads of a group moves four 16-byte pieces per tile through registers.
    // Group 0 thread (u, c): keys 4u..4u+3, dims 8c..8c+7 (16 consecutive lanes
    // read 16 different keys, so the transposed 8-byte LDS writes hit 16
    // different bank pairs). Group 1 thread (u, c): bytes 16u.. of key rows
    // c + 16i, written at their permuted row positions 16i + perm_row(c).
    // Rows past the end of the sequence load as zeros.
    const int gt = tid & 255;
    const int su = gt & 15, sc = gt >> 4;
    int soff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) soff[i] = grp ? (16 * i + sc) * kss + 16 * su : (4 * su + i) * vss + 16 * sc;
    const int wr_size = grp ? kKBytes : kVBytes;
    const uint32_t wr_lane = grp ? (kKStride * perm_row(sc) + 8 * su) * 2 : (kVStride * 8 * sc + 4 * su) * 2;
    const uint32_t wr0 = (grp ? 0 : kVBase) + wr_lane;  // slot 0
    u32x4 st[4];
    // The group is a compile-time tag (G = 0 or 1) in everything the loops
    // call, so that no branch on it remains inside them.
    auto stage_load = [&](int t, auto gtag) __attribute__((always_inline)) {
        constexpr int G = decltype(gtag)::value;
        const int key0 = t * kN;
        const int rows = min(kN, p.Lkv - key0);
        const __amdgpu_buffer_rsrc_t r =
            G ? rows_rsrc(kbase + (int64_t)key0 * kss, rows, kss) : rows_rsrc(vbase + (int64_t)key0 * vss, rows, vss);
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] = load16(r, soff[i]);
    };
    auto stage_store = [&](uint32_t wr, auto gtag) __attribute__((always_inline)) {
        constexpr int G = decltype(gtag)::value;
        if constexpr (G == 0) {
            // 4x8 transpose: dims 8c+e of keys 4u..4u+3 -> V^T row 8c+e, columns 4u..4u+3
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                u32x2 o;
                o[0] = __builtin_amdgcn_perm(st[1][e >> 1], st[0][e >> 1], sel);
                o[1] = __builtin_amdgcn_perm(st[3][e >> 1], st[2][e >> 1], sel);
                *reinterpret_cast<u32x2*>(lds + wr + e * kVStride * 2) = o;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(lds + wr + 16 * i * kKStride * 2) = st[i];
        }
    };

    f32x16 sacc[2];  // scores of the tile whose softmax is next
    u32x4 pk[2][2];  // bf16 weights of the tile whose P.V is next

    // ---- M phase: P.V of tile j, then the scores of tile j+1. Each product is
    // 16 MFMAs whose operands are read from LDS six ahead. `vrd` and `krd` are
    // this lane's read offsets in the slots of V^T tile j and K tile j+1.
    constexpr int kAhead = 6;
    auto pv_block = [&](uint32_t vrd) __attribute__((always_inline)) {
        // operand i: key block i >> 3, dim block (i >> 1) & 3, half i & 1
        auto addr = [&](int i) __attribute__((always_inline)) {
            return reinterpret_cast<const bf16x8*>(lds + vrd +
                                                   2 * (32 * ((i >> 1) & 3) * kVStride + 32 * (i >> 3) + 16 * (i & 1)));
        };
        bf16x8 opnd[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) opnd[i] = *addr(i);
        // the scheduling fences keep the reads six MFMAs ahead
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bf16x8 a = opnd[i % kAhead];
            if (i + kAhead < 16) opnd[i % kAhead] = *addr(i + kAhead);
            const int kb = i >> 3, dblk = (i >> 1) & 3, half = i & 1;
            oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pk[kb][half]),
                                                                 oacc[dblk], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto qk_block = [&](uint32_t krd) __attribute__((always_inline)) {
        // operand i: key block i >> 3, d-step i & 7
        auto addr = [&](int i) __attribute__((always_inline)) {
            return reinterpret_cast<const bf16x8*>(lds + krd + 2 * (32 * (i >> 3) * kKStride + 16 * (i & 7)));
        };
        bf16x8 opnd[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) opnd[i] = *addr(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bf16x8 a = opnd[i % kAhead];
            if (i + kAhead < 16) opnd[i % kAhead] = *addr(i + kAhead);
            const int kb = i >> 3, ks = i & 7;
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], ks ? sacc[kb] : (f32x16){}, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- V phase: mask, running max, exponentials and bf16 weights of tile j.
    auto vphase = [&](int j) __attribute__((always_inline)) {
        const int key0 = j * kN;
        // mask keys past the diagonal or past the end
        const bool edge = (key0 + kN > p.Lkv) || (p.causal && key0 + kN - 1 > q0 + off);
        if (edge) {
            // largest visible key offset within the tile, relative to this
            // lane's first key (8hb), so each test is against a constant
            const int lim = (p.causal ? min(qabs, p.Lkv - 1) : p.Lkv - 1) - key0 - 8 * hb;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const float x = sacc[kb][jj];
                    sacc[kb][jj] = (32 * kb + key_of(jj, 0) > lim) ? kNegInf : x;
                }
        }
        // Lazy running max: the exponentials use m_run as long as no score of
        // the lane exceeds it by the headroom; only then (wave vote) the row max
        // over the lane pair is taken and the accumulators rescaled.
        float lm = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int jj = 0; jj < 16; jj += 2) lm = fmaxf(lm, fmaxf(sacc[kb][jj], sacc[kb][jj + 1]));
        if (__builtin_amdgcn_ballot_w64(lm * c2 > m_run + kHeadroom) != 0) {
            const float m_new = fmaxf(m_run, pair_max(lm) * c2);
            const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) oacc[i][jj] *= alpha;
        }
        const float nm = -m_run;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float pr[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(fmaf(sacc[kb][8 * half + e], c2, nm));
                ls += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[kb][half][e] = pack_bf16(pr[2 * e], pr[2 * e + 1]);
            }
        l_run += ls;
    };

    // Writes piece `t` of this group (V^T for group 0, K for group 1) at `wr`
    // and requests piece t+1.
    auto stage = [&](int t, uint32_t wr, auto gtag) __attribute__((always_inline)) {
        if (t < ntiles) {
            // the piece was requested two segments ago
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            stage_store(wr, gtag);
            if (t + 1 < ntiles) stage_load(t + 1, gtag);
        }
    };
    // M phase of tile j (P.V of j, scores of j+1) for this wave, if any, after
    // the group's staging step.
    auto mstep = [&](int j, int t, uint32_t wr, uint32_t vrd, uint32_t krd, auto gtag) __attribute__((always_inline)) {
        const bool pv = j >= 0 && j * kN <= wave_last_key;
        const bool qk = j + 1 < ntiles && (j + 1) * kN <= wave_last_key;
        __builtin_amdgcn_s_setprio(1);
        stage(t, wr, gtag);
        if (pv) pv_block(vrd);
        if (qk) qk_block(krd);
        __builtin_amdgcn_s_setprio(0);
    };
    auto vstep = [&](int j) __attribute__((always_inline)) {
        if (j >= 0 && j < ntiles && j * kN <= wave_last_key) vphase(j);
    };

    // ---- Schedule. Per wave, tile j goes through M(j-1) (its scores, with the
    // P.V of tile j-1), V(j) (softmax) and M(j) (its P.V, with the scores of
    // tile j+1). The two wave groups run this sequence one segment apart, with
    // a workgroup barrier between segments, so that on every SIMD one wave
    // issues MFMAs while the other one computes exponentials:
    //   segment 2k:   group 0 M(k-1)   group 1 V(k-1)
    //   segment 2k+1: group 0 V(k)     group 1 M(k-1)
    // The V phase is the softmax alone; LDS staging rides in the M phase, whose
    // vector ALU is otherwise idle. LDS holds three tiles (slot = tile % 3):
    // group 0 writes V^T of tile k in segment 2k (read from segment 2k+2 on),
    // group 1 writes K of tile k+1 in segment 2k+1 (read from segment 2k+2
    // on); a slot is rewritten only after both groups have passed the M phase
    // that read its previous tile. Each group requests its next piece from
    // global memory two segments before writing it. Both groups pass the same
    // 2(ntiles + 1) barriers.
    // In iteration k the read offsets point at slots (k+2)%3 (V^T of tile
    // k-1) and k%3 (K of tile k); the write offset at k%3 (group 0) or
    // (k+1)%3 (group 1). All move one slot per iteration.
    auto run = [&](auto gtag) __attribute__((always_inline)) {
        constexpr int G = decltype(gtag)::value;
        uint32_t vrd = kVBase + 2 * kVBytes + (row * kVStride + 8 * hb) * 2;
        uint32_t krd = (row * kKStride + 8 * hb) * 2;
        uint32_t wr = G ? wr0 + wr_size : wr0;
        stage_load(0, gtag);
        if constexpr (G == 1) {
            stage_store(wr0, gtag);
            if (ntiles > 1) stage_load(1, gtag);
        }
        __syncthreads();
        for (int k = 0; k <= ntiles; ++k) {
            const int s0 = k % 3;
            if constexpr (G == 0) {
                mstep(k - 1, k, wr, vrd, krd, gtag);
                __syncthreads();
                vstep(k);
                __syncthreads();
            } else {
                vstep(k - 1);
                __syncthreads();
                mstep(k - 1, k + 1, wr, vrd, krd, gtag);
                __syncthreads();
            }
            vrd = next_slot(vrd, (s0 + 2) % 3, kVBytes);
            krd = next_slot(krd, s0, kKBytes);
            wr = next_slot(wr, G ? (s0 + 1) % 3 : s0, wr_size);
        }
    };
    if (grp == 0)
        run(std::integral_constant<int, 0>{});
    else
        run(std::integral_constant<int, 1>{});

    // Keep the staging registers live to here, so that both loops (and the
    // prologue) stage through the same registers and no other loop-carried
    // value is given a register that a load of the other group's loop writes
    // (the compiler would then wait for those loads before using it).
    asm volatile("" ::"v"(st[0]), "v"(st[1]), "v"(st[2]), "v"(st[3]));

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
