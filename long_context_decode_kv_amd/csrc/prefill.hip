// Fused prefill attention for gfx950 (bf16, head dim 128 or 64, causal or not).
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
// go from global memory straight into a four-tile LDS ring (buffer loads with
// an LDS destination, no registers; out-of-range rows arrive as zeros): group
// 0 moves V, group 1 moves K.
//
// Both products are computed transposed so that one query row lives in one
// lane and the softmax needs no cross-lane reduction except one lane-pair exchange:
//   S^T (32 keys x 32 rows) = K Q^T      v_mfma_f32_32x32x16_bf16, 8 steps over d
//   O^T (32 dims x 32 rows) += V^T P^T   same instruction, 16 keys per step
// Lane l holds query row (l & 31) and 16 of the 32 keys of each key block; the
// K rows are fed to the MFMA in a permuted order (bits 2 and 3 of the row
// index swapped) so that those 16 keys come as two runs of 8 consecutive keys,
// which makes P^T usable directly as the B operand of the second product.
// V stays row-major in LDS; its V^T operands come from the transposed LDS
// read (ds_read_b64_tr_b16: 16 lanes read a 4-key x 16-dim block and each
// lane receives the 4 keys of its own dim), two per operand.
//
// LDS layout (per slot): K and V tiles of 64 rows x 256 bytes, unpadded, with
// the 16-byte chunks of K rows and the 64-byte segments of V rows rotated by
// row so that every operand read is free of bank conflicts (details at the
// staging code).
//
// Causal masking (bottom-right aligned: query i sees keys <= Lkv - Lq + i) is
// applied only on tiles that cross the diagonal; tiles past it are skipped.
// Workgroups are issued heaviest (latest) query block first.
#include "internal.h"

#include <algorithm>
#include <type_traits>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 32;        // query rows per wave
constexpr int kN = 64;           // keys per tile

// Sizes that follow the head dim D (128 or 64) and the number of wave groups
// NG (2: eight waves, a four-tile ring; 1: four waves, a two-tile ring): a K
// or V row of 2D bytes in 2D / 16 chunks of 16 bytes, a 64-row tile, a ring
// slot of one K and one V tile, the ring, the 32 x D fp32 output tile a wave
// stages (4D bytes a row).
template <int D, int NG>
struct Geom {
    static_assert(D == 128 || D == 64, "head dim");
    static_assert(NG == 1 || NG == 2, "wave groups");
    static constexpr int kWaves = 4 * NG;
    static constexpr int kSlots = NG == 2 ? 4 : 2;
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = kRowBytes / 16;
    static constexpr int kTileBytes = kN * kRowBytes;
    static constexpr int kSlotBytes = 2 * kTileBytes;
    static constexpr int kLdsBytes = kSlots * kSlotBytes;  // also holds the Q rows and the output tiles
    static constexpr int kKSteps = D / 16;     // k-steps of the scores over d
    static constexpr int kDimBlocks = D / 32;  // 32-dim output blocks
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one 1 KB LDS-destination load fills
    static constexpr int kOutRow = 4 * D;                  // bytes of a staged fp32 output row
};

// LDS position of 16-byte chunk c of a K (or staged Q) row r, chosen so that
// the 16 rows one operand read touches per 16 lanes (same chunk) hit 16
// different 16-byte bank groups: with 256-byte rows c ^ (r & 15); with
// 128-byte rows two rows share a 256-byte bank window, so the rows of each
// parity take c ^ ((r >> 1) & 7).
template <int D>
__device__ __forceinline__ int kchunk(int r, int c) {
    if constexpr (D == 128) return c ^ (r & 15);
    else return c ^ ((r >> 1) & 7);
}
// Position of the 64-byte segment sg (32 dims) of V row r: the four rows a
// transposed read touches per 32 lanes must cover all 64 banks once. 256-byte
// rows: (sg + r) & 3. 128-byte rows (two segments, rows r and r + 1 in
// different bank halves): (sg + ((r & 3) >> 1)) & 1.
template <int D>
__device__ __forceinline__ int vseg(int r, int sg) {
    if constexpr (D == 128) return (sg + r) & 3;
    else return (sg + ((r & 3) >> 1)) & 1;
}
// The segment of V row r that position ps holds (the inverse of vseg).
template <int D>
__device__ __forceinline__ int vseg_at(int r, int ps) {
    if constexpr (D == 128) return (ps - r) & 3;
    else return (ps + ((r & 3) >> 1)) & 1;
}
constexpr float kHeadroom = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
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
// or past the resource's byte size return zero (also into LDS).
constexpr int kRsrcWord3 = 0x00020000;

// Buffer resource over `rows` rows of `row_bytes` bytes starting at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int rows, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, rows * row_bytes, kRsrcWord3);
}

typedef __attribute__((address_space(3))) char lds_char;

// Workgroup barrier for the main loop. Unlike __syncthreads it does not wait
// for outstanding loads into LDS (the compiler's release fence would): those
// are completed explicitly, one M phase after they are issued, so they stay
// in flight across the barriers in between. It waits for this wave's own LDS
// reads (lgkmcnt(0)), so no slot is overwritten while a read of it is in
// flight, and the empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void loop_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
typedef short v4i16 __attribute__((ext_vector_type(4)));

// BAND: the key set of a query at position qpos = i + p.diag is bounded on
// both sides, keys j with qpos - p.window <= j <= qpos (no lower bound when
// p.window < 0; p.diag may be negative, so a row can see no key at all: it
// gets O = 0 and lse = -inf). Used for pi-Attention's window and its strided
// skip classes; without BAND the kernel is plain causal (diag = Lkv - Lq) or
// full attention.
//
// NG = 2 is the two-group workgroup described at the top of the file. NG = 1
// is a four-wave workgroup (one wave per SIMD) with a two-tile ring, of which
// two fit on a compute unit, so that one workgroup's loads, barrier waits and
// stores overlap the other's products (launches whose workgroups walk only a
// few tiles); each wave runs scores, softmax and P.V of a tile in turn, with
// one barrier per tile (at the loop). Both compute every row the same way:
// the same tiles, the same products in the same order, so the outputs are
// bit-identical.
template <bool BAND, int D, int NG>
__global__ __launch_bounds__(256 * NG, 3 - NG) void prefill_fwd(PrefillParams p) {
    using Gm = Geom<D, NG>;
    constexpr int kRowBytes = Gm::kRowBytes, kTileBytes = Gm::kTileBytes, kSlotBytes = Gm::kSlotBytes;
    constexpr int kLdsBytes = Gm::kLdsBytes, kKSteps = Gm::kKSteps, kDB = Gm::kDimBlocks;
    constexpr int kWaves = Gm::kWaves, kSlots = Gm::kSlots;
    __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes + kWaves * kRows * 4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = w >> 2;  // wave group: 0 = waves 0-3, 1 = waves 4-7 (one of each per SIMD)
    const int wv = w & 3;    // wave within its group
    const int hb = lane >> 5, row = lane & 31;
    const int G = p.Hq / p.Hkv;
    const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);  // query heads per workgroup
    const int PW = kWaves / HW;                                // 32-position blocks per workgroup
    const int span = kRows * PW;                               // positions per workgroup
    const int nqb = (p.Lq + span - 1) / span;
    const int hgroups = G / HW;

    // Workgroup -> (position block, batch, KV head, head group). Plain:
    // heaviest (latest) position block first. Banded: batch entry first (a
    // residue class of a skip launch), then its position blocks, KV head
    // fastest, so the blocks of one class run together on the XCD of their
    // KV head (round-robin by workgroup index) and share its K/V tiles in L2.
    const int id = blockIdx.x;
    int qb, hgi, b, g;
    if constexpr (BAND) {
        const int inner = nqb * p.Hkv * hgroups;
        b = id / inner;
        const int rem = id % inner;
        g = rem % p.Hkv;
        const int r2 = rem / p.Hkv;
        hgi = r2 % hgroups;
        qb = nqb - 1 - r2 / hgroups;
    } else {
        const int per_qb = p.B * p.Hkv * hgroups;
        qb = nqb - 1 - id / per_qb;
        const int rem = id % per_qb;
        hgi = rem % hgroups;
        const int bg = rem / hgroups;
        b = bg / p.Hkv;
        g = bg % p.Hkv;
    }
    const int h = g * G + hgi * HW + (w % HW);

    const int off = BAND ? p.diag : p.Lkv - p.Lq;  // bottom-right alignment unless banded
    const int p0 = qb * span;
    const int q0 = p0 + kRows * (w / HW);  // first query row of this wave
    const int kv_limit = p.causal ? min(p.Lkv, p0 + span + off) : p.Lkv;
    // tiles t0 .. t0 + ntiles - 1 hold this workgroup's keys
    const bool lower = BAND && p.window >= 0;
    const int t0 = lower ? max(0, p0 + off - p.window) / kN : 0;
    const int ntiles = max(0, (kv_limit + kN - 1) / kN - t0);
    const int wave_last_key = p.causal ? min(p.Lkv - 1, q0 + kRows - 1 + off) : p.Lkv - 1;
    // local tiles [jw_lo, jw_hi] hold keys some row of this wave sees
    // (wave_last_key may be negative when banded; floor division)
    const int jw_hi = (wave_last_key >= 0 ? wave_last_key / kN : -1) - t0;
    const int jw_lo = lower ? max(0, max(0, q0 + off - p.window) / kN - t0) : 0;

    const char* kbase = static_cast<const char*>(p.k) + (b * p.k_sb + g * p.k_sh) * 2;
    const char* vbase = static_cast<const char*>(p.v) + (b * p.v_sb + g * p.v_sh) * 2;
    const int kss = (int)(p.k_ss * 2), vss = (int)(p.v_ss * 2);  // row strides in bytes

    // Q^T operand: column `row` is query q0 + row; k-slots are dims 16ks + 8hb + e.
    // The wave's 32 rows come through LDS (8 KB per wave in the last NG ring
    // slots, which the first tiles leave free): buffer loads with an LDS
    // destination, 16 lanes per 256-byte row, so the global reads are whole
    // rows; chunk c of row r lands at position c ^ (r & 15), so the operand
    // reads (chunk 2ks + hb of rows 0..15 per 16 lanes) hit distinct banks.
    // Rows past the end of the queries arrive as zeros.
    // Register arrays are sized for d = 128 (only the first kKSteps / kDB
    // entries are used at d = 64): an array whose size depends on D would make
    // the builtin calls that take its elements type-dependent, and the host
    // pass would then emit no launch stub for the kernel.
    bf16x8 qop[8];
    const uint32_t qstage = (kSlots - NG) * kSlotBytes + w * (kRows * kRowBytes);
    {
        const int qrows = max(0, min(kRows, p.Lq - q0));
        const int qss = (int)(p.q_ss * 2);
        const char* qbase = static_cast<const char*>(p.q) + (b * p.q_sb + h * p.q_sh + (int64_t)q0 * p.q_ss) * 2;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(qbase), 0, qrows > 0 ? (qrows - 1) * qss + kRowBytes : 0, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < kRows / Gm::kRowsPerLoad; ++i) {
            const int rr = Gm::kRowsPerLoad * i + lane / Gm::kChunks, pc = lane % Gm::kChunks;
            const int goff = rr * qss + 16 * kchunk<D>(rr, pc);  // a plain int: see the arrays above
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_char*)lds + qstage + 1024 * i, 16, goff, 0, 0, 0);
        }
    }
    const float c2 = p.scale_log2;
    const int qabs = q0 + row + off;  // absolute position of this lane's query row
    // pi-Attention merge inputs of this lane's row, loaded now so the epilogue
    // does not wait for them: the prior alpha and the lse of the part already
    // in `out`
    const int64_t li = b * p.lse_sb + h * p.lse_sh + (int64_t)(q0 + row) * p.lse_ss;
    float alpha_row = 1.f, lse_prev = kNegInf;
    if constexpr (BAND) {
        if (p.merge && q0 + row < p.Lq) {
            if (p.alpha) alpha_row = p.alpha[li];
            if (p.merge != 2) lse_prev = p.lse_w[li];
        }
    }

    f32x16 oacc[4];
#pragma unroll
    for (int i = 0; i < kDB; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    // ---- LDS tiles. Slot s holds K of one tile at s * kSlotBytes and V of the
    // same tile right after it, both as 64 rows of 256 bytes, no padding:
    //  * K row r holds the key whose row in the MFMA order is r (rows are fed
    //    with bits 2 and 3 of the index swapped), and its 16-byte chunk c sits
    //    at position c ^ (r & 15), so the 16 rows one operand read touches per
    //    16 lanes hit 16 different bank groups;
    //  * V row r holds key r, and its 64-byte segment d (dims 32d..32d+31)
    //    sits at position (d + r) & 3, so the four rows one transposed read
    //    touches per 32 lanes cover all 64 banks once.
    // Tiles go from global memory straight into LDS (buffer loads with an LDS
    // destination, no registers): each wave moves 4 KB per tile with four
    // 1 KB instructions, lane i writing bytes 16i..16i+15 of each; the global
    // address each lane asks for makes the layout above. With two groups,
    // group 0 moves V and group 1 moves K; with one, every wave moves its
    // rows of both. Rows past the end of the sequence arrive as zeros.
    constexpr int kLoads = 16 / Gm::kRowsPerLoad;  // 1 KB loads a wave issues per K or V tile
    // NG = 1: soff holds the K offsets; the V rows of load i are those of
    // load 0 plus kRowsPerLoad * i, in the same segment order (which follows
    // the row mod 4), so their offset is vsoff0 plus a multiple of the stride.
    int soff[4];
    int vsoff0 = 0;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        // LDS row and 16-byte chunk position written
        const int r = 16 * wv + Gm::kRowsPerLoad * i + lane / Gm::kChunks, q = lane % Gm::kChunks;
        if (NG == 1 || grp) {
            const int key = (r & ~31) | perm_row(r & 31);
            soff[i] = key * kss + 16 * kchunk<D>(r, q);  // kchunk is its own inverse
        } else {
            soff[i] = r * vss + 64 * vseg_at<D>(r, q >> 2) + 16 * (q & 3);
        }
        if (NG == 1 && i == 0) vsoff0 = r * vss + 64 * vseg_at<D>(r, q >> 2) + 16 * (q & 3);
    }
    // Requests this wave's piece of K (GG = 1) or V (GG = 0) of tile t into
    // LDS slot t % kSlots.
    auto dma = [&](int t, auto gtag) __attribute__((always_inline)) {
        constexpr int GG = decltype(gtag)::value;
        const int key0 = (t0 + t) * kN;
        const int rows = min(kN, p.Lkv - key0);
        const __amdgpu_buffer_rsrc_t r = GG ? rows_rsrc(kbase + (int64_t)key0 * kss, rows, kss)
                                            : rows_rsrc(vbase + (int64_t)key0 * vss, rows, vss);
        lds_char* dst = (lds_char*)lds + (t % kSlots) * kSlotBytes + (GG ? 0 : kTileBytes) + wv * (kTileBytes / 4);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            // the whole offset in the vector operand (the bounds check that
            // zero-fills rows past the end covers only that one), as a plain
            // int: see the arrays above
            int off = soff[i];
            if constexpr (NG == 1 && GG == 0) off = vsoff0 + Gm::kRowsPerLoad * i * vss;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + 1024 * i, 16, off, 0, 0, 0);
        }
    };

    // Per-lane read offsets within a slot. K operand (key block kb, d-step
    // ks): row 32kb + row, chunk (2ks + hb) ^ (row & 15). V^T operand (dim
    // block dblk, keys kk..kk+3 for the transposed read): this lane supplies
    // the address of keys kk + (i16 >> 2), dims 32dblk + 16g + 4(i16 & 3).
    uint32_t kofs[8], vofs[4];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) kofs[ks] = row * kRowBytes + 16 * kchunk<D>(row, 2 * ks + hb);
    {
        const int i16 = lane & 15, ga = i16 >> 2, gb = i16 & 3, gg = (lane >> 4) & 1;
#pragma unroll
        for (int dblk = 0; dblk < kDB; ++dblk)
            vofs[dblk] = kTileBytes + (8 * hb + ga) * kRowBytes + 64 * vseg<D>(ga, dblk) + 32 * gg + 8 * gb;
    }

    f32x16 sacc[2];  // scores of the tile whose softmax is next
    u32x4 pk[2][2];  // bf16 weights of the tile whose P.V is next

    // ---- M phase: P.V of tile j, then the scores of tile j+1. Each product is
    // 16 MFMAs whose operands are read from LDS four (V^T: transposed reads,
    // two per operand) or six (K) MFMAs ahead. Consecutive MFMAs accumulate
    // into different tiles (the four dim blocks of O, the two key blocks of
    // S); each tile still sums its steps in the same order.
    constexpr int kAhead = NG == 2 ? 6 : 4;
    auto pv_block = [&](uint32_t slot) __attribute__((always_inline)) {
        // operand i: key block kb = i / (2 kDB), dim block i % kDB, half (i / kDB) & 1:
        // keys 32kb + 16half + 8hb + (0..7), dim 32dblk + (lane & 31)
        auto rd = [&](int i) __attribute__((always_inline)) {
            const int kb = i / (2 * kDB), dblk = i % kDB, half = (i / kDB) & 1;
            const uint32_t a0 = slot + vofs[dblk] + (32 * kb + 16 * half) * kRowBytes;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)((lds_char*)lds + a0));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)((lds_char*)lds + a0 + 4 * kRowBytes));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        constexpr int kA = 4;
        bf16x8 opnd[kA];
#pragma unroll
        for (int i = 0; i < kA; ++i) opnd[i] = rd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4 * kDB; ++i) {
            const bf16x8 a = opnd[i % kA];
            if (i + kA < 4 * kDB) opnd[i % kA] = rd(i + kA);
            const int kb = i / (2 * kDB), dblk = i % kDB, half = (i / kDB) & 1;
            oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pk[kb][half]),
                                                                 oacc[dblk], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto qk_block = [&](uint32_t slot) __attribute__((always_inline)) {
        // operand i: key block i & 1, d-step i >> 1
        auto rd = [&](int i) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8*>(lds + slot + kofs[i >> 1] + 32 * (i & 1) * kRowBytes);
        };
        bf16x8 opnd[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) opnd[i] = rd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2 * kKSteps; ++i) {
            const bf16x8 a = opnd[i % kAhead];
            if (i + kAhead < 2 * kKSteps) opnd[i % kAhead] = rd(i + kAhead);
            const int kb = i & 1, ks = i >> 1;
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], ks ? sacc[kb] : (f32x16){}, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- V phase: mask, running max, exponentials and bf16 weights of tile j.
    auto vphase = [&](int j) __attribute__((always_inline)) {
        const int key0 = (t0 + j) * kN;
        // mask keys past the diagonal or past the end (and, banded, below the window)
        const bool edge = (key0 + kN > p.Lkv) || (p.causal && key0 + kN - 1 > q0 + off) ||
                          (lower && key0 < q0 + kRows - 1 + off - p.window);
        if (edge) {
            // largest visible key offset within the tile, relative to this
            // lane's first key (8hb), so each test is against a constant
            const int lim = (p.causal ? min(qabs, p.Lkv - 1) : p.Lkv - 1) - key0 - 8 * hb;
            if constexpr (BAND) {
                // visible offsets [lo, lim] as one unsigned range test
                int lo = lower ? qabs - p.window - key0 - 8 * hb : -kN;
                int wd = lim - lo;
                if (wd < 0) {  // nothing visible: a range no offset falls in
                    lo = 1 << 20;
                    wd = 0;
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) {
                        const float x = sacc[kb][jj];
                        const int ko = 32 * kb + key_of(jj, 0);
                        sacc[kb][jj] = ((uint32_t)(ko - lo) > (uint32_t)wd) ? kNegInf : x;
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) {
                        const float x = sacc[kb][jj];
                        sacc[kb][jj] = (32 * kb + key_of(jj, 0) > lim) ? kNegInf : x;
                    }
            }
        }
        // Lazy running max: the exponentials use m_run as long as no score of
        // the lane exceeds it by the headroom; only then (wave vote) the row max
        // over the lane pair is taken and the accumulators rescaled.
        // one chain of three-input maxima (two new scores per step)
        float lm = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int jj = kb ? 0 : 2; jj < 16; jj += 2) lm = fmaxf(fmaxf(lm, sacc[kb][jj]), sacc[kb][jj + 1]);
        if (__builtin_amdgcn_ballot_w64(lm * c2 > m_run + kHeadroom) != 0) {
            const float m_new = fmaxf(m_run, pair_max(lm) * c2);
            const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < kDB; ++i)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) oacc[i][jj] *= alpha;
        }
        // banded rows may have seen no key yet (m_run = -inf): their masked
        // scores must give weight 0, not exp2(-inf + inf)
        const float nm = (BAND && m_run == kNegInf) ? 0.f : -m_run;
        float ls;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float pr[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(fmaf(sacc[kb][8 * half + e], c2, nm));
                const float gs = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
                ls = (kb == 0 && half == 0) ? gs : ls + gs;
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[kb][half][e] = pack_bf16(pr[2 * e], pr[2 * e + 1]);
            }
        l_run += ls;
        // Issue order: one exponential (transcendental, mask 0x400), then
        // three other vector instructions (mask 0x2), instead of runs of four
        // exponentials: the partner wave issues its MFMAs between them (same
        // results; 16K prefill about 0.5 % faster).
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x2, 3, 0);
        }
    };

    // M phase of tile j (P.V of j, scores of j+1) for this wave, if any, after
    // requesting the group's piece of tile j+3. The wait at the end (vmcnt)
    // completes the previous request, tile j+2's piece, before the barrier
    // that precedes its first reader.
    auto mstep = [&](int j, auto gtag) __attribute__((always_inline)) {
        const bool pv = j >= jw_lo && j <= jw_hi;
        const bool qk = j + 1 < ntiles && j + 1 >= jw_lo && j + 1 <= jw_hi;
        __builtin_amdgcn_s_setprio(1);
        const bool more = j + 3 < ntiles;
        // the request goes after the transposed V reads: the compiler makes
        // those wait for every outstanding LDS load
        if (pv) pv_block((uint32_t)((j % kSlots) * kSlotBytes));
        if (more) dma(j + 3, gtag);
        if (qk) qk_block((uint32_t)(((j + 1) % kSlots) * kSlotBytes));
        __builtin_amdgcn_s_setprio(0);
        if (more)
            __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4): all but the four just issued
        else
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    };
    auto vstep = [&](int j) __attribute__((always_inline)) {
        if (j >= jw_lo && j < ntiles && j <= jw_hi) vphase(j);
    };

    // ---- Schedule. Per wave, tile j goes through M(j-1) (its scores, with the
    // P.V of tile j-1), V(j) (softmax) and M(j) (its P.V, with the scores of
    // tile j+1). The two wave groups run this sequence one segment apart, with
    // a workgroup barrier between segments, so that on every SIMD one wave
    // issues MFMAs while the other one computes exponentials:
    //   segment 2k:   group 0 M(k-1)   group 1 V(k-1)
    //   segment 2k+1: group 0 V(k)     group 1 M(k-1)
    // Tile t lives in LDS slot t % 4. In M(j) (segment 2j+2+g for group g)
    // each group requests its piece of tile j+3, after its P.V reads: the
    // slot's previous tile, j-1, was last read as K in M(j-2) and as V in
    // M(j-1), both in earlier segments. The request is complete at the end of
    // the group's next M phase, M(j+1), before the barrier that precedes the
    // first reader of tile j+3, M(j+2) of group 0. Tiles 0 and 1 are
    // requested before the loop. Both groups pass the same 2(ntiles + 1)
    // barriers.
    auto run = [&](auto gtag) __attribute__((always_inline)) {
        constexpr int GG = decltype(gtag)::value;
        if (ntiles > 0) dma(0, gtag);
        if (ntiles > 1) dma(1, gtag);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): tiles 0-1 and this wave's Q rows
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks)
            qop[ks] = *reinterpret_cast<const bf16x8*>(lds + qstage + row * kRowBytes +
                                                       16 * kchunk<D>(row, 2 * ks + hb));
        loop_barrier();  // every wave holds its Q before tile 2 is requested into slot 2
        for (int k = 0; k <= ntiles; ++k) {
            if constexpr (GG == 0) {
                mstep(k - 1, gtag);
                loop_barrier();
                vstep(k);
                loop_barrier();
            } else {
                vstep(k - 1);
                loop_barrier();
                mstep(k - 1, gtag);
                loop_barrier();
            }
        }
    };
    // One group: tile t in slot t % 2. Iteration k: P.V of tile k-1; wait for
    // this wave's piece of tile k (requested in iteration k-1); barrier (every
    // piece of tile k is in, every wave is done with slot (k-1) % 2); request
    // tile k+1 into that slot; scores and softmax of tile k. The request has
    // the scores and the softmax to land before the P.V reads it. Every wave
    // passes the same ntiles + 1 barriers.
    auto run1 = [&]() __attribute__((always_inline)) {
        const std::integral_constant<int, 1> kt{};
        const std::integral_constant<int, 0> vt{};
        if (ntiles > 0) {
            dma(0, kt);
            dma(0, vt);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): tile 0 and this wave's Q rows
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks)
            qop[ks] = *reinterpret_cast<const bf16x8*>(lds + qstage + row * kRowBytes +
                                                       16 * kchunk<D>(row, 2 * ks + hb));
        for (int k = 0; k <= ntiles; ++k) {
            if (k >= 1 && k - 1 >= jw_lo && k - 1 <= jw_hi) pv_block((uint32_t)(((k - 1) % kSlots) * kSlotBytes));
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's piece of tile k
            loop_barrier();  // also: every wave holds its Q before tile 1 goes into the Q rows' slot
            if (k + 1 < ntiles) {
                dma(k + 1, kt);
                dma(k + 1, vt);
            }
            if (k < ntiles && k >= jw_lo && k <= jw_hi) {
                qk_block((uint32_t)((k % kSlots) * kSlotBytes));
                vphase(k);
            }
        }
    };
    if constexpr (NG == 1) {
        run1();
    } else {
        if (grp == 0)
            run(std::integral_constant<int, 0>{});
        else
            run(std::integral_constant<int, 1>{});
    }

    // epilogue: O = acc / l, lse = m ln2 + ln l. The rows go out through LDS
    // (the ring is free after the loop's last barrier): each wave stages its
    // 32 x D fp32 tile (4D bytes a row, chunk c of row r at c ^ (r & 15), so
    // the writes and the row reads both hit distinct banks), then 16 lanes
    // write each 128-byte piece of a bf16 row, so the global stores (and the
    // reads of the part already in `out` when merging) are whole lines.
    const bool merge_prev = BAND && (p.merge == 1 || p.merge == 3);
    uint16_t* obase = static_cast<uint16_t*>(p.out) + b * p.o_sb + h * p.o_sh;
    // the part already in `out` (merging): rows 4i + (lane >> 4), dims 4c .. 4c + 3
    // with c = 16 hh + (lane & 15), requested before the staging below
    constexpr int kHH = D / 64;  // 128-byte pieces of a bf16 output row
    u32x2 prev[8][2];
    if (merge_prev) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int hh = 0; hh < kHH; ++hh) {
                const int r = 4 * i + (lane >> 4), c = 16 * hh + (lane & 15);
                prev[i][hh] = q0 + r < p.Lq
                                  ? *reinterpret_cast<const u32x2*>(obase + (int64_t)(q0 + r) * p.o_ss + 4 * c)
                                  : u32x2{0u, 0u};
            }
    }
    const float l_tot = pair_sum(l_run);
    const int qr = q0 + row;
    const bool empty = BAND && !(l_tot > 0.f);  // a banded row that saw no key
    float inv = empty ? 0.f : 1.0f / l_tot;
    float lse = empty ? kNegInf : fmaf(m_run, kLn2, logf(l_tot));  // one rounding in every instantiation
    float wprev = 0.f;  // weight of the part already in `out` (merge 1 and 3)
    if constexpr (BAND) {
        if (p.merge && qr < p.Lq) {
            // pi-Attention's log-priors: + ln(alpha) on the window part,
            // + ln(1 - alpha) on the skip part
            float bw = 0.f, bs = 0.f;
            if (p.alpha) {
                const float a = fminf(fmaxf(alpha_row, 0.f), 1.f);
                bw = logf(a);
                bs = logf(1.f - a);
            }
            if (p.merge == 2) {  // the window alone
                lse += bw;
                if (lse == kNegInf) inv = 0.f;
            } else {
                // this launch's part is skip keys; the part already in
                // out / lse_w is the window (merge 1: its prior still to
                // add) or the window and the other skip keys (merge 3:
                // priors included)
                if (p.merge == 3) bw = 0.f;
                const float mw = lse_prev + bw, ms = lse + bs;
                const float M = fmaxf(mw, ms);
                const float ww = (mw == kNegInf) ? 0.f : fast_exp2((mw - M) * kLog2e);
                const float ws = (ms == kNegInf) ? 0.f : fast_exp2((ms - M) * kLog2e);
                const float z = ww + ws;
                const float iz = (M == kNegInf) ? 0.f : 1.f / z;
                wprev = ww * iz;
                inv *= ws * iz;
                lse = (M == kNegInf) ? kNegInf : M + logf(z);
            }
        }
    }
    if (qr < p.Lq && p.lse && hb == 0) p.lse[li] = lse;
    const uint32_t ostage = w * (kRows * Gm::kOutRow);
    float* wstage = reinterpret_cast<float*>(lds + kLdsBytes) + w * kRows;
#pragma unroll
    for (int dblk = 0; dblk < kDB; ++dblk)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            // dims 32 dblk + 8 jj + 4 hb .. +3: 16-byte chunk 8 dblk + 2 jj + hb
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = oacc[dblk][4 * jj + e] * inv;
            *reinterpret_cast<f32x4*>(lds + ostage + row * Gm::kOutRow + 16 * ((8 * dblk + 2 * jj + hb) ^ (row & 15))) = o;
        }
    if (hb == 0) wstage[row] = wprev;
    loop_barrier();  // LDS writes done; the loads of the part in `out` stay in flight
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        if (q0 + r >= p.Lq) continue;
        uint16_t* orow = obase + (int64_t)(q0 + r) * p.o_ss;
        const float wp = merge_prev ? wstage[r] : 0.f;
#pragma unroll
        for (int hh = 0; hh < kHH; ++hh) {
            const int c = 16 * hh + (lane & 15);  // dims 4c .. 4c + 3
            f32x4 o = *reinterpret_cast<const f32x4*>(lds + ostage + r * Gm::kOutRow + 16 * (c ^ (r & 15)));
            if (merge_prev) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w2 = prev[i][hh][e >> 1];
                    const float x = __builtin_bit_cast(float, (e & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
                    o[e] = fmaf(wp, x, o[e]);
                }
            }
            u32x2 pk;
            pk[0] = pack_bf16(o[0], o[1]);
            pk[1] = pack_bf16(o[2], o[3]);
            *reinterpret_cast<u32x2*>(orow + 4 * c) = pk;
        }
    }
}

}  // namespace

namespace {
template <int NG>
hipError_t launch_prefill_ng(const PrefillParams& p, hipStream_t stream) {
    constexpr int kWaves = 4 * NG;
    const int G = p.Hq / p.Hkv;
    const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
    const int span = kRows * (kWaves / HW);
    const int64_t nqb = (p.Lq + span - 1) / span;
    const int64_t wgs = nqb * p.B * p.Hkv * (G / HW);
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    if (wgs == 0) return hipSuccess;
    const dim3 grid((unsigned)wgs), block(64 * kWaves);
    if (p.d == 128) {
        if (p.band) hipLaunchKernelGGL((prefill_fwd<true, 128, NG>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((prefill_fwd<false, 128, NG>), grid, block, 0, stream, p);
    } else if constexpr (NG == 1) {  // d = 64 always takes four-wave workgroups
        if (p.band) hipLaunchKernelGGL((prefill_fwd<true, 64, NG>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((prefill_fwd<false, 64, NG>), grid, block, 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

// Four-wave workgroups (two per compute unit) when no workgroup walks more
// than sixteen 64-key tiles: then a workgroup's start, barrier waits and
// stores weigh about as much as its products, and the second workgroup on the
// compute unit hides them. Longer walks keep the eight-wave workgroup, whose
// K/V tiles serve twice the rows. Causal prefills, 32q/8kv, d = 128, eight
// and four waves: 64 x 256 tokens 0.116 / 0.096 ms, 32 x 512 0.149 / 0.134 ms,
// 16 x 1024 0.188 / 0.185 ms, 4 x 4096 0.493 / 0.528 ms, 16K 1.81 / 1.98 ms;
// the 16K pi-Attention prefill (window 512, period 64: a window launch of
// 576-key walks and skip-class launches of 256 keys) 0.350 / 0.327 ms.
// At d = 64 a tile's products take half the MFMA time while the softmax work
// stays, and the four-wave form (139 VGPRs, 32.5 KB of LDS: three workgroups
// per compute unit) wins at every length: 16K causal 1.159 / 1.087 ms,
// 4 x 4096 0.315 / 0.288 ms, 16 x 1024 0.114 / 0.092 ms.
static bool narrow_prefill(const PrefillParams& p) {
    if (p.d == 64) return true;
    int64_t keys = p.Lkv;  // keys one workgroup may walk
    if (p.band && p.window >= 0) keys = std::min<int64_t>(keys, (int64_t)p.window + 2 * kRows);
    return keys <= 16 * kN;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    if (p.d != 128 && p.d != 64) return hipErrorInvalidValue;
    return narrow_prefill(p) ? launch_prefill_ng<1>(p, stream) : launch_prefill_ng<2>(p, stream);
}

}  // namespace attn
