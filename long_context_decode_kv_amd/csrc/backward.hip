// Backward pass of exact attention for gfx950 (bf16 inputs, head dim 128).
//
// The gradient of the attention output with respect to its inputs (attention
// as the gradient of a scalar energy function is the starting point of the
// Tree Attention explainer, section 3; the backward pass differentiates that
// forward once more). With logits z = sigma q.k, P the row softmax over the
// visible keys, O = P V and the incoming gradient dO:
//   D_i = dO_i . O_i,  dP_ij = dO_i . v_j,  dz_ij = P_ij (dP_ij - D_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = sigma sum_i dz_ij q_i,  dQ_i = sigma sum_j dz_ij k_j.
// P is recomputed from the forward's lse (P_ij = exp(z_ij - lse_i)), so
// nothing of size L x L is stored.
//
// Three kernels, no atomics (results are deterministic):
//  * bwd_prep:  D per row (one wave per row).
//  * bwd_dkdv:  one workgroup per 64-key block of one KV head; it walks the
//    64-row query blocks of every query head of the group that see the block,
//    recomputes P and dz for the 64 x 64 tile, and accumulates dV = P^T dO and
//    dK = dz^T Q in registers.
//  * bwd_dq:    one workgroup per 128-row query block of one query head; it
//    walks the key blocks the rows see and accumulates dQ = dz K, with dz
//    fed from the accumulator registers (no LDS round trip) and the K/V
//    blocks in two LDS buffers used in turn (one barrier per block).
// Every product runs on v_mfma_f32_32x32x16_bf16 with 32 x 32 tiles, one or
// two per wave (4 waves per workgroup). Operands come from LDS tiles laid
// out so that fragment reads hit distinct banks (16-byte chunks swizzled by
// row in the 128-wide tiles, 16 bytes of padding per row in the 64-wide
// ones); the products that contract over the sequence take Q, dO and K
// through transposed LDS reads of the same row-major tiles. The next
// block's global loads are issued before the current block is computed. P
// and dz are rounded to bf16 as MFMA operands, like P in the forward pass.
#include "internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 64;                 // rows or keys per block
constexpr int kD = 128;                  // head dim
constexpr int kPitch = kD * 2;           // bytes per [.][128] bf16 row (16-byte chunks swizzled, below)
constexpr int kTPitch = kBlk * 2 + 16;   // bytes per padded [.][64] bf16 row
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kInf = __builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (M index) of accumulator register j of a lane in half hb of a 32 x 32
// MFMA tile; the lane's column (N index) is lane & 31.
__device__ __forceinline__ int acc_row(int j, int hb) { return 8 * (j >> 2) + 4 * hb + (j & 3); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 lds_frag(const char* lds, int byte_off) {
    return *reinterpret_cast<const bf16x8*>(lds + byte_off);
}

// [.][128] tiles keep 16-byte chunk c of row r at chunk position c ^ swz(r),
// swz swapping the two low 2-bit fields of r. Sixteen consecutive rows then
// cover all 16 positions (row-wise 16-byte reads and writes of 16 lanes hit
// distinct banks), and the four rows of a transposed read fall on four
// different chunk pairs (its 8-byte pieces hit distinct banks too).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int chunk_at(int r, int c) { return r * kPitch + 16 * (c ^ swz(r)); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// One thread's share of a 64 x 128 bf16 block: lane r of a wave takes row
// r, chunks (tid >> 6) + 4i (16 bytes each, dims 8c .. 8c + 7). Rows past
// `nrows` repeat the last row (their results are masked).
struct BlockRegs {
    u32x4 x[4];
};

__device__ __forceinline__ void load_block(BlockRegs& br, const uint16_t* base, int64_t ss, int row0, int nrows,
                                           int tid) {
    const int row = min(row0 + (tid & 63), nrows - 1);
    const uint16_t* src = base + (int64_t)row * ss;
#pragma unroll
    for (int i = 0; i < 4; ++i) br.x[i] = *reinterpret_cast<const u32x4*>(src + 8 * ((tid >> 6) + 4 * i));
}

__device__ __forceinline__ void store_block(const BlockRegs& br, char* dst, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + chunk_at(tid & 63, (tid >> 6) + 4 * i)) = br.x[i];
}

typedef __attribute__((address_space(3))) char lds_char;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// B operand of a product over the sequence from a row-major [seq][128] LDS
// tile: k = rows 16ks + 8hb + (0..7), n = dim 32dblk + (lane & 31), built from
// two transposed reads (ds_read_b64_tr_b16: in each group of 16 lanes, lane
// 4a + b names row a and dims 4b .. 4b + 3 of a 4 x 16 block, and lane i
// receives the four rows of dim i).
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int ks, int dblk, int lane) {
    const int i16 = lane & 15, ga = i16 >> 2, gb = i16 & 3, gg = (lane >> 4) & 1, hb = lane >> 5;
    const int r = 16 * ks + 8 * hb + ga, c = 4 * dblk + 2 * gg + (gb >> 1), half = 8 * (gb & 1);
    lds_char* t = (lds_char*)tile;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(t + chunk_at(r, c) + half));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(t + chunk_at(r + 4, c) + half));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------- D = rowsum(dO * O)
__global__ __launch_bounds__(256) void bwd_prep_kernel(BackwardParams p) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t R = (int64_t)p.B * p.Hq * p.Lq;
    if (r >= R) return;
    const int i = (int)(r % p.Lq);
    const int64_t bh = r / p.Lq;
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const uint32_t o = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.o) + b * p.o_sb + h * p.o_sh +
                                                         (int64_t)i * p.o_ss)[lane];
    const uint32_t g = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.dout) + b * p.do_sb +
                                                         h * p.do_sh + (int64_t)i * p.do_ss)[lane];
    float acc = fmaf(bf16_lo(o), bf16_lo(g), bf16_hi(o) * bf16_hi(g));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) p.delta[r] = acc;
}

// Stores one 32 x 32 fp32 accumulator tile whose rows are sequence positions
// (row0 + acc_row) and columns dims (col0 + lane & 31), as bf16 or fp32.
__device__ __forceinline__ void store_tile(void* base, int dtype, int64_t ss, int row0, int nrows, int col0,
                                           const f32x16& acc, float mul, int lane) {
    const int hb = lane >> 5, col = col0 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int row = row0 + acc_row(j, hb);
        if (row < nrows) {
            const float v = acc[j] * mul;
            if (dtype == DT_BF16) {
                static_cast<__bf16*>(base)[(int64_t)row * ss + col] = (__bf16)v;
            } else {
                static_cast<float*>(base)[(int64_t)row * ss + col] = v;
            }
        }
    }
}

// ---------------------------------------------------------------- dK, dV
struct DkdvLds {
    char q[kBlk * kPitch];
    char dout[kBlk * kPitch];
    char pT[kBlk * kTPitch];   // P^T  [key][row] bf16
    char dsT[kBlk * kTPitch];  // dz^T [key][row] bf16
    float lse2[kBlk];          // lse * log2(e), +inf for rows without weights
    float delta[kBlk];
};

__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BackwardParams p) {
    __shared__ __attribute__((aligned(16))) DkdvLds s;
    // grid (Hkv, key blocks, B): the heads of one key block are issued
    // together, the blocks most queries see (the first, when causal) first
    const int g = blockIdx.x, kb = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, hb = lane >> 5, w = tid >> 6;
    const int kt = w >> 1;  // this wave's 32-key half of the block
    const int rt = w & 1;   // its 32-row half for S and dP; its 64-dim half for dK and dV
    const int G = p.Hq / p.Hkv;
    const int off = p.Lkv - p.Lq;  // query i sits at position i + off
    const int key0 = kb * kBlk;
    const float c2 = p.scale_log2;

    // K and V of the wave's 32 keys as B operands (column = key, k = dims)
    const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + b * p.k_sb + g * p.k_sh;
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + b * p.v_sb + g * p.v_sh;
    const int mykey = min(key0 + 32 * kt + (lane & 31), p.Lkv - 1);
    bf16x8 kf[8], vf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        kf[ks] = *reinterpret_cast<const bf16x8*>(kbase + (int64_t)mykey * p.k_ss + 16 * ks + 8 * hb);
        vf[ks] = *reinterpret_cast<const bf16x8*>(vbase + (int64_t)mykey * p.v_ss + 16 * ks + 8 * hb);
    }
    f32x16 dk[2], dv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) dk[u][j] = dv[u][j] = 0.f;

    // (head, query block) pairs whose rows see some key of this block, in
    // order; the next pair's Q and dO are loaded while this one is computed
    const int nqb = (p.Lq + kBlk - 1) / kBlk;
    const int qb0 = p.causal ? max(0, (key0 - off) / kBlk) : 0;
    const int nq = max(0, nqb - qb0), nit = G * nq;
    BlockRegs qr, dr;
    float lse_n = 0.f, dl_n = 0.f;
    auto fetch = [&](int it) __attribute__((always_inline)) {
        const int h = g * G + it / nq, row0 = (qb0 + it % nq) * kBlk;
        load_block(qr, static_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh, p.q_ss, row0, p.Lq, tid);
        load_block(dr, static_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh, p.do_ss, row0, p.Lq, tid);
        if (tid < kBlk) {
            const int i = row0 + tid;
            const int64_t ri = ((int64_t)b * p.Hq + h) * p.Lq + i;
            lse_n = i < p.Lq ? p.lse[ri] : -kInf;
            dl_n = i < p.Lq ? p.delta[ri] : 0.f;
        }
    };
    if (nit > 0) fetch(0);
    for (int it = 0; it < nit; ++it) {
        const int row0 = (qb0 + it % nq) * kBlk;
        __syncthreads();  // the previous pair's readers are done
        store_block(qr, s.q, tid);
        store_block(dr, s.dout, tid);
        if (tid < kBlk) {
            s.lse2[tid] = (lse_n == -kInf) ? kInf : lse_n * kLog2e;
            s.delta[tid] = dl_n;
        }
        __syncthreads();
        if (it + 1 < nit) fetch(it + 1);

        // S and dP for rows 32rt.., keys 32kt.. (row = M, key = N)
        f32x16 sa = {}, dpa = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int ao = chunk_at(32 * rt + (lane & 31), 2 * ks + hb);
            sa = mfma(lds_frag(s.q, ao), kf[ks], sa);
            dpa = mfma(lds_frag(s.dout, ao), vf[ks], dpa);
        }
        // P and dz; stored transposed ([key][row]) as bf16, four rows per write.
        // A tile with every key visible to every row needs no mask.
        const int key = key0 + 32 * kt + (lane & 31);
        const bool full = key0 + kBlk <= p.Lkv && row0 + kBlk <= p.Lq && (!p.causal || key0 + kBlk - 1 <= row0 + off);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r0 = 32 * rt + 8 * t + 4 * hb;  // rows r0 .. r0 + 3
            const float4 l4 = *reinterpret_cast<const float4*>(&s.lse2[r0]);
            const float4 d4 = *reinterpret_cast<const float4*>(&s.delta[r0]);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dlv[4] = {d4.x, d4.y, d4.z, d4.w};
            float pv[4], dz[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * t + e;
                const int i = row0 + r0 + e;
                const bool vis = full || (key < p.Lkv && i < p.Lq && (!p.causal || key <= i + off));
                pv[e] = vis ? __builtin_amdgcn_exp2f(fmaf(sa[j], c2, -lv[e])) : 0.f;
                dz[e] = pv[e] * (dpa[j] - dlv[e]);
            }
            const int rbyte = 2 * (32 * rt + 8 * t + 4 * hb);
            const int kr = 32 * kt + (lane & 31);
            *reinterpret_cast<u32x2*>(s.pT + kr * kTPitch + rbyte) = (u32x2){pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
            *reinterpret_cast<u32x2*>(s.dsT + kr * kTPitch + rbyte) = (u32x2){pack_bf16(dz[0], dz[1]), pack_bf16(dz[2], dz[3])};
        }
        __syncthreads();

        // dV += P^T dO and dK += dz^T Q for keys 32kt.., dims 64rt + 32u..
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ao = (32 * kt + (lane & 31)) * kTPitch + 32 * ks + 16 * hb;
            const bf16x8 pa = lds_frag(s.pT, ao), da = lds_frag(s.dsT, ao);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                dv[u] = mfma(pa, tr_frag(s.dout, ks, 2 * rt + u, lane), dv[u]);
                dk[u] = mfma(da, tr_frag(s.q, ks, 2 * rt + u, lane), dk[u]);
            }
        }
    }
    const float sigma = p.scale_log2 / kLog2e;
    void* dkb = static_cast<char*>(p.dk) + (b * p.dk_sb + g * p.dk_sh) * (p.grad_dtype == DT_BF16 ? 2 : 4);
    void* dvb = static_cast<char*>(p.dv) + (b * p.dv_sb + g * p.dv_sh) * (p.grad_dtype == DT_BF16 ? 2 : 4);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        store_tile(dkb, p.grad_dtype, p.dk_ss, key0 + 32 * kt, p.Lkv, 64 * rt + 32 * u, dk[u], sigma, lane);
        store_tile(dvb, p.grad_dtype, p.dv_ss, key0 + 32 * kt, p.Lkv, 64 * rt + 32 * u, dv[u], 1.f, lane);
    }
}

// ---------------------------------------------------------------- dQ
// One workgroup per 128-row query block of one query head (a wave per 32
// rows); K/V blocks of 64 keys pass through two LDS buffers used in turn.
// Per block and 32-key half, a wave computes S^T and dP^T (keys x its rows)
// and dz, and feeds dz straight from the accumulator registers to
// dQ += dz K as the A operand: the C layout gives lane l its row l & 31 and,
// for k-step t, the keys 16t + swap23(kappa) of its k-slots kappa = 8hb + e
// (bits 2 and 3 swapped), so the K operand is read in that key order (two
// transposed reads of rows 16t + 4hb .. +3 and 16t + 8 + 4hb .. +3).
struct DqLds {
    char k[2][kBlk * kPitch];
    char v[2][kBlk * kPitch];
};

// B operand of dQ += dz K for k-step t of key half hk, dim block dblk: keys
// 32hk + 16t + swap23(8hb + e), dim 32dblk + (lane & 31).
__device__ __forceinline__ bf16x8 tr_frag_sw(const char* tile, int row0, int dblk, int lane) {
    const int i16 = lane & 15, ga = i16 >> 2, gb = i16 & 3, gg = (lane >> 4) & 1, hb = lane >> 5;
    const int r = row0 + 4 * hb + ga, c = 4 * dblk + 2 * gg + (gb >> 1), half = 8 * (gb & 1);
    lds_char* t = (lds_char*)tile;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(t + chunk_at(r, c) + half));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(t + chunk_at(r + 8, c) + half));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr int kDqRows = 128;  // query rows per dQ workgroup

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BackwardParams p) {
    __shared__ __attribute__((aligned(16))) DqLds s;
    // grid (Hq, query blocks, B): the heads of one query block are issued
    // together, the blocks that see the most keys (the last, when causal) first
    const int h = blockIdx.x, qb = gridDim.y - 1 - blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, hb = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's 32-row quarter
    const int G = p.Hq / p.Hkv, g = h / G;
    const int off = p.Lkv - p.Lq;
    const int row0 = qb * kDqRows, wrow0 = row0 + 32 * w;
    const float c2 = p.scale_log2;

    // Q and dO of the wave's 32 rows as B operands (column = row, k = dims)
    const int myrow = wrow0 + (lane & 31);
    const int qrw = min(myrow, p.Lq - 1);
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)qrw * p.q_ss;
    const uint16_t* dorow = static_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)qrw * p.do_ss;
    bf16x8 qf[8], df[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * hb);
        df[ks] = *reinterpret_cast<const bf16x8*>(dorow + 16 * ks + 8 * hb);
    }
    float lse2 = kInf, dlt = 0.f;
    if (myrow < p.Lq) {
        const float l = p.lse[((int64_t)b * p.Hq + h) * p.Lq + myrow];
        lse2 = (l == -kInf) ? kInf : l * kLog2e;
        dlt = p.delta[((int64_t)b * p.Hq + h) * p.Lq + myrow];
    }
    f32x16 dq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) dq[u][j] = 0.f;

    const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + b * p.k_sb + g * p.k_sh;
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + b * p.v_sb + g * p.v_sh;
    const int nkb_all = (p.Lkv + kBlk - 1) / kBlk;
    // key blocks some row of the workgroup sees, and those of this wave
    const int last_key = min(p.Lkv - 1, row0 + kDqRows - 1 + off);
    const int nkb = p.causal ? (last_key >= 0 ? last_key / kBlk + 1 : 0) : nkb_all;
    const int wlast = min(p.Lkv - 1, wrow0 + 31 + off);
    const int nkb_w = p.causal ? (wlast >= 0 ? wlast / kBlk + 1 : 0) : nkb_all;
    BlockRegs kr, vr;  // the block after the one being stored, loaded while this one is computed
    if (nkb > 0) {
        load_block(kr, kbase, p.k_ss, 0, p.Lkv, tid);
        load_block(vr, vbase, p.v_ss, 0, p.Lkv, tid);
        store_block(kr, s.k[0], tid);
        store_block(vr, s.v[0], tid);
    }
    if (nkb > 1) {
        load_block(kr, kbase, p.k_ss, kBlk, p.Lkv, tid);
        load_block(vr, vbase, p.v_ss, kBlk, p.Lkv, tid);
    }
    for (int kb = 0; kb < nkb; ++kb) {
        const int key0 = kb * kBlk;
        // block kb's buffer is complete; the other one was last read in
        // iteration kb - 1, which every wave has finished
        __syncthreads();
        if (kb + 1 < nkb) {
            store_block(kr, s.k[(kb + 1) & 1], tid);
            store_block(vr, s.v[(kb + 1) & 1], tid);
            if (kb + 2 < nkb) {
                load_block(kr, kbase, p.k_ss, key0 + 2 * kBlk, p.Lkv, tid);
                load_block(vr, vbase, p.v_ss, key0 + 2 * kBlk, p.Lkv, tid);
            }
        }
        if (kb >= nkb_w) continue;  // past this wave's rows (causal): nothing to add
        const char* sk = s.k[kb & 1];
        const char* sv = s.v[kb & 1];
        // a block every key of which every row of the wave sees needs no mask
        const bool full = key0 + kBlk <= p.Lkv && wrow0 + 32 <= p.Lq && (!p.causal || key0 + kBlk - 1 <= wrow0 + off);
#pragma unroll
        for (int hk = 0; hk < 2; ++hk) {
            // S^T and dP^T for keys 32hk.. (M) and the wave's rows (N)
            f32x16 sa = {}, dpa = {};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int ao = chunk_at(32 * hk + (lane & 31), 2 * ks + hb);
                sa = mfma(lds_frag(sk, ao), qf[ks], sa);
                dpa = mfma(lds_frag(sv, ao), df[ks], dpa);
            }
            // dz of this lane's row at keys 32hk + acc_row(j, hb), packed as bf16
            u32x4 dz[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float z[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int j = 8 * t + 2 * e2 + u;
                        const int key = key0 + 32 * hk + acc_row(j, hb);
                        const bool vis = full || (key < p.Lkv && myrow < p.Lq && (!p.causal || key <= myrow + off));
                        const float pv = vis ? __builtin_amdgcn_exp2f(fmaf(sa[j], c2, -lse2)) : 0.f;
                        z[u] = pv * (dpa[j] - dlt);
                    }
                    dz[t][e2] = pack_bf16(z[0], z[1]);
                }
            // dQ += dz K over the half's 32 keys (two k-steps of 16)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    dq[u] = mfma(__builtin_bit_cast(bf16x8, dz[t]), tr_frag_sw(sk, 32 * hk + 16 * t, u, lane), dq[u]);
        }
    }
    const float sigma = p.scale_log2 / kLog2e;
    void* dqb = static_cast<char*>(p.dq) + (b * p.dq_sb + h * p.dq_sh) * (p.grad_dtype == DT_BF16 ? 2 : 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) store_tile(dqb, p.grad_dtype, p.dq_ss, wrow0, p.Lq, 32 * u, dq[u], sigma, lane);
}

}  // namespace

hipError_t launch_backward(const BackwardParams& p, hipStream_t stream) {
    if (p.d != kD) return hipErrorInvalidValue;
    const int64_t R = (int64_t)p.B * p.Hq * p.Lq;
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(p.Hkv, (p.Lkv + kBlk - 1) / kBlk, p.B), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(p.Hq, (p.Lq + kDqRows - 1) / kDqRows, p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace attn
