// Split-KV grouped-query decode for gfx950: one query token, four query heads
// per KV head, head dim 128, KV cache spans in bf16, OCP fp8-e4m3 or OCP MX
// fp4.
//
// Work split (the single-GPU form of the sequence-axis tree reduction in the
// explainer of "Tree Attention: Topology-aware Decoding for Long-Context
// Attention on GPU Clusters", section 3): workgroup (s, g, b) owns one chunk of
// keys of KV head g of sequence b and emits one partial (o, m, l) per query
// head. The four waves of the workgroup interleave 32-key tiles of the chunk;
// each wave's products sum over all its keys, so its partial is complete in
// registers. The waves' partials are merged in LDS -- the level-1 tree. The
// level-2 tree across workgroups runs either here (the last workgroup of each
// (sequence, KV head) to finish merges its group's partials, see FUSED) or in
// combine.hip.
//
// Per 32-key tile and wave (tile32 below): scores S^T = K Q^T and the product
// O^T += V^T P^T both on v_mfma_f32_16x16x32_bf16, with the four query heads
// repeated in the 16 columns (MFMA is used because both are dense
// contractions; the repeated columns cost nothing that matters at a few
// flop/byte). The softmax keeps scores in base-2 units (scale folded with
// log2 e); the running maximum moves only when a score exceeds it by 8 (2^8
// headroom in fp32), so rescaling the accumulators is rare, and the result is
// the same exact quantity, normalised with the same maximum in o and l (the
// max subtraction the Grayskull explainer names in section 3). K and V are
// read as whole rows per load instruction with non-temporal buffer loads (K
// then goes through a small wave-private LDS stage into the MFMA operand
// layout); every valid key is read from HBM exactly once, and the next tile's
// loads are issued before the current tile is computed.
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
constexpr float kHeadroom = 8.0f;  // base-2 units a score may exceed the running max by
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Storage precision of a span of the cache: bf16; OCP fp8-e4m3 with one fp32
// scale per (sequence, KV head); OCP MX fp4 (E2M1 codes, two per byte with
// the first in the low nibble, and one E8M0 power-of-two scale per 32
// consecutive elements of a row, in a separate array of 4 bytes per row).
constexpr int kBf16 = 0, kFp8 = 1, kFp4 = 2;

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

// Eight MX fp4 codes (a dword, first code in the low nibble) times 2^scale ->
// eight bf16, in the code order (exact: a one-bit mantissa times a power of
// two; a probe of every code at every scale byte matched the fp32 form).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float sc) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Four OCP e4m3 codes of a dword pair -> eight bf16 (exact widening).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ---- 32-key tiles per wave, both products on the MFMA.
//
// Scores: S^T = K Q^T as two v_mfma_f32_16x16x32_bf16 chains over d. Product
// a takes the tile's keys 8(m >> 2) + (m & 3) as its A rows m, product b
// those keys + 4, so lane l receives head l & 3 of keys 8(l >> 4) + r (from
// a) and 8(l >> 4) + 4 + r (from b), r < 4: the eight keys 8(l >> 4) .. +7
// that the same lane feeds to the P.V product as its B operand. No lane
// exchange is needed between the two products.
// P.V: O^T = V^T P^T as eight products j = 0..7 over the 32 keys. Product j's
// A row m is dim 8m + j (lane l holds those of the eight values it loaded per
// key, dims 8(l & 15) .. +7), its B column n is head n & 3 (the four heads
// repeat across the 16 columns, as in the scores), so lane l ends with head
// l & 3 at dims 32(l >> 4) + 8r + j in acc[j][r].
// bf16 values feed the MFMA as stored; fp8 and fp4 codes widen exactly to
// bf16 (fp8-e4m3: three mantissa bits; MX fp4: one mantissa bit times the
// block's power-of-two scale). P is rounded to bf16 for the MFMA, the sum l
// takes the fp32 weights. The running max is shared by
// the 16 lanes of a head, because every product sums over all lanes' keys.
// fp8's per-head K scale is folded into the score scale and its V scale is
// applied to the partial; fp4's block scales are applied in the conversion.
constexpr int kTile32 = 32;

// Geometry of a span's 32-key tile with head dim D: bytes of a K or V row,
// 16-byte chunks a K row has, and K loads a lane issues per tile (one 16-byte
// chunk each: a load instruction covers 64 / kChunks whole rows).
template <int P, int D>
struct Geo {
    static constexpr int kRowBytes = P == kBf16 ? 2 * D : (P == kFp8 ? D : D / 2);
    static constexpr int kChunks = kRowBytes / 16;
    static constexpr int kRowsPerLoad = 64 / kChunks;
    static constexpr int kLoads = kTile32 / kRowsPerLoad;
    static constexpr int kSteps = D / 32;  // MFMA steps over d for the scores
    static_assert(kChunks == 4 || kChunks == 8 || kChunks == 16, "tile geometry");
};

template <int P, int D>
struct Tile32;
template <int D>
struct Tile32<kBf16, D> {
    u32x4 k[Geo<kBf16, D>::kLoads];  // key row lane / kChunks + kRowsPerLoad i: chunk lane % kChunks
    u32x4 v[8];  // key 8*(lane >> 4) + u: its 8 values at dims 8*(lane & (D/8 - 1)) .. +7
};
template <int D>
struct Tile32<kFp8, D> {
    u32x4 k[Geo<kFp8, D>::kLoads];
    u32x2 v[8];  // key 8*(lane >> 4) + u: its 8 codes at dims 8*(lane & (D/8 - 1)) .. +7
};
template <int D>
struct Tile32<kFp4, D> {
    static_assert(D == 128, "MX fp4 spans take d = 128");
    u32x4 k[2];      // key rows lane >> 2 and 16 + (lane >> 2): 16-byte chunk lane & 3 (32 codes, block lane & 3)
    uint32_t ks[2];  // scale words of key rows row_a(lane & 15) and that + 4 (byte i: block i)
    uint32_t v[8];   // key 8*(lane >> 4) + u: its 8 codes at dims 8*(lane & 15) .. +7
    uint32_t vs[8];  // that key's scale word
};

// The tile row score product a takes as its A row m.
__device__ __forceinline__ int row_a(int m) { return 8 * (m >> 2) + (m & 3); }

// K stages of a 32-row tile (u32x4 units), by chunks a row. Four chunks
// (fp4 at d = 128, fp8 at d = 64): chunk c of row r at c ^ ((r >> 3) & 3);
// the operand reads (16 bytes, or for fp4 4-byte word lane >> 4, of chunk
// lane >> 4 or i of row row_a(lane & 15), or that + 4) hit distinct bank
// groups. Eight chunks (fp8 at d = 128, bf16 at d = 64): chunk c of row r at
// c ^ s(r) with s(r) = 2((r >> 3) & 3) + ((r >> 1) & 1), distinct over the
// eight rows of each parity that one read touches, so the 16-byte operand
// reads (chunk 4h + (lane >> 4)) and the row writes both take the minimum of
// four passes. Sixteen chunks (bf16 at d = 128): chunk c of row r at c ^ t(r)
// with t(r) = (r & 3) + 4((r >> 3) & 3), distinct over the 16 rows
// row_a(0..15) (and over those + 4) that one operand read touches, so every
// 16 lanes of the read hit 16 different 16-byte bank groups; a row write
// spans all 16 chunks of a row.
template <int CH>
__device__ __forceinline__ int kidx32(int row, int chunk) {
    if constexpr (CH == 4) return row * 4 + (chunk ^ ((row >> 3) & 3));
    else if constexpr (CH == 16) return row * 16 + (chunk ^ ((row & 3) | (((row >> 3) & 3) << 2)));
    else return row * 8 + (chunk ^ ((((row >> 3) & 3) << 1) | ((row >> 1) & 1)));
}

// Word 3 of a raw buffer resource (32-bit data format, no swizzle): loads at
// or past the resource's byte size return zero.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 2;  // cache policy of the streaming buffer loads

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const char* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kRsrcWord3);
}

// This lane's byte offsets inside a 32-key tile, the same for every tile of a
// split: K (row lane / kChunks, chunk lane % kChunks), K scales (fp4) of row
// row_a(lane & 15), V of row 8(lane >> 4) at dims 8(lane & (D/8 - 1)) (at
// d = 64 lanes l and l + 8 of each 16 read the same bytes: the products'
// rows for dims past 64 are computed and dropped), V scales (fp4) of row
// 8(lane >> 4). The other rows a lane reads are these plus a multiple of the
// row stride, passed as the loads' scalar offset.
struct Lanes32 {
    uint32_t k, ks, v, vs;
};
template <int P, int D>
__device__ __forceinline__ Lanes32 lanes32(int ik, int iks, int iv, int ivs, int lane) {
    using Gm = Geo<P, D>;
    Lanes32 o;
    o.k = (lane / Gm::kChunks) * ik + 16 * (lane % Gm::kChunks);
    constexpr int kVBytes = P == kBf16 ? 16 : (P == kFp8 ? 8 : 4);  // 8 values of a V row
    o.v = 8 * (lane >> 4) * iv + kVBytes * (lane & (D / 8 - 1));
    if constexpr (P == kFp4) {
        o.ks = row_a(lane & 15) * iks;
        o.vs = 8 * (lane >> 4) * ivs;
    } else {
        o.ks = 0;
        o.vs = 0;
    }
    return o;
}

// Loads the 32-key tile starting at key tok0. Buffer loads over the tile's
// valid rows (up to key tlast): rows past it read as zero, so the tail needs
// no clamping (a zero key scores 0 and is masked; a zero value adds nothing),
// and the lanes' addresses are fixed offsets (the host keeps row strides below
// 2^26 bytes, so 32 rows fit 32-bit offsets).
template <int P, int D>
__device__ __forceinline__ void load_tile32(Tile32<P, D>& t, const char* kbase, const char* vbase, int ik, int iv,
                                            const ScaleRows& sc, int iks, int ivs, const Lanes32& ln, int tok0,
                                            int tlast) {
    using Gm = Geo<P, D>;
    const int last = min(tlast - tok0, kTile32 - 1);
    const __amdgpu_buffer_rsrc_t rk = bytes_rsrc(kbase + (int64_t)tok0 * ik, last * ik + Gm::kRowBytes);
    const __amdgpu_buffer_rsrc_t rv = bytes_rsrc(vbase + (int64_t)tok0 * iv, last * iv + Gm::kRowBytes);
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i)
        t.k[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ln.k, Gm::kRowsPerLoad * i * ik, kNonTemporal));
    if constexpr (P == kFp4) {
        const __amdgpu_buffer_rsrc_t rks = bytes_rsrc(sc.k + (int64_t)tok0 * iks, last * iks + 4);
        const __amdgpu_buffer_rsrc_t rvs = bytes_rsrc(sc.v + (int64_t)tok0 * ivs, last * ivs + 4);
        t.ks[0] = __builtin_amdgcn_raw_buffer_load_b32(rks, ln.ks, 0, kNonTemporal);
        t.ks[1] = __builtin_amdgcn_raw_buffer_load_b32(rks, ln.ks, 4 * iks, kNonTemporal);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            t.v[u] = __builtin_amdgcn_raw_buffer_load_b32(rv, ln.v, u * iv, kNonTemporal);
            t.vs[u] = __builtin_amdgcn_raw_buffer_load_b32(rvs, ln.vs, u * ivs, kNonTemporal);
        }
    } else if constexpr (P == kBf16) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            t.v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ln.v, u * iv, kNonTemporal));
    } else {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            t.v[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, ln.v, u * iv, kNonTemporal));
    }
}

// P.V products 2 SEL and 2 SEL + 1: values 2 SEL and 2 SEL + 1 of every key
// (dims 8m + 2 SEL and 8m + 2 SEL + 1 of A row m).
template <int P, int D, int SEL>
__device__ __forceinline__ void pv_pair(const Tile32<P, D>& t, const float (&sc)[8], const bf16x8& pb, f32x4& acc0,
                                        f32x4& acc1) {
    bf16x8 a0, a1;
    if constexpr (P == kBf16) {
        // word SEL of a key's 16 bytes holds dims 2 SEL (low half) and 2 SEL + 1
        u32x4 w0, w1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t x = t.v[2 * q][SEL], y = t.v[2 * q + 1][SEL];
            w0[q] = __builtin_amdgcn_perm(y, x, 0x05040100u);
            w1[q] = __builtin_amdgcn_perm(y, x, 0x07060302u);
        }
        a0 = __builtin_bit_cast(bf16x8, w0);
        a1 = __builtin_bit_cast(bf16x8, w1);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, pb, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, pb, acc1, 0, 0, 0);
        return;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        f32x2 x;
        if constexpr (P == kFp4) x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(t.v[u], sc[u], SEL);
        else x = __builtin_amdgcn_cvt_pk_f32_fp8(t.v[u][SEL >> 1], (SEL & 1) != 0);
        a0[u] = (__bf16)x[0];
        a1[u] = (__bf16)x[1];
    }
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, pb, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, pb, acc1, 0, 0, 0);
}

// One 32-key tile of a wave: scores, softmax update, P.V (see above).
template <int P, int D, int G>
__device__ __forceinline__ void tile32(const Tile32<P, D>& t, u32x4* ks, const float* e8m0, const bf16x8 (&qop)[4],
                                       float scale2, int tok0, int tend, int lane, float& m_run, float& l_run,
                                       f32x4 (&acc)[8]) {
    using Gm = Geo<P, D>;
    constexpr int CH = Gm::kChunks;
    const int g = lane >> 4, ra = row_a(lane & 15);
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i) ks[kidx32<CH>(lane / CH + Gm::kRowsPerLoad * i, lane % CH)] = t.k[i];
    if constexpr (P == kBf16) {
        // step i: dims 32i + 8g .. +7 (chunk 4i + g), the Q operand's bf16 dim order
#pragma unroll
        for (int i = 0; i < Gm::kSteps; ++i) {
            const u32x4 a = ks[kidx32<CH>(ra, 4 * i + g)];
            const u32x4 b = ks[kidx32<CH>(ra + 4, 4 * i + g)];
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qop[i], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), qop[i], sb, 0, 0, 0);
        }
    } else if constexpr (P == kFp4) {
        const uint32_t* ks32 = reinterpret_cast<const uint32_t*>(ks);
        // step i is scale block i: dims 32i + 8g .. +7 of this lane's rows
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 a = fp4x8_to_bf16(ks32[4 * kidx32<CH>(ra, i) + g], e8m0[(t.ks[0] >> (8 * i)) & 255u]);
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[i], sa, 0, 0, 0);
            const bf16x8 b = fp4x8_to_bf16(ks32[4 * kidx32<CH>(ra + 4, i) + g], e8m0[(t.ks[1] >> (8 * i)) & 255u]);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, qop[i], sb, 0, 0, 0);
        }
    } else {
        // steps 2h and 2h + 1 take the two halves of chunk 4h + g: dims
        // 64h + 16g .. +7 and +8 .. +15 (the Q operand's fp8 dim order)
#pragma unroll
        for (int h = 0; h < Gm::kSteps / 2; ++h) {
            const u32x4 a = ks[kidx32<CH>(ra, 4 * h + g)];
            const u32x4 b = ks[kidx32<CH>(ra + 4, 4 * h + g)];
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(a[0], a[1]), qop[2 * h], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(b[0], b[1]), qop[2 * h], sb, 0, 0, 0);
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(a[2], a[3]), qop[2 * h + 1], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(b[2], b[3]), qop[2 * h + 1], sb, 0, 0, 0);
        }
    }
    const int kb = tok0 + 8 * g;
    float s[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        s[r] = sa[r] * scale2;
        s[4 + r] = sb[r] * scale2;
    }
    if (tok0 + kTile32 > tend) {  // the split's last tile: mask the keys past its end
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = (kb + r < tend) ? s[r] : kNegInf;
            s[4 + r] = (kb + 4 + r < tend) ? s[4 + r] : kNegInf;
        }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, fmaxf(s[r], s[4 + r]));
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kHeadroom) != 0) {
        // the new running max of each head: over the 64 / G lanes with its
        // lane & (G - 1)
        float hm = tmax;
#pragma unroll
        for (int off = G; off < 64; off <<= 1) hm = fmaxf(hm, __shfl_xor(hm, off));
        const float m_new = fmaxf(m_run, hm);
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    }
    // m_run is finite here: every tile has a valid key for every head (key
    // tok0), so the first tile set it; masked scores give exp2(-inf) = 0
    bf16x8 pb;
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const float pu = fast_exp2(s[u] - m_run);
        lsum += pu;
        pb[u] = (__bf16)pu;
    }
    l_run += lsum;
    float sc[8];
    if constexpr (P == kFp4) {
        // dims 8*(lane & 15) .. +7 lie in scale block (lane & 15) >> 2
        const int sh = 8 * ((lane & 15) >> 2);
#pragma unroll
        for (int u = 0; u < 8; ++u) sc[u] = e8m0[(t.vs[u] >> sh) & 255u];
    }
    pv_pair<P, D, 0>(t, sc, pb, acc[0], acc[1]);
    pv_pair<P, D, 1>(t, sc, pb, acc[2], acc[3]);
    pv_pair<P, D, 2>(t, sc, pb, acc[4], acc[5]);
    pv_pair<P, D, 3>(t, sc, pb, acc[6], acc[7]);
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
// workgroup publishes its partial (agent-scope stores, released at agent
// scope), then takes a ticket in its block of `ticket_block` splits; the last of a block merges
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
    // The barrier orders every thread's partial stores before thread 0's
    // ticket, which releases them at agent scope (happens-before is
    // transitive across the two scopes); the threads of the workgroup that
    // draws the last ticket acquire at agent scope before they read the other
    // workgroups' partials.
    __syncthreads();
    if (tid == 0) {
        uint32_t* blk = line + (1 + bi) * kCounterStride;
        const uint32_t o1 = __hip_atomic_fetch_add(blk, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        role = (o1 == (uint32_t)(in_block - 1)) ? 1 : 0;
        if (role) __hip_atomic_store(blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!role) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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
        __syncthreads();
        if (tid == 0) {
            const uint32_t o2 = __hip_atomic_fetch_add(line, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            role = (o2 == (uint32_t)(nb - 1)) ? 2 : 0;
            if (role) __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!role) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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
constexpr int kMaxG = 8;  // query heads per KV head, at most
struct DecodeLds {
    u32x4 kstage[kWaves][512];
    float o[kWaves][kMaxG][128];
    float m[kWaves][kMaxG];
    float l[kWaves][kMaxG];
    float e8m0[256];  // MX fp4 spans: the value of every E8M0 scale byte
};

// One workgroup: split s of span `sp`, publishing partial s_out of its rows.
// TWO (two-span launches): the span's key geometry and log-prior apply; every
// split of the launch publishes a partial (an empty one the identity) and
// takes part in the fused merge, which covers all p.S of them.
template <int P, int D, int G, bool FUSED, bool TWO>
__device__ __forceinline__ void decode_wg(const DecodeParams& p, const KvSpan& sp, int s, int s_out,
                                          DecodeLds& lds) {
    constexpr bool FP8 = P == kFp8;
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "query heads per KV head");
    static_assert((G == 4 && D == 128) || !FUSED, "the fused merge takes four heads of 128 dims a group");
    static_assert(D == 64 || D == 128, "head dim");
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
        for (int i = tid; i < G * D; i += 256) {
            const int64_t row = (int64_t)b * p.Hq + g * G + i / D;
            if constexpr (FUSED && TWO) {
                st_agent(p.o_part + (row * p.S + s_out) * D + i % D, 0.f);
                if (i % D == 0) {
                    st_agent(p.m_part + row * p.S + s_out, kNegInf);
                    st_agent(p.l_part + row * p.S + s_out, 0.f);
                }
            } else {
                p.o_part[(row * p.S + s_out) * D + i % D] = 0.f;
                if (i % D == 0) {
                    p.m_part[row * p.S + s_out] = kNegInf;
                    p.l_part[row * p.S + s_out] = 0.f;
                }
            }
        }
        if constexpr (FUSED && TWO) merge_group_if_last(p, b, g, n_merge, tid);
        if (FUSED && !TWO && L_b == 0 && s == 0) {
            // an empty sequence: O = 0, lse = -inf (no workgroup of it merges)
            for (int i = tid; i < G * 128; i += 256) {
                uint16_t* orow = static_cast<uint16_t*>(p.out) + b * p.out_sb + (int64_t)(g * G + i / 128) * p.out_sh;
                orow[i % 128] = 0;
                if (p.lse && i % 128 == 0) p.lse[(int64_t)b * p.Hq + g * G + i / 128] = kNegInf;
            }
        }
        return;
    }
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

    // Q^T operand: column (lane & 15) is query head G g + (lane & (G - 1)) (the
    // G heads repeat across the 16 columns); its k-slots follow the same dim
    // order as the K operand.
    const __bf16* qrow =
        static_cast<const __bf16*>(p.q) + b * p.q_sb + (int64_t)(g * G + (lane & (G - 1))) * p.q_sh;
    bf16x8 qop[4];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
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
    u32x4* ks = lds.kstage[w];
    int k = w;
    {
        // 32-key tiles, both products on the MFMA (tile32); two tiles in flight
        const int ntiles32 = (t_end - t_begin + kTile32 - 1) / kTile32;
        f32x4 acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (P == kFp4) {
            // scale bytes are widened by a table lookup (exact, 2^-127 and NaN included)
            lds.e8m0[tid] = e8m0_to_f32((uint32_t)tid);
            __syncthreads();
        }
        if (k < ntiles32) {
            const int ik = (int)kss, iv = (int)vss, iks = (int)sc.kss, ivs = (int)sc.vss;
            const Lanes32 ln = lanes32<P, D>(ik, iks, iv, ivs, lane);
            Tile32<P, D> ta, tb;
            load_tile32<P, D>(ta, kbase, vbase, ik, iv, sc, iks, ivs, ln, t_begin + kTile32 * k, t_end - 1);
            while (true) {
                const bool more_b = k + kWaves < ntiles32;
                if (more_b)
                    load_tile32<P, D>(tb, kbase, vbase, ik, iv, sc, iks, ivs, ln, t_begin + kTile32 * (k + kWaves), t_end - 1);
                tile32<P, D, G>(ta, ks, lds.e8m0, qop, scale2, t_begin + kTile32 * k, t_end, lane, m_run, l_run, acc);
                if (!more_b) break;
                k += kWaves;
                const bool more_a = k + kWaves < ntiles32;
                if (more_a)
                    load_tile32<P, D>(ta, kbase, vbase, ik, iv, sc, iks, ivs, ln, t_begin + kTile32 * (k + kWaves), t_end - 1);
                tile32<P, D, G>(tb, ks, lds.e8m0, qop, scale2, t_begin + kTile32 * k, t_end, lane, m_run, l_run, acc);
                if (!more_a) break;
                k += kWaves;
            }
        }
        // The MFMA summed over every key of the wave, so the wave's partial is
        // complete: lane l holds head l & (G - 1) at dims 32*(l>>4) + 8r + j
        // (acc[j][r]), the same in the 16 / G lanes with equal l & (G - 1) and
        // l >> 4; l_run counts the keys of lane group l >> 4 once per lane of a
        // head.
        float lw = l_run + __shfl_xor(l_run, 16);
        lw += __shfl_xor(lw, 32);
        if ((lane & 15) < G && (lane >> 4) < D / 32) {
            float* orow = lds.o[w][lane & (G - 1)] + 32 * (lane >> 4);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) orow[8 * r + j] = acc[j][r];
        }
        if (lane < G) {
            lds.m[w][lane] = m_run;
            lds.l[w][lane] = lw;
        }
    }
    // Level 1b: merge the four waves in LDS; thread pass q takes head h and
    // columns c, c + 1 (G * D / 2 column pairs over 256 threads).
    __syncthreads();
    constexpr int kPairs = D / 2;
#pragma unroll
    for (int q0 = 0; q0 < G * kPairs; q0 += 256) {
        const int qi = q0 + tid;
        if (qi >= G * kPairs) break;
        const int h = qi / kPairs;
        const int c = (qi % kPairs) * 2;
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
        const int64_t row = (int64_t)b * p.Hq + g * G + h;
        float m_out = Mx * kLn2;
        if constexpr (TWO) {
            // the span's log-prior shifts its partial's max (natural-log units)
            if (sp.prior && p.alpha) {
                const float a = fminf(fmaxf(p.alpha[row], 0.f), 1.f);
                m_out += logf(sp.prior == 1 ? a : 1.f - a);
            }
        }
        if constexpr (FUSED) {
            st_agent2(p.o_part + (row * p.S + s_out) * D + c, out);
            if (qi % kPairs == 0) {
                st_agent(p.m_part + row * p.S + s_out, m_out);
                st_agent(p.l_part + row * p.S + s_out, L);
            }
        } else {
            *reinterpret_cast<f32x2*>(p.o_part + (row * p.S + s_out) * D + c) = out;
            if (qi % kPairs == 0) {
                p.m_part[row * p.S + s_out] = m_out;
                p.l_part[row * p.S + s_out] = L;
            }
        }
    }
    if constexpr (FUSED) merge_group_if_last(p, b, g, n_merge, tid);
}

__device__ __forceinline__ KvSpan main_span(const DecodeParams& p) {
    return KvSpan{p.k,       p.k_sb, p.k_sh,  p.k_ss,    p.v, p.v_sb, p.v_sh, p.v_ss, p.kv_lens,
                  1,         0,      p.L_cap, p.chunk,   kGeomAll, 0, 1, 0};
}

template <int D, int G, bool FP8, bool FUSED>
__global__ __launch_bounds__(256, 2) void decode_gqa(DecodeParams p) {
    __shared__ DecodeLds lds;
    decode_wg<FP8 ? kFp8 : kBf16, D, G, FUSED, false>(p, main_span(p), blockIdx.x, blockIdx.x, lds);
}

// Two spans in one launch (a two-precision cache, or pi-Attention's window
// and skip keys): splits [0, S0) stream span sp0, the others span sp1; one
// merge over all splits.
template <int D, int G, int P0, int P1, bool FUSED>
__global__ __launch_bounds__(256, 2) void decode_gqa_two(DecodeParams p) {
    __shared__ DecodeLds lds;  // one copy for both branches
    const int s = blockIdx.x;
    if (s < p.S0) decode_wg<P0, D, G, FUSED, true>(p, p.sp0, s, s, lds);
    else decode_wg<P1, D, G, FUSED, true>(p, p.sp1, s - p.S0, s, lds);
}

// Three spans in one launch (a cache kept in bf16, fp8 and MX fp4): splits
// [0, S0) stream sp0, [S0, S1) sp1, the others sp2; one merge over all
// splits. Each workgroup reads one precision, so no wave branches between
// formats.
template <int G, int P0, int P1, int P2, bool FUSED>
__global__ __launch_bounds__(256, 2) void decode_gqa_three(DecodeParams p) {
    __shared__ DecodeLds lds;
    const int s = blockIdx.x;
    if (s < p.S0) decode_wg<P0, 128, G, FUSED, true>(p, p.sp0, s, s, lds);
    else if (s < p.S1) decode_wg<P1, 128, G, FUSED, true>(p, p.sp1, s - p.S0, s, lds);
    else decode_wg<P2, 128, G, FUSED, true>(p, p.sp2, s - p.S1, s, lds);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int G, hipStream_t stream) {
    dim3 grid(p.S, p.Hkv, p.B);
    const bool fused = p.counters != nullptr;
    const bool fp8 = kv_dtype == DT_FP8;
    const int D = p.d;
    if (fused && (G != 4 || D != 128)) return hipErrorInvalidValue;  // the fused merge: four heads of 128 dims
#define ATTN_ONE(DD, GG, F8)                                                                                       \
    if (D == DD && G == GG && fp8 == F8) {                                                                         \
        if (fused) hipLaunchKernelGGL((decode_gqa<DD, GG, F8, GG == 4 && DD == 128>), grid, dim3(256), 0, stream, \
                                      p);                                                                          \
        else hipLaunchKernelGGL((decode_gqa<DD, GG, F8, false>), grid, dim3(256), 0, stream, p);                   \
        return hipGetLastError();                                                                                  \
    }
#define ATTN_ONE_G(DD, F8) ATTN_ONE(DD, 4, F8) ATTN_ONE(DD, 8, F8) ATTN_ONE(DD, 2, F8) ATTN_ONE(DD, 1, F8)
    ATTN_ONE_G(128, false)
    ATTN_ONE_G(128, true)
    ATTN_ONE_G(64, false)
    ATTN_ONE_G(64, true)
#undef ATTN_ONE_G
#undef ATTN_ONE
    return hipErrorInvalidValue;  // no kernel for this head dim or head ratio
}

hipError_t launch_decode_mfma_two(const DecodeParams& p, int prec0, int prec1, hipStream_t stream) {
    dim3 grid(p.S, p.Hkv, p.B);
    const bool f = p.counters != nullptr;
    const int G = p.Hkv > 0 ? p.Hq / p.Hkv : 0;
    const int D = p.d;
    if (f && (G != 4 || D != 128)) return hipErrorInvalidValue;  // the fused merge: four heads of 128 dims
#define ATTN_TWO(DD, GG, P0, P1)                                                                                \
    if (D == DD && G == GG && prec0 == P0 && prec1 == P1) {                                                     \
        if (f) hipLaunchKernelGGL((decode_gqa_two<DD, GG, P0, P1, GG == 4 && DD == 128>), grid, dim3(256), 0,  \
                                  stream, p);                                                                   \
        else hipLaunchKernelGGL((decode_gqa_two<DD, GG, P0, P1, false>), grid, dim3(256), 0, stream, p);        \
        return hipGetLastError();                                                                               \
    }
#define ATTN_TWO_G(DD, P0, P1) ATTN_TWO(DD, 4, P0, P1) ATTN_TWO(DD, 8, P0, P1) ATTN_TWO(DD, 2, P0, P1) ATTN_TWO(DD, 1, P0, P1)
    ATTN_TWO_G(128, kBf16, kFp8)
    ATTN_TWO_G(128, kBf16, kBf16)
    ATTN_TWO_G(128, kFp8, kFp8)
    ATTN_TWO_G(128, kBf16, kFp4)
    ATTN_TWO_G(64, kBf16, kFp8)
    ATTN_TWO_G(64, kBf16, kBf16)
    ATTN_TWO_G(64, kFp8, kFp8)
#undef ATTN_TWO_G
#undef ATTN_TWO
    return hipErrorInvalidValue;  // no kernel for this pair of precisions, head dim or head ratio
}

hipError_t launch_decode_mfma_three(const DecodeParams& p, int prec0, int prec1, int prec2, hipStream_t stream) {
    if (prec0 != kBf16 || prec1 != kFp8 || prec2 != kFp4 || p.d != 128) return hipErrorInvalidValue;
    dim3 grid(p.S, p.Hkv, p.B);
    const bool f = p.counters != nullptr;
    const int G = p.Hkv > 0 ? p.Hq / p.Hkv : 0;
    if (f && G != 4) return hipErrorInvalidValue;
#define ATTN_THREE(GG)                                                                                           \
    if (G == GG) {                                                                                               \
        if (f) hipLaunchKernelGGL((decode_gqa_three<GG, kBf16, kFp8, kFp4, GG == 4>), grid, dim3(256), 0, stream, \
                                  p);                                                                            \
        else hipLaunchKernelGGL((decode_gqa_three<GG, kBf16, kFp8, kFp4, false>), grid, dim3(256), 0, stream, p); \
        return hipGetLastError();                                                                                \
    }
    ATTN_THREE(4)
    ATTN_THREE(8)
    ATTN_THREE(2)
    ATTN_THREE(1)
#undef ATTN_THREE
    return hipErrorInvalidValue;
}

}  // namespace attn
