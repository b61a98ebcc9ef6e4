// Matrix-core (MFMA) split-K decode attention over the compressed cache, gfx950.
//
// What it computes (pages by title and section):
//  * the quantcpp article's progressive cache (4-bit codes with fp16 scale/zero per 32 channels,
//    newest 128 tokens read in FP32) and the KVarN post's Walsh-Hadamard + Sinkhorn-balanced
//    4-bit cache: out = softmax(q k^T * scale) v with k, v the dequantized tokens, scores in the
//    rotated/balanced domain via q' = R(q) .* c, output un-rotated at the end (merge kernel);
//  * the TurboQuant row of "LLM memory saving ... 2026": a key scores
//    n <R q, mu[code]> + gamma * sqrt(pi/2)/128 * sum_i (2 b_i - 1) (S R q)_i, a TurboQuant-MSE
//    value is n mu[code] in the rotated domain.
//
// How (one workgroup = NW waves per (sequence, kv head, token split); each wave streams 64-token
// chunks; all products on v_mfma_f32_16x16x32_f16, every code operand exact):
//  * Uniform K: A = (head, group) rows of q' as fp16 hi and remainder lo, both products in one
//    accumulator chain, B = raw codes: 4-bit codes as fp16
//    subnormal bit patterns (code * 2^-24, odd nibbles x16 compensated in A), 8-bit codes as
//    zero-extended bytes.  The fp16 scale and zero fold in afterwards:
//    s_t = sum_g scale_g,t dot_g + zero_g,t sum_{j in g} q'_j.
//  * TurboQuant K: the 8 Lloyd-Max centroids are odd-symmetric, so with code bits c0, c1, c2 and
//    b = 2c - 1, mu[code] = a0 b0 + a1 b1 + a2 b2 + a3 b0 b1 b2, and b0 b1 b2 = 2 (c0^c1^c2) - 1.
//    <q', mu[code]> is then four dot products of q' with 0/1 bit planes (plus a constant), and
//    the QJL term a fifth.  A bit plane enters B as a masked word (bit * 2^(k-24) for a bit at
//    position k < 10, compensated in A); A rows are (head; q' hi, q' lo, Sq' hi, Sq' lo).
//  * Split K (the outlier split on keys): q' is taken into the split domain (its channels gathered
//    by the key permutation, then the two 64-point transforms); the A rows carry the outlier
//    half's q' and the rest's separately (each zero on the other half's channels), so one product
//    with a bit plane yields both halves' sums, which take their own norms; the outliers' top
//    plane (and at 3.5 bits their parity monomial) and the QJL term are the remaining products.
//  * Online softmax in the log2 domain (q' carries softmax_scale * log2(e) and a per-head power
//    of two that keeps 16 q' inside fp16 range).
//  * PV: A = p * (scale_g | -n * a_p) as fp16 hi (rows 0-7) + remainder lo (rows 8-15), staged
//    through LDS in operand order; B = centred V codes c - 8 (c - 128) as exact fp16 integers,
//    or the TurboQuant-MSE bit planes as -+1, plus a vector-ALU sum of p (zero + 8 scale).
//    Centring keeps every accumulator of the order of the output itself.
//  * Each split writes one partial (running max, sum, acc[128]) per query head; the merge
//    kernel combines them in a fixed order and applies c_V and R_V^-1.
//  * The FP32 window (progressive mode) is one extra split computed on the vector ALU.
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_lanes.h"
#include "kvq_mfma_ops.h"
#include "kvq_quant_dev.h"

namespace kvq {
namespace {

using namespace mops;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kPRow = 72;                 // halves per staged P row: 64 tokens + 8 pad
constexpr int kPWave = 4 * 16 * kPRow;    // halves per wave: [group | plane][16 rows][token]
constexpr float kKappa = 0.0097915166977774f; // sqrt(pi/2) / 128
// cache kinds (template parameters)
// uniform 4-bit, uniform 8-bit, TurboQuant 3-bit, TurboQuant-MSE 4-bit (V only), the split
// TurboQuant-MSE V with 3 / 4 bits on the outlier half (2.5 / 3.5 bits per channel), uniform
// 3-bit (bit planes in the TurboQuant 3-bit layout, uniform scale / zero), and the split key
// at b = 3 / 4 (b - 1 bits on the outliers, b - 2 on the rest, plus the QJL sketch; K only)
constexpr int kU4 = 0, kU8 = 1, kTb = 2, kTb4 = 3, kTs3 = 4, kTs4 = 5, kU3 = 6, kSk3 = 7, kSk4 = 8;

// Eight one-bit operands from a half-interleaved word: quarter q (0..3) of each half, i.e. bits
// 4q + v and 16 + 4q + v (v = 0..3).  Operand 2v + h is that bit times 2^(4(q%2) + v - 24).
__device__ __forceinline__ u4 bits8(uint32_t w, int q) {
    const uint32_t x = (q & 2) ? (w >> 8) : w;
    const uint32_t m = 0x00010001u << (4 * (q & 1));
    u4 r;
    r.x = x & m;
    r.y = x & (m << 1);
    r.z = x & (m << 2);
    r.w = x & (m << 3);
    return r;
}

// Eight 3-bit codes from the three bit-plane words of a half-interleaved group, quarter q of each
// half: operand 2v + h is the code whose bits sit at 16h + 4q + v of the three words, as the fp16
// subnormal code * 2^(4(q%2) + v - 24) (the three bits land on consecutive mantissa bits).
__device__ __forceinline__ u4 codes3x8(uint32_t p0, uint32_t p1, uint32_t p2, int q) {
    const uint32_t x0 = (q & 2) ? (p0 >> 8) : p0, x1 = (q & 2) ? (p1 >> 8) : p1, x2 = (q & 2) ? (p2 >> 8) : p2;
    const uint32_t m = 0x00010001u << (4 * (q & 1));
    u4 r;
    r.x = (x0 & m) | ((x1 & m) << 1) | ((x2 & m) << 2);
    r.y = (x0 & (m << 1)) | ((x1 & (m << 1)) << 1) | ((x2 & (m << 1)) << 2);
    r.z = (x0 & (m << 2)) | ((x1 & (m << 2)) << 1) | ((x2 & (m << 2)) << 2);
    r.w = (x0 & (m << 3)) | ((x1 & (m << 3)) << 1) | ((x2 & (m << 3)) << 2);
    return r;
}

// The same eight codes centred, as exact fp16 (code - 4) * 2^(4(q%2) + v): the code bits are
// placed in the mantissa of 1024 (0x6400) and 1024 + 4 * 2^(4(q%2) + v) is subtracted with one
// packed fp16 add per operand pair.
__device__ __forceinline__ h8 centred3x8(uint32_t p0, uint32_t p1, uint32_t p2, int q) {
    const u4 c = codes3x8(p0, p1, p2, q);
    const _Float16 b = (_Float16)(q & 1 ? 16.0f : 1.0f);
    const h2v k0 = {(_Float16)1024.0f + (_Float16)4.0f * b, (_Float16)1024.0f + (_Float16)4.0f * b};
    const h2v k1 = {(_Float16)1024.0f + (_Float16)8.0f * b, (_Float16)1024.0f + (_Float16)8.0f * b};
    const h2v k2 = {(_Float16)1024.0f + (_Float16)16.0f * b, (_Float16)1024.0f + (_Float16)16.0f * b};
    const h2v k3 = {(_Float16)1024.0f + (_Float16)32.0f * b, (_Float16)1024.0f + (_Float16)32.0f * b};
    const h2v a0 = __builtin_bit_cast(h2v, c.x | 0x64006400u) - k0;
    const h2v a1 = __builtin_bit_cast(h2v, c.y | 0x64006400u) - k1;
    const h2v a2 = __builtin_bit_cast(h2v, c.z | 0x64006400u) - k2;
    const h2v a3 = __builtin_bit_cast(h2v, c.w | 0x64006400u) - k3;
    h8 r;
    r[0] = a0[0];
    r[1] = a0[1];
    r[2] = a1[0];
    r[3] = a1[1];
    r[4] = a2[0];
    r[5] = a2[1];
    r[6] = a3[0];
    r[7] = a3[1];
    return r;
}

// TurboQuant-MSE V bits as fp16 -1 (bit set) / +1 (bit clear), quarter q of a half-interleaved
// word: operand 2v + h comes from bit 16h + 4q + v.
__device__ __forceinline__ u4 pm1x8(uint32_t w, int q) {
    u4 r;
    r.x = and_or(w << (15 - 4 * q), 0x80008000u, 0x3C003C00u);
    r.y = and_or(w << (14 - 4 * q), 0x80008000u, 0x3C003C00u);
    r.z = and_or(w << (13 - 4 * q), 0x80008000u, 0x3C003C00u);
    r.w = and_or(w << (12 - 4 * q), 0x80008000u, 0x3C003C00u);
    return r;
}

__device__ __forceinline__ float wave_max(float v) {
    return xor_reduce<64>(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
    return xor_reduce<64>(v, [](float x, float y) { return x + y; });
}

__device__ __forceinline__ void hadamard_wave(float& a, float& b, int) { qdev::hadamard_wave(a, b); }

// Per-lane registers of one 64-token chunk.  K: sub-tile j = rows 16j + (lane % 16) of the
// 64-token block (tokens 4 (lane % 16) + j).  Uniform: the lane's quarter of the code row and the
// row's 16-byte meta.  TurboQuant: the three plane words of group lane / 16, QJL word lane / 16,
// and (n, gamma).  V: uniform = 32*VB/4 bytes of each 32-token block at lane * 32*VB/4 plus the
// 16-byte meta of tokens 4 (lane % 16) + 0..3; TurboQuant-MSE = the lane's six words of each
// 32-token block plus the norms of tokens 4 (lane % 16) + 0..3.
template <int KT>
struct KRegs {
    static constexpr int KB = KT == kU4 ? 4 : 8;
    u4 kc[4][KB / 4], km[4];
};
template <>
struct KRegs<kTb> {
    uint32_t pw[4][3], qw[4], nm[4];
};
// split K: the plane words of group lane / 16 (b - 1 on the outlier groups 0, 1, b - 2 on the
// others, unused words zero), QJL word lane / 16, and the row's (n_outlier | n_rest, gamma | 0)
template <>
struct KRegs<kSk3> {
    uint32_t pw[4][3], qw[4];
    uint2 nm[4];
};
template <>
struct KRegs<kSk4> {
    uint32_t pw[4][3], qw[4];
    uint2 nm[4];
};
// uniform 3-bit K: the three plane words of group lane / 16 and the 16-byte meta row
template <>
struct KRegs<kU3> {
    uint32_t pw[4][3];
    u4 km[4];
};
template <int VT>
struct VRegs {
    static constexpr int VB = VT == kU4 ? 4 : 8;
    u4 vc[2][VB / 2], vm[4];
};
template <>
struct VRegs<kTb> {
    uint2 w[2][3];
    uint2 nm;
};
// uniform 3-bit V: the lane's six plane words of each 32-token block (TurboQuant-MSE V layout) and
// the 16-byte meta of tokens 4 (lane % 16) + 0..3
template <>
struct VRegs<kU3> {
    uint2 w[2][3];
    u4 vm[4];
};
template <>
struct VRegs<kTb4> {
    uint2 w[2][4];
    uint2 nm;
};
// split V: the lane's W = 2 bo - 1 words (outlier planes, then the rest's) of each 32-token
// block, and the (outlier, rest) norm pairs of tokens 4 (lane % 16) + 0..3
template <>
struct VRegs<kTs3> {
    uint32_t w[2][5];
    u4 nm;
};
template <>
struct VRegs<kTs4> {
    uint32_t w[2][7];
    u4 nm;
};

// Coefficients of a b-bit odd-symmetric codebook as a sum over the odd monomials of the code's
// +-1 bits (b = 1: b0; b = 2: b0, b1; b = 3: b0, b1, b2, b0b1b2; b = 4: b0, b1, b2, b3, b0b1b2, b0b1b3,
// b0b2b3, b1b2b3): a_S = mean over the upper half of mu[c] prod_S b (the top bit is 1 there).
template <int B>
__device__ __forceinline__ void odd_coeffs(const float* mu, float* a) {
    constexpr int H = 1 << (B - 1);
#pragma unroll
    for (int s = 0; s < H; ++s) a[s] = 0.0f;
#pragma unroll
    for (int c = H; c < 2 * H; ++c) {
        const float m = mu[c];
        const float b0 = (c & 1) ? 1.0f : -1.0f, b1 = (c & 2) ? 1.0f : -1.0f, b2 = (c & 4) ? 1.0f : -1.0f;
        if constexpr (B == 1) {
            a[0] += m;
        } else if constexpr (B == 2) {
            a[0] += m * b0;
            a[1] += m;
        } else if constexpr (B == 3) {
            a[0] += m * b0;
            a[1] += m * b1;
            a[2] += m;
            a[3] += m * (b0 * b1);
        } else {
            a[0] += m * b0;
            a[1] += m * b1;
            a[2] += m * b2;
            a[3] += m;
            a[4] += m * (b0 * b1 * b2);
            a[5] += m * (b0 * b1);
            a[6] += m * (b0 * b2);
            a[7] += m * (b1 * b2);
        }
    }
#pragma unroll
    for (int s = 0; s < H; ++s) a[s] *= 1.0f / (float)H;
}

// PV products of one 16-channel tile with a b-bit plane set: w[k] = plane k's word, the
// monomials in odd_coeffs order as -+1 operands (an odd product of +-1 bits is 2 parity - 1).
template <int B>
__device__ __forceinline__ f4 pv_planes(const h8* Pg, const uint32_t* w, int q, f4 acc) {
    acc = mfma16(Pg[0], as_h8(pm1x8(w[0], q)), acc);
    acc = mfma16(Pg[1], as_h8(pm1x8(w[1], q)), acc);
    if constexpr (B == 3) {
        acc = mfma16(Pg[2], as_h8(pm1x8(w[2], q)), acc);
        acc = mfma16(Pg[3], as_h8(pm1x8(w[0] ^ w[1] ^ w[2], q)), acc);
    } else if constexpr (B == 4) {
        const uint32_t x01 = w[0] ^ w[1];
        acc = mfma16(Pg[2], as_h8(pm1x8(w[2], q)), acc);
        acc = mfma16(Pg[3], as_h8(pm1x8(w[3], q)), acc);
        acc = mfma16(Pg[4], as_h8(pm1x8(x01 ^ w[2], q)), acc);
        acc = mfma16(Pg[5], as_h8(pm1x8(x01 ^ w[3], q)), acc);
        acc = mfma16(Pg[6], as_h8(pm1x8(w[0] ^ w[2] ^ w[3], q)), acc);
        acc = mfma16(Pg[7], as_h8(pm1x8(w[1] ^ w[2] ^ w[3], q)), acc);
    }
    return acc;
}

template <int KT, int VT, int MB, int kNW>
__global__ __launch_bounds__(kNW * 64) void decode_mfma_kernel(DecodeParams p) {
    // K kinds: uniform (4 / 8 / 3-bit codes), TurboQuant-QJL, split (outlier / rest codes + QJL)
    constexpr bool KQ = KT == kTb, KS = KT == kSk3 || KT == kSk4, KU = !KQ && !KS;
    constexpr int kKb = KT == kSk4 ? 4 : 3; // split K: b (outliers b - 1 bits, the rest b - 2)
    constexpr bool VU = VT == kU4 || VT == kU8 || VT == kU3, VT4 = VT == kTb4;
    constexpr bool VS = VT == kTs3 || VT == kTs4;
    constexpr bool K3 = KT == kU3, V3 = VT == kU3; // uniform 3-bit planes
    constexpr int KB = KT == kU4 ? 4 : 8, VB = VT == kU4 ? 4 : (V3 ? 3 : 8);
    // split V: bo bits on the outlier half (kSo monomials), bo - 1 on the rest (kSr), W words
    constexpr int kBo = VT == kTs4 ? 4 : 3, kSo = 1 << (kBo - 1), kSr = kSo / 2, kWv = 2 * kBo - 1;
    // P staging slots per wave: 4 (uniform groups, or the 3-bit planes), 8 (the 4-bit
    // monomials), kSo + kSr (split V)
    // 4-bit and split TurboQuant V with one head block (G <= 4) stage 8 rows per slot (heads' hi
    // in rows 0-3, lo in 4-7; lanes of rows 8-15 take zeros), which halves the LDS so that 8
    // waves fit
    constexpr bool kCmp = (VS || VT4) && MB == 1;
    constexpr int kRows = kCmp ? 8 : 16;
    // halves per wave: the staged P slots, and at least the 2 x 8 x 128 fp32 accumulator rows the
    // epilogue stores in the same memory
    constexpr int kSlots = VT4 ? 8 : (VS ? kSo + kSr : 4);
    constexpr int kPW = (kSlots * kRows * kPRow > 2 * 8 * kDim * 2) ? kSlots * kRows * kPRow : 2 * 8 * kDim * 2;
    static_assert(kPW * 2 >= 2 * 8 * kDim * 4, "the epilogue's accumulator rows fit in the staging area");
    __shared__ float s_q[kMaxGroupHeads][kDim];   // q' in the rotated/balanced domain, scaled
    __shared__ float s_qw[kMaxGroupHeads][kDim];  // plain q * scale * log2e (FP32 window)
    __shared__ float s_sp[KU ? 1 : kMaxGroupHeads][kDim]; // S q' (TurboQuant K)
    __shared__ float s_qsum[kMaxGroupHeads][4];
    __shared__ float s_spsum[kMaxGroupHeads];
    __shared__ float s_qfac[kMaxGroupHeads];
    __shared__ __align__(16) _Float16 s_p[kNW * kPW];
    __shared__ float s_wm[kNW][kMaxGroupHeads], s_wl[kNW][kMaxGroupHeads];
    __shared__ float s_wz[kNW][kMaxGroupHeads][4];
    __shared__ float2 s_vmap[2][64]; // value plane's c_V and signs per lane pair (output map)
    __shared__ int2 s_vperm[64];     // split V: channels of the lane's two positions

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
    const int G = p.G, W = p.window;
    const int n = p.len[b];
    const int nq = (W > 0) ? max(0, n - W) : n;
    const bool wsplit = (W > 0) && (split >= p.n_splits); // FP32-window workgroups come last
    const PlaneGeom& KG = p.geom[0];
    const PlaneGeom& VG = p.geom[1];
    const char* slot = p.layer_base + (size_t)b * p.seq_stride + (size_t)kvh * p.head_stride;
    const uint8_t* kcodes = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.codes_off);
    const uint8_t* kmeta = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.meta_off);
    const uint8_t* kqjl = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.qjl_off);
    const float* kring = reinterpret_cast<const float*>(slot + p.plane_off[0] + KG.ring_off);
    const uint8_t* vcodes = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.codes_off);
    const uint8_t* vmeta = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.meta_off);
    const float* vring = reinterpret_cast<const float*>(slot + p.plane_off[1] + VG.ring_off);
    // Fused append: the workgroup whose split holds the newest token (the window split in
    // progressive mode, else the code split of token n - 1) quantizes it first, K on wave 0 and
    // V on wave 1; the barrier makes its stores visible to the workgroup's own loads below.
    if (p.fuse) {
        const int owner = (W > 0) ? p.n_splits + min(p.n_win_splits - 1, (n - 1 - nq) / ((kWindowMax + p.n_win_splits - 1) / p.n_win_splits))
                                  : (n - 1) / p.split_tokens;
        if (split == owner && n > 0) {
            if (wave < 2) qdev::quantize_wave(p.append, wave, b, kvh, 0, reinterpret_cast<float*>(s_p) + wave * kDim);
            __syncthreads();
        }
    }
    const float UK = (KB == 4 && !K3) ? 1048576.0f : 16777216.0f; // 2^20 / 2^24: unit of a code product
    const float UV = (VB == 4) ? 0.0625f : 1.0f; // 4-bit: half the weights carry x16

    // ---------------- the query-side loads go out first (they are small and the preparation
    // waits on them), then this wave's first chunk, so the memory pipe starts immediately
    constexpr int kHPW = (kMaxGroupHeads + kNW - 1) / kNW; // heads prepared per wave
    float qa[kHPW], qc[kHPW];
#pragma unroll
    for (int i = 0; i < kHPW; ++i) {
        const int h = wave + i * kNW;
        qa[i] = qc[i] = 0.0f;
        if (h < G) {
            const size_t off = ((size_t)b * p.Hq + kvh * G + h) * kDim;
            if (p.dtype == 0) {
                const float2 v = reinterpret_cast<const float2*>(static_cast<const float*>(p.q) + off)[l];
                qa[i] = v.x;
                qc[i] = v.y;
            } else {
                const uint32_t v = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + off)[l];
                qa[i] = in16_to_f32(v & 0xffff, p.dtype);
                qc[i] = in16_to_f32(v >> 16, p.dtype);
            }
        }
    }
    const float2 sgn = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 0) * kDim)[l];
    // the value plane's output-map tables, staged once for the epilogue (read after barriers)
    if (wave == 0 && !wsplit) {
        const size_t vtab = (size_t)(kvh * 2 + 1) * kDim;
        s_vmap[0][l] = VG.sinkhorn ? reinterpret_cast<const float2*>(p.cs + vtab)[l] : make_float2(1.0f, 1.0f);
        s_vmap[1][l] = (VG.rotate || VS) ? reinterpret_cast<const float2*>(p.signs + vtab)[l] : make_float2(1.0f, 1.0f);
        s_vperm[l] = VS ? reinterpret_cast<const int2*>(p.perm + (size_t)kvh * kDim)[l] : make_int2(2 * l, 2 * l + 1);
    }
    const float2 csk = reinterpret_cast<const float2*>(p.cs + (size_t)(kvh * 2 + 0) * kDim)[l];
    int2 pmk = make_int2(0, 0);
    if constexpr (KS) pmk = reinterpret_cast<const int2*>(p.perm_k + (size_t)kvh * kDim)[l];
    // TurboQuant tables: centroids 4..7, and this thread's slice of S^T (stored [j][i]) for S q'
    constexpr int kParts = kNW * 64 / kDim, kJ = kDim / kParts;
    float mu4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float st[KU ? 1 : kJ];
    if constexpr (KQ || VT == kTb) {
#pragma unroll
        for (int c = 0; c < 4; ++c) mu4[c] = p.mu[4 + c];
    }
    if constexpr (!KU) {
        if (!wsplit) {
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj) st[jj] = p.qjl_st[((tid >> 7) * kJ + jj) * kDim + (tid & 127)];
        }
    }
    const int lr = l & 15, lq = l >> 4; // column / quarter of the 16x16 tiles
    const int tok_begin = split * p.split_tokens;
    const int tok_end = wsplit ? tok_begin : min(nq, tok_begin + p.split_tokens);
    const int nch = (tok_end > tok_begin) ? (tok_end - tok_begin + 63) / 64 : 0;

    // kBuf register sets per wave: with 4 waves (one per SIMD) each wave keeps two chunks in
    // flight (uniform K; TurboQuant K has no registers to spare); with 8 waves, two waves share
    // a SIMD and each keeps one
    constexpr int kBuf = (kNW == 4 && KU) ? 2 : 1;
    KRegs<KT> krs[kBuf];
    VRegs<VT> vrs[kBuf];
    auto load_k = [&](KRegs<KT>& kr, int ci) {
        const size_t r0 = (size_t)tok_begin + 64 * ci + lr; // row of sub-tile 0
        if constexpr (K3) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t* c = reinterpret_cast<const uint32_t*>(kcodes + (r0 + 16 * j) * 48 + 12 * lq);
                kr.pw[j][0] = c[0];
                kr.pw[j][1] = c[1];
                kr.pw[j][2] = c[2];
                kr.km[j] = *reinterpret_cast<const u4*>(kmeta + (r0 + 16 * j) * 16);
            }
        } else if constexpr (KU) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint8_t* c = kcodes + (r0 + 16 * j) * (16 * KB) + (16 * KB / 4) * lq;
#pragma unroll
                for (int u = 0; u < KB / 4; ++u) kr.kc[j][u] = *reinterpret_cast<const u4*>(c + 16 * u);
                kr.km[j] = *reinterpret_cast<const u4*>(kmeta + (r0 + 16 * j) * 16);
            }
        } else if constexpr (KS) {
            // group lq's planes start at word split_k_group_word(lq, b) of the row
            const int nbk = lq < 2 ? kKb - 1 : kKb - 2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t* c = reinterpret_cast<const uint32_t*>(kcodes + (r0 + 16 * j) * split_k_row_bytes(kKb)) +
                                    split_k_group_word(lq, kKb);
#pragma unroll
                for (int k = 0; k < 3; ++k) kr.pw[j][k] = (k < nbk) ? c[k] : 0u;
                kr.qw[j] = *reinterpret_cast<const uint32_t*>(kqjl + (r0 + 16 * j) * 16 + 4 * lq);
                kr.nm[j] = *reinterpret_cast<const uint2*>(kmeta + (r0 + 16 * j) * 8);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t* c = reinterpret_cast<const uint32_t*>(kcodes + (r0 + 16 * j) * 48 + 12 * lq);
                kr.pw[j][0] = c[0];
                kr.pw[j][1] = c[1];
                kr.pw[j][2] = c[2];
                kr.qw[j] = *reinterpret_cast<const uint32_t*>(kqjl + (r0 + 16 * j) * 16 + 4 * lq);
                kr.nm[j] = *reinterpret_cast<const uint32_t*>(kmeta + (r0 + 16 * j) * 4);
            }
        }
    };
    auto load_v = [&](VRegs<VT>& vr, int ci) {
        const size_t t0 = (size_t)tok_begin + 64 * ci;
        if constexpr (V3) {
            const uint8_t* c = vcodes + (t0 / 32) * 1536 + 24 * l;
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int u = 0; u < 3; ++u) vr.w[k][u] = *reinterpret_cast<const uint2*>(c + k * 1536 + 8 * u);
#pragma unroll
            for (int j = 0; j < 4; ++j) vr.vm[j] = *reinterpret_cast<const u4*>(vmeta + (t0 + 4 * lr + j) * 16);
        } else if constexpr (VU) {
            const uint8_t* c = vcodes + (t0 / 32) * (512 * VB) + (size_t)(32 * VB / 4) * l;
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int u = 0; u < VB / 2; ++u)
                    vr.vc[k][u] = *reinterpret_cast<const u4*>(c + k * 512 * VB + 16 * u);
#pragma unroll
            for (int j = 0; j < 4; ++j) vr.vm[j] = *reinterpret_cast<const u4*>(vmeta + (t0 + 4 * lr + j) * 16);
        } else if constexpr (VS) {
            const uint32_t* c = reinterpret_cast<const uint32_t*>(vcodes + (t0 / 32) * (256 * kWv)) + kWv * l;
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int u = 0; u < kWv; ++u) vr.w[k][u] = c[k * 64 * kWv + u];
            vr.nm = *reinterpret_cast<const u4*>(vmeta + (t0 + 4 * lr) * 4);
        } else if constexpr (VT4) {
            const uint8_t* c = vcodes + (t0 / 32) * 2048 + 32 * l;
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int u = 0; u < 4; ++u) vr.w[k][u] = *reinterpret_cast<const uint2*>(c + k * 2048 + 8 * u);
            vr.nm = *reinterpret_cast<const uint2*>(vmeta + (t0 + 4 * lr) * 2);
        } else {
            const uint8_t* c = vcodes + (t0 / 32) * 1536 + 24 * l;
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int u = 0; u < 3; ++u) vr.w[k][u] = *reinterpret_cast<const uint2*>(c + k * 1536 + 8 * u);
            vr.nm = *reinterpret_cast<const uint2*>(vmeta + (t0 + 4 * lr) * 2);
        }
    };
    // The wave's first chunk is requested right away; each later chunk is requested as soon as
    // the registers it goes into have been consumed (K after the scores, V after PV).
    if (wave < nch) {
        load_k(krs[0], wave);
        load_v(vrs[0], wave);
    }
    if (kBuf == 2 && wave + kNW < nch) {
        load_k(krs[kBuf - 1], wave + kNW);
        load_v(vrs[kBuf - 1], wave + kNW);
    }

    // ---------------- query preparation (once per workgroup) ----------------
#pragma unroll
    for (int i = 0; i < kHPW; ++i) {
        const int h = wave + i * kNW;
        if (h >= G) break;
        float a = qa[i], c = qc[i];
        s_qw[h][2 * l] = a * p.qscale;
        s_qw[h][2 * l + 1] = c * p.qscale;
        if constexpr (KS) {
            // the split domain: positions 2l, 2l+1 take channels perm_k[2l], perm_k[2l+1] (lane
            // pm / 2, component pm % 2), then signs by position and the two 64-point transforms
            const float ax = __shfl(a, pmk.x >> 1), ay = __shfl(c, pmk.x >> 1);
            const float bx = __shfl(a, pmk.y >> 1), by = __shfl(c, pmk.y >> 1);
            a = (pmk.x & 1) ? ay : ax;
            c = (pmk.y & 1) ? by : bx;
            qdev::rotate64_signed(a, c, sgn.x, sgn.y);
        } else if (KG.rotate) {
            if (sgn.x < 0.0f) a = -a;
            if (sgn.y < 0.0f) c = -c;
            hadamard_wave(a, c, l);
            a *= c0f();
            c *= c0f();
        }
        if (KG.sinkhorn) {
            a *= csk.x;
            c *= csk.y;
        }
        a *= p.qscale;
        c *= p.qscale;
        // exact power-of-two normalisation: 16 * max|q'| lands in [2^10, 2^11)
        const float mx = wave_max(fmaxf(fabsf(a), fabsf(c)));
        int e2 = 0;
        if (mx > 0.0f) frexpf(mx, &e2);
        const int e = (mx > 0.0f) ? min(max(7 - e2, -100), 100) : 0;
        const float f = ldexpf(1.0f, e);
        a *= f;
        c *= f;
        s_q[h][2 * l] = a;
        s_q[h][2 * l + 1] = c;
        const float gs = row_sum16(a + c);
        if ((l & 15) == 0) s_qsum[h][l >> 4] = gs;
        if (l == 0) s_qfac[h] = ldexpf(1.0f, -e);
    }
    __syncthreads();
    if constexpr (!KU) {
        // S q' for the QJL term: thread (i, part) sums 128/kParts values of j for every head, then
        // the parts are added in order
        float* s_spp = reinterpret_cast<float*>(s_p); // [kParts][8][128] scratch
        if (!wsplit) {
            const int i = tid & 127, part = tid >> 7;
#pragma unroll
            for (int h = 0; h < kMaxGroupHeads; ++h) {
                if (h >= G) break;
                float a = 0.0f;
#pragma unroll
                for (int jj = 0; jj < kJ; ++jj) a = fmaf(st[jj], s_q[h][part * kJ + jj], a);
                s_spp[(part * 8 + h) * kDim + i] = a;
            }
        }
        __syncthreads();
        if (!wsplit) {
            for (int idx = tid; idx < G * kDim; idx += kNW * 64) {
                const int h = idx >> 7, i = idx & 127;
                float a = 0.0f;
#pragma unroll
                for (int q = 0; q < kParts; ++q) a += s_spp[(q * 8 + h) * kDim + i];
                s_sp[h][i] = a;
            }
        }
        __syncthreads();
        for (int h = wave; h < G; h += kNW) {
            const float v = wave_sum(s_sp[h][2 * l] + s_sp[h][2 * l + 1]);
            if (l == 0) s_spsum[h] = v;
        }
        __syncthreads();
    }

    // TurboQuant centroids as odd bit functions: mu[c] = a0 b0 + a1 b1 + a2 b2 + a3 b0 b1 b2
    float al[4] = {0.0f, 0.0f, 0.0f, 0.0f}, asum = 0.0f;
    // 16-level (4-bit V) centroids: mu[c] = sum over the odd monomials of b0..b3 (b0, b1, b2, b3,
    // b0b1b2, b0b1b3, b0b2b3, b1b2b3) of a_S prod b; the codebook's odd symmetry makes each a_S
    // the mean of mu[c] prod_S b over the upper half c = 8 .. 15 (where b3 = 1)
    float a16[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (VT4) {
#pragma unroll
        for (int c = 8; c < 16; ++c) {
            const float m = p.mu16[c];
            const float b0 = (c & 1) ? 1.0f : -1.0f, b1 = (c & 2) ? 1.0f : -1.0f, b2 = (c & 4) ? 1.0f : -1.0f;
            a16[0] += m * b0;
            a16[1] += m * b1;
            a16[2] += m * b2;
            a16[3] += m;
            a16[4] += m * (b0 * b1 * b2);
            a16[5] += m * (b0 * b1);
            a16[6] += m * (b0 * b2);
            a16[7] += m * (b1 * b2);
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) a16[g] *= 0.125f;
    }
    // split V: the outlier and rest codebooks of N(0, 1/64) (tables at levels - 4)
    float aO[kSo], aR[kSr];
    if constexpr (VS) {
        odd_coeffs<kBo>(p.mu64 + ((1 << kBo) - 4), aO);
        odd_coeffs<kBo - 1>(p.mu64 + ((1 << (kBo - 1)) - 4), aR);
    }
    // split K: the outlier (b - 1 bits) and rest (b - 2 bits) codebooks of N(0, 1/64)
    float aKO[KS ? (1 << (kKb - 2)) : 1], aKR[KS ? (1 << (kKb - 3)) : 1], aKOs = 0.0f, aKRs = 0.0f;
    if constexpr (KS) {
        odd_coeffs<kKb - 1>(p.mu64 + split_table_off(1 << (kKb - 1)), aKO);
        odd_coeffs<kKb - 2>(p.mu64 + split_table_off(1 << (kKb - 2)), aKR);
#pragma unroll
        for (int k = 0; k < (1 << (kKb - 2)); ++k) aKOs += aKO[k];
#pragma unroll
        for (int k = 0; k < (1 << (kKb - 3)); ++k) aKRs += aKR[k];
    }
    if constexpr (KQ || VT == kTb) {
        const float m4 = mu4[0], m5 = mu4[1], m6 = mu4[2], m7 = mu4[3];
        al[0] = 0.25f * ((m5 - m4) + (m7 - m6));
        al[1] = 0.25f * ((m6 - m4) + (m7 - m5));
        al[2] = 0.25f * ((m4 + m5) + (m6 + m7));
        al[3] = 0.25f * ((m4 - m5) + (m7 - m6));
        asum = (al[0] + al[1]) + (al[2] + al[3]);
    }

    // per-wave softmax state, in the score layout (lane: head 4*mb + lq, column lr)
    float m_run[MB], l_run[MB], z_run[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        m_run[mb] = kNegInf;
        l_run[mb] = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) z_run[mb][g] = 0.0f;
    }
    // PV accumulators: tile N = channels 16N..16N+15; rows 4*lq + v: lq 0,1 = fp16-hi part of
    // heads 4*lq + v, lq 2,3 = fp16-lo part of heads 4*(lq-2) + v
    f4 acc[8];
#pragma unroll
    for (int N = 0; N < 8; ++N) acc[N] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    // window split results (plain domain), lane = channel pair
    float wacc0[kMaxGroupHeads], wacc1[kMaxGroupHeads], wm[kMaxGroupHeads], wl[kMaxGroupHeads];
#pragma unroll
    for (int h = 0; h < kMaxGroupHeads; ++h) {
        wacc0[h] = wacc1[h] = 0.0f;
        wm[h] = kNegInf;
        wl[h] = 0.0f;
    }

    _Float16* my_p = s_p + wave * kPW;

    if (!wsplit) {
        // ---------------- A operands ----------------
        // uniform K: Ahi/Alo[mb][g] = (head, group) rows of q' (fp16 hi / lo), zero outside g.
        // TurboQuant K: At[mb][s] rows (head 4mb + lr/4; q' hi, q' lo, Sq' hi, Sq' lo), k-slice s
        // = channels 32*lq + 8s + 0..7, pre-scaled by 2^-(4(s%2) + i/2) for the bit operands.
        // split K: At rows (head 4mb + lr/4; q'_O hi, q'_O lo, q'_R hi, q'_R lo) -- each half's
        // rows zero on the other half's channels, so one bit-plane product yields both halves'
        // sums -- and AtS rows (Sq' hi, Sq' lo, 0, 0) for the QJL term, with the same pre-scaling.
        constexpr int NA = KU ? 4 : 1;
        h8 Ahi[MB][NA], Alo[MB][NA], At[MB][KU ? 1 : 4], AtS[MB][KS ? 4 : 1];
        float qs_l[MB][4], F[MB], cQ[MB], cS[MB], cQR[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int hs = min(4 * mb + lq, G - 1); // score-layout head of this lane
            if constexpr (K3) {
                // uniform 3-bit K: the product over k-slice s takes channels 32 lq + 8 s + i from
                // quarter lq, i.e. group lq; row (head, group gq) keeps only the quarter gq, and
                // each value is pre-scaled by 2^-(4(s%2) + i/2) for the code operand's position
                const int h = 4 * mb + (lr >> 2), gq = lr & 3;
                const int hc = min(h, G - 1);
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    h8 hi, lo;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float sc = __uint_as_float((uint32_t)(127 - 4 * (sl & 1) - (i >> 1)) << 23);
                        const float x = (h < G && lq == gq) ? s_q[hc][32 * lq + 8 * sl + i] * sc : 0.0f;
                        const _Float16 xh = (_Float16)x;
                        hi[i] = xh;
                        lo[i] = (_Float16)(x - (float)xh); // unscaled: accumulates with hi
                    }
                    Ahi[mb][sl] = hi;
                    Alo[mb][sl] = lo;
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) qs_l[mb][g] = s_qsum[hs][g] * (1.0f / UK);
                F[mb] = UK * s_qfac[hs];
            } else if constexpr (KU) {
                const int h = 4 * mb + (lr >> 2), gq = lr & 3;
                const int hc = min(h, G - 1);
                h8 hi, lo;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float w = (KB == 4 && (i == 0 || i == 1 || i == 4 || i == 5)) ? 16.0f : 1.0f;
                    const float x = (h < G) ? s_q[hc][32 * gq + 8 * lq + i] * w : 0.0f;
                    const _Float16 xh = (_Float16)x;
                    hi[i] = xh;
                    // the remainder unscaled: it shares the hi product's accumulator (its absolute
                    // precision, 2^-24 where it is subnormal, is 2^-30 of the largest |q'|)
                    lo[i] = (_Float16)(x - (float)xh);
                }
                const h8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    Ahi[mb][g] = (g == gq) ? hi : zero;
                    Alo[mb][g] = (g == gq) ? lo : zero;
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) qs_l[mb][g] = s_qsum[hs][g] * (1.0f / UK);
                F[mb] = UK * s_qfac[hs];
            } else if constexpr (KS) {
                const int h = 4 * mb + (lr >> 2), v = lr & 3;
                const int hc = min(h, G - 1);
                const bool mine = (v < 2) == (lq < 2); // outlier rows on channels < 64, rest rows above
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    h8 a, as;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int c = 32 * lq + 8 * s + i;
                        const float sc = __uint_as_float((uint32_t)(127 - 4 * (s & 1) - (i >> 1)) << 23);
                        const float x = (h < G && mine) ? s_q[hc][c] * sc : 0.0f;
                        const _Float16 xh = (_Float16)x;
                        a[i] = (v & 1) ? (_Float16)((x - (float)xh) * kLoScale) : xh;
                        const float y = (h < G && v < 2) ? s_sp[hc][c] * sc : 0.0f;
                        const _Float16 yh = (_Float16)y;
                        as[i] = (v & 1) ? (_Float16)((y - (float)yh) * kLoScale) : yh;
                    }
                    At[mb][s] = a;
                    AtS[mb][s] = as;
                }
                cQ[mb] = aKOs * (s_qsum[hs][0] + s_qsum[hs][1]) * 5.9604644775390625e-8f; // 2^-24
                cQR[mb] = aKRs * (s_qsum[hs][2] + s_qsum[hs][3]) * 5.9604644775390625e-8f;
                cS[mb] = s_spsum[hs] * 5.9604644775390625e-8f;
                F[mb] = 16777216.0f * s_qfac[hs];
            } else {
                const int h = 4 * mb + (lr >> 2), v = lr & 3;
                const int hc = min(h, G - 1);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    h8 a;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int c = 32 * lq + 8 * s + i;
                        const float sc = __uint_as_float((uint32_t)(127 - 4 * (s & 1) - (i >> 1)) << 23);
                        const float x = (h < G) ? ((v < 2) ? s_q[hc][c] : s_sp[hc][c]) * sc : 0.0f;
                        const _Float16 xh = (_Float16)x;
                        a[i] = (v & 1) ? (_Float16)((x - (float)xh) * kLoScale) : xh;
                    }
                    At[mb][s] = a;
                }
                const float qtot = (s_qsum[hs][0] + s_qsum[hs][1]) + (s_qsum[hs][2] + s_qsum[hs][3]);
                cQ[mb] = asum * qtot * 5.9604644775390625e-8f; // 2^-24
                cS[mb] = s_spsum[hs] * 5.9604644775390625e-8f;
                F[mb] = 16777216.0f * s_qfac[hs];
            }
        }

        auto chunk = [&](KRegs<KT>& kr, VRegs<VT>& vr, int ci) __attribute__((always_inline)) {
            const int c0 = tok_begin + 64 * ci;
            const int nci = ci + kBuf * kNW; // the chunk these registers are refilled with
            const bool more = nci < nch;

            // ---- scores
            float raw[MB][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool valid = (c0 + 4 * lr + j) < tok_end;
                if constexpr (KU) {
                    const auto& km = kr.km;
                    h8 B[4]; // uniform 4 / 8-bit: B[g] = 8 codes of group g; 3-bit: B[s] = slice s
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        if constexpr (K3)
                            B[g] = as_h8(codes3x8(kr.pw[j][0], kr.pw[j][1], kr.pw[j][2], g));
                        else if constexpr (KB == 4)
                            B[g] = as_h8(unpack4(kr.kc[j][0][g]));
                        else
                            B[g] = as_h8(unpack8(kr.kc[j][g >> 1][2 * (g & 1)], kr.kc[j][g >> 1][2 * (g & 1) + 1]));
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        f4 D = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            D = mfma16(Ahi[mb][g], B[g], D);
                            D = mfma16(Alo[mb][g], B[g], D);
                        }
                        float r = lo_h(km[j].x) * D[0];
                        r = fmaf(hi_h(km[j].x), D[1], r);
                        r = fmaf(lo_h(km[j].y), D[2], r);
                        r = fmaf(hi_h(km[j].y), D[3], r);
                        r = fmaf(lo_h(km[j].z), qs_l[mb][0], r);
                        r = fmaf(hi_h(km[j].z), qs_l[mb][1], r);
                        r = fmaf(lo_h(km[j].w), qs_l[mb][2], r);
                        r = fmaf(hi_h(km[j].w), qs_l[mb][3], r);
                        raw[mb][j] = valid ? r : kNegInf;
                    }
                } else if constexpr (KS) {
                    // planes 0 .. b - 3 exist in both halves (one product gives the outlier sum in
                    // rows 0, 1 and the rest's in rows 2, 3); the outliers' top plane (and at b = 4
                    // their parity monomial b0 b1 b2) only in lanes of groups 0, 1
                    constexpr int NP = kKb == 3 ? 2 : 4;
                    const uint32_t P0 = kr.pw[j][0], P1 = kr.pw[j][1], P2 = kr.pw[j][2];
                    const uint32_t W[4] = {P0, P1, P2, lq < 2 ? (P0 ^ P1 ^ P2) : 0u};
                    f4 D[MB][NP + 1];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int k = 0; k <= NP; ++k) D[mb][k] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        h8 B[NP];
#pragma unroll
                        for (int k = 0; k < NP; ++k) B[k] = as_h8(bits8(W[k], s));
                        const h8 BQ = as_h8(bits8(kr.qw[j], s));
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                            for (int k = 0; k < NP; ++k) D[mb][k] = mfma16(At[mb][s], B[k], D[mb][k]);
                            D[mb][NP] = mfma16(AtS[mb][s], BQ, D[mb][NP]);
                        }
                    }
                    const float nO = lo_h(kr.nm[j].x), nR = hi_h(kr.nm[j].x), gam = lo_h(kr.nm[j].y);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        // outlier monomials: b0, b1 (b = 3); b0, b1, b2, b0 b1 b2 (b = 4); the rest:
                        // b0 (b = 3); b0, b1 (b = 4)
                        float mo = 0.0f, mr = 0.0f;
#pragma unroll
                        for (int k = 0; k < (1 << (kKb - 2)); ++k)
                            mo = fmaf(aKO[k], fmaf(D[mb][k][1], kLoInv, D[mb][k][0]), mo);
#pragma unroll
                        for (int k = 0; k < (1 << (kKb - 3)); ++k)
                            mr = fmaf(aKR[k], fmaf(D[mb][k][3], kLoInv, D[mb][k][2]), mr);
                        const float qj = fmaf(D[mb][NP][1], kLoInv, D[mb][NP][0]);
                        float r = fmaf(nO, fmaf(2.0f, mo, -cQ[mb]), nR * fmaf(2.0f, mr, -cQR[mb]));
                        r = fmaf(gam * kKappa, fmaf(2.0f, qj, -cS[mb]), r);
                        raw[mb][j] = valid ? r : kNegInf;
                    }
                } else {
                    const uint32_t P0 = kr.pw[j][0], P1 = kr.pw[j][1], P2 = kr.pw[j][2];
                    const uint32_t X = P0 ^ P1 ^ P2, Q = kr.qw[j];
                    f4 D[MB][5];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int k = 0; k < 5; ++k) D[mb][k] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const h8 B0 = as_h8(bits8(P0, s)), B1 = as_h8(bits8(P1, s)), B2 = as_h8(bits8(P2, s));
                        const h8 B3 = as_h8(bits8(X, s)), BQ = as_h8(bits8(Q, s));
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            D[mb][0] = mfma16(At[mb][s], B0, D[mb][0]);
                            D[mb][1] = mfma16(At[mb][s], B1, D[mb][1]);
                            D[mb][2] = mfma16(At[mb][s], B2, D[mb][2]);
                            D[mb][3] = mfma16(At[mb][s], B3, D[mb][3]);
                            D[mb][4] = mfma16(At[mb][s], BQ, D[mb][4]);
                        }
                    }
                    const float nrm = lo_h(kr.nm[j]), gam = hi_h(kr.nm[j]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        float mse = al[0] * fmaf(D[mb][0][1], kLoInv, D[mb][0][0]);
                        mse = fmaf(al[1], fmaf(D[mb][1][1], kLoInv, D[mb][1][0]), mse);
                        mse = fmaf(al[2], fmaf(D[mb][2][1], kLoInv, D[mb][2][0]), mse);
                        mse = fmaf(al[3], fmaf(D[mb][3][1], kLoInv, D[mb][3][0]), mse);
                        const float qj = fmaf(D[mb][4][3], kLoInv, D[mb][4][2]);
                        const float r = fmaf(nrm, fmaf(2.0f, mse, -cQ[mb]), gam * kKappa * fmaf(2.0f, qj, -cS[mb]));
                        raw[mb][j] = valid ? r : kNegInf;
                    }
                }
            }

            // the next chunk's K is requested as soon as this chunk's scores are formed
            if (more) load_k(kr, nci);

            // ---- online softmax
            float pj[MB][4], alpha[MB];
            bool grew = false;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float t = fmaxf(fmaxf(raw[mb][0], raw[mb][1]), fmaxf(raw[mb][2], raw[mb][3]));
                t = row_max16(t);
                const float mnew = fmaxf(m_run[mb], t * F[mb]);
                const bool inf = (mnew == kNegInf);
                // the hardware exp2 (no denormal-range fix-up: a weight below 2^-126 is zero once it
                // becomes an fp16 operand, and negligible in the running sum)
                alpha[mb] = inf ? 1.0f : __builtin_amdgcn_exp2f(m_run[mb] - mnew);
                grew |= (mnew > m_run[mb]);
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pj[mb][j] = inf ? 0.0f : __builtin_amdgcn_exp2f(fmaf(raw[mb][j], F[mb], -mnew));
                    s += pj[mb][j];
                }
                l_run[mb] = l_run[mb] * alpha[mb] + s;
                m_run[mb] = mnew;
#pragma unroll
                for (int g = 0; g < 4; ++g) z_run[mb][g] *= alpha[mb];
            }
            if (__ballot(grew) != 0) {
                // rescale the PV accumulators: rows 4*lq + v hold head 4*(lq % 2) + v
                float av[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float a0 = readlane_f(alpha[0], 16 * v);
                    float a1 = 1.0f;
                    if (MB == 2) a1 = readlane_f(alpha[MB - 1], 16 * v);
                    av[v] = (kCmp || !(lq & 1)) ? a0 : a1; // compact: rows 4-7 are lo of heads 0-3
                }
#pragma unroll
                for (int N = 0; N < 8; ++N)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[N][v] *= av[v];
            }

            // ---- zero-point / centroid-constant term, and the PV A operand staged in LDS:
            // [g][row][token], row = head (fp16 hi) or 8 + head (fp16 lo)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = 4 * mb + lq;
                // operand [g][j] = PA[g][j] * PB[g][j]: the token's weight factor times the slot's
                // scale or codebook coefficient, split into fp16 hi and scaled lo below
                float PA[kSlots][4], PB[kSlots][4];
                if constexpr (VU) {
                    const auto& vm = vr.vm;
                    constexpr float mid = (VB == 4) ? 8.0f : (V3 ? 4.0f : 128.0f); // codes enter as c - mid
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        z_run[mb][0] = fmaf(pj[mb][j], fmaf(mid, lo_h(vm[j].x), lo_h(vm[j].z)), z_run[mb][0]);
                        z_run[mb][1] = fmaf(pj[mb][j], fmaf(mid, hi_h(vm[j].x), hi_h(vm[j].z)), z_run[mb][1]);
                        z_run[mb][2] = fmaf(pj[mb][j], fmaf(mid, lo_h(vm[j].y), lo_h(vm[j].w)), z_run[mb][2]);
                        z_run[mb][3] = fmaf(pj[mb][j], fmaf(mid, hi_h(vm[j].y), hi_h(vm[j].w)), z_run[mb][3]);
                        // 4-bit: half the operands carry x16; 3-bit: token 4 lr + j enters its
                        // operand at 2^((4 lr + j) % 8 / 2), undone here
                        const float w = V3 ? __uint_as_float((uint32_t)(127 - 2 * (lr & 1) - (j >> 1)) << 23)
                                           : ((VB == 4 && j < 2) ? 16.0f : 1.0f);
                        const float pw = pj[mb][j] * w;
#pragma unroll
                        for (int g = 0; g < 4; ++g) PA[g][j] = pw;
                        PB[0][j] = lo_h(vm[j].x);
                        PB[1][j] = hi_h(vm[j].x);
                        PB[2][j] = lo_h(vm[j].y);
                        PB[3][j] = hi_h(vm[j].y);
                    }
                } else if constexpr (VS) {
                    // outlier slots -p n_O a_S, then the rest's -p n_R a_S
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t nw = (j == 0) ? vr.nm.x : (j == 1) ? vr.nm.y : (j == 2) ? vr.nm.z : vr.nm.w;
                        const float po = pj[mb][j] * lo_h(nw), pr = pj[mb][j] * hi_h(nw);
#pragma unroll
                        for (int g = 0; g < kSo; ++g) {
                            PA[g][j] = -po;
                            PB[g][j] = aO[g];
                        }
#pragma unroll
                        for (int g = 0; g < kSr; ++g) {
                            PA[kSo + g][j] = -pr;
                            PB[kSo + g][j] = aR[g];
                        }
                    }
                } else {
                    // weight of plane p = -p n a_p: the bit operands are -b = -(2 bit - 1)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t nw = (j < 2) ? vr.nm.x : vr.nm.y;
                        const float nt = (j & 1) ? hi_h(nw) : lo_h(nw);
                        const float pn = pj[mb][j] * nt;
#pragma unroll
                        for (int g = 0; g < kSlots; ++g) {
                            PA[g][j] = -pn;
                            PB[g][j] = VT4 ? a16[g] : al[g & 3];
                        }
                    }
                }
#pragma unroll
                for (int g = 0; g < kSlots; ++g) {
                    h4 hv, lv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // hi = fp16(a b); lo = fp16(a b - hi) from one fused product (a mixed-
                        // precision fma when b is an fp16 scale), unscaled: where it is subnormal
                        // its absolute precision is 2^-25 of operands whose weights are at most 1
                        const float a = PA[g][j], b = PB[g][j];
                        const _Float16 ph = (_Float16)(a * b);
                        hv[j] = ph;
                        lv[j] = (_Float16)fmaf(a, b, -(float)ph);
                    }
                    *reinterpret_cast<h4*>(my_p + (g * kRows + row) * kPRow + 4 * lr) = hv;
                    *reinterpret_cast<h4*>(my_p + (g * kRows + kRows / 2 + row) * kPRow + 4 * lr) = lv;
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

            // ---- PV over the two 32-token blocks of the chunk
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                h8 Pg[kSlots];
#pragma unroll
                for (int g = 0; g < kSlots; ++g)
                    Pg[g] = (kCmp && lr >= 8) ? h8{0, 0, 0, 0, 0, 0, 0, 0}
                                              : *reinterpret_cast<const h8*>(my_p + (g * kRows + lr) * kPRow + 32 * k + 8 * lq);
                if constexpr (V3) {
                    // centred 3-bit codes from the three plane words of the tile's half; tiles
                    // with odd N carry x16 (their quarter's position), undone in the epilogue
#pragma unroll
                    for (int N = 0; N < 8; ++N) {
                        const int hN = N >> 2;
                        const uint32_t p0 = hN ? vr.w[k][0].y : vr.w[k][0].x;
                        const uint32_t p1 = hN ? vr.w[k][1].y : vr.w[k][1].x;
                        const uint32_t p2 = hN ? vr.w[k][2].y : vr.w[k][2].x;
                        acc[N] = mfma16(Pg[N >> 1], centred3x8(p0, p1, p2, N & 3), acc[N]);
                    }
                } else if constexpr (VU) {
                    const auto& vc = vr.vc;
#pragma unroll
                    for (int N = 0; N < 8; ++N) {
                        h8 Bv;
                        if (VB == 4)
                            Bv = as_h8(centred4(vc[k][N >> 2][N & 3]));
                        else
                            Bv = as_h8(centred8(vc[k][N >> 1][2 * (N & 1)], vc[k][N >> 1][2 * (N & 1) + 1]));
                        acc[N] = mfma16(Pg[N >> 1], Bv, acc[N]);
                    }
                } else if constexpr (VS) {
                    // channels 0..63 (N < 4) are the outlier subset's positions, 64..127 the rest's
#pragma unroll
                    for (int N = 0; N < 8; ++N) {
                        if (N < 4)
                            acc[N] = pv_planes<kBo>(Pg, vr.w[k], N & 3, acc[N]);
                        else
                            acc[N] = pv_planes<kBo - 1>(Pg + kSo, vr.w[k] + kBo, N & 3, acc[N]);
                    }
                } else if constexpr (VT4) {
                    // four planes; the cubic monomials are XORs of three (b_i b_j b_k = 2 (c_i ^
                    // c_j ^ c_k) - 1, an operand -b like the linear ones)
                    const uint32_t w0[2] = {vr.w[k][0].x, vr.w[k][0].y};
                    const uint32_t w1[2] = {vr.w[k][1].x, vr.w[k][1].y};
                    const uint32_t w2[2] = {vr.w[k][2].x, vr.w[k][2].y};
                    const uint32_t w3[2] = {vr.w[k][3].x, vr.w[k][3].y};
#pragma unroll
                    for (int N = 0; N < 8; ++N) {
                        const int hN = N >> 2, q = N & 3;
                        const uint32_t x01 = w0[hN] ^ w1[hN];
                        acc[N] = mfma16(Pg[0], as_h8(pm1x8(w0[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[1], as_h8(pm1x8(w1[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[2], as_h8(pm1x8(w2[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[3], as_h8(pm1x8(w3[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[4], as_h8(pm1x8(x01 ^ w2[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[5], as_h8(pm1x8(x01 ^ w3[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[6], as_h8(pm1x8(w0[hN] ^ w2[hN] ^ w3[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[7], as_h8(pm1x8(w1[hN] ^ w2[hN] ^ w3[hN], q)), acc[N]);
                    }
                } else {
                    // words: [plane 0, N<4], [plane 0, N>=4], [plane 1, ...], [plane 2, ...]
                    const uint32_t w0[2] = {vr.w[k][0].x, vr.w[k][0].y};
                    const uint32_t w1[2] = {vr.w[k][1].x, vr.w[k][1].y};
                    const uint32_t w2[2] = {vr.w[k][2].x, vr.w[k][2].y};
#pragma unroll
                    for (int N = 0; N < 8; ++N) {
                        const int hN = N >> 2, q = N & 3;
                        acc[N] = mfma16(Pg[0], as_h8(pm1x8(w0[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[1], as_h8(pm1x8(w1[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[2], as_h8(pm1x8(w2[hN], q)), acc[N]);
                        acc[N] = mfma16(Pg[3], as_h8(pm1x8(w0[hN] ^ w1[hN] ^ w2[hN], q)), acc[N]);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            if (more) load_v(vr, nci);
        };
        for (int ci = wave; ci < nch; ci += kBuf * kNW) {
            chunk(krs[0], vrs[0], ci);
            if (kBuf == 2 && ci + kNW < nch) chunk(krs[kBuf - 1], vrs[kBuf - 1], ci + kNW);
        }
        // reduce the per-lane softmax sums over each row of 16 lanes
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            l_run[mb] = row_sum16(l_run[mb]);
#pragma unroll
            for (int g = 0; g < 4; ++g) z_run[mb][g] = row_sum16(z_run[mb][g]);
        }
    } else {
        // ---------------- FP32 window (vector ALU): tokens nq .. n-1 ----------------
        // The window is spread over p.n_win_splits workgroups.  A wave takes 4 tokens at a time:
        // 16 lanes per token form its G scores (8 channels per lane, then a row reduction), the
        // four tokens update the running softmax, and every lane accumulates two channels of V.
        const int per_wg = (kWindowMax + p.n_win_splits - 1) / p.n_win_splits;
        const int wb = nq + (split - p.n_splits) * per_wg;
        const int we = min(n, wb + per_wg);
        for (int t4 = wb + 4 * wave; t4 < we; t4 += 4 * kNW) {
            const int tok = t4 + lq;
            const bool valid = tok < we;
            const float* krow = kring + (size_t)((valid ? tok : t4) % W) * kDim + 8 * lr;
            const float4 k0 = *reinterpret_cast<const float4*>(krow);
            const float4 k1 = *reinterpret_cast<const float4*>(krow + 4);
            float2 vv[4];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const int tt = min(t4 + tau, we - 1);
                vv[tau] = reinterpret_cast<const float2*>(vring + (size_t)(tt % W) * kDim)[l];
            }
#pragma unroll
            for (int h = 0; h < kMaxGroupHeads; ++h) {
                if (h >= G) continue;
                const float* qh = &s_qw[h][8 * lr];
                float d = k0.x * qh[0] + k0.y * qh[1] + k0.z * qh[2] + k0.w * qh[3] +
                          k1.x * qh[4] + k1.y * qh[5] + k1.z * qh[6] + k1.w * qh[7];
                d = row_sum16(d);
                const float sv = valid ? d : kNegInf;
                const float s0 = readlane_f(sv, 0), s1 = readlane_f(sv, 16), s2 = readlane_f(sv, 32),
                            s3 = readlane_f(sv, 48);
                const float mnew = fmaxf(wm[h], fmaxf(fmaxf(s0, s1), fmaxf(s2, s3)));
                const float a = (mnew == kNegInf) ? 1.0f : exp2f(wm[h] - mnew);
                const float p0 = (s0 == kNegInf) ? 0.0f : exp2f(s0 - mnew);
                const float p1 = (s1 == kNegInf) ? 0.0f : exp2f(s1 - mnew);
                const float p2 = (s2 == kNegInf) ? 0.0f : exp2f(s2 - mnew);
                const float p3 = (s3 == kNegInf) ? 0.0f : exp2f(s3 - mnew);
                wl[h] = wl[h] * a + ((p0 + p1) + (p2 + p3));
                wm[h] = mnew;
                wacc0[h] = fmaf(p3, vv[3].x, fmaf(p2, vv[2].x, fmaf(p1, vv[1].x, fmaf(p0, vv[0].x, wacc0[h] * a))));
                wacc1[h] = fmaf(p3, vv[3].y, fmaf(p2, vv[2].y, fmaf(p1, vv[1].y, fmaf(p0, vv[0].y, wacc1[h] * a))));
            }
        }
    }

    // ---------------- combine the waves of this workgroup ----------------
    if (!wsplit) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int h = 4 * mb + lq;
            if (lr == 0 && h < G) {
                s_wm[wave][h] = m_run[mb];
                s_wl[wave][h] = l_run[mb];
#pragma unroll
                for (int g = 0; g < 4; ++g) s_wz[wave][h][g] = VU ? z_run[mb][g] : 0.0f;
            }
        }
    } else if (l == 0) {
        for (int h = 0; h < G; ++h) {
            s_wm[wave][h] = wm[h];
            s_wl[wave][h] = wl[h];
#pragma unroll
            for (int g = 0; g < 4; ++g) s_wz[wave][h][g] = 0.0f;
        }
    }
    __syncthreads(); // every wave is done with its staging area: reuse it for the accumulators
    float* s_acc = reinterpret_cast<float*>(s_p);  // [kNW][8][128], fp16-hi rows / window
    float* s_acc2 = s_acc + kNW * 8 * kDim;         // [kNW][8][128], fp16-lo rows
    if (!wsplit) {
#pragma unroll
        for (int N = 0; N < 8; ++N) {
            const float u = V3 ? ((N & 1) ? 0.0625f : 1.0f) : (VU ? UV : 1.0f);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                // rows 4 lq + v: head 4 (lq % 2) + v, hi part for lq < 2 (compact: head v, hi for
                // lq = 0, lo for lq = 1, nothing in rows 8-15)
                const int h = kCmp ? v : 4 * (lq & 1) + v;
                const bool lo_part = kCmp ? (lq == 1) : (lq >= 2);
                if (h < G && (!kCmp || lq < 2)) {
                    if (!lo_part)
                        s_acc[(wave * 8 + h) * kDim + 16 * N + lr] = acc[N][v] * u;
                    else
                        s_acc2[(wave * 8 + h) * kDim + 16 * N + lr] = acc[N][v] * u;
                }
            }
        }
    } else {
        for (int h = 0; h < G; ++h) {
            s_acc[(wave * 8 + h) * kDim + 2 * l] = wacc0[h];
            s_acc[(wave * 8 + h) * kDim + 2 * l + 1] = wacc1[h];
            s_acc2[(wave * 8 + h) * kDim + 2 * l] = 0.0f;
            s_acc2[(wave * 8 + h) * kDim + 2 * l + 1] = 0.0f;
        }
    }
    __syncthreads();
    const float2 cs2 = wsplit ? make_float2(1.0f, 1.0f) : s_vmap[0][l];
    const float2 sg2 = wsplit ? make_float2(1.0f, 1.0f) : s_vmap[1][l];
    const int2 pm2 = wsplit ? make_int2(2 * l, 2 * l + 1) : s_vperm[l];
    // partial of this split for each of its query heads, [b][hq][split][m, l, -, -, acc[128]], in
    // the plain channel domain: one wave per head, lane l the channel pair 2l, 2l + 1 (code-domain
    // positions, mapped back by the value plane's output map; the FP32-window split is plain)
    for (int h = wave; h < G; h += kNW) {
        float M = kNegInf;
        for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_wm[w][h]);
        float A0 = 0.0f, A1 = 0.0f, L = 0.0f;
        if (M != kNegInf) {
            for (int w = 0; w < kNW; ++w) {
                if (s_wm[w][h] == kNegInf) continue;
                const float f = exp2f(s_wm[w][h] - M);
                const int o = (w * 8 + h) * kDim + 2 * l;
                const float z = s_wz[w][h][l >> 4];
                A0 = fmaf(f, (s_acc[o] + s_acc2[o]) + z, A0);
                A1 = fmaf(f, (s_acc[o + 1] + s_acc2[o + 1]) + z, A1);
                L = fmaf(f, s_wl[w][h], L);
            }
        }
        if (!wsplit) value_out_map(A0, A1, VS, VG.sinkhorn, VG.rotate, cs2, sg2);
        float* part = p.partials + (((size_t)b * p.Hq + kvh * G + h) * p.n_splits_total + split) * kPartialFloats;
        part[4 + pm2.x] = A0;
        part[4 + pm2.y] = A1;
        if (l == 0) {
            part[0] = M;
            part[1] = L;
        }
    }
}

template <int KT, int VT, int MB>
hipError_t launch_t(const DecodeParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    // 8 waves where registers allow (the 4-bit and split TurboQuant V stage 8 or 12 P slots, in
    // the compact 8-row form with one head block)
    constexpr int NW = (MB == 1 && !(KT == kU8 && VT == kU8)) ? 8 : 4;
    dim3 grid(p.n_splits_total, p.Hkv, p.batch);
    hipExtLaunchKernelGGL((decode_mfma_kernel<KT, VT, MB, NW>), grid, dim3(NW * 64), 0, s, ev0, ev1, 0, p);
    return hipGetLastError();
}

template <int KT, int VT>
hipError_t launch_mb(const DecodeParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    return p.G > 4 ? launch_t<KT, VT, 2>(p, s, ev0, ev1) : launch_t<KT, VT, 1>(p, s, ev0, ev1);
}

template <int KT>
hipError_t launch_v(const DecodeParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const PlaneGeom& V = p.geom[1];
    if (V.scheme == kTurboSplit)
        return V.bits == 4 ? launch_mb<KT, kTs4>(p, s, ev0, ev1) : launch_mb<KT, kTs3>(p, s, ev0, ev1);
    if (V.scheme != kUniform) return V.bits == 4 ? launch_mb<KT, kTb4>(p, s, ev0, ev1) : launch_mb<KT, kTb>(p, s, ev0, ev1);
    if (V.bits == 3) return launch_mb<KT, kU3>(p, s, ev0, ev1);
    return V.bits == 4 ? launch_mb<KT, kU4>(p, s, ev0, ev1) : launch_mb<KT, kU8>(p, s, ev0, ev1);
}

} // namespace

bool mfma_path_supported(const DecodeParams& p) {
    const PlaneGeom& K = p.geom[0];
    const PlaneGeom& V = p.geom[1];
    const bool k_ok = (K.scheme == kUniform && (K.bits == 3 || K.bits == 4 || K.bits == 8)) || K.scheme == kTurboQjl ||
                      (K.scheme == kTurboSplit && (K.bits == 3 || K.bits == 4));
    const bool v_ok = (V.scheme == kUniform && (V.bits == 3 || V.bits == 4 || V.bits == 8)) || V.scheme == kTurboMse ||
                      (V.scheme == kTurboSplit && (V.bits == 3 || V.bits == 4));
    return k_ok && v_ok && p.G <= kMaxGroupHeads;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const PlaneGeom& K = p.geom[0];
    if (K.scheme == kTurboSplit) return K.bits == 4 ? launch_v<kSk4>(p, s, ev0, ev1) : launch_v<kSk3>(p, s, ev0, ev1);
    if (K.scheme != kUniform) return launch_v<kTb>(p, s, ev0, ev1);
    if (K.bits == 3) return launch_v<kU3>(p, s, ev0, ev1);
    return K.bits == 4 ? launch_v<kU4>(p, s, ev0, ev1) : launch_v<kU8>(p, s, ev0, ev1);
}

} // namespace kvq
