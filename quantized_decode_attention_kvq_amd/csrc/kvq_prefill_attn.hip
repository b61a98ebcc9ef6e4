// Multi-query attention of a prefill chunk over the compressed cache, gfx950 matrix cores.
//
// What it computes (pages by title and section):
//  * quantcpp article "Beyond RAG...", v3.2 batched prefill: a prompt is processed as whole
//    chunks.  Here the n_q newest tokens of each sequence (already appended to the cache) are the
//    chunk's queries; query i, at position pos_i = len - n_q + i, attends to the cache as it
//    stands, up to its own position: out_i = softmax(q_i k_t^T * scale | t <= pos_i) v.
//  * quantcpp article, progressive table and "how it works" (4-bit codes with fp16 scale and
//    zero per 32 channels), and the KVarN post, TL;DR (Walsh-Hadamard + Sinkhorn-balanced
//    cache): keys and values are the dequantized uniform codes (the newest 128 tokens from the
//    FP32 window in progressive mode); scores are taken in the rotated / balanced domain with
//    q' = R(q) .* c, and the output is mapped back with c_V and R_V^-1.
//  * "LLM memory saving ... 2026", TurboQuant row and application rules (K = Q8, V = TurboQuant),
//    with the outlier split of its 2.5 / 3.5-bit figures: values may be TurboQuant-MSE codes,
//    n mu[code] in the rotated domain (two 64-channel halves for the split).  Keys may be
//    TurboQuant-QJL codes (same row, 1-bit QJL for an unbiased inner product): the score of key t
//    is n_t <rho_q, mu[code_t]> + gamma_t sqrt(pi/2) / 128 sum_i (2 b_ti - 1) (S rho_q)_i with
//    rho_q = R(q), i.e. a 256-long contraction of [n mu[code], f_t signs] with [rho_q, S rho_q].
//
// How.  The (query, head) pairs of one (sequence, kv head) are rows r = G * i + h (query i,
// query head h of the kv head's group).  A workgroup of 8 waves owns 128 consecutive rows (16 per
// wave, one 16-row MFMA column block) and one share of the key chunks up to its last row's
// position ("split"; the host picks the number of splits from a cost model).  Per 64-token
// chunk:
//  * the workgroup dequantizes the chunk's keys and values (z + s * code in fp32) into LDS as
//    fp16 pairs (hi = the value rounded, lo = the remainder rounded), once for its 128 rows,
//    while the waves work on the previous chunk (two LDS buffers, global loads one chunk ahead);
//  * each wave forms the transposed scores S^T = K q'^T on v_mfma_f32_16x16x32_f16 with three
//    products per slice (K_hi q_hi, K_hi q_lo, K_lo q_hi: close to fp32 accuracy);
//    key rows are ordered in LDS so that each lane's score values are exactly the P^T operand
//    of the PV product, which therefore never leaves the registers;
//  * an online softmax per row in the log2 domain (tokens after the row's position are masked),
//    then O^T += V_hi^T P^T + V_lo^T P^T (values as the A operand, fp16 weights as B; the
//    softmax sum adds the same fp16 weights).
// With one split, each row's output is divided by its softmax sum and mapped back with c_V and
// R_V^-1 in the same kernel; with several, each split writes (m, l, acc) and a merge kernel
// combines them in a fixed order.
// TurboQuant-QJL keys: the key rows hold n mu[code] (hi, lo) like any dequantized key; the QJL
// signs stay in LDS as their 16-byte words, and each lane expands its eight signs of a k-slice
// into the A operands +-f_t hi and lo (f_t = gamma_t sqrt(pi/2) / 128 per key row) against
// S q' as fp16 hi and lo, three more products per slice accumulated with the others.
// FP32 window: in the plain domain the window tokens' original values overwrite their LDS units
// in the dequantizer's own thread mapping; beside rotated or balanced codes, a chunk holding
// window tokens gets one more barrier after which each wave maps whole window tokens into the
// code domain (R(x) .* 1/c for uniform planes, R(x) for TurboQuant, the two 64-point rotations
// of the permuted channels for a split V) before writing them, and their QJL scale f_t is zero.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_lanes.h"
#include "kvq_mfma_ops.h"
#include "kvq_quant_dev.h"

namespace kvq {
namespace {

using namespace mops;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazy = 8.0f; // log2 headroom of the running softmax maximum
constexpr int kQB = 1;                            // 16-row column blocks per wave
constexpr int kWaveRows = 16 * kQB;
constexpr int kWaves = kPrefillRowsPerBlock / kWaveRows;
constexpr int kThreads = 64 * kWaves;
// Row pitches (halves) of the dequantized chunk: 144 and 80 halves put the rows that one
// ds_read_b128 gathers (16 rows, 16 B each, four column offsets) on disjoint banks; measured on
// gfx950, pitches of 136 / 72 halves cost about 3 conflict cycles per read.
constexpr int kKS = 144; // key row: 128 channels + pad
constexpr int kVS = 80;  // value row: 64 tokens + pad
constexpr int kKBuf = 2 * 64 * kKS;               // one chunk's keys: 64 hi rows, then 64 lo rows
constexpr int kVBuf = 2 * 128 * kVS;              // one chunk's values [channel][token]: hi, lo
constexpr int kLdsHalves = 2 * (kKBuf + kVBuf);   // two buffers of each
constexpr int kVmRow = 80;                        // value meta row, fp16 (64 tokens + pad: the
                                                  // groups on different banks)
constexpr int kUnits = 64 * 16 / kThreads;        // 8-code units of a chunk per thread (K; V alike)
static_assert(kWaves == 8, "two waves per SIMD");
static_assert(kUnits * kThreads == 1024, "a chunk is 1024 key units and 1024 value units");
static_assert(kLdsHalves * 2 >= 2 * kWaves * 16 * kDim * 4, "the q' rows and the S q' rows fit in the chunk buffers");

// LDS row of chunk token t (0..63) in the key buffer.  Score tile b (16 key rows) holds at row
// 4u + v the token 32 (b / 2) + 8u + 4 (b % 2) + v, so that a lane's four score values of tile
// 2k and its four of tile 2k + 1 are tokens 32k + 8u .. 32k + 8u + 7: the lane's B operand of the
// PV product over the chunk's k-th 32 tokens.
__device__ __forceinline__ int key_lds_row(int t) {
    return 16 * (2 * (t >> 5) + ((t >> 2) & 1)) + 4 * ((t >> 3) & 3) + (t & 3);
}

// Prefetched global words of one chunk: kUnits key units (8 codes + their group's scale and
// zero), kUnits value units (8 codes), and one token's value meta (threads 0..63).
struct ChunkRegs {
    uint2 kc[kUnits], vc[kUnits];
    uint32_t kc3[kUnits]; // 3-bit keys: the third plane word of the unit's group
    uint32_t ks[kUnits], kz[kUnits]; // fp16 bits of the key unit's scale and zero (QJL: n, gamma)
    uint32_t kq;          // QJL keys: one sign word of the chunk (threads 0..255)
    u4 vm;
};

struct Planes {
    const uint8_t *kcodes, *kmeta, *kqjl, *vcodes, *vmeta;
};

// Key kinds: KB = 4 or 8 (uniform codes), 3 (uniform 3-bit codes as three bit planes in the
// TurboQuant 3-bit K row layout), or kQjlK (TurboQuant-QJL: 3-bit Lloyd-Max codes in that row
// layout, fp16 n and gamma per row, 16 bytes of QJL signs per row).
constexpr int kQjlK = -3;
// Split keys at b = 3 or 4 (kSplitK - b): per-group plane words (b - 1 planes on groups 0, 1,
// b - 2 on groups 2, 3) in a split_k_row_bytes(b) row, fp16 n_outlier, n_rest, gamma per row,
// and the QJL signs of a TurboQuant key.
constexpr int kSplitK = -20;
__host__ __device__ constexpr bool split_k_kind(int kb) { return kb <= kSplitK - 3 && kb >= kSplitK - 4; }
__host__ __device__ constexpr int split_k_bits(int kb) { return kSplitK - kb; }
constexpr float kKappa = 0.0097915166977774f; // sqrt(pi/2) / 128
// Value kinds: VB = 4 or 8 (uniform codes), 3 (uniform 3-bit codes as three bit planes in the
// TurboQuant-MSE V layout, read by TurboQuant value units), -b for TurboQuant-MSE V with b = 3 or
// 4 bit planes,
// or kSplitV - bo for the split TurboQuant V with bo = 3 or 4 outlier bits (channel quads
// N / 4 = 0 are the outlier half's positions, bo planes; N / 4 = 1 the rest's, bo - 1 planes).
// A TurboQuant value unit is one thread's (block half, octet kb, lane column n, channel quad
// N / 4, token parity): the b plane words of (kb, n, N / 4), whose nibble 4 (N % 4) of the
// half-word of that parity holds tokens par, par + 2, par + 4, par + 6 of the octet.
constexpr int kSplitV = -10;
__host__ __device__ constexpr bool split_kind(int vb) { return vb <= kSplitV; }

// Thread -> TurboQuant value unit: token parity in lane bit 0 (the swap partner is lane ^ 1),
// lane column n in bits 1-4, octet kb in bits 5-6, channel quad N / 4 in bit 7 and block half in
// bit 8, so that the quad (and with it a split V's half and codebook) is uniform per wave.
struct TUnit {
    int half, kb, n, hN, par;
};
__device__ __forceinline__ TUnit turbo_unit(int tid) {
    return TUnit{tid >> 8, (tid >> 5) & 3, (tid >> 1) & 15, (tid >> 7) & 1, tid & 1};
}

template <int KB, int VB>
__device__ __forceinline__ void load_codes(const Planes& P, int ci, int tid, ChunkRegs& R) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
        const int u = tid + kThreads * j, g = (u >> 2) & 3, word = 4 * (u & 3) + g;
        const size_t row = (size_t)64 * ci + (u >> 4);
        if constexpr (split_k_kind(KB)) {
            // the plane words of position group g (planes beyond the group's count read as 0)
            constexpr int B = split_k_bits(KB);
            const uint32_t* pw = reinterpret_cast<const uint32_t*>(P.kcodes + row * split_k_row_bytes(B)) +
                                 split_k_group_word(g, B);
            const int nb = g < 2 ? B - 1 : B - 2;
            R.kc[j].x = pw[0];
            R.kc[j].y = nb > 1 ? pw[1] : 0u;
            R.kc3[j] = nb > 2 ? pw[2] : 0u;
        } else if constexpr (KB == 3 || KB == kQjlK) {
            // the three plane words of group g (the unit's codes are their nibble u % 4)
            const uint32_t* pw = reinterpret_cast<const uint32_t*>(P.kcodes + row * 48 + 12 * g);
            R.kc[j].x = pw[0];
            R.kc[j].y = pw[1];
            R.kc3[j] = pw[2];
        } else if constexpr (KB == 4) R.kc[j].x = reinterpret_cast<const uint32_t*>(P.kcodes + row * 64)[word];
        else R.kc[j] = reinterpret_cast<const uint2*>(P.kcodes + row * 128)[word];
        if constexpr (KB == kQjlK) {
            const uint16_t* m = reinterpret_cast<const uint16_t*>(P.kmeta + row * 4);
            R.ks[j] = m[0]; // n
            R.kz[j] = m[1]; // gamma
        } else if constexpr (split_k_kind(KB)) {
            const uint16_t* m = reinterpret_cast<const uint16_t*>(P.kmeta + row * 8);
            R.ks[j] = m[g < 2 ? 0 : 1]; // the half's norm
            R.kz[j] = m[2];             // gamma
        } else {
            const uint16_t* m = reinterpret_cast<const uint16_t*>(P.kmeta + row * 16);
            R.ks[j] = m[g]; // kept apart until the dequantization: no wait on the load here
            R.kz[j] = m[4 + g];
        }
    }
    if constexpr (KB == kQjlK || split_k_kind(KB)) {
        // sign word tid % 4 of physical row tid / 4
        if (tid < 256) R.kq = reinterpret_cast<const uint32_t*>(P.kqjl + ((size_t)64 * ci + (tid >> 2)) * 16)[tid & 3];
    }
    if constexpr (split_kind(VB)) {
        constexpr int BO = kSplitV - VB, W = 2 * BO - 1;
        const TUnit U = turbo_unit(tid);
        const int hN = U.hN;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(P.vcodes + ((size_t)2 * ci + U.half) * (256 * W)) +
                            W * (16 * U.kb + U.n) + (hN ? BO : 0);
        const int nb = hN ? BO - 1 : BO;
        R.vc[0].x = w[0];
        R.vc[0].y = w[1];
        R.vc[1].x = (nb > 2) ? w[2] : 0u;
        R.vc[1].y = (nb > 3) ? w[3] : 0u;
    } else if constexpr (VB < 0 || VB == 3) {
        constexpr int NB = VB == 3 ? 3 : -VB;
        const TUnit U = turbo_unit(tid);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(P.vcodes + ((size_t)2 * ci + U.half) * (512 * NB)) +
                            2 * NB * (16 * U.kb + U.n) + U.hN;
        R.vc[0].x = w[0];
        R.vc[0].y = w[2];
        R.vc[1].x = w[4];
        R.vc[1].y = (NB == 4) ? w[6] : 0u;
    } else {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int u = tid + kThreads * j;
            const size_t blk = (size_t)2 * ci + (u >> 9);
            if constexpr (VB == 4) R.vc[j].x = reinterpret_cast<const uint32_t*>(P.vcodes + blk * 2048)[u & 511];
            else R.vc[j] = reinterpret_cast<const uint2*>(P.vcodes + blk * 4096)[u & 511];
        }
    }
}

template <int VB>
__device__ __forceinline__ void load_vmeta(const Planes& P, int ci, int tid, ChunkRegs& R) {
    if constexpr (split_kind(VB)) {
        if (tid < 64) R.vm.x = reinterpret_cast<const uint32_t*>(P.vmeta)[(size_t)64 * ci + tid]; // two fp16 norms
    } else if constexpr (VB < 0) {
        if (tid < 64) R.vm.x = reinterpret_cast<const uint16_t*>(P.vmeta)[(size_t)64 * ci + tid]; // fp16 norm
    } else {
        if (tid < 64) R.vm = *reinterpret_cast<const u4*>(P.vmeta + ((size_t)64 * ci + tid) * 16);
    }
}

// value meta of one chunk -> sm[scale | zero][group][token] (fp16); TurboQuant: sm[0][0][token]
// = the token's norm; split: sm[0][0 | 1][token] = the outlier / rest norm
template <int VB>
__device__ __forceinline__ void store_vmeta(_Float16 (*sm)[4][kVmRow], int tid, const ChunkRegs& R) {
    if constexpr (split_kind(VB)) {
        if (tid < 64) {
            sm[0][0][tid] = __builtin_bit_cast(_Float16, (uint16_t)(R.vm.x & 0xffffu));
            sm[0][1][tid] = __builtin_bit_cast(_Float16, (uint16_t)(R.vm.x >> 16));
        }
    } else if constexpr (VB < 0) {
        if (tid < 64) sm[0][0][tid] = __builtin_bit_cast(_Float16, (uint16_t)R.vm.x);
    } else if (tid < 64) {
        const uint32_t w[4] = {R.vm.x, R.vm.y, R.vm.z, R.vm.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const h2v v = __builtin_bit_cast(h2v, w[k]);
            sm[k >> 1][2 * (k & 1)][tid] = v[0];
            sm[k >> 1][2 * (k & 1) + 1][tid] = v[1];
        }
    }
}

// Codes 2k and 2k + 1 of an 8-code unit as exact fp16 integers: each code is placed in the
// mantissa of 1024 (bits 0x6400 | c) and 1024 is subtracted with one packed fp16 add.
template <int BITS>
__device__ __forceinline__ h2v code_pair(uint2 w, int k) {
    uint32_t b;
    if constexpr (BITS == 4) {
        b = ((w.x >> (4 * k)) & 0x000F000Fu) | 0x64006400u; // codes at bits 4k and 16 + 4k
    } else {
        const uint32_t src = (k < 2) ? w.x : w.y;          // codes at bytes 2k and 2k + 1
        b = __builtin_amdgcn_perm(0x64646464u, src, (k & 1) ? 0x04030402u : 0x04010400u);
    }
    return __builtin_bit_cast(h2v, b) - h2v{(_Float16)1024.0f, (_Float16)1024.0f};
}

// Codes 2k and 2k + 1 of nibble kb of three half-interleaved plane words (bits 4 kb + k and
// 16 + 4 kb + k) as exact fp16 integers, the same way.
__device__ __forceinline__ h2v code_pair3(uint32_t p0, uint32_t p1, uint32_t p2, int kb, int k) {
    const int sh = 4 * kb + k;
    const uint32_t b = ((p0 >> sh) & 0x00010001u) | (((p1 >> sh) & 0x00010001u) << 1) |
                       (((p2 >> sh) & 0x00010001u) << 2) | 0x64006400u;
    return __builtin_bit_cast(h2v, b) - h2v{(_Float16)1024.0f, (_Float16)1024.0f};
}

// y = s c + z for a pair: hi = fp16 of y in one rounding (packed fp16 fma), lo = fp16(y - hi)
// with y - hi formed in fp32.
struct Pair {
    uint32_t hi, lo;
};
__device__ __forceinline__ Pair dequant_pair(h2v s, h2v c, h2v z, float mone) {
    const h2v h = __builtin_elementwise_fma(s, c, z);
    h2v r;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float y = fmaf((float)s[e], (float)c[e], (float)z[e]);
        r[e] = (_Float16)fmaf((float)h[e], mone, y); // mixed fp16 / fp32 fma, rounded once to fp16
    }
    return Pair{__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, r)};
}

// Dequantize the prefetched chunk into one key buffer and one value buffer.
//  key unit u: physical row p = u / 16 (token 4 (p % 16) + p / 16 of the chunk), w = u % 16 =
//    4 g + kb: code word 4 kb + g, channels 32 g + 8 kb + i (so consecutive lanes fill
//    consecutive 16 B of the LDS row);
//  value unit u: 32-token block u / 512, word w = u % 512 = 8 (16 kb + n) + N (channel
//    d = 16 N + n, tokens 8 kb + i of the block).  Value rows [channel][token] store the 8-token
//    slot s at slot s ^ (d / 16), which keeps both these writes and the operand reads free of
//    bank conflicts.
// Centroid of a b-bit TurboQuant code from the upper half of its odd-symmetric codebook
// (mg[j] = mu[2^(b-1) + j]): mu[c] = mg[c - h] for c >= h, -mg[h - 1 - c] below.
template <int NB>
__device__ __forceinline__ float centroid(uint32_t c, const float* mg) {
    constexpr uint32_t H = 1u << (NB - 1);
    const bool up = (c & H) != 0;
    const uint32_t j = (c & (H - 1)) ^ (up ? 0u : H - 1);
    float a = (j & 1) ? mg[1] : mg[0];
    float b = (j & 1) ? mg[3] : mg[2];
    float m = (j & 2) ? b : a;
    if constexpr (NB == 4) {
        const float e = (j & 1) ? mg[5] : mg[4];
        const float f = (j & 1) ? mg[7] : mg[6];
        const float g = (j & 2) ? f : e;
        m = (j & 4) ? g : m;
    }
    return up ? m : -m;
}

// z + s code for the 4 channels x 4 tokens of a 3-bit uniform value unit (the TurboQuant value
// unit mapping): v[q][m] = channel 16 (4 hN + q) + n, token t0 + 2m + par, with the fp16 scale
// and zero of the channel's group from sm[scale | zero][group][token].
__device__ __forceinline__ void uniform3_values(const uint32_t* wd, const _Float16 (*sm)[4][kVmRow], int t0, int hN,
                                                int par, float (&v)[4][4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int t = t0 + 2 * m + par;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int g = 2 * hN + (q >> 1), sh = 16 * par + 4 * q + m;
            const uint32_t c = ((wd[0] >> sh) & 1u) | (((wd[1] >> sh) & 1u) << 1) | (((wd[2] >> sh) & 1u) << 2);
            v[q][m] = fmaf((float)sm[0][g][t], (float)c, (float)sm[1][g][t]);
        }
    }
}

// n_t mu[code] for the 4 channels x 4 tokens of a TurboQuant value unit: v[q][m] = channel quad
// q, token 2m + par of the octet; NB-bit codes from the plane words wd, norms from nrm[token].
template <int NB>
__device__ __forceinline__ void turbo_values(const uint32_t* wd, const _Float16* nrm, const float* mg, int par,
                                             float (&v)[4][4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float nt = (float)nrm[2 * m + par];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int sh = 16 * par + 4 * q + m;
            uint32_t c = 0;
#pragma unroll
            for (int k = 0; k < NB; ++k) c |= ((wd[k] >> sh) & 1u) << k;
            v[q][m] = nt * centroid<NB>(c, mg);
        }
    }
}

// QJL and split keys: the (up to) 3-bit code of each of a key unit's elements 2k, 2k + 1 (bits
// 4 kb + k and 16 + 4 kb + k of the plane words; missing planes are 0)
__device__ __forceinline__ uint32_t code3_at(uint32_t p0, uint32_t p1, uint32_t p2, int sh) {
    return ((p0 >> sh) & 1u) | (((p1 >> sh) & 1u) << 1) | (((p2 >> sh) & 1u) << 2);
}

// Centroid of an nb-bit code (nb = 1, 2 or 3, known at run time) from the upper half of its
// odd-symmetric codebook (mg[j] = mu[2^(nb-1) + j], unused entries ignored).
__device__ __forceinline__ float centroid_rt(uint32_t c, int nb, const float* mg) {
    const uint32_t H = 1u << (nb - 1);
    const bool up = (c & H) != 0;
    const uint32_t j = (c & (H - 1)) ^ (up ? 0u : H - 1);
    const float a = (j & 1) ? mg[1] : mg[0];
    const float b = (j & 1) ? mg[3] : mg[2];
    const float m = (j & 2) ? b : a;
    return up ? m : -m;
}

template <int KB, int VB>
__device__ __forceinline__ void dequant_chunk(_Float16* sk, _Float16* sv, const _Float16 (*sm)[4][kVmRow], int tid,
                                              const ChunkRegs& R, const float* mg, const float* mgk, uint32_t* ssg,
                                              uint32_t* sf) {
    // -1 in a register the compiler cannot see through: hi * (-1) + y stays one mixed-precision
    // fma (v_fma_mix*) instead of being rewritten as a conversion and a subtraction
    float mone = -1.0f;
    asm volatile("" : "+v"(mone));
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
        const int u = tid + kThreads * j, p = u >> 4, w = u & 15;
        const int t = 4 * (p & 15) + (p >> 4);
        const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)R.ks[j]);
        const _Float16 zr = __builtin_bit_cast(_Float16, (uint16_t)R.kz[j]);
        u4 hi, lo;
        if constexpr (KB == kQjlK || split_k_kind(KB)) {
            // n mu[code] in fp32, then fp16 hi + remainder lo; the row's first unit writes f_t.
            // Split keys: the unit's position group g picks the half (norm loaded per unit), its
            // code width and its codebook (mgk[0..3] outliers, mgk[4..7] the rest)
            const float n = (float)sc;
            int nb = 3;
            float mgu[4] = {mgk[0], mgk[1], mgk[2], mgk[3]};
            if constexpr (split_k_kind(KB)) {
                constexpr int B = split_k_bits(KB);
                const bool out = ((u >> 2) & 3) < 2;
                nb = out ? B - 1 : B - 2;
#pragma unroll
                for (int i = 0; i < 4; ++i) mgu[i] = out ? mgk[i] : mgk[4 + i];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int sh = 4 * (u & 3) + k;
                float ye = n * centroid_rt(code3_at(R.kc[j].x, R.kc[j].y, R.kc3[j], sh), nb, mgu);
                float yo = n * centroid_rt(code3_at(R.kc[j].x, R.kc[j].y, R.kc3[j], sh + 16), nb, mgu);
                // the products are rounded to fp32 once, here: with contraction the compiler may
                // otherwise take hi from the fp32 product and lo from the exact one, which differ
                // by one fp16 ulp where the fp32 product is an fp16 tie
                asm volatile("" : "+v"(ye), "+v"(yo));
                const h2v h = h2v{(_Float16)ye, (_Float16)yo};
                const h2v r = h2v{(_Float16)(ye - (float)h[0]), (_Float16)(yo - (float)h[1])};
                hi[k] = __builtin_bit_cast(uint32_t, h);
                lo[k] = __builtin_bit_cast(uint32_t, r);
            }
            if (w == 0) {
                const float f = (float)zr * kKappa;
                const _Float16 fh = (_Float16)f, fl = (_Float16)(f - (float)fh);
                sf[key_lds_row(t)] = (uint32_t)__builtin_bit_cast(uint16_t, fh) |
                                     ((uint32_t)__builtin_bit_cast(uint16_t, fl) << 16);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                h2v c;
                if constexpr (KB == 3) c = code_pair3(R.kc[j].x, R.kc[j].y, R.kc3[j], u & 3, k);
                else c = code_pair<KB>(R.kc[j], k);
                const Pair q = dequant_pair(h2v{sc, sc}, c, h2v{zr, zr}, mone);
                hi[k] = q.hi;
                lo[k] = q.lo;
            }
        }
        _Float16* dst = sk + key_lds_row(t) * kKS + 8 * w; // channels 32 (w / 4) + 8 (w % 4) + i
        *reinterpret_cast<u4*>(dst) = hi;
        *reinterpret_cast<u4*>(dst + 64 * kKS) = lo;
    }
    if constexpr (KB == kQjlK || split_k_kind(KB)) {
        if (tid < 256) {
            const int p = tid >> 2, t = 4 * (p & 15) + (p >> 4);
            ssg[4 * key_lds_row(t) + (tid & 3)] = R.kq;
        }
    }
    if constexpr (VB < 0 || VB == 3) {
        // TurboQuant-MSE values n_t mu[code] (fp32 product), or 3-bit uniform values z + s c
        // (one fp32 fma), then fp16 hi + remainder lo.  The
        // two parity threads of a unit (adjacent lanes) swap halves so that each ends up with two
        // whole channels of the octet: channels 4 hN + 2 par + {0, 1}.
        // split V: the thread's half (hN) fixes its norm row, code bits and codebook (mg holds
        // the outlier table in 0..7 and the rest's in 8..11)
        constexpr bool SPL = split_kind(VB);
        constexpr int NB = SPL ? kSplitV - VB : (VB == 3 ? 3 : -VB);
        const TUnit U = turbo_unit(tid);
        const int half = U.half, kb = U.kb, n = U.n, hN = U.hN, par = U.par;
        const uint32_t wd[4] = {R.vc[0].x, R.vc[0].y, R.vc[1].x, R.vc[1].y};
        const int t0 = 32 * half + 8 * kb;
        float v[4][4]; // [channel quad q][token pair m]: token 2m + par
        if constexpr (VB == 3)
            uniform3_values(wd, sm, t0, hN, par, v);
        else if (SPL && hN) // the rest half of a split V (uniform per wave): one bit fewer, own table
            turbo_values<(SPL ? NB - 1 : NB)>(wd, &sm[0][1][t0], mg + 8, par, v);
        else
            turbo_values<NB>(wd, &sm[0][0][t0], mg, par, v);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            float tok[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float keep = par ? v[2 + qq][m] : v[qq][m];  // this thread's channel
                const float give = par ? v[qq][m] : v[2 + qq][m];  // the partner's channel
                const float got = xor_lane<1>(give);
                tok[2 * m] = par ? got : keep;
                tok[2 * m + 1] = par ? keep : got;
            }
            h8 hi, lo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float y = tok[i];
                asm volatile("" : "+v"(y)); // one fp32 value for hi and lo (see the QJL keys)
                const _Float16 h = (_Float16)y;
                hi[i] = h;
                lo[i] = (_Float16)(y - (float)h);
            }
            const int N = 4 * hN + 2 * par + qq, d = 16 * N + n;
            _Float16* dst = sv + d * kVS + 8 * ((4 * half + kb) ^ N);
            *reinterpret_cast<h8*>(dst) = hi;
            *reinterpret_cast<h8*>(dst + 128 * kVS) = lo;
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
        const int u = tid + kThreads * j, half = u >> 9, w = u & 511;
        const int kb = w >> 7, n = (w >> 3) & 15, N = w & 7, d = 16 * N + n, g = N >> 1;
        const int t0 = 32 * half + 8 * kb;
        const u4 sw = *reinterpret_cast<const u4*>(&sm[0][g][t0]);
        const u4 zw = *reinterpret_cast<const u4*>(&sm[1][g][t0]);
        u4 hi, lo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // bit_cast a named scalar: clang's bit_cast of an ext_vector element reads element 0
            const uint32_t s2 = sw[k], z2 = zw[k];
            const Pair q = dequant_pair(__builtin_bit_cast(h2v, s2), code_pair<VB>(R.vc[j], k),
                                        __builtin_bit_cast(h2v, z2), mone);
            hi[k] = q.hi;
            lo[k] = q.lo;
        }
        _Float16* dst = sv + d * kVS + 8 * ((4 * half + kb) ^ N);
        *reinterpret_cast<u4*>(dst) = hi;
        *reinterpret_cast<u4*>(dst + 128 * kVS) = lo;
    }
}

// FP32 window (progressive caches): tokens nqd .. len - 1 of the chunk take their original
// values (in the code domain: the rings themselves, or their mapped copies) instead of the codes.
// Each thread rewrites exactly the LDS units it dequantized (same unit mapping, so program order
// makes the ring values final); a value unit straddling nqd keeps its dequantized tokens below
// it.  A QJL key's scale f_t becomes 0: its signs carry no estimate for a window token.
template <int KB, int VB>
__device__ __forceinline__ void window_overwrite(_Float16* sk, _Float16* sv, uint32_t* sf, int chunk, int nqd,
                                                 int len, int W, const float* kring, const float* vring, int tid) {
    if (W == 0 || 64 * chunk + 63 < nqd || 64 * chunk >= len) return;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
        const int u = tid + kThreads * j, pr = u >> 4, w = u & 15;
        const int t = 4 * (pr & 15) + (pr >> 4), tok = 64 * chunk + t;
        if (tok < nqd || tok >= len) continue;
        const float4* r = reinterpret_cast<const float4*>(kring + (size_t)(tok % W) * kDim + 8 * w);
        const float4 a = r[0], c = r[1];
        const float y[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        h8 hi, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 h = (_Float16)y[i];
            hi[i] = h;
            lo[i] = (_Float16)(y[i] - (float)h);
        }
        _Float16* dst = sk + key_lds_row(t) * kKS + 8 * w;
        *reinterpret_cast<h8*>(dst) = hi;
        *reinterpret_cast<h8*>(dst + 64 * kKS) = lo;
        if constexpr (KB == kQjlK || split_k_kind(KB)) {
            if (w == 0) sf[key_lds_row(t)] = 0u;
        }
    }
    if constexpr (VB == 3 || VB < 0) {
        // 3-bit uniform, TurboQuant and split values were dequantized by TurboQuant value units:
        // the thread rewrites its own two channel (split: position) slots, 16 (4 hN + 2 par + qq)
        // + n, tokens t0 .. t0 + 7
        const TUnit U = turbo_unit(tid);
        const int tok0 = 64 * chunk + 32 * U.half + 8 * U.kb;
        if (tok0 + 7 >= nqd && tok0 < len) {
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int N = 4 * U.hN + 2 * U.par + qq, d = 16 * N + U.n;
                _Float16* dst = sv + d * kVS + 8 * ((4 * U.half + U.kb) ^ N);
                h8 hi = *reinterpret_cast<const h8*>(dst), lo = *reinterpret_cast<const h8*>(dst + 128 * kVS);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int tok = tok0 + i;
                    if (tok >= nqd && tok < len) {
                        const float y = vring[(size_t)(tok % W) * kDim + d];
                        const _Float16 h = (_Float16)y;
                        hi[i] = h;
                        lo[i] = (_Float16)(y - (float)h);
                    }
                }
                *reinterpret_cast<h8*>(dst) = hi;
                *reinterpret_cast<h8*>(dst + 128 * kVS) = lo;
            }
        }
    } else if constexpr (VB > 0) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int u = tid + kThreads * j, half = u >> 9, w = u & 511;
            const int kb = w >> 7, n = (w >> 3) & 15, N = w & 7, d = 16 * N + n;
            const int tok0 = 64 * chunk + 32 * half + 8 * kb;
            if (tok0 + 7 < nqd || tok0 >= len) continue;
            _Float16* dst = sv + d * kVS + 8 * ((4 * half + kb) ^ N);
            h8 hi = *reinterpret_cast<const h8*>(dst), lo = *reinterpret_cast<const h8*>(dst + 128 * kVS);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tok = tok0 + i;
                if (tok >= nqd && tok < len) {
                    const float y = vring[(size_t)(tok % W) * kDim + d];
                    const _Float16 h = (_Float16)y;
                    hi[i] = h;
                    lo[i] = (_Float16)(y - (float)h);
                }
            }
            *reinterpret_cast<h8*>(dst) = hi;
            *reinterpret_cast<h8*>(dst + 128 * kVS) = lo;
        }
    }
}

// FP32 window beside rotated or balanced codes: the window tokens' originals mapped into the
// domain their tensor's codes live in, the one the scores and the value accumulator use (uniform
// planes: R(x) when rotated, then .* 1/c when balanced; TurboQuant planes: R(x); a split V: the
// two 64-point rotations of the permuted channels, position j holding channel perm[j]).  One
// workgroup per (kv head, sequence), one wave per token at a time (lane l: channels or positions
// 2l, 2l + 1); the copy keeps the ring layout, wring[b][kv head][tensor][t % 128][128].
__global__ __launch_bounds__(256) void prefill_window_kernel(PrefillParams p) {
    const int kvh = blockIdx.x, b = blockIdx.y, wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const PlaneGeom& KG = p.geom[0];
    const PlaneGeom& VG = p.geom[1];
    const char* slot = p.layer_base + (size_t)b * p.seq_stride + (size_t)kvh * p.head_stride;
    const float* kring = reinterpret_cast<const float*>(slot + p.plane_off[0] + KG.ring_off);
    const float* vring = reinterpret_cast<const float*>(slot + p.plane_off[1] + VG.ring_off);
    float* kdst = p.wring + ((size_t)b * p.Hkv + kvh) * 2 * kWindowMax * kDim;
    float* vdst = kdst + kWindowMax * kDim;
    const size_t tk = (size_t)(kvh * 2 + 0) * kDim, tv = (size_t)(kvh * 2 + 1) * kDim;
    const float2 ksg = reinterpret_cast<const float2*>(p.signs + tk)[l];
    const float2 vsg = reinterpret_cast<const float2*>(p.signs + tv)[l];
    const float2 kic = KG.sinkhorn ? reinterpret_cast<const float2*>(p.inv_c + tk)[l] : make_float2(1.0f, 1.0f);
    const float2 vic = VG.sinkhorn ? reinterpret_cast<const float2*>(p.inv_c + tv)[l] : make_float2(1.0f, 1.0f);
    const bool vsplit = VG.scheme == kTurboSplit, ksplit = KG.scheme == kTurboSplit;
    const int2 pm = vsplit ? reinterpret_cast<const int2*>(p.perm + (size_t)kvh * kDim)[l] : make_int2(0, 0);
    const int2 pmk = ksplit ? reinterpret_cast<const int2*>(p.perm_k + (size_t)kvh * kDim)[l] : make_int2(0, 0);
    const int N = p.len[b];
    for (int tok = max(0, N - kWindowMax) + wave; tok < N; tok += 4) { // wave-uniform: shuffles are safe
        const size_t r = (size_t)(tok % kWindowMax) * kDim;
        float2 k = reinterpret_cast<const float2*>(kring + r)[l];
        float2 v = reinterpret_cast<const float2*>(vring + r)[l];
        if (ksplit) {
            const float ax = __shfl(k.x, pmk.x >> 1), ay = __shfl(k.y, pmk.x >> 1);
            const float bx = __shfl(k.x, pmk.y >> 1), by = __shfl(k.y, pmk.y >> 1);
            k = make_float2((pmk.x & 1) ? ay : ax, (pmk.y & 1) ? by : bx);
            qdev::rotate64_signed(k.x, k.y, ksg.x, ksg.y);
        } else if (KG.rotate) {
            qdev::rotate_signed(k.x, k.y, ksg.x, ksg.y);
        }
        if (KG.sinkhorn) {
            k.x *= kic.x;
            k.y *= kic.y;
        }
        if (vsplit) {
            // channel pm.x sits in lane pm.x / 2, component pm.x % 2 (pm.y alike)
            const float ax = __shfl(v.x, pm.x >> 1), ay = __shfl(v.y, pm.x >> 1);
            const float bx = __shfl(v.x, pm.y >> 1), by = __shfl(v.y, pm.y >> 1);
            v = make_float2((pm.x & 1) ? ay : ax, (pm.y & 1) ? by : bx);
            qdev::rotate64_signed(v.x, v.y, vsg.x, vsg.y);
        } else {
            if (VG.rotate) qdev::rotate_signed(v.x, v.y, vsg.x, vsg.y);
            if (VG.sinkhorn) {
                v.x *= vic.x;
                v.y *= vic.y;
            }
        }
        reinterpret_cast<float2*>(kdst + r)[l] = k;
        reinterpret_cast<float2*>(vdst + r)[l] = v;
    }
}

// out row = R_V^-1(c_V .* x) for a row held as two channels per lane (2l, 2l + 1).
__device__ __forceinline__ void store_out_row(float a, float c, const PlaneGeom& VG, float2 csv, float2 sgv,
                                              int2 pm, float* out_row, int l) {
    if (VG.scheme == kTurboSplit) {
        // two 64-point inverse rotations (the 128-point butterflies without the last span), then
        // positions 2l, 2l + 1 go to their channels
        const float s = a + c, d = a - c;
        a = s;
        c = d;
        qdev::hadamard_step<1>(a, c, l);
        qdev::hadamard_step<2>(a, c, l);
        qdev::hadamard_step<4>(a, c, l);
        qdev::hadamard_step<8>(a, c, l);
        qdev::hadamard_step<16>(a, c, l);
        a *= 0.125f;
        c *= 0.125f;
        if (sgv.x < 0.0f) a = -a;
        if (sgv.y < 0.0f) c = -c;
        out_row[pm.x] = a;
        out_row[pm.y] = c;
        return;
    }
    if (VG.sinkhorn) {
        a *= csv.x;
        c *= csv.y;
    }
    if (VG.rotate) {
        qdev::hadamard_wave(a, c);
        a *= c0f();
        c *= c0f();
        if (sgv.x < 0.0f) a = -a;
        if (sgv.y < 0.0f) c = -c;
    }
    reinterpret_cast<float2*>(out_row)[l] = make_float2(a, c);
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int KB, int VB>
__global__ __launch_bounds__(kThreads) void prefill_attn_kernel(PrefillParams p) {
    constexpr bool KQ = KB == kQjlK || split_k_kind(KB); // keys with the QJL sketch
    __shared__ __align__(16) _Float16 s_lds[kLdsHalves];
    __shared__ __align__(16) _Float16 s_vm[2][2][4][kVmRow]; // [buffer][scale | zero][group][token]
    __shared__ float s_qf[kWaves][kWaveRows];          // 2^-e of each row's q' scaling
    // QJL keys, per buffer: the sign words [key row][4] and the scale f_t per key row as fp16
    // hi | lo << 16
    __shared__ __align__(16) uint32_t s_sg[2][KQ ? 256 : 1];
    __shared__ __align__(16) uint32_t s_f[2][KQ ? 64 : 1];

    const int S = p.n_splits;
    const int kvh = blockIdx.x % p.Hkv, rest = blockIdx.x / p.Hkv;
    const int split = rest % S, tile = rest / S, b = blockIdx.y;
    const int G = p.G, nrows = p.n_q * G;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, lr = l & 15, lq = l >> 4;
    const int N = p.len[b], P0 = N - p.n_q;
    const int row0 = tile * kPrefillRowsPerBlock + kWaveRows * wave; // this wave's first row
    const PlaneGeom& KG = p.geom[0];
    const PlaneGeom& VG = p.geom[1];
    const char* slot = p.layer_base + (size_t)b * p.seq_stride + (size_t)kvh * p.head_stride;
    Planes P;
    P.kcodes = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.codes_off);
    P.kmeta = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.meta_off);
    P.kqjl = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.qjl_off);
    P.vcodes = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.codes_off);
    P.vmeta = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.meta_off);
    // FP32 window: the newest min(len, W) tokens are read from the rings, or beside rotated or
    // balanced codes from their copies mapped into the code domain by prefill_window_kernel
    const int Wn = p.window, nqd = (Wn > 0) ? max(0, N - Wn) : N;
    const float* kring = reinterpret_cast<const float*>(slot + p.plane_off[0] + KG.ring_off);
    const float* vring = reinterpret_cast<const float*>(slot + p.plane_off[1] + VG.ring_off);
    if (p.wring) {
        kring = p.wring + ((size_t)b * p.Hkv + kvh) * 2 * kWindowMax * kDim;
        vring = kring + kWindowMax * kDim;
    }
    // QJL keys: the upper half of the 3-bit codebook; split keys: the upper halves of the outlier
    // (0..3) and the rest (4..7) codebooks of N(0, 1/64)
    float mgk[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (KB == kQjlK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) mgk[j] = p.mu[4 + j];
    } else if constexpr (split_k_kind(KB)) {
        constexpr int B = split_k_bits(KB), LO = 1 << (B - 1), LR = 1 << (B - 2);
#pragma unroll
        for (int j = 0; j < LO / 2; ++j) mgk[j] = p.mu64[split_table_off(LO) + LO / 2 + j];
#pragma unroll
        for (int j = 0; j < LR / 2; ++j) mgk[4 + j] = p.mu64[split_table_off(LR) + LR / 2 + j];
    }
    // TurboQuant-MSE V: the upper half of the codebook (the lower half is its mirror image)
    float mg[12] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (split_kind(VB)) {
        // upper halves of the N(0, 1/64) codebooks (tables at levels - 4): outliers, then the rest
        constexpr int BO = kSplitV - VB, LO = 1 << BO, LR = 1 << (BO - 1);
#pragma unroll
        for (int j = 0; j < LO / 2; ++j) mg[j] = p.mu64[(LO - 4) + LO / 2 + j];
#pragma unroll
        for (int j = 0; j < LR / 2; ++j) mg[8 + j] = p.mu64[(LR - 4) + LR / 2 + j];
    } else if constexpr (VB == -3) {
#pragma unroll
        for (int j = 0; j < 4; ++j) mg[j] = p.mu[4 + j];
    } else if constexpr (VB == -4) {
#pragma unroll
        for (int j = 0; j < 8; ++j) mg[j] = p.mu16[8 + j];
    }

    // ---------------- q' = R_K(q) .* c_K * scale * log2(e) * 2^e per row (2^e keeps max|q'| in
    // [64, 128)), then the B operands of the score product (column = row lr of the block,
    // k = channel 32 ks + 8 lq + i): hi = fp16(q'), lo = fp16(q' - hi)
    h8 Bh[4][kQB], Bl[4][kQB];
    h8 Ph[KQ ? 4 : 1][kQB], Pl[KQ ? 4 : 1][kQB]; // QJL keys: p = S q' per row as fp16 hi + lo (the
                                                 // operand layout of q')
    {
        const float2 sgn = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 0) * kDim)[l];
        const float2 csk = reinterpret_cast<const float2*>(p.cs + (size_t)(kvh * 2 + 0) * kDim)[l];
        const int2 pmk = split_k_kind(KB) ? reinterpret_cast<const int2*>(p.perm_k + (size_t)kvh * kDim)[l]
                                          : make_int2(0, 0);
        float* s_rows = reinterpret_cast<float*>(s_lds) + wave * 16 * kDim;
        for (int qb = 0; qb < kQB; ++qb) {
            for (int rr = 0; rr < 16; ++rr) {
                const int r = 16 * qb + rr, gr = row0 + r;
                float a = 0.0f, c = 0.0f;
                if (gr < nrows) {
                    const int i = gr / G, hq = kvh * G + (gr - i * G);
                    const size_t off = (((size_t)b * p.n_q + i) * p.Hq + hq) * kDim;
                    if (p.dtype == 0) {
                        const float2 v = reinterpret_cast<const float2*>(static_cast<const float*>(p.q) + off)[l];
                        a = v.x;
                        c = v.y;
                    } else {
                        const uint32_t v = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + off)[l];
                        a = in16_to_f32(v & 0xffff, p.dtype);
                        c = in16_to_f32(v >> 16, p.dtype);
                    }
                }
                if constexpr (split_k_kind(KB)) {
                    // the split domain: positions 2l, 2l + 1 take channels pmk (lane pmk / 2,
                    // component pmk % 2), then the two 64-point rotations
                    const float ax = __shfl(a, pmk.x >> 1), ay = __shfl(c, pmk.x >> 1);
                    const float bx = __shfl(a, pmk.y >> 1), by = __shfl(c, pmk.y >> 1);
                    a = (pmk.x & 1) ? ay : ax;
                    c = (pmk.y & 1) ? by : bx;
                    qdev::rotate64_signed(a, c, sgn.x, sgn.y);
                } else if (KG.rotate) {
                    if (sgn.x < 0.0f) a = -a;
                    if (sgn.y < 0.0f) c = -c;
                    qdev::hadamard_wave(a, c);
                    a *= c0f();
                    c *= c0f();
                }
                if (KG.sinkhorn) {
                    a *= csk.x;
                    c *= csk.y;
                }
                a *= p.qscale;
                c *= p.qscale;
                const float mx = xor_reduce<64>(fmaxf(fabsf(a), fabsf(c)), [](float x, float y) { return fmaxf(x, y); });
                int e2 = 0;
                if (mx > 0.0f) frexpf(mx, &e2);
                const int e = (mx > 0.0f) ? min(max(7 - e2, -100), 100) : 0;
                const float f = ldexpf(1.0f, e);
                reinterpret_cast<float2*>(s_rows + rr * kDim)[l] = make_float2(a * f, c * f);
                if (l == 0) s_qf[wave][r] = ldexpf(1.0f, -e);
            }
            wave_lds_sync();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const float4 x0 = *reinterpret_cast<const float4*>(s_rows + lr * kDim + 32 * ks + 8 * lq);
                const float4 x1 = *reinterpret_cast<const float4*>(s_rows + lr * kDim + 32 * ks + 8 * lq + 4);
                const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const _Float16 h = (_Float16)xs[i];
                    Bh[ks][qb][i] = h;
                    Bl[ks][qb][i] = (_Float16)(xs[i] - (float)h);
                }
            }
            if constexpr (KQ) {
                // p_r = S q'_r for the wave's 16 rows (lane: projections 2l, 2l + 1; S^T rows from
                // global memory, q' broadcast from LDS), then through LDS into the operand layout
                float pa[16], pc[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) pa[r] = pc[r] = 0.0f;
                for (int j = 0; j < kDim; j += 4) {
                    float2 s4[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        s4[jj] = reinterpret_cast<const float2*>(p.qjl_st + (size_t)(j + jj) * kDim)[l];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float4 x = *reinterpret_cast<const float4*>(s_rows + r * kDim + j);
                        pa[r] = fmaf(s4[0].x, x.x, fmaf(s4[1].x, x.y, fmaf(s4[2].x, x.z, fmaf(s4[3].x, x.w, pa[r]))));
                        pc[r] = fmaf(s4[0].y, x.x, fmaf(s4[1].y, x.y, fmaf(s4[2].y, x.z, fmaf(s4[3].y, x.w, pc[r]))));
                    }
                }
                float* s_prows = reinterpret_cast<float*>(s_lds) + (kWaves + wave) * 16 * kDim;
#pragma unroll
                for (int r = 0; r < 16; ++r) reinterpret_cast<float2*>(s_prows + r * kDim)[l] = make_float2(pa[r], pc[r]);
                wave_lds_sync();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const float4 x0 = *reinterpret_cast<const float4*>(s_prows + lr * kDim + 32 * ks + 8 * lq);
                    const float4 x1 = *reinterpret_cast<const float4*>(s_prows + lr * kDim + 32 * ks + 8 * lq + 4);
                    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const _Float16 h = (_Float16)xs[i];
                        Ph[ks][qb][i] = h;
                        Pl[ks][qb][i] = (_Float16)(xs[i] - (float)h);
                    }
                }
            }
            wave_lds_sync();
        }
    }
    // the lane's column (query row lr of each block): scale back, position (-1: an absent row
    // sees no token)
    float F[kQB], m_run[kQB], l_run[kQB];
    int pos[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int gr = row0 + 16 * qb + lr;
        F[qb] = s_qf[wave][16 * qb + lr];
        pos[qb] = (gr < nrows) ? P0 + gr / G : -1;
        m_run[qb] = kNegInf;
        l_run[qb] = 0.0f;
    }
    int pmin = pos[0];
#pragma unroll
    for (int qb = 1; qb < kQB; ++qb) pmin = min(pmin, pos[qb]);
    const float pos_min = xor_reduce<64>((float)pmin, [](float x, float y) { return fminf(x, y); });
    f4 O[8][kQB];
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) O[n][qb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    // ---------------- this split's chunks of the keys the workgroup's rows can see
    const int last_row = min(tile * kPrefillRowsPerBlock + kPrefillRowsPerBlock, nrows) - 1;
    const int nch = (P0 + last_row / G + 1 + 63) / 64;
    const int cps = (nch + S - 1) / S;
    const int c0 = split * cps, c1 = min(nch, c0 + cps);
    __syncthreads(); // the q' rows are consumed; the LDS becomes the chunk buffers

    ChunkRegs R;
    const bool late = wave >= kWaves / 2; // dequantizes before its matrix products
    if (c0 < c1) {
        load_vmeta<VB>(P, c0, tid, R);
        store_vmeta<VB>(s_vm[0], tid, R);
        load_codes<KB, VB>(P, c0, tid, R);
        if (c0 + 1 < c1) load_vmeta<VB>(P, c0 + 1, tid, R);
        __syncthreads();
        dequant_chunk<KB, VB>(s_lds, s_lds + 2 * kKBuf, s_vm[0], tid, R, mg, mgk, s_sg[0], s_f[0]);
        window_overwrite<KB, VB>(s_lds, s_lds + 2 * kKBuf, s_f[0], c0, nqd, N, Wn, kring, vring, tid);
        if (c0 + 1 < c1) store_vmeta<VB>(s_vm[1], tid, R);
        if (late && c0 + 1 < c1) load_codes<KB, VB>(P, c0 + 1, tid, R);
        __syncthreads();
    }
    for (int ci = c0; ci < c1; ++ci) {
        const int buf = (ci - c0) & 1;
        const bool more = ci + 1 < c1;
        // The two waves sharing a SIMD (w and w + 4) take the iteration in opposite order: one
        // dequantizes the next chunk (vector ALU) while the other multiplies (matrix cores).  The
        // waves that dequantize first hold their global words one chunk further ahead.
        auto dequant_next = [&]() {
            if (more) {
                dequant_chunk<KB, VB>(s_lds + (buf ^ 1) * kKBuf, s_lds + 2 * kKBuf + (buf ^ 1) * kVBuf,
                                      s_vm[buf ^ 1], tid, R, mg, mgk, s_sg[buf ^ 1], s_f[buf ^ 1]);
                window_overwrite<KB, VB>(s_lds + (buf ^ 1) * kKBuf, s_lds + 2 * kKBuf + (buf ^ 1) * kVBuf,
                                         s_f[buf ^ 1], ci + 1, nqd, N, Wn, kring, vring, tid);
                if (ci + 2 < c1) store_vmeta<VB>(s_vm[buf], tid, R);
            }
        };
        if (!late) {
            if (ci + 2 < c1) load_vmeta<VB>(P, ci + 2, tid, R); // first: it may wait on its register
            if (more) load_codes<KB, VB>(P, ci + 1, tid, R);
        } else {
            dequant_next();
            if (ci + 2 < c1) load_codes<KB, VB>(P, ci + 2, tid, R);
        }
        const _Float16* sk = s_lds + buf * kKBuf;
        const _Float16* sv = s_lds + 2 * kKBuf + buf * kVBuf;
        const uint32_t* sg = s_sg[buf];
        const uint32_t* sfb = s_f[buf];
        const bool masked = 64 * ci + 63 > (int)pos_min;
        // ---- S^T for the chunk's four 16-token tiles (tile b, row 4 lq + v = token
        // 32 (b / 2) + 8 lq + 4 (b % 2) + v); three accumulators per tile (K_hi q_hi, K_hi q_lo,
        // K_lo q_hi) keep the matrix-core dependency chains four products long
        f4 Sa[4][kQB], Sb[4][kQB], Sd[4][kQB];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) Sa[b][qb] = Sb[b][qb] = Sd[b][qb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const _Float16* kr = sk + (16 * b + lr) * kKS + 32 * ks + 8 * lq;
                const h8 Ah = *reinterpret_cast<const h8*>(kr);
                const h8 Al = *reinterpret_cast<const h8*>(kr + 64 * kKS);
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    Sa[b][qb] = mfma16(Ah, Bh[ks][qb], Sa[b][qb]);
                    Sb[b][qb] = mfma16(Ah, Bl[ks][qb], Sb[b][qb]);
                    // QJL keys keep two chains per tile (registers: S q' is one more operand set)
                    if constexpr (KQ) Sb[b][qb] = mfma16(Al, Bh[ks][qb], Sb[b][qb]);
                    else Sd[b][qb] = mfma16(Al, Bh[ks][qb], Sd[b][qb]);
                }
                if constexpr (KQ) {
                    // QJL: A = +-f_t (hi, then lo) of the row's eight signs of this slice
                    // (projections 32 ks + 8 lq + i at bits 16 (i % 2) + 4 lq + i / 2 of word ks; a
                    // clear bit is -1: the sign bit of f flipped)
                    const uint32_t nw = ~sg[4 * (16 * b + lr) + ks] >> (4 * lq);
                    const uint32_t fw = sfb[16 * b + lr];
                    const uint32_t fh = (fw & 0xffffu) * 0x00010001u, fl = (fw >> 16) * 0x00010001u;
                    u4 a2h, a2l;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t m = ((nw >> k) & 0x00010001u) << 15;
                        a2h[k] = m ^ fh;
                        a2l[k] = m ^ fl;
                    }
#pragma unroll
                    for (int qb = 0; qb < kQB; ++qb) {
                        Sa[b][qb] = mfma16(__builtin_bit_cast(h8, a2h), Ph[ks][qb], Sa[b][qb]);
                        Sb[b][qb] = mfma16(__builtin_bit_cast(h8, a2h), Pl[ks][qb], Sb[b][qb]);
                        Sa[b][qb] = mfma16(__builtin_bit_cast(h8, a2l), Ph[ks][qb], Sa[b][qb]);
                    }
                }
            }
        }
        // ---- online softmax of each column over the chunk's 64 tokens.  The running maximum m
        // moves only when a score exceeds it by more than kLazy (log2 units), so the accumulator
        // is rescaled rarely; weights stay below 2^kLazy.
        h8 Pb[2][kQB]; // [k-slice hh][column block]: element i = token 32 hh + 8 lq + i
        float al[kQB];
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            float raw[16]; // raw[8 hh + 4 tb + v]: token 32 hh + 8 lq + 4 tb + v
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) raw[4 * b + v] = Sa[b][qb][v] + (Sb[b][qb][v] + Sd[b][qb][v]);
            if (__builtin_expect(masked, 0)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = 64 * ci + 32 * (i >> 3) + 8 * lq + (i & 7);
                    if (t > pos[qb]) raw[i] = kNegInf;
                }
            }
            float mx = raw[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, raw[i]);
            mx = fmaxf(mx, xor_lane<16>(mx));
            mx = fmaxf(mx, xor_lane<32>(mx)) * F[qb];
            const bool up = mx > m_run[qb] + kLazy;
            al[qb] = up ? __builtin_amdgcn_exp2f(m_run[qb] - mx) : 1.0f;
            if (up) m_run[qb] = mx;
            need |= up;
            const float m = m_run[qb];
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // the sum takes the fp16 weights the PV product uses: the output stays a convex
                // combination of the values (exactly so when one weight dominates)
                const float pv = (m == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(raw[i], F[qb], -m));
                const _Float16 ph = (_Float16)pv;
                sum += (float)ph;
                Pb[i >> 3][qb][i & 7] = ph;
            }
            l_run[qb] = fmaf(l_run[qb], al[qb], sum);
        }
        if (__ballot(need) != 0) {
#pragma unroll
            for (int n = 0; n < 8; ++n)
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) O[n][qb][v] *= al[qb];
        }
        // ---- O^T += V^T P^T over the chunk's two 32-token k-slices (A = values [channel
        // 16 n + lr][token 32 hh + 8 lq + i])
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const _Float16* vr = sv + (16 * n + lr) * kVS + 8 * ((4 * hh + lq) ^ n);
                const h8 Vh = *reinterpret_cast<const h8*>(vr);
                const h8 Vl = *reinterpret_cast<const h8*>(vr + 128 * kVS);
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    O[n][qb] = mfma16(Vh, Pb[hh][qb], O[n][qb]);
                    O[n][qb] = mfma16(Vl, Pb[hh][qb], O[n][qb]);
                }
            }
        }
        if (!late) dequant_next();
        __syncthreads();
    }

    // ---------------- rows out: softmax sum over the column's four lanes; O^T lane (lr, lq) holds
    // channels 16 n + 4 lq + v of row lr
    float lt[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        lt[qb] = l_run[qb] + xor_lane<16>(l_run[qb]);
        lt[qb] += xor_lane<32>(lt[qb]);
    }
    if (S > 1) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int gr = row0 + 16 * qb + lr;
            if (gr < nrows) {
                const int i = gr / G, hq = kvh * G + (gr - i * G);
                float* P_ = p.partials + ((((size_t)b * p.n_q + i) * p.Hq + hq) * S + split) * kPartialFloats;
                if (lq == 0) {
                    P_[0] = m_run[qb];
                    P_[1] = lt[qb];
                }
#pragma unroll
                for (int n = 0; n < 8; ++n) *reinterpret_cast<f4*>(P_ + 4 + 16 * n + 4 * lq) = O[n][qb];
            }
        }
        return;
    }
    __syncthreads(); // c0 >= c1 workgroups skipped the loop's barriers
    const float2 csv = reinterpret_cast<const float2*>(p.cs + (size_t)(kvh * 2 + 1) * kDim)[l];
    const float2 sgv = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 1) * kDim)[l];
    const int2 pmv = VG.scheme == kTurboSplit ? reinterpret_cast<const int2*>(p.perm + (size_t)kvh * kDim)[l]
                                              : make_int2(2 * l, 2 * l + 1);
    float* s_rows = reinterpret_cast<float*>(s_lds) + wave * 8 * kDim;
#pragma unroll
    for (int ps = 0; ps < 2 * kQB; ++ps) { // register indexes must stay compile-time: unrolled
        const int qb = ps >> 1, h8r = ps & 1;
        if ((lr >> 3) == h8r) {
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                f4 o = O[n][qb];
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = (lt[qb] > 0.0f) ? o[v] / lt[qb] : 0.0f;
                *reinterpret_cast<f4*>(s_rows + (lr & 7) * kDim + 16 * n + 4 * lq) = o;
            }
        }
        wave_lds_sync();
        for (int rr = 0; rr < 8; ++rr) {
            const int gr = row0 + 16 * qb + 8 * h8r + rr;
            if (gr >= nrows) break;
            const int i = gr / G, hq = kvh * G + (gr - i * G);
            const float2 x = reinterpret_cast<const float2*>(s_rows + rr * kDim)[l];
            store_out_row(x.x, x.y, VG, csv, sgv, pmv, p.out + (((size_t)b * p.n_q + i) * p.Hq + hq) * kDim, l);
        }
        wave_lds_sync();
    }
}

// One wave per output row: combine the splits' (m, l, acc) in split order, divide, map back.
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p) {
    const int l = threadIdx.x & 63;
    const int rr = blockIdx.x * 4 + (threadIdx.x >> 6); // (b * n_q + i) * Hq + hq
    if (rr >= p.batch * p.n_q * p.Hq) return;
    const int hq = rr % p.Hq, kvh = hq / p.G;
    const int S = p.n_splits;
    const float* P_ = p.partials + (size_t)rr * S * kPartialFloats;
    float M = kNegInf;
    for (int s = 0; s < S; ++s) M = fmaxf(M, P_[s * kPartialFloats]);
    float a = 0.0f, c = 0.0f, L = 0.0f;
    for (int s = 0; s < S; ++s) {
        const float m = P_[s * kPartialFloats];
        const float w = (m == kNegInf) ? 0.0f : exp2f(m - M);
        L = fmaf(w, P_[s * kPartialFloats + 1], L);
        const float2 v = reinterpret_cast<const float2*>(P_ + s * kPartialFloats + 4)[l];
        a = fmaf(w, v.x, a);
        c = fmaf(w, v.y, c);
    }
    a = (L > 0.0f) ? a / L : 0.0f;
    c = (L > 0.0f) ? c / L : 0.0f;
    const float2 csv = reinterpret_cast<const float2*>(p.cs + (size_t)(kvh * 2 + 1) * kDim)[l];
    const float2 sgv = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 1) * kDim)[l];
    const int2 pmv = p.geom[1].scheme == kTurboSplit ? reinterpret_cast<const int2*>(p.perm + (size_t)kvh * kDim)[l]
                                                      : make_int2(2 * l, 2 * l + 1);
    store_out_row(a, c, p.geom[1], csv, sgv, pmv, p.out + (size_t)rr * kDim, l);
}

template <int KB, int VB>
hipError_t launch_t(const PrefillParams& p, hipStream_t s) {
    const int tiles = (p.n_q * p.G + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock;
    const dim3 grid(p.Hkv * p.n_splits * tiles, p.batch);
    hipLaunchKernelGGL((prefill_attn_kernel<KB, VB>), grid, dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_splits == 1) return e;
    const int rows = p.batch * p.n_q * p.Hq;
    hipLaunchKernelGGL(prefill_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, p);
    return hipGetLastError();
}

} // namespace

bool prefill_attn_supported(const PrefillParams& p) {
    const PlaneGeom& K = p.geom[0];
    const PlaneGeom& V = p.geom[1];
    auto ok = [](const PlaneGeom& g) { return g.scheme == kUniform && (g.bits == 3 || g.bits == 4 || g.bits == 8); };
    const bool k_qjl = (K.scheme == kTurboQjl && K.bits == 3) || (K.scheme == kTurboSplit && (K.bits == 3 || K.bits == 4));
    const bool v_turbo = (V.scheme == kTurboMse || V.scheme == kTurboSplit) && (V.bits == 3 || V.bits == 4);
    const bool win_ok = p.window == 0 || p.window == kWindowMax;
    return (ok(K) || k_qjl) && (ok(V) || v_turbo) && win_ok && p.G >= 1 && p.G <= kMaxGroupHeads;
}

template <int KB>
hipError_t launch_k(const PrefillParams& p, hipStream_t s) {
    const int vb = p.geom[1].bits;
    if (p.geom[1].scheme == kTurboSplit)
        return vb == 4 ? launch_t<KB, kSplitV - 4>(p, s) : launch_t<KB, kSplitV - 3>(p, s);
    if (p.geom[1].scheme == kTurboMse) return vb == 4 ? launch_t<KB, -4>(p, s) : launch_t<KB, -3>(p, s);
    if (vb == 3) return launch_t<KB, 3>(p, s);
    return vb == 4 ? launch_t<KB, 4>(p, s) : launch_t<KB, 8>(p, s);
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
    if (p.wring) {
        hipLaunchKernelGGL(prefill_window_kernel, dim3(p.Hkv, p.batch), dim3(256), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int kb = p.geom[0].bits;
    if (p.geom[0].scheme == kTurboQjl) return launch_k<kQjlK>(p, s);
    if (p.geom[0].scheme == kTurboSplit) return kb == 4 ? launch_k<kSplitK - 4>(p, s) : launch_k<kSplitK - 3>(p, s);
    if (kb == 3) return launch_k<3>(p, s);
    return kb == 4 ? launch_k<4>(p, s) : launch_k<8>(p, s);
}

} // namespace kvq
