// Bulk (prefill) quantizer, lane-dense.  A wave owns one (tensor, sequence, kv head) and loops
// over its 8-token octets; an octet is quantized in two rounds of four tokens, lane L holding
// channels 8j .. 8j+7 (j = L % 16) of octet token 4r + L / 16.  The binary32 operations that
// decide a code are the same, in the same order, as in quantize_wave (spans 1, 2, 4 of the
// Walsh-Hadamard butterflies inside the lane, spans 8 .. 64 across lanes j ^ 1, 2, 4, 8; the same
// group min / max, fp16 zero and scale, and rounding; the same pairwise norm tree; the same
// sequential QJL fma chain), so the bytes are identical; only the integer packing differs in how
// it is done.
//
// Method sources (pages by title and section):
//  - quantcpp article "Beyond RAG...", progressive table + "how it works": 4-bit codes with fp16
//    scale and zero per 32 channels, newest 128 tokens kept in FP32.
//  - KVarN-on-Bonsai post, TL;DR: Walsh-Hadamard transform and Sinkhorn variance balancing
//    before 4-bit quantization.
//  - "LLM memory saving ... 2026", TurboQuant row of the method table: random rotation,
//    per-coordinate optimal scalar quantizer, 1-bit QJL of the residual.
#pragma once

#include <utility>

#include "kvq_quant_dev.h"

namespace kvq {
namespace qbulk {

using qdev::c0f;
using qdev::f16_rd;
using qdev::f16_rn;
using qdev::f16_val;
using qdev::k_row;
using qdev::lane_id;

// 2^23: adding it to a value u in [0, 2^23) rounds u to an integer (ties to even) and leaves
// that integer in the low mantissa bits.
__device__ __forceinline__ float magic23() { return __uint_as_float(0x4B000000u); }

// Source values of one octet: v[r][i] = channel 8j + i of octet token 4r + L / 16 (zero for
// tokens outside the append).
struct OctetIn {
    float v[2][8];
};

// What a wave keeps for its (tensor, sequence, kv head) across octets.
struct WavePlane {
    const char* src;  // source of channel 8j of append token 0
    size_t tok_bytes; // bytes between consecutive tokens of the source
    int dtype, start, end, window;
    uint8_t* codes;
    uint8_t* meta;
    float* ring;
};

__device__ __forceinline__ WavePlane wave_plane(const QuantParams& p, int tensor, int b, int head) {
    const int j = lane_id() & 15;
    const PlaneGeom& G = p.geom[tensor];
    char* slot = p.layer_base + (size_t)b * p.seq_stride + (size_t)head * p.head_stride +
                 p.plane_off[tensor];
    WavePlane w;
    const size_t esz = p.dtype == 0 ? 4 : 2;
    w.tok_bytes = (size_t)p.Hkv * kDim * esz;
    w.src = static_cast<const char*>(p.src[tensor]) + ((size_t)b * p.T * p.Hkv + head) * kDim * esz +
            8 * j * esz;
    w.dtype = p.dtype;
    w.start = p.start[b];
    w.end = w.start + p.T;
    w.window = p.window;
    w.codes = reinterpret_cast<uint8_t*>(slot + G.codes_off);
    w.meta = reinterpret_cast<uint8_t*>(slot + G.meta_off);
    w.ring = reinterpret_cast<float*>(slot + G.ring_off);
    return w;
}

__device__ __forceinline__ void load_octet(const WavePlane& w, int g, OctetIn& in) {
    const int tk = lane_id() >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = 8 * g + 4 * r + tk;
#pragma unroll
        for (int i = 0; i < 8; ++i) in.v[r][i] = 0.0f;
        if (t >= w.start && t < w.end) {
            const char* s = w.src + (size_t)(t - w.start) * w.tok_bytes;
            if (w.dtype == 0) {
                const float4 a = reinterpret_cast<const float4*>(s)[0];
                const float4 c = reinterpret_cast<const float4*>(s)[1];
                in.v[r][0] = a.x; in.v[r][1] = a.y; in.v[r][2] = a.z; in.v[r][3] = a.w;
                in.v[r][4] = c.x; in.v[r][5] = c.y; in.v[r][6] = c.z; in.v[r][7] = c.w;
            } else {
                const uint4 a = *reinterpret_cast<const uint4*>(s);
                const uint32_t x[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    in.v[r][2 * i] = in16_to_f32(x[i] & 0xffff, w.dtype);
                    in.v[r][2 * i + 1] = in16_to_f32(x[i] >> 16, w.dtype);
                }
            }
        }
    }
}

// Span 8 D of the butterflies across lanes j and j ^ D: the lower lane forms own + partner, the
// upper lane partner + (-own), the same binary32 value as partner - own.
template <int D>
__device__ __forceinline__ void cross8(float* e, int j) {
    const uint32_t neg = (j & D) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float pv = xor_lane<D>(e[i]);
        e[i] = pv + __uint_as_float(__float_as_uint(e[i]) ^ neg);
    }
}

// R(x) = c0 H (d .* x) of the lane's 8 values; sgm[i] is the sign bit of d for channel 8j + i.
__device__ __forceinline__ void rotate(float* e, const uint32_t* sgm, int j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = __uint_as_float(__float_as_uint(e[i]) ^ sgm[i]);
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & h)) {
                const float x = e[i], y = e[i + h];
                e[i] = x + y;
                e[i + h] = x - y;
            }
    cross8<1>(e, j);
    cross8<2>(e, j);
    cross8<4>(e, j);
    cross8<8>(e, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = e[i] * c0f();
}

// Group code of the lane's 8 values (group = lanes 4g .. 4g+3 of the token): fp16 zero = the
// largest fp16 <= min, fp16 scale = fp16((max - zero) / L), code = min(rint((x - zero) / scale), L)
// (x - zero >= 0, so the lower clamp never acts).  r[i] holds 2^23 + code as binary32 bits, so its
// low byte is the code.
template <int BITS>
__device__ __forceinline__ void group_codes(const float* e, uint32_t* r, uint16_t& s16, uint16_t& z16) {
    float mn = e[0], mx = e[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, e[i]);
        mx = fmaxf(mx, e[i]);
    }
    mn = xor_reduce<4>(mn, [](float x, float y) { return fminf(x, y); });
    mx = xor_reduce<4>(mx, [](float x, float y) { return fmaxf(x, y); });
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    constexpr float L = (float)((1 << BITS) - 1);
    z16 = f16_rd(mn);
    const float z = f16_val(z16);
    const float s32 = (mx - z) / L;
    s16 = f16_rn(s32);
    const float s = f16_val(s16);
    const float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
    const float top = magic23() + L;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float u = (e[i] - z) * inv;
        r[i] = __float_as_uint(fminf(u + magic23(), top));
    }
}

// Symmetric 8-bit (q8_0-style) code of the lane's 8 values (group = lanes 4g .. 4g+3 of the
// token): d = fp16(max|x| / 127), q = rint(x * fp32(1/d)) clamped to [-127, 127], code q + 128
// (r[i] = 2^23 + code as binary32 bits), zero field fp16(-128 d).
__device__ __forceinline__ void group_codes_sym8(const float* e, uint32_t* r, uint16_t& s16, uint16_t& z16) {
    float amax = fabsf(e[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) amax = fmaxf(amax, fabsf(e[i]));
    amax = xor_reduce<4>(amax, [](float x, float y) { return fmaxf(x, y); });
    s16 = f16_rn(amax / 127.0f);
    const float d = f16_val(s16);
    z16 = f16_rn(-128.0f * d);
    const float inv = (d > 0.0f) ? 1.0f / d : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = fminf(fmaxf(rintf(e[i] * inv), -127.0f), 127.0f);
        r[i] = __float_as_uint((magic23() + 128.0f) + q);
    }
}

// Low bytes of a and b at bytes 0 and 2: a | b << 16 for codes below 256.
__device__ __forceinline__ uint32_t pair16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x0C040C00u);
}

// K row word of 8 4-bit codes: element i at bit 16 (i % 2) + 4 (i / 2).
__device__ __forceinline__ uint32_t pack_k4(const uint32_t* r) {
    const uint32_t a = pair16(r[0], r[1]), b = pair16(r[2], r[3]);
    const uint32_t c = pair16(r[4], r[5]), d = pair16(r[6], r[7]);
    return (d << 12) | (c << 8) | (b << 4) | a;
}

// Low bytes of r[0..3] in byte order.
__device__ __forceinline__ uint32_t pack_bytes(const uint32_t* r) {
    const uint32_t lo = __builtin_amdgcn_perm(r[1], r[0], 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(r[3], r[2], 0x04000C0Cu);
    return lo | hi;
}

// V word of one channel from its 8 token codes in byte order (lo = tokens 0..3, hi = 4..7):
// token i at bit 16 (i % 2) + 4 (i / 2).
__device__ __forceinline__ uint32_t pack_v4(uint32_t lo, uint32_t hi) {
    uint32_t ev = __builtin_amdgcn_perm(hi, lo, 0x06040200u); // tokens 0, 2, 4, 6
    uint32_t od = __builtin_amdgcn_perm(hi, lo, 0x07050301u); // tokens 1, 3, 5, 7
    ev = ev | (ev >> 4);
    od = od | (od >> 4);
    return __builtin_amdgcn_perm(od, ev, 0x06040200u);
}

// Bits of the V word that belong to tokens i of the octet with lo <= i < hi.
template <int BITS>
__device__ __forceinline__ uint64_t v_token_mask(int lo, int hi) {
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int sh = BITS == 4 ? 16 * (i % 2) + 4 * (i / 2) : 8 * i;
        if (i >= lo && i < hi) m |= (uint64_t)((1u << BITS) - 1) << sh;
    }
    return m;
}

// Byte of bit k of the four bytes of x (byte 0 -> bit 0), as a nibble.
__device__ __forceinline__ uint32_t byte_bits(uint32_t x, int k) {
    x = (x >> k) & 0x01010101u;
    x = x | (x >> 7);
    x = x | (x >> 14);
    return x & 0xFu;
}

// Block words of an octet of 3-bit codes in the TurboQuant-MSE V layout (TurboQuant V, and the
// 3-bit uniform V planes, which share it): bit k of channel d -> word 6 (16 o + d % 16) + 2k +
// (d / 16) / 4, token i at bit 16 (i % 2) + 4 ((d / 16) % 4) + i / 2.  wv: the octet's codes as
// [token][channel] bytes in the wave's LDS.  Lane L (< 32) forms the three words of n = L % 16,
// h = L / 16 (channels 16 N + n, N = 4h .. 4h + 3); lanes 32 + L take channels N = 4h + 2, 4h + 3
// of the same words, merged by the lane 32 apart.  Tokens of the octet outside [t_lo, t_hi) keep
// their bits.
__device__ __forceinline__ void v3_plane_words(const WavePlane& w, int g, int t_lo, int t_hi, const uint8_t* wv) {
    const int L = lane_id();
    const int n = L & 15, h = (L >> 4) & 1, half = L >> 5;
    uint32_t wk0 = 0u, wk1 = 0u, wk2 = 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int Nl = 2 * half + c; // N % 4
        const int d = 16 * (4 * h + Nl) + n;
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (uint32_t)wv[i * kDim + d] << (8 * i);
            hi |= (uint32_t)wv[(i + 4) * kDim + d] << (8 * i);
        }
        const uint32_t ev = __builtin_amdgcn_perm(hi, lo, 0x06040200u); // tokens 0, 2, 4, 6
        const uint32_t od = __builtin_amdgcn_perm(hi, lo, 0x07050301u); // tokens 1, 3, 5, 7
        wk0 |= (byte_bits(ev, 0) | (byte_bits(od, 0) << 16)) << (4 * Nl);
        wk1 |= (byte_bits(ev, 1) | (byte_bits(od, 1) << 16)) << (4 * Nl);
        wk2 |= (byte_bits(ev, 2) | (byte_bits(od, 2) << 16)) << (4 * Nl);
    }
    wk0 |= xor_lane<32>(wk0);
    wk1 |= xor_lane<32>(wk1);
    wk2 |= xor_lane<32>(wk2);
    __builtin_amdgcn_wave_barrier();
    if (half == 0) {
        const int o = g & 3;
        uint32_t* blk = reinterpret_cast<uint32_t*>(w.codes + (size_t)(g >> 2) * 1536) + 6 * (16 * o + n) + h;
        if (t_hi - t_lo == 8) {
            blk[0] = wk0;
            blk[2] = wk1;
            blk[4] = wk2;
        } else {
            // token bits of the octet present in this append
            uint32_t m = 0u;
            for (int i = t_lo - 8 * g; i < t_hi - 8 * g; ++i) m |= 0x1111u << (16 * (i & 1) + (i >> 1));
            blk[0] = (blk[0] & ~m) | (wk0 & m);
            blk[2] = (blk[2] & ~m) | (wk1 & m);
            blk[4] = (blk[4] & ~m) | (wk2 & m);
        }
    }
}

// One octet g of a uniform plane.  wv: 1 KiB of the wave's LDS (V planes: codes staged as
// [channel][token] bytes).
template <int BITS, bool ROT, bool SINK, bool SYM = false>
__device__ __forceinline__ void uniform_octet(const WavePlane& w, bool IS_V, int g, const OctetIn& in,
                                              const uint32_t* sgm, const float* ic, uint8_t* wv) {
    static_assert(!SYM || BITS == 8, "the symmetric quantizer is 8-bit");
    const int L = lane_id(), tk = L >> 4, j = L & 15;
    const int t_lo = max(w.start, 8 * g), t_hi = min(w.end, 8 * g + 8);
    if (t_lo >= t_hi) return;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i_tok = 4 * r + tk, t = 8 * g + i_tok;
        const bool valid = t >= t_lo && t < t_hi;
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = in.v[r][i];
        if (w.window > 0 && valid && t >= w.end - w.window) {
            float4* ring = reinterpret_cast<float4*>(w.ring + (size_t)(t % w.window) * kDim + 8 * j);
            ring[0] = make_float4(e[0], e[1], e[2], e[3]);
            ring[1] = make_float4(e[4], e[5], e[6], e[7]);
        }
        if (ROT) rotate(e, sgm, j);
        if (SINK) {
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = e[i] * ic[i];
        }
        uint32_t c[8];
        uint16_t s16, z16;
        if constexpr (SYM)
            group_codes_sym8(e, c, s16, z16);
        else
            group_codes<BITS>(e, c, s16, z16);
        const int g4 = j >> 2, kb = j & 3;
        const int row = IS_V ? t : k_row(t);
        if constexpr (BITS == 3) {
            // bit planes in the TurboQuant 3-bit layout: K rows hold three words per group
            // (channel 8j + i = value 8 (j % 4) + i of group j / 4, at bit 16 (v % 2) + v / 2);
            // V codes are staged as [token][channel] bytes for the block words
            if (IS_V) {
                *reinterpret_cast<uint2*>(wv + (size_t)i_tok * kDim + 8 * j) = make_uint2(pack_bytes(c), pack_bytes(c + 4));
            } else {
                uint32_t pw0 = 0u, pw1 = 0u, pw2 = 0u;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int v = 8 * (j & 3) + i;
                    const uint32_t bit = 1u << (16 * (v & 1) + (v >> 1));
                    pw0 |= (c[i] & 1u) ? bit : 0u;
                    pw1 |= (c[i] & 2u) ? bit : 0u;
                    pw2 |= (c[i] & 4u) ? bit : 0u;
                }
                pw0 = qdev::or_reduce<4>(pw0);
                pw1 = qdev::or_reduce<4>(pw1);
                pw2 = qdev::or_reduce<4>(pw2);
                if (valid && kb == 0) {
                    uint32_t* kw = reinterpret_cast<uint32_t*>(w.codes + (size_t)row * 48 + 12 * g4);
                    kw[0] = pw0;
                    kw[1] = pw1;
                    kw[2] = pw2;
                }
            }
        } else if (!IS_V && valid) {
            uint8_t* rp = w.codes + (size_t)row * (16 * BITS);
            if (BITS == 4) {
                reinterpret_cast<uint32_t*>(rp)[4 * kb + g4] = pack_k4(c);
            } else {
                *reinterpret_cast<uint2*>(rp + 8 * (4 * kb + g4)) = make_uint2(pack_bytes(c), pack_bytes(c + 4));
            }
        }
        if (IS_V && BITS != 3) {
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[(8 * j + i) * 8 + i_tok] = (uint8_t)c[i];
        }
        if (valid && kb == 0) {
            uint16_t* m = reinterpret_cast<uint16_t*>(w.meta + (size_t)row * 16);
            m[g4] = s16;
            m[4 + g4] = z16;
        }
    }
    if (IS_V && BITS == 3) {
        __builtin_amdgcn_wave_barrier();
        v3_plane_words(w, g, t_lo, t_hi, wv);
        __builtin_amdgcn_wave_barrier();
    } else if (IS_V) {
        // lane L forms V words w = 2L and 2L + 1 of the octet's 128 (word w holds channel
        // 16 (w % 8) + w / 8): channels 32 (L % 4) + L / 4 and that + 16
        __builtin_amdgcn_wave_barrier();
        const int da = 32 * (L & 3) + (L >> 2);
        const uint2 ca = *reinterpret_cast<const uint2*>(wv + da * 8);
        const uint2 cb = *reinterpret_cast<const uint2*>(wv + (da + 16) * 8);
        __builtin_amdgcn_wave_barrier();
        const int blk = g >> 2, kb = g & 3;
        const bool full = t_hi - t_lo == 8;
        if (BITS == 4) {
            uint2 v = make_uint2(pack_v4(ca.x, ca.y), pack_v4(cb.x, cb.y));
            uint2* dst = reinterpret_cast<uint2*>(w.codes + (size_t)blk * 2048 + 4 * (128 * kb + 2 * L));
            if (!full) {
                const uint32_t m = (uint32_t)v_token_mask<4>(t_lo - 8 * g, t_hi - 8 * g);
                const uint2 old = *dst;
                v.x = (old.x & ~m) | (v.x & m);
                v.y = (old.y & ~m) | (v.y & m);
            }
            *dst = v;
        } else {
            uint4 v = make_uint4(ca.x, ca.y, cb.x, cb.y);
            uint4* dst = reinterpret_cast<uint4*>(w.codes + (size_t)blk * 4096 + 8 * (128 * kb + 2 * L));
            if (!full) {
                const uint64_t m = v_token_mask<8>(t_lo - 8 * g, t_hi - 8 * g);
                const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
                const uint4 old = *dst;
                v.x = (old.x & ~ml) | (v.x & ml);
                v.y = (old.y & ~mh) | (v.y & mh);
                v.z = (old.z & ~ml) | (v.z & ml);
                v.w = (old.w & ~mh) | (v.w & mh);
            }
            *dst = v;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// TurboQuant planes
// ---------------------------------------------------------------------------------------------

// Pairwise tree sum of the squares of the 128 values a 16-lane group holds, 8 per lane: three
// levels inside the lane, then lane partners at distances 1, 2, 4, 8 (the index-order tree).
__device__ __forceinline__ float tree_sum_sq16(const float* e) {
    const float l0 = e[0] * e[0] + e[1] * e[1], l1 = e[2] * e[2] + e[3] * e[3];
    const float l2 = e[4] * e[4] + e[5] * e[5], l3 = e[6] * e[6] + e[7] * e[7];
    const float t = (l0 + l1) + (l2 + l3);
    return xor_reduce<16>(t, [](float x, float y) { return x + y; });
}

// Bytes of LDS per wave of the TurboQuant bulk kernels: 128 channels x 4 tokens of binary32
// residuals (QJL K planes, one round) or 128 channels x 8 tokens of one-byte codes (V planes).
constexpr int kTurboWaveLds = 4 * kDim * 4;

// Per-wave constants of a TurboQuant plane: the 7 ascending thresholds and the 8 levels, as
// separate values (kept in registers; selects between them never become indexed loads).
struct TurboTabs {
    float t0, t1, t2, t3, t4, t5, t6;
    float m0, m1, m2, m3, m4, m5, m6, m7;
};

// Lloyd-Max code of u: the number of thresholds below u, found by a binary search over the
// ascending thresholds (the same count as comparing u with each of them).  b0, b1, b2: its bits.
__device__ __forceinline__ void turbo_code(float u, const TurboTabs T, bool& b0, bool& b1, bool& b2) {
    const float t0 = T.t0, t1 = T.t1, t2 = T.t2, t3 = T.t3, t4 = T.t4, t5 = T.t5, t6 = T.t6;
    b2 = u > t3;
    b1 = u > (b2 ? t5 : t1);
    b0 = u > (b2 ? (b1 ? t6 : t4) : (b1 ? t2 : t0));
}

__device__ __forceinline__ float turbo_level(bool b0, bool b1, bool b2, const TurboTabs T) {
    const float hi = b1 ? (b0 ? T.m7 : T.m6) : (b0 ? T.m5 : T.m4);
    const float lo = b1 ? (b0 ? T.m3 : T.m2) : (b0 ? T.m1 : T.m0);
    return b2 ? hi : lo;
}


// acc = (r of lane LN of this 16-lane row) * s + acc with one rounding: v_fmac_f32 with a
// row_newbcast DPP source, the same binary32 result as fmaf(s, r_LN, acc).
template <int LN>
__device__ __forceinline__ void fmac_row_bcast(float& acc, float r, float s) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(r), "v"(s), "n"(LN));
}

// Step j = JJ of the QJL chains of a round's 4 tokens (residual (JJ, token) is value 4 JJ + token,
// held by lane JJ % 16 of every row in register (JJ / 16, token)).
template <int JJ>
__device__ __forceinline__ void qjl_step(const float (&rv)[8][4], const float* st, int L, float* acc0,
                                         float* acc1) {
    constexpr int lane = JJ % 16, m = JJ / 16;
    const float s0 = st[JJ * kDim + L], s1 = st[JJ * kDim + 64 + L];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        fmac_row_bcast<lane>(acc0[c], rv[m][c], s0);
        fmac_row_bcast<lane>(acc1[c], rv[m][c], s1);
    }
}

template <int... JJ>
__device__ __forceinline__ void qjl_chain(const float (&rv)[8][4], const float* st, int L, float* acc0,
                                          float* acc1, std::integer_sequence<int, JJ...>) {
    (qjl_step<JJ>(rv, st, L, acc0, acc1), ...);
}

// One octet g of a TurboQuant plane (QJL: TurboQuant-QJL K plane; else TurboQuant-MSE, K or V).
// wl: kTurboWaveLds bytes of the wave's LDS.  st: S^T ([j][i] = S[i][j], 128 x 128) in LDS (QJL).
// kbit[i]: 1 << (the bit of channel 8j + i in its K plane words).
template <bool QJL>
__device__ __forceinline__ void turbo_octet(const WavePlane& w, bool IS_V, int g, const OctetIn& in,
                                            const uint32_t* sgm, const TurboTabs T,
                                            const uint32_t* kbit, float* wl, const float* st,
                                            uint8_t* qjl_base) {
    const int L = lane_id(), tk = L >> 4, j = L & 15;
    const int t_lo = max(w.start, 8 * g), t_hi = min(w.end, 8 * g + 8);
    if (t_lo >= t_hi) return;
    uint8_t* wv = reinterpret_cast<uint8_t*>(wl);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i_tok = 4 * r + tk, t = 8 * g + i_tok;
        const bool valid = t >= t_lo && t < t_hi;
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = in.v[r][i];
        if (w.window > 0 && valid && t >= w.end - w.window) {
            float4* ring = reinterpret_cast<float4*>(w.ring + (size_t)(t % w.window) * kDim + 8 * j);
            ring[0] = make_float4(e[0], e[1], e[2], e[3]);
            ring[1] = make_float4(e[4], e[5], e[6], e[7]);
        }
        rotate(e, sgm, j);
        const uint16_t n16 = f16_rn(sqrtf(tree_sum_sq16(e)));
        const float n = f16_val(n16);
        const float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
        uint32_t pw0 = 0u, pw1 = 0u, pw2 = 0u, codes_lo = 0u, codes_hi = 0u;
        float rr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bool b0, b1, b2;
            turbo_code(e[i] * inv, T, b0, b1, b2);
            if (IS_V) {
                const uint32_t q = (b0 ? 1u : 0u) | (b1 ? 2u : 0u) | (b2 ? 4u : 0u);
                if (i < 4) codes_lo |= q << (8 * i);
                else codes_hi |= q << (8 * (i - 4));
            } else {
                pw0 |= b0 ? kbit[i] : 0u;
                pw1 |= b1 ? kbit[i] : 0u;
                pw2 |= b2 ? kbit[i] : 0u;
            }
            if (QJL) rr[i] = e[i] - n * turbo_level(b0, b1, b2, T);
        }
        if (IS_V) {
            *reinterpret_cast<uint2*>(wv + (size_t)i_tok * kDim + 8 * j) = make_uint2(codes_lo, codes_hi);
            if (valid && j == 0) reinterpret_cast<uint16_t*>(w.meta)[t] = n16;
            continue;
        }
        // K row of token t: plane words of group j / 4, merged over its 4 lanes
        pw0 = qdev::or_reduce<4>(pw0);
        pw1 = qdev::or_reduce<4>(pw1);
        pw2 = qdev::or_reduce<4>(pw2);
        const int row = k_row(t);
        if (valid && (j & 3) == 0) {
            uint32_t* kw = reinterpret_cast<uint32_t*>(w.codes + (size_t)row * 48 + 12 * (j >> 2));
            kw[0] = pw0;
            kw[1] = pw1;
            kw[2] = pw2;
        }
        if (QJL) {
            const uint16_t g16 = f16_rn(sqrtf(tree_sum_sq16(rr)));
            if (valid && j == 0) {
                uint16_t* m = reinterpret_cast<uint16_t*>(w.meta + (size_t)row * 4);
                m[0] = n16;
                m[1] = g16;
            }
            // sign(S r) of this round's 4 tokens: lane L forms projections L and 64 + L, each a
            // sequential fma chain over j = 0 .. 127.  The residual of channel 8j + i of token
            // tk goes to wl[(8j + i) * 4 + tk]; then every 16-lane row holds all 512 of them
            // (value v at lane (v % 64) / 4, register (v / 64, v % 4)) and each fma takes its
            // residual by a row broadcast; only the rows of S^T come from LDS.
#pragma unroll
            for (int i = 0; i < 8; ++i) wl[(8 * j + i) * 4 + tk] = rr[i];
            __builtin_amdgcn_wave_barrier();
            float rv[8][4];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float4 x = *reinterpret_cast<const float4*>(wl + 64 * m + 4 * j);
                rv[m][0] = x.x;
                rv[m][1] = x.y;
                rv[m][2] = x.z;
                rv[m][3] = x.w;
            }
            __builtin_amdgcn_wave_barrier();
            float acc0[4], acc1[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc0[c] = acc1[c] = 0.0f;
            qjl_chain(rv, st, L, acc0, acc1, std::make_integer_sequence<int, kDim>{});
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint64_t m0 = __ballot(acc0[c] >= 0.0f);
                const uint64_t m1 = __ballot(acc1[c] >= 0.0f);
                const int tc = 8 * g + 4 * r + c;
                if (L == c && tc >= t_lo && tc < t_hi) {
                    uint4 qw;
                    qw.x = qdev::unshuffle32((uint32_t)m0);
                    qw.y = qdev::unshuffle32((uint32_t)(m0 >> 32));
                    qw.z = qdev::unshuffle32((uint32_t)m1);
                    qw.w = qdev::unshuffle32((uint32_t)(m1 >> 32));
                    *reinterpret_cast<uint4*>(qjl_base + (size_t)k_row(tc) * 16) = qw;
                }
            }
        } else if (valid && j == 0) {
            reinterpret_cast<uint16_t*>(w.meta)[row] = n16;
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (IS_V) v3_plane_words(w, g, t_lo, t_hi, wv);
    __builtin_amdgcn_wave_barrier();
}

// 15 thresholds of the 16-level codebook, by value (a select-of-array would index scratch).
struct TurboTabs4 {
    float t0, t1, t2, t3, t4, t5, t6, t7, t8, t9, t10, t11, t12, t13, t14;
};

// 4-bit Lloyd-Max code of u: the number of thresholds below u, by a binary search over the
// ascending thresholds (bit 3 against t7, bit 2 against t3 / t11, bit 1 against t(4q + 1), bit 0
// against t(2q), q = the code's bits found so far).
__device__ __forceinline__ uint32_t turbo_code4(float u, const TurboTabs4 T) {
    const bool b3 = u > T.t7;
    const bool b2 = u > (b3 ? T.t11 : T.t3);
    const float x1 = b3 ? (b2 ? T.t13 : T.t9) : (b2 ? T.t5 : T.t1);
    const bool b1 = u > x1;
    const float x0 = b3 ? (b2 ? (b1 ? T.t14 : T.t12) : (b1 ? T.t10 : T.t8))
                        : (b2 ? (b1 ? T.t6 : T.t4) : (b1 ? T.t2 : T.t0));
    const bool b0 = u > x0;
    return (b3 ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

// One octet g of a 4-bit TurboQuant-MSE V plane (four bit planes).  wl: kTurboWaveLds bytes of
// the wave's LDS (codes staged as [token][channel] bytes).
__device__ __forceinline__ void turbo4_v_octet(const WavePlane& w, int g, const OctetIn& in, const uint32_t* sgm,
                                               const TurboTabs4 T, float* wl) {
    const int L = lane_id(), tk = L >> 4, j = L & 15;
    const int t_lo = max(w.start, 8 * g), t_hi = min(w.end, 8 * g + 8);
    if (t_lo >= t_hi) return;
    uint8_t* wv = reinterpret_cast<uint8_t*>(wl);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i_tok = 4 * r + tk, t = 8 * g + i_tok;
        const bool valid = t >= t_lo && t < t_hi;
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = in.v[r][i];
        if (w.window > 0 && valid && t >= w.end - w.window) {
            float4* ring = reinterpret_cast<float4*>(w.ring + (size_t)(t % w.window) * kDim + 8 * j);
            ring[0] = make_float4(e[0], e[1], e[2], e[3]);
            ring[1] = make_float4(e[4], e[5], e[6], e[7]);
        }
        rotate(e, sgm, j);
        const uint16_t n16 = f16_rn(sqrtf(tree_sum_sq16(e)));
        const float n = f16_val(n16);
        const float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
        uint32_t codes_lo = 0u, codes_hi = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t q = turbo_code4(e[i] * inv, T);
            if (i < 4) codes_lo |= q << (8 * i);
            else codes_hi |= q << (8 * (i - 4));
        }
        *reinterpret_cast<uint2*>(wv + (size_t)i_tok * kDim + 8 * j) = make_uint2(codes_lo, codes_hi);
        if (valid && j == 0) reinterpret_cast<uint16_t*>(w.meta)[t] = n16;
    }
    __builtin_amdgcn_wave_barrier();
    // block words: bit k of channel d -> word 8 (16 o + d % 16) + 2k + (d / 16) / 4, token i at bit
    // 16 (i % 2) + 4 ((d / 16) % 4) + i / 2.  Lane L (< 32) forms the four words of n = L % 16,
    // h = L / 16 (channels 16 N + n, N = 4h .. 4h + 3); lanes 32 + L take channels N = 4h + 2,
    // 4h + 3 of the same words, merged by the lane 32 apart.
    const int n = L & 15, h = (L >> 4) & 1, half = L >> 5;
    uint32_t wk0 = 0u, wk1 = 0u, wk2 = 0u, wk3 = 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int Nl = 2 * half + c; // N % 4
        const int d = 16 * (4 * h + Nl) + n;
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (uint32_t)wv[i * kDim + d] << (8 * i);
            hi |= (uint32_t)wv[(i + 4) * kDim + d] << (8 * i);
        }
        const uint32_t ev = __builtin_amdgcn_perm(hi, lo, 0x06040200u); // tokens 0, 2, 4, 6
        const uint32_t od = __builtin_amdgcn_perm(hi, lo, 0x07050301u); // tokens 1, 3, 5, 7
        wk0 |= (byte_bits(ev, 0) | (byte_bits(od, 0) << 16)) << (4 * Nl);
        wk1 |= (byte_bits(ev, 1) | (byte_bits(od, 1) << 16)) << (4 * Nl);
        wk2 |= (byte_bits(ev, 2) | (byte_bits(od, 2) << 16)) << (4 * Nl);
        wk3 |= (byte_bits(ev, 3) | (byte_bits(od, 3) << 16)) << (4 * Nl);
    }
    wk0 |= xor_lane<32>(wk0);
    wk1 |= xor_lane<32>(wk1);
    wk2 |= xor_lane<32>(wk2);
    wk3 |= xor_lane<32>(wk3);
    __builtin_amdgcn_wave_barrier();
    if (half == 0) {
        const int o = g & 3;
        uint32_t* blk = reinterpret_cast<uint32_t*>(w.codes + (size_t)(g >> 2) * 2048) + 8 * (16 * o + n) + h;
        if (t_hi - t_lo == 8) {
            blk[0] = wk0;
            blk[2] = wk1;
            blk[4] = wk2;
            blk[6] = wk3;
        } else {
            // token bits of the octet present in this append
            uint32_t m = 0u;
            for (int i = t_lo - 8 * g; i < t_hi - 8 * g; ++i) m |= 0x1111u << (16 * (i & 1) + (i >> 1));
            blk[0] = (blk[0] & ~m) | (wk0 & m);
            blk[2] = (blk[2] & ~m) | (wk1 & m);
            blk[4] = (blk[4] & ~m) | (wk2 & m);
            blk[6] = (blk[6] & ~m) | (wk3 & m);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------------------------
// Split TurboQuant V (outlier split): one wave per (octet, half).  Lane L takes token L / 8 of
// the octet and positions 8 (L % 8) .. + 7 of the wave's half (channels perm[.] of the source row,
// gathered); the 64-point rotation runs inside the lane (spans 1, 2, 4) and across lanes L ^ 1,
// 2, 4 (spans 8, 16, 32); the norm is the index-order tree over the half; the half's codebook
// is uniform per wave.  Codes are staged as [token][position] bytes in the wave's LDS and formed
// into the half's plane words: word W (16 o + n) + k (outliers) or + bo + k (the rest).
// ---------------------------------------------------------------------------------------------
struct SplitIn {
    float v[8];
};

__device__ __forceinline__ void load_split(const WavePlane& w, int g, const int* pm, SplitIn& in) {
    const int t = 8 * g + (lane_id() >> 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) in.v[i] = 0.0f;
    if (t >= w.start && t < w.end) {
        // w.src points at channel 8 (lane % 16) of the row; step back to channel 0
        const int j16 = lane_id() & 15;
        const char* row = w.src + (size_t)(t - w.start) * w.tok_bytes - (size_t)8 * j16 * (w.dtype == 0 ? 4 : 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (w.dtype == 0) in.v[i] = reinterpret_cast<const float*>(row)[pm[i]];
            else in.v[i] = in16_to_f32(reinterpret_cast<const uint16_t*>(row)[pm[i]], w.dtype);
        }
    }
}

// Code of u with NB bits: the number of thresholds below u, by binary search over the ascending
// thresholds t0 .. t(2^NB - 2) (named values: a select over an array would index scratch).
template <int NB>
__device__ __forceinline__ uint32_t split_code(float u, const TurboTabs4& T) {
    if constexpr (NB == 2) {
        const bool b1 = u > T.t1;
        const bool b0 = u > (b1 ? T.t2 : T.t0);
        return (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
    } else if constexpr (NB == 3) {
        const bool b2 = u > T.t3;
        const bool b1 = u > (b2 ? T.t5 : T.t1);
        const bool b0 = u > (b2 ? (b1 ? T.t6 : T.t4) : (b1 ? T.t2 : T.t0));
        return (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
    } else {
        return turbo_code4(u, T);
    }
}

// NB = the half's code bits (bo for the outliers, bo - 1 for the rest), hv = the half.
template <int BO, int NB>
__device__ __forceinline__ void split_v_octet(const WavePlane& w, int g, int hv, const SplitIn& in, const int* pm,
                                              const uint32_t* sgm, const TurboTabs4& th, float* wl) {
    constexpr int W = 2 * BO - 1;
    const int L = lane_id(), tk = L >> 3, j = L & 7;
    const int t_lo = max(w.start, 8 * g), t_hi = min(w.end, 8 * g + 8);
    if (t_lo >= t_hi) return;
    uint8_t* wv = reinterpret_cast<uint8_t*>(wl);
    const int t = 8 * g + tk;
    const bool valid = t >= t_lo && t < t_hi;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = in.v[i];
    if (w.window > 0 && valid && t >= w.end - w.window) {
        float* ring = w.ring + (size_t)(t % w.window) * kDim;
#pragma unroll
        for (int i = 0; i < 8; ++i) ring[pm[i]] = e[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = __uint_as_float(__float_as_uint(e[i]) ^ sgm[i]);
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & h)) {
                const float x = e[i], y = e[i + h];
                e[i] = x + y;
                e[i + h] = x - y;
            }
    cross8<1>(e, j);
    cross8<2>(e, j);
    cross8<4>(e, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = e[i] * 0.125f;
    const float l0 = e[0] * e[0] + e[1] * e[1], l1 = e[2] * e[2] + e[3] * e[3];
    const float l2 = e[4] * e[4] + e[5] * e[5], l3 = e[6] * e[6] + e[7] * e[7];
    const float nsq = xor_reduce<8>((l0 + l1) + (l2 + l3), [](float x, float y) { return x + y; });
    const uint16_t n16 = f16_rn(sqrtf(nsq));
    const float n = f16_val(n16);
    const float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t q = split_code<NB>(e[i] * inv, th);
        if (i < 4) lo |= q << (8 * i);
        else hi |= q << (8 * (i - 4));
    }
    *reinterpret_cast<uint2*>(wv + (size_t)tk * 64 + 8 * j) = make_uint2(lo, hi);
    if (valid && j == 0) reinterpret_cast<uint16_t*>(w.meta)[2 * t + hv] = n16;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // lane L < 32: column n = L % 16, quads Nq = 2 (L / 16) + {0, 1} of the half's positions
    // 16 Nq + n; lanes L and L + 16 then hold complementary nibbles of the same words
    const int n_ = L & 15, cp = (L >> 4) & 1;
    uint32_t wk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int Nq = 2 * cp + c, d = 16 * Nq + n_;
        uint32_t lo4 = 0u, hi4 = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo4 |= (uint32_t)wv[i * 64 + d] << (8 * i);
            hi4 |= (uint32_t)wv[(i + 4) * 64 + d] << (8 * i);
        }
        const uint32_t ev = __builtin_amdgcn_perm(hi4, lo4, 0x06040200u); // tokens 0, 2, 4, 6
        const uint32_t od = __builtin_amdgcn_perm(hi4, lo4, 0x07050301u); // tokens 1, 3, 5, 7
#pragma unroll
        for (int k = 0; k < NB; ++k) wk[k] |= (byte_bits(ev, k) | (byte_bits(od, k) << 16)) << (4 * Nq);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) wk[k] |= xor_lane<16>(wk[k]);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (L < 16) {
        const int o = g & 3;
        uint32_t* blk = reinterpret_cast<uint32_t*>(w.codes + (size_t)(g >> 2) * (256 * W)) + W * (16 * o + n_) +
                        (hv ? BO : 0);
        if (t_hi - t_lo == 8) {
#pragma unroll
            for (int k = 0; k < NB; ++k) blk[k] = wk[k];
        } else {
            uint32_t m = 0u;
            for (int i = t_lo - 8 * g; i < t_hi - 8 * g; ++i) m |= 0x1111u << (16 * (i & 1) + (i >> 1));
#pragma unroll
            for (int k = 0; k < NB; ++k) blk[k] = (blk[k] & ~m) | (wk[k] & m);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

} // namespace qbulk
} // namespace kvq
