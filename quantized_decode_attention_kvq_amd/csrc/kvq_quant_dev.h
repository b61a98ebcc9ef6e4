// Device code of quantize-on-append, shared by the append kernel and the fused append + decode
// kernel.  Every translation unit that includes it is compiled with -ffp-contract=off, so each
// binary32 operation rounds separately, in the order written, and the packed codes and fp16
// scales are bit-identical to any other implementation of the same format; fmaf() is used only
// where the format fuses (the QJL projection).
//
// Method sources (pages by title and section):
//  - quantcpp article "Beyond RAG...", progressive table + "how it works": 4-bit codes with fp16
//    scale and zero per 32 channels (6.4x), newest 128 tokens kept in FP32.
//  - KVarN-on-Bonsai post, TL;DR: Walsh-Hadamard transform and Sinkhorn variance balancing
//    before 4-bit quantization.
//  - "LLM memory saving ... 2026", TurboQuant row of the method table: random rotation,
//    per-coordinate optimal scalar quantizer, 1-bit QJL of the residual.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_lanes.h"

namespace kvq {
namespace qdev {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float c0f() { return __uint_as_float(0x3DB504F3u); } // 2^-3.5

__device__ __forceinline__ uint16_t f16_rn(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ float f16_val(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Largest binary16 <= x: round to nearest, step down one binary16 ulp if that overshot.
__device__ __forceinline__ uint16_t f16_rd(float x) {
    uint16_t h = f16_rn(x);
    if (f16_val(h) > x) {
        if ((h & 0x7fff) == 0)
            h = 0x8001;
        else if (h & 0x8000)
            h = (uint16_t)(h + 1);
        else
            h = (uint16_t)(h - 1);
    }
    return h;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Lane l loads channels 2l and 2l+1 of one 128-vector.
__device__ __forceinline__ void load_pair(const void* base, size_t elem_off, int dtype, float& a,
                                          float& b) {
    const int l = lane_id();
    if (dtype == 0) {
        const float2 v = reinterpret_cast<const float2*>(
            static_cast<const float*>(base) + elem_off)[l];
        a = v.x;
        b = v.y;
    } else {
        const uint32_t v = reinterpret_cast<const uint32_t*>(
            static_cast<const uint16_t*>(base) + elem_off)[l];
        a = bf16_to_f32((uint16_t)(v & 0xffff));
        b = bf16_to_f32((uint16_t)(v >> 16));
    }
}

// Sylvester-Hadamard butterflies over a wave (lane l holds elements 2l, 2l+1), spans
// h = 1, 2, ..., 64 in ascending order; pair (i, i+h) with bit h of i clear maps to
// (t_i + t_{i+h}, t_i - t_{i+h}).  The lane holding the upper element forms partner - own,
// which is the same binary32 value as t_i - t_{i+h}.
template <int M>
__device__ __forceinline__ void hadamard_step(float& a, float& b, int l) {
    const float pa = xor_lane<M>(a), pb = xor_lane<M>(b);
    const bool lower = (l & M) == 0;
    a = lower ? (a + pa) : (pa - a);
    b = lower ? (b + pb) : (pb - b);
}
__device__ __forceinline__ void hadamard_wave(float& a, float& b) {
    const int l = lane_id();
    const float s = a + b, d = a - b;
    a = s;
    b = d;
    hadamard_step<1>(a, b, l);
    hadamard_step<2>(a, b, l);
    hadamard_step<4>(a, b, l);
    hadamard_step<8>(a, b, l);
    hadamard_step<16>(a, b, l);
    hadamard_step<32>(a, b, l);
}

// R(x) = c0 * H (d .* x).
__device__ __forceinline__ void rotate_wave(float& a, float& b, const float* signs) {
    const int l = lane_id();
    if (signs[2 * l] < 0.0f) a = -a;
    if (signs[2 * l + 1] < 0.0f) b = -b;
    hadamard_wave(a, b);
    a = a * c0f();
    b = b * c0f();
}

// R(x) = c0 * H (d .* x) with the lane's two signs already loaded.
__device__ __forceinline__ void rotate_signed(float& a, float& b, float s0, float s1) {
    if (s0 < 0.0f) a = -a;
    if (s1 < 0.0f) b = -b;
    hadamard_wave(a, b);
    a = a * c0f();
    b = b * c0f();
}

// Index-order pairwise sum of v^2 over the 128 elements (level 1 inside the lane, then lane
// pairs at distance 1, 2, ..., 32); every lane returns the total.
__device__ __forceinline__ float tree_sum_sq(float a, float b) {
    const float t = a * a + b * b;
    return xor_reduce<64>(t, [](float x, float y) { return x + y; });
}

template <int W>
__device__ __forceinline__ uint32_t or_reduce(uint32_t v) {
    return xor_reduce<W>(v, [](uint32_t x, uint32_t y) { return x | y; });
}

// Half-interleave: bit e of x moves to bit 16*(e%2) + e/2 (even bits to the low half, odd bits
// to the high half, order kept), by four swaps of bit fields.
__device__ __forceinline__ uint32_t unshuffle32(uint32_t x) {
    x = ((x & 0x22222222u) << 1) | ((x >> 1) & 0x22222222u) | (x & 0x99999999u);
    x = ((x & 0x0C0C0C0Cu) << 2) | ((x >> 2) & 0x0C0C0C0Cu) | (x & 0xC3C3C3C3u);
    x = ((x & 0x00F000F0u) << 4) | ((x >> 4) & 0x00F000F0u) | (x & 0xF00FF00Fu);
    x = ((x & 0x0000FF00u) << 8) | ((x >> 8) & 0x0000FF00u) | (x & 0xFF0000FFu);
    return x;
}

__device__ __forceinline__ int k_row(int t) { return 64 * (t / 64) + 16 * ((t % 64) % 4) + (t % 64) / 4; }

// Uniform quantizer of the two elements a lane holds; the lane's group is lanes 16g..16g+15.
__device__ __forceinline__ void quant_uniform(float a, float b, int bits, uint32_t& c0, uint32_t& c1,
                                              uint16_t& s16, uint16_t& z16) {
    float mn = fminf(a, b), mx = fmaxf(a, b);
    mn = xor_reduce<16>(mn, [](float x, float y) { return fminf(x, y); });
    mx = xor_reduce<16>(mx, [](float x, float y) { return fmaxf(x, y); });
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    const float L = (float)((1 << bits) - 1);
    z16 = f16_rd(mn);
    const float z = f16_val(z16);
    const float s32 = (mx - z) / L;
    s16 = f16_rn(s32);
    const float s = f16_val(s16);
    const float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
    float u0 = (a - z) * inv, u1 = (b - z) * inv;
    u0 = fminf(fmaxf(rintf(u0), 0.0f), L);
    u1 = fminf(fmaxf(rintf(u1), 0.0f), L);
    c0 = (uint32_t)u0;
    c1 = (uint32_t)u1;
}

struct Unit {
    int tensor, b, head, grp;
};

// Quantize-on-append of one wave's unit: the tokens of (tensor, sequence b, kv head, 8-token
// octet `unit` counted from the octet of p.start[b]) that this call appends.  rbuf: 128 floats of
// LDS owned by the wave (QJL residual staging).  Owning whole octets makes the V
// read-modify-write race free.
__device__ __forceinline__ void quantize_wave(const QuantParams& p, int tensor, int b, int head,
                                              int unit, float* rbuf) {
    const int l = lane_id();
    if (unit >= p.groups8) return;
    const int start = p.start[b];
    const int end = start + p.T;
    const int g0 = start / 8 + unit;
    const int t_lo = max(start, 8 * g0), t_hi = min(end, 8 * g0 + 8);
    if (t_lo >= t_hi) return;

    const PlaneGeom& G = p.geom[tensor];
    char* slot = p.layer_base + (size_t)b * p.seq_stride + (size_t)head * p.head_stride +
                 p.plane_off[tensor];
    uint8_t* codes = reinterpret_cast<uint8_t*>(slot + G.codes_off);
    uint8_t* meta = reinterpret_cast<uint8_t*>(slot + G.meta_off);
    const float* signs = p.signs[tensor] ? p.signs[tensor] + (size_t)(head * 2 + tensor) * kDim : nullptr;
    const float* inv_c = p.inv_c[tensor] ? p.inv_c[tensor] + (size_t)(head * 2 + tensor) * kDim : nullptr;

    // V uniform accumulators for the group's packed words (channels 2l and 2l+1).
    uint64_t vacc0 = 0, vacc1 = 0, vmask = 0;
    // V turbo bit-plane words of channels 2l and 2l+1 for this octet, and the bits written.
    uint32_t tv_a[3] = {0u, 0u, 0u}, tv_c[3] = {0u, 0u, 0u}, tv_mask = 0u;

    // all of the octet's source values are requested before the first is used, so a wave pays
    // one memory round trip instead of one per token
    float pa[8], pc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        pa[i] = pc[i] = 0.0f;
        if (t_lo + i < t_hi) {
            const size_t elem = (((size_t)b * p.T + (t_lo + i - start)) * p.Hkv + head) * kDim;
            load_pair(p.src[tensor], elem, p.dtype, pa[i], pc[i]);
        }
    }
    const float* sg_l = signs ? signs + 2 * l : nullptr;
    const float* ic_l = inv_c ? inv_c + 2 * l : nullptr;
    float sg0 = 1.0f, sg1 = 1.0f, ic0 = 1.0f, ic1 = 1.0f;
    if (sg_l) {
        sg0 = sg_l[0];
        sg1 = sg_l[1];
    }
    if (G.scheme == kUniform && G.sinkhorn) {
        ic0 = ic_l[0];
        ic1 = ic_l[1];
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = t_lo + i;
        if (t >= t_hi) break;
        float a = pa[i], c = pc[i];

        if (p.window > 0 && t >= end - p.window) {
            float* ring = reinterpret_cast<float*>(slot + G.ring_off) + (size_t)(t % p.window) * kDim;
            reinterpret_cast<float2*>(ring)[l] = make_float2(a, c);
        }

        if (G.scheme == kUniform) {
            if (G.rotate) rotate_signed(a, c, sg0, sg1);
            if (G.sinkhorn) {
                a = a * ic0;
                c = c * ic1;
            }
            uint32_t q0, q1;
            uint16_t s16, z16;
            quant_uniform(a, c, G.bits, q0, q1, s16, z16);
            const int g = l >> 4;
            if (tensor == 0) {
                const int row = k_row(t);
                uint8_t* r = codes + (size_t)row * (16 * G.bits);
                const int kb = (l & 15) >> 2, i = 2 * (l & 3);
                if (G.bits == 4) {
                    uint32_t w = (q0 << (4 * (l & 3))) | (q1 << (16 + 4 * (l & 3)));
                    w = or_reduce<4>(w);
                    if ((l & 3) == 0) reinterpret_cast<uint32_t*>(r)[4 * kb + g] = w;
                } else {
                    *reinterpret_cast<uint16_t*>(r + 8 * (4 * kb + g) + i) = (uint16_t)(q0 | (q1 << 8));
                }
                if ((l & 15) == 0) {
                    uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)row * 16);
                    m[g] = s16;
                    m[4 + g] = z16;
                }
            } else {
                const int i = t % 8;
                const int sh = (G.bits == 4) ? 16 * (i % 2) + 4 * (i / 2) : 8 * i;
                vacc0 |= (uint64_t)q0 << sh;
                vacc1 |= (uint64_t)q1 << sh;
                vmask |= (uint64_t)((1u << G.bits) - 1) << sh;
                if ((l & 15) == 0) {
                    uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)t * 16);
                    m[g] = s16;
                    m[4 + g] = z16;
                }
            }
        } else {
            // TurboQuant code: rho = R(x); n = fp16(|rho|); codes = #thresholds below rho/n;
            // residual r = rho - n mu[code]; QJL bits = sign(S r) with a sequential fma chain.
            rotate_signed(a, c, sg0, sg1);
            const float nsq = tree_sum_sq(a, c);
            const uint16_t n16 = f16_rn(sqrtf(nsq));
            const float n = f16_val(n16);
            const float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
            const float ua = a * inv, uc = c * inv;
            uint32_t qa = 0, qc = 0;
#pragma unroll
            for (int k = 0; k < 7; ++k) {
                const float th = p.theta[k];
                qa += (ua > th) ? 1u : 0u;
                qc += (uc > th) ? 1u : 0u;
            }
            const float pa = n * p.mu[qa], pc = n * p.mu[qc];
            const float ra = a - pa, rc = c - pc;
            if (tensor == 0) {
                // K row: bit planes of group g (lanes 16g..16g+15 hold its channels 2lg, 2lg+1,
                // i.e. half-interleaved values lg and 16 + lg)
                const int lg = l & 15, g = l >> 4;
                const int row = k_row(t);
                uint32_t pw[3];
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    pw[k] = or_reduce<16>((((qa >> k) & 1u) << lg) | (((qc >> k) & 1u) << (16 + lg)));
                if (lg == 0) {
                    uint32_t* w = reinterpret_cast<uint32_t*>(codes + (size_t)row * 48 + 12 * g);
                    w[0] = pw[0];
                    w[1] = pw[1];
                    w[2] = pw[2];
                }
                if (G.scheme == kTurboQjl) {
                    const uint16_t g16 = f16_rn(sqrtf(tree_sum_sq(ra, rc)));
                    rbuf[2 * l] = ra;
                    rbuf[2 * l + 1] = rc;
                    __builtin_amdgcn_wave_barrier();
                    float acc0 = 0.0f, acc1 = 0.0f;
                    for (int j = 0; j < kDim; ++j) {
                        const float rj = rbuf[j];
                        acc0 = fmaf(p.qjl_st[j * kDim + l], rj, acc0);
                        acc1 = fmaf(p.qjl_st[j * kDim + 64 + l], rj, acc1);
                    }
                    __builtin_amdgcn_wave_barrier();
                    const uint64_t b0 = __ballot(acc0 >= 0.0f);
                    const uint64_t b1 = __ballot(acc1 >= 0.0f);
                    if (l == 0) {
                        uint32_t* qj = reinterpret_cast<uint32_t*>(slot + G.qjl_off + (size_t)row * 16);
                        qj[0] = unshuffle32((uint32_t)b0);
                        qj[1] = unshuffle32((uint32_t)(b0 >> 32));
                        qj[2] = unshuffle32((uint32_t)b1);
                        qj[3] = unshuffle32((uint32_t)(b1 >> 32));
                        uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)row * 4);
                        m[0] = n16;
                        m[1] = g16;
                    }
                } else if (l == 0) {
                    reinterpret_cast<uint16_t*>(meta)[row] = n16;
                }
            } else {
                // V block: bit k of channel 2l (2l+1) goes to word 6(16 o + n) + 2k + N/4 with
                // n = 2(l%8) (+1), N = l/8; token i of the octet at bit 16(i%2) + 4(N%4) + i/2
                const int i = t % 8, N = l >> 3;
                const uint32_t pos = 1u << (16 * (i & 1) + 4 * (N & 3) + (i >> 1));
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    tv_a[k] |= ((qa >> k) & 1u) ? pos : 0u;
                    tv_c[k] |= ((qc >> k) & 1u) ? pos : 0u;
                }
                tv_mask |= pos;
                if (l == 0) reinterpret_cast<uint16_t*>(meta)[t] = n16;
            }
        }
    }

    if (tensor == 1 && G.scheme != kUniform) {
        // merge the four lanes (l ^ 8, l ^ 16) whose channels share each word, then
        // read-modify-write this octet's words
        uint32_t m = tv_mask;
        m |= xor_lane<8>(m);
        m |= xor_lane<16>(m);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            tv_a[k] |= xor_lane<8>(tv_a[k]);
            tv_a[k] |= xor_lane<16>(tv_a[k]);
            tv_c[k] |= xor_lane<8>(tv_c[k]);
            tv_c[k] |= xor_lane<16>(tv_c[k]);
        }
        if (((l >> 3) & 3) == 0) {
            const int o = (t_lo % 32) / 8, n0 = 2 * (l & 7), N = l >> 3;
            uint32_t* blk = reinterpret_cast<uint32_t*>(codes + (size_t)(t_lo / 32) * 1536);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                uint32_t* wa = blk + 6 * (16 * o + n0) + 2 * k + (N >> 2);
                uint32_t* wc = wa + 6;
                *wa = (*wa & ~m) | tv_a[k];
                *wc = (*wc & ~m) | tv_c[k];
            }
        }
    }

    if (tensor == 1 && G.scheme == kUniform) {
        // read-modify-write the packed words of channels 2l, 2l+1 for this 8-token group
        const int blk = t_lo / 32, kb = (t_lo % 32) / 8;
        const int d0 = 2 * l, n0 = d0 % 16, N = d0 / 16;
        const int w0 = 8 * (16 * kb + n0) + N, w1 = w0 + 8;
        if (G.bits == 4) {
            uint32_t* bp = reinterpret_cast<uint32_t*>(codes + (size_t)blk * 2048);
            const uint32_t m = (uint32_t)vmask;
            bp[w0] = (bp[w0] & ~m) | (uint32_t)vacc0;
            bp[w1] = (bp[w1] & ~m) | (uint32_t)vacc1;
        } else {
            uint64_t* bp = reinterpret_cast<uint64_t*>(codes + (size_t)blk * 4096);
            bp[w0] = (bp[w0] & ~vmask) | vacc0;
            bp[w1] = (bp[w1] & ~vmask) | vacc1;
        }
    }
}



// ---------------------------------------------------------------------------------------------
// Bulk (prefill) quantizer, lane-dense: a wave quantizes the tokens of one octet of one
// (tensor, sequence, kv head) in two rounds of four tokens.  In round r lane L holds channels
// 8j .. 8j+7 (j = L % 16) of octet token 4r + L / 16.  Every binary32 operation is the same, and
// in the same order, as in quantize_wave (in-lane butterflies for spans 1, 2, 4; lane partners
// at distances 1, 2, 4, 8 for spans 8 .. 64; the same pairwise norm tree; the same sequential
// QJL fma chain), so the packed bytes are identical.
// ---------------------------------------------------------------------------------------------

// Pairwise tree sum of the squares of 128 values held 8 per lane by a 16-lane group.
__device__ __forceinline__ float tree_sum_sq16(const float* e) {
    const float l0 = e[0] * e[0] + e[1] * e[1], l1 = e[2] * e[2] + e[3] * e[3];
    const float l2 = e[4] * e[4] + e[5] * e[5], l3 = e[6] * e[6] + e[7] * e[7];
    const float t = (l0 + l1) + (l2 + l3);
    return xor_reduce<16>(t, [](float x, float y) { return x + y; });
}

// Butterfly span 8 D across lanes j and j ^ D: the lower lane forms own + partner, the upper lane
// partner + (-own), which is the same binary32 value as partner - own.
template <int D>
__device__ __forceinline__ void hadamard_cross8(float* e, int j) {
    const uint32_t neg = (j & D) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float pv = xor_lane<D>(e[i]);
        e[i] = pv + __uint_as_float(__float_as_uint(e[i]) ^ neg);
    }
}

// R(x) for the lane's 8 values: sign flips, Sylvester butterflies (spans 1, 2, 4 in the lane,
// 8, 16, 32, 64 across lanes j ^ 1, 2, 4, 8), then the final c0.
__device__ __forceinline__ void rotate8(float* e, const float* sg, int j) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (sg[i] < 0.0f) e[i] = -e[i];
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & h)) {
                const float x = e[i], y = e[i + h];
                e[i] = x + y;
                e[i + h] = x - y;
            }
    hadamard_cross8<1>(e, j);
    hadamard_cross8<2>(e, j);
    hadamard_cross8<4>(e, j);
    hadamard_cross8<8>(e, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = e[i] * c0f();
}

// Uniform group code of the lane's 8 values; the group is the 4 lanes 4g .. 4g+3 of its token.
__device__ __forceinline__ void quant_uniform8(const float* e, int bits, uint32_t* c, uint16_t& s16,
                                               uint16_t& z16) {
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
    const float L = (float)((1 << bits) - 1);
    z16 = f16_rd(mn);
    const float z = f16_val(z16);
    const float s32 = (mx - z) / L;
    s16 = f16_rn(s32);
    const float s = f16_val(s16);
    const float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float u = (e[i] - z) * inv;
        u = fminf(fmaxf(rintf(u), 0.0f), L);
        c[i] = (uint32_t)u;
    }
}

__device__ __forceinline__ float select8(uint32_t c, const float* mu) {
    const float a = (c & 1) ? mu[1] : mu[0], b = (c & 1) ? mu[3] : mu[2];
    const float d = (c & 1) ? mu[5] : mu[4], f = (c & 1) ? mu[7] : mu[6];
    const float ab = (c & 2) ? b : a, df = (c & 2) ? f : d;
    return (c & 4) ? df : ab;
}

// Bytes of LDS one wave of the bulk quantizer uses: 8 tokens x 128 residuals (binary32) for the
// QJL projection, or 8 tokens x 128 codes (one byte each) for the V words.
constexpr int kBulkWaveLds = 8 * kDim * 4;

// Source values of one octet as the bulk quantizer holds them: v[r][i] = channel 8j + i of octet
// token 4r + L / 16 (zero for tokens outside the append).
struct OctetSrc {
    float v[2][8];
};

struct OctetSpan {
    int start, end, g0, t_lo, t_hi;
};

__device__ __forceinline__ bool octet_span(const QuantParams& p, int b, int unit, OctetSpan& o) {
    if (unit >= p.groups8) return false;
    o.start = p.start[b];
    o.end = o.start + p.T;
    o.g0 = o.start / 8 + unit;
    o.t_lo = max(o.start, 8 * o.g0);
    o.t_hi = min(o.end, 8 * o.g0 + 8);
    return o.t_lo < o.t_hi;
}

__device__ __forceinline__ void load_octet(const QuantParams& p, int tensor, int b, int head,
                                           int unit, OctetSrc& src) {
    const int L = lane_id(), tk = L >> 4, j = L & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) src.v[r][i] = 0.0f;
    OctetSpan o;
    if (!octet_span(p, b, unit, o)) return;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = 8 * o.g0 + 4 * r + tk;
        if (t >= o.t_lo && t < o.t_hi) {
            const size_t elem = (((size_t)b * p.T + (t - o.start)) * p.Hkv + head) * kDim + 8 * j;
            if (p.dtype == 0) {
                const float4* s4 = reinterpret_cast<const float4*>(static_cast<const float*>(p.src[tensor]) + elem);
                const float4 v0 = s4[0], v1 = s4[1];
                src.v[r][0] = v0.x; src.v[r][1] = v0.y; src.v[r][2] = v0.z; src.v[r][3] = v0.w;
                src.v[r][4] = v1.x; src.v[r][5] = v1.y; src.v[r][6] = v1.z; src.v[r][7] = v1.w;
            } else {
                const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.src[tensor]) + elem);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    src.v[r][2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xffff));
                    src.v[r][2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
                }
            }
        }
    }
}

// One octet of the bulk quantizer, tensor scheme SCH, from its loaded source values.  wl:
// kBulkWaveLds bytes of LDS owned by the wave.  st: the 128 x 128 QJL matrix S^T ([j][i] =
// S[i][j]) in LDS when SCH is TurboQuant-QJL (a K plane), else unused.
template <int SCH>
__device__ __forceinline__ void quantize_octet_dense(const QuantParams& p, int tensor, int b,
                                                     int head, int unit, const OctetSrc& src,
                                                     float* wl, const float* st) {
    const int L = lane_id(), tk = L >> 4, j = L & 15;
    OctetSpan o;
    if (!octet_span(p, b, unit, o)) return;
    const int end = o.end, g0 = o.g0, t_lo = o.t_lo, t_hi = o.t_hi;

    const PlaneGeom& G = p.geom[tensor];
    char* slot = p.layer_base + (size_t)b * p.seq_stride + (size_t)head * p.head_stride +
                 p.plane_off[tensor];
    uint8_t* codes = reinterpret_cast<uint8_t*>(slot + G.codes_off);
    uint8_t* meta = reinterpret_cast<uint8_t*>(slot + G.meta_off);
    uint8_t* wcodes = reinterpret_cast<uint8_t*>(wl);
    constexpr bool qjl = SCH == kTurboQjl;

    float sg[8], ic[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sg[i] = ic[i] = 1.0f;
    if (G.rotate) {
        const float4* s4 = reinterpret_cast<const float4*>(p.signs[tensor] + (size_t)(head * 2 + tensor) * kDim + 8 * j);
        const float4 a = s4[0], c = s4[1];
        sg[0] = a.x; sg[1] = a.y; sg[2] = a.z; sg[3] = a.w;
        sg[4] = c.x; sg[5] = c.y; sg[6] = c.z; sg[7] = c.w;
    }
    if (SCH == kUniform && G.sinkhorn) {
        const float4* c4 = reinterpret_cast<const float4*>(p.inv_c[tensor] + (size_t)(head * 2 + tensor) * kDim + 8 * j);
        const float4 a = c4[0], c = c4[1];
        ic[0] = a.x; ic[1] = a.y; ic[2] = a.z; ic[3] = a.w;
        ic[4] = c.x; ic[5] = c.y; ic[6] = c.z; ic[7] = c.w;
    }

#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i_tok = 4 * r + tk, t = 8 * g0 + i_tok;
        const bool valid = t >= t_lo && t < t_hi;
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = src.v[r][i];
        if (valid && p.window > 0 && t >= end - p.window) {
            float4* ring = reinterpret_cast<float4*>(reinterpret_cast<float*>(slot + G.ring_off) +
                                                     (size_t)(t % p.window) * kDim + 8 * j);
            ring[0] = make_float4(e[0], e[1], e[2], e[3]);
            ring[1] = make_float4(e[4], e[5], e[6], e[7]);
        }
        if constexpr (SCH == kUniform) {
            if (G.rotate) rotate8(e, sg, j);
            if (G.sinkhorn) {
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = e[i] * ic[i];
            }
            uint32_t c[8];
            uint16_t s16, z16;
            quant_uniform8(e, G.bits, c, s16, z16);
            const int g = j >> 2, kb = j & 3;
            if (tensor == 0) {
                const int row = k_row(t);
                if (valid) {
                    if (G.bits == 4) {
                        uint32_t w = 0;
#pragma unroll
                        for (int i = 0; i < 8; ++i) w |= c[i] << (16 * (i & 1) + 4 * (i >> 1));
                        reinterpret_cast<uint32_t*>(codes + (size_t)row * 64)[4 * kb + g] = w;
                    } else {
                        uint32_t w0 = 0, w1 = 0;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            w0 |= c[i] << (8 * i);
                            w1 |= c[4 + i] << (8 * i);
                        }
                        *reinterpret_cast<uint2*>(codes + (size_t)row * 128 + 8 * (4 * kb + g)) = make_uint2(w0, w1);
                    }
                    if (kb == 0) {
                        uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)row * 16);
                        m[g] = s16;
                        m[4 + g] = z16;
                    }
                }
            } else {
                uint2 cw;
                cw.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
                cw.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
                *reinterpret_cast<uint2*>(wcodes + i_tok * kDim + 8 * j) = cw;
                if (valid && kb == 0) {
                    uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)t * 16);
                    m[g] = s16;
                    m[4 + g] = z16;
                }
            }
        } else {
            rotate8(e, sg, j);
            const float nsq = tree_sum_sq16(e);
            const uint16_t n16 = f16_rn(sqrtf(nsq));
            const float n = f16_val(n16);
            const float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
            uint32_t c[8];
            float rr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float u = e[i] * inv;
                uint32_t q = 0;
#pragma unroll
                for (int k = 0; k < 7; ++k) q += (u > p.theta[k]) ? 1u : 0u;
                c[i] = q;
                const float pq = n * select8(q, p.mu);
                rr[i] = e[i] - pq;
            }
            if (tensor == 0) {
                // K row: plane words of group g = j / 4; this lane's channels are values
                // v = 8 (j % 4) + i of the group, at half-interleaved bit 16 (v % 2) + v / 2
                const int row = k_row(t), g = j >> 2, v0 = 8 * (j & 3);
                uint32_t pw[3] = {0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int v = v0 + i, bit = 16 * (v & 1) + (v >> 1);
#pragma unroll
                    for (int k = 0; k < 3; ++k) pw[k] |= ((c[i] >> k) & 1u) << bit;
                }
#pragma unroll
                for (int k = 0; k < 3; ++k) pw[k] = or_reduce<4>(pw[k]);
                if (valid && (j & 3) == 0) {
                    uint32_t* w = reinterpret_cast<uint32_t*>(codes + (size_t)row * 48 + 12 * g);
                    w[0] = pw[0];
                    w[1] = pw[1];
                    w[2] = pw[2];
                }
                if constexpr (qjl) {
                    const uint16_t g16 = f16_rn(sqrtf(tree_sum_sq16(rr)));
                    // residual of channel 8j + i, token i_tok at wl[(8j + i) * 8 + i_tok]
#pragma unroll
                    for (int i = 0; i < 8; ++i) wl[(8 * j + i) * 8 + i_tok] = rr[i];
                    if (valid && j == 0) {
                        uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)row * 4);
                        m[0] = n16;
                        m[1] = g16;
                    }
                } else if (valid && j == 0) {
                    reinterpret_cast<uint16_t*>(meta)[row] = n16;
                }
            } else {
                uint2 cw;
                cw.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
                cw.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
                *reinterpret_cast<uint2*>(wcodes + i_tok * kDim + 8 * j) = cw;
                if (valid && j == 0) reinterpret_cast<uint16_t*>(meta)[t] = n16;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();

    if constexpr (qjl) {
        // sign(S r) for the octet's 8 tokens: lane L forms projections L and 64 + L, each a
        // sequential fma chain over j = 0 .. 127; S^T rows are shared by the 8 tokens
        float acc0[8], acc1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc0[i] = acc1[i] = 0.0f;
#pragma unroll 4
        for (int jj = 0; jj < kDim; ++jj) {
            const float s0 = st[jj * kDim + L], s1 = st[jj * kDim + 64 + L];
            const float4 ra = *reinterpret_cast<const float4*>(wl + jj * 8);
            const float4 rb = *reinterpret_cast<const float4*>(wl + jj * 8 + 4);
            const float rj[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                acc0[i] = fmaf(s0, rj[i], acc0[i]);
                acc1[i] = fmaf(s1, rj[i], acc1[i]);
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint64_t b0 = __ballot(acc0[i] >= 0.0f);
            const uint64_t b1 = __ballot(acc1[i] >= 0.0f);
            const int t = 8 * g0 + i;
            if (L == i && t >= t_lo && t < t_hi) {
                uint4 w;
                w.x = unshuffle32((uint32_t)b0);
                w.y = unshuffle32((uint32_t)(b0 >> 32));
                w.z = unshuffle32((uint32_t)b1);
                w.w = unshuffle32((uint32_t)(b1 >> 32));
                *reinterpret_cast<uint4*>(slot + G.qjl_off + (size_t)k_row(t) * 16) = w;
            }
        }
    }

    if (tensor == 1) {
        // V words of channels 2L, 2L+1 for this octet from the staged codes, then a
        // read-modify-write of the octet's bits (tokens outside [t_lo, t_hi) keep theirs)
        const int d0 = 2 * L;
        if constexpr (SCH == kUniform) {
            uint64_t vacc0 = 0, vacc1 = 0, vmask = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = 8 * g0 + i;
                if (t < t_lo || t >= t_hi) continue;
                const int sh = (G.bits == 4) ? 16 * (i % 2) + 4 * (i / 2) : 8 * i;
                const uint32_t pr = *reinterpret_cast<const uint16_t*>(wcodes + i * kDim + d0);
                vacc0 |= (uint64_t)(pr & 0xffu) << sh;
                vacc1 |= (uint64_t)(pr >> 8) << sh;
                vmask |= (uint64_t)((1u << G.bits) - 1) << sh;
            }
            const int blk = t_lo / 32, kb = (t_lo % 32) / 8;
            const int n0 = d0 % 16, N = d0 / 16;
            const int w0 = 8 * (16 * kb + n0) + N, w1 = w0 + 8;
            if (G.bits == 4) {
                uint32_t* bp = reinterpret_cast<uint32_t*>(codes + (size_t)blk * 2048);
                const uint32_t m = (uint32_t)vmask;
                bp[w0] = (bp[w0] & ~m) | (uint32_t)vacc0;
                bp[w1] = (bp[w1] & ~m) | (uint32_t)vacc1;
            } else {
                uint64_t* bp = reinterpret_cast<uint64_t*>(codes + (size_t)blk * 4096);
                bp[w0] = (bp[w0] & ~vmask) | vacc0;
                bp[w1] = (bp[w1] & ~vmask) | vacc1;
            }
        } else {
            // TurboQuant-MSE V: bit k of channel d goes to word 6 (16 o + d % 16) + 2k + (d / 16) / 4
            // of the block, token i of the octet at bit 16 (i % 2) + 4 ((d / 16) % 4) + i / 2; lanes
            // L ^ 8 and L ^ 16 hold the other channel slots of the same words
            const int N = L >> 3;
            uint32_t ta[3] = {0u, 0u, 0u}, tc[3] = {0u, 0u, 0u}, msk = 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = 8 * g0 + i;
                if (t < t_lo || t >= t_hi) continue;
                const uint32_t pos = 1u << (16 * (i & 1) + 4 * (N & 3) + (i >> 1));
                const uint32_t pr = *reinterpret_cast<const uint16_t*>(wcodes + i * kDim + d0);
                const uint32_t qa = pr & 0xffu, qc = pr >> 8;
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    ta[k] |= ((qa >> k) & 1u) ? pos : 0u;
                    tc[k] |= ((qc >> k) & 1u) ? pos : 0u;
                }
                msk |= pos;
            }
            msk |= xor_lane<8>(msk);
            msk |= xor_lane<16>(msk);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                ta[k] |= xor_lane<8>(ta[k]);
                ta[k] |= xor_lane<16>(ta[k]);
                tc[k] |= xor_lane<8>(tc[k]);
                tc[k] |= xor_lane<16>(tc[k]);
            }
            if ((N & 3) == 0) {
                const int o = (t_lo % 32) / 8, n0 = 2 * (L & 7);
                uint32_t* blkp = reinterpret_cast<uint32_t*>(codes + (size_t)(t_lo / 32) * 1536);
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    uint32_t* wa = blkp + 6 * (16 * o + n0) + 2 * k + (N >> 2);
                    uint32_t* wc = wa + 6;
                    *wa = (*wa & ~msk) | ta[k];
                    *wc = (*wc & ~msk) | tc[k];
                }
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

} // namespace qdev
} // namespace kvq
