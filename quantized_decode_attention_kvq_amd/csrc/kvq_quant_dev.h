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
        a = in16_to_f32(v & 0xffff, dtype);
        b = in16_to_f32(v >> 16, dtype);
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

// 64-point R64(x) = (1/8) H64 (d .* x) on each half of the wave (lanes 0-31: positions 0..63,
// lanes 32-63: positions 64..127): the butterflies of hadamard_wave without the last span.
__device__ __forceinline__ void rotate64_signed(float& a, float& b, float s0, float s1) {
    const int l = lane_id();
    if (s0 < 0.0f) a = -a;
    if (s1 < 0.0f) b = -b;
    const float s = a + b, d = a - b;
    a = s;
    b = d;
    hadamard_step<1>(a, b, l);
    hadamard_step<2>(a, b, l);
    hadamard_step<4>(a, b, l);
    hadamard_step<8>(a, b, l);
    hadamard_step<16>(a, b, l);
    a = a * 0.125f;
    b = b * 0.125f;
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

// QJL projections of the residual held in the wave's LDS row r[0..127]: lane l forms
// (S r)_l and (S r)_{64+l} as sequential fma chains over j = 0..127 (S^T stored [j][i]).  The
// sixteen S^T loads of each 8-j step are issued together and pinned to registers before the
// chain consumes them: left to itself, the scheduler of a register-heavy caller (the fused
// append inside the decode kernel) waited on every load in turn.
__device__ __forceinline__ void qjl_project(const float* __restrict__ st, const float* r, int l, float& acc0,
                                            float& acc1) {
    acc0 = 0.0f;
    acc1 = 0.0f;
    for (int j0 = 0; j0 < kDim; j0 += 8) {
        float x[8], y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            x[u] = st[(j0 + u) * kDim + l];
            y[u] = st[(j0 + u) * kDim + 64 + l];
        }
        asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]),
                     "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]), "v"(y[6]), "v"(y[7]));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float rj = r[j0 + u];
            acc0 = fmaf(x[u], rj, acc0);
            acc1 = fmaf(y[u], rj, acc1);
        }
    }
}

// Symmetric 8-bit (q8_0-style) quantizer of the two elements a lane holds: d = fp16(max|y| / 127),
// q = rint(y * fp32(1/d)) clamped to [-127, 127], code q + 128, zero field fp16(-128 d).
__device__ __forceinline__ void quant_sym8(float a, float b, uint32_t& c0, uint32_t& c1, uint16_t& s16,
                                           uint16_t& z16) {
    float amax = fmaxf(fabsf(a), fabsf(b));
    amax = xor_reduce<16>(amax, [](float x, float y) { return fmaxf(x, y); });
    s16 = f16_rn(amax / 127.0f);
    const float d = f16_val(s16);
    z16 = f16_rn(-128.0f * d);
    const float inv = (d > 0.0f) ? 1.0f / d : 0.0f;
    const float u0 = fminf(fmaxf(rintf(a * inv), -127.0f), 127.0f);
    const float u1 = fminf(fmaxf(rintf(b * inv), -127.0f), 127.0f);
    c0 = (uint32_t)(int)(u0 + 128.0f);
    c1 = (uint32_t)(int)(u1 + 128.0f);
}

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
    // V turbo bit-plane words (3 or 4 planes) of channels 2l and 2l+1 for this octet, and the
    // bits written.
    uint32_t tv_a[4] = {0u, 0u, 0u, 0u}, tv_c[4] = {0u, 0u, 0u, 0u}, tv_mask = 0u;

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
    // split V / K: this lane codes positions 2l, 2l+1, i.e. channels perm[2l], perm[2l+1]
    int pm0 = 0, pm1 = 0;
    if (G.scheme == kTurboSplit) {
        const int2 pm = reinterpret_cast<const int2*>((tensor == 0 ? p.perm_k : p.perm) + (size_t)head * kDim)[l];
        pm0 = pm.x;
        pm1 = pm.y;
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
            if (G.symmetric)
                quant_sym8(a, c, q0, q1, s16, z16);
            else
                quant_uniform(a, c, G.bits, q0, q1, s16, z16);
            const int g = l >> 4;
            if (G.bits == 3) {
                // 3-bit codes go to bit planes laid out as the TurboQuant 3-bit planes (K: three
                // words per group in the 48-byte row, channels 2 lg, 2 lg + 1 at bits lg, 16 + lg;
                // V: the block words written after the octet), the meta as for any uniform plane
                const int lg = l & 15;
                const int row = tensor == 0 ? k_row(t) : t;
                if (tensor == 0) {
                    uint32_t pw[3];
#pragma unroll
                    for (int k = 0; k < 3; ++k)
                        pw[k] = or_reduce<16>((((q0 >> k) & 1u) << lg) | (((q1 >> k) & 1u) << (16 + lg)));
                    if (lg == 0) {
                        uint32_t* w = reinterpret_cast<uint32_t*>(codes + (size_t)row * 48 + 12 * g);
                        w[0] = pw[0];
                        w[1] = pw[1];
                        w[2] = pw[2];
                    }
                } else {
                    const int i = t % 8, N = l >> 3;
                    const uint32_t pos = 1u << (16 * (i & 1) + 4 * (N & 3) + (i >> 1));
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        tv_a[k] |= ((q0 >> k) & 1u) ? pos : 0u;
                        tv_c[k] |= ((q1 >> k) & 1u) ? pos : 0u;
                    }
                    tv_mask |= pos;
                }
                if (lg == 0) {
                    uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)row * 16);
                    m[g] = s16;
                    m[4 + g] = z16;
                }
            } else if (tensor == 0) {
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
        } else if (G.scheme == kTurboSplit && tensor == 0) {
            // split key (b = G.bits): the split's MSE codes -- outliers (lanes 0-31) b - 1 bits,
            // the rest b - 2, each half its own rotation, norm and codebook -- in the K row
            // layout, then gamma and the QJL bits of the whole residual as for a TurboQuant key
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            rbuf[2 * l] = a;
            rbuf[2 * l + 1] = c;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            a = rbuf[pm0];
            c = rbuf[pm1];
            rotate64_signed(a, c, sg0, sg1);
            const float nsq = xor_reduce<32>(a * a + c * c, [](float x, float y) { return x + y; });
            const uint16_t n16 = f16_rn(sqrtf(nsq));
            const float n = f16_val(n16);
            const float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
            const float ua = a * inv, uc = c * inv;
            const int nb = (l < 32) ? G.bits - 1 : G.bits - 2, levels = 1 << nb;
            const float* th = p.theta64 + split_table_off(levels);
            uint32_t qa = 0, qc = 0;
#pragma unroll
            for (int k = 0; k < 7; ++k) {
                if (k < levels - 1) {
                    const float thk = th[k];
                    qa += (ua > thk) ? 1u : 0u;
                    qc += (uc > thk) ? 1u : 0u;
                }
            }
            const float* mu = p.mu64 + split_table_off(levels);
            const float pa_ = n * mu[qa], pc_ = n * mu[qc];
            const float ra = a - pa_, rc = c - pc_;
            // K row: group g = l / 16 (positions 32g .. 32g+31) keeps its nb planes as words
            // starting at split_k_group_word(g, b); lane lg holds half-interleaved values lg and
            // 16 + lg of its group
            const int lg = l & 15, g = l >> 4;
            const int row = k_row(t);
            uint32_t pw[3];
#pragma unroll
            for (int k = 0; k < 3; ++k)
                pw[k] = or_reduce<16>((((qa >> k) & 1u) << lg) | (((qc >> k) & 1u) << (16 + lg)));
            if (lg == 0) {
                uint32_t* w = reinterpret_cast<uint32_t*>(codes + (size_t)row * split_k_row_bytes(G.bits)) +
                              split_k_group_word(g, G.bits);
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    if (k < nb) w[k] = pw[k];
            }
            const uint16_t g16 = f16_rn(sqrtf(tree_sum_sq(ra, rc)));
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            rbuf[2 * l] = ra;
            rbuf[2 * l + 1] = rc;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            float acc0, acc1;
            qjl_project(p.qjl_st, rbuf, l, acc0, acc1);
            __builtin_amdgcn_wave_barrier();
            const uint64_t b0 = __ballot(acc0 >= 0.0f);
            const uint64_t b1 = __ballot(acc1 >= 0.0f);
            uint16_t* m = reinterpret_cast<uint16_t*>(meta + (size_t)row * 8);
            if (l == 0) {
                uint32_t* qj = reinterpret_cast<uint32_t*>(slot + G.qjl_off + (size_t)row * 16);
                qj[0] = unshuffle32((uint32_t)b0);
                qj[1] = unshuffle32((uint32_t)(b0 >> 32));
                qj[2] = unshuffle32((uint32_t)b1);
                qj[3] = unshuffle32((uint32_t)(b1 >> 32));
                m[0] = n16;
                m[2] = g16;
                m[3] = 0;
            }
            if (l == 32) m[1] = n16;
        } else if (G.scheme == kTurboSplit) {
            // outlier split: gather the lane's two positions through the wave's LDS row, then
            // per half of the wave rho = R64(x_h), n_h = fp16(|rho|), codes = #thresholds of the
            // half's codebook (outliers G.bits bits, the rest one fewer) below rho / n_h
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            rbuf[2 * l] = a;
            rbuf[2 * l + 1] = c;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            a = rbuf[pm0];
            c = rbuf[pm1];
            rotate64_signed(a, c, sg0, sg1);
            const float nsq = xor_reduce<32>(a * a + c * c, [](float x, float y) { return x + y; });
            const uint16_t n16 = f16_rn(sqrtf(nsq));
            const float n = f16_val(n16);
            const float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
            const float ua = a * inv, uc = c * inv;
            const int levels = (l < 32) ? (1 << G.bits) : (1 << (G.bits - 1));
            const float* th = p.theta64 + (levels - 4);
            uint32_t qa = 0, qc = 0;
#pragma unroll
            for (int k = 0; k < 15; ++k) {
                if (k < levels - 1) {
                    const float thk = th[k];
                    qa += (ua > thk) ? 1u : 0u;
                    qc += (uc > thk) ? 1u : 0u;
                }
            }
            const int i = t % 8, N = l >> 3;
            const uint32_t pos = 1u << (16 * (i & 1) + 4 * (N & 3) + (i >> 1));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                tv_a[k] |= ((qa >> k) & 1u) ? pos : 0u;
                tv_c[k] |= ((qc >> k) & 1u) ? pos : 0u;
            }
            tv_mask |= pos;
            if ((l & 31) == 0) reinterpret_cast<uint16_t*>(meta)[2 * t + (l >> 5)] = n16;
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
            if (G.bits == 4) {
                // 4-bit TurboQuant-MSE V: the 16-level codebook
#pragma unroll
                for (int k = 0; k < 15; ++k) {
                    const float th = p.theta16[k];
                    qa += (ua > th) ? 1u : 0u;
                    qc += (uc > th) ? 1u : 0u;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 7; ++k) {
                    const float th = p.theta[k];
                    qa += (ua > th) ? 1u : 0u;
                    qc += (uc > th) ? 1u : 0u;
                }
            }
            const float* mu = (G.bits == 4) ? p.mu16 : p.mu;
            const float pa = n * mu[qa], pc = n * mu[qc];
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
                    float acc0, acc1;
                    qjl_project(p.qjl_st, rbuf, l, acc0, acc1);
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
                // V block (b = G.bits planes): bit k of channel 2l (2l+1) goes to word
                // 2b(16 o + n) + 2k + N/4 with n = 2(l%8) (+1), N = l/8; token i of the octet at
                // bit 16(i%2) + 4(N%4) + i/2
                const int i = t % 8, N = l >> 3;
                const uint32_t pos = 1u << (16 * (i & 1) + 4 * (N & 3) + (i >> 1));
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    tv_a[k] |= ((qa >> k) & 1u) ? pos : 0u;
                    tv_c[k] |= ((qc >> k) & 1u) ? pos : 0u;
                }
                tv_mask |= pos;
                if (l == 0) reinterpret_cast<uint16_t*>(meta)[t] = n16;
            }
        }
    }

    if (tensor == 1 && (G.scheme != kUniform || G.bits == 3)) {
        // merge the four lanes (l ^ 8, l ^ 16) whose channels share each word, then
        // read-modify-write this octet's words (TurboQuant planes, and 3-bit uniform planes in
        // the same layout)
        uint32_t m = tv_mask;
        m |= xor_lane<8>(m);
        m |= xor_lane<16>(m);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            tv_a[k] |= xor_lane<8>(tv_a[k]);
            tv_a[k] |= xor_lane<16>(tv_a[k]);
            tv_c[k] |= xor_lane<8>(tv_c[k]);
            tv_c[k] |= xor_lane<16>(tv_c[k]);
        }
        if (((l >> 3) & 3) == 0 && G.scheme == kTurboSplit) {
            // W = 2 bits - 1 words per (octet, lane column): the outlier planes, then the rest's
            const int W = 2 * G.bits - 1, o = (t_lo % 32) / 8, n0 = 2 * (l & 7);
            const int first = (l < 32) ? 0 : G.bits, nb = (l < 32) ? G.bits : G.bits - 1;
            uint32_t* blk = reinterpret_cast<uint32_t*>(codes + (size_t)(t_lo / 32) * (256 * W));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (k >= nb) break;
                uint32_t* wa = blk + W * (16 * o + n0) + first + k;
                uint32_t* wc = wa + W;
                *wa = (*wa & ~m) | tv_a[k];
                *wc = (*wc & ~m) | tv_c[k];
            }
        } else if (((l >> 3) & 3) == 0) {
            const int b = G.bits; // bit planes
            const int o = (t_lo % 32) / 8, n0 = 2 * (l & 7), N = l >> 3;
            uint32_t* blk = reinterpret_cast<uint32_t*>(codes + (size_t)(t_lo / 32) * (512 * b));
#pragma unroll
            for (int k = 0; k < 4; ++k) { // register indexes stay compile-time; planes k < b
                if (k >= b) break;
                uint32_t* wa = blk + 2 * b * (16 * o + n0) + 2 * k + (N >> 2);
                uint32_t* wc = wa + 2 * b;
                *wa = (*wa & ~m) | tv_a[k];
                *wc = (*wc & ~m) | tv_c[k];
            }
        }
    }

    if (tensor == 1 && G.scheme == kUniform && G.bits != 3) {
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

} // namespace qdev
} // namespace kvq
