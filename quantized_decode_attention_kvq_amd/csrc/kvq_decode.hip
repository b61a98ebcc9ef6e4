// Decode attention over the compressed cache: split-K partials (vector-ALU kernel for every
// scheme) and the fixed-order log-sum-exp merge with the inverse rotation of V.
//
// Method sources (pages by title and section):
//  - quantcpp article "Beyond RAG...", "how it works": the newest 128 tokens are read in FP32,
//    everything older from the 4-bit codes.
//  - KVarN-on-Bonsai post, TL;DR: keys and values were rotated (Walsh-Hadamard) and balanced
//    (Sinkhorn) before coding, so scores use R(q) .* c and the output is R^-1(c .* acc).
//  - "LLM memory saving ... 2026", TurboQuant row: the score of a TurboQuant key is
//    n <R q, mu[code]> plus the 1-bit QJL estimate of the residual's inner product.
//
// Scores are kept in the log2 domain: q' = q * softmax_scale * log2(e), p = exp2(s - m).
#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"
#include "kvq_lanes.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ float c0f() { return __uint_as_float(0x3DB504F3u); }
__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ __forceinline__ float wave_max(float v) {
    return xor_reduce<64>(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
    return xor_reduce<64>(v, [](float x, float y) { return x + y; });
}

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

// The split domain of a vector held as channel pairs (lane l: 2l, 2l+1): positions 2l, 2l+1 take
// channels pm.x, pm.y (lane pm / 2, component pm % 2), then the signs by position and the two
// 64-point Walsh-Hadamard transforms (the butterflies without the last span), scale 1/8.
__device__ __forceinline__ void split_rotate(float& a, float& c, int2 pm, float2 sg) {
    const int l = lane_id();
    const float ax = __shfl(a, pm.x >> 1), ay = __shfl(c, pm.x >> 1);
    const float bx = __shfl(a, pm.y >> 1), by = __shfl(c, pm.y >> 1);
    a = (pm.x & 1) ? ay : ax;
    c = (pm.y & 1) ? by : bx;
    if (sg.x < 0.0f) a = -a;
    if (sg.y < 0.0f) c = -c;
    const float s = a + c, d = a - c;
    a = s;
    c = d;
    hadamard_step<1>(a, c, l);
    hadamard_step<2>(a, c, l);
    hadamard_step<4>(a, c, l);
    hadamard_step<8>(a, c, l);
    hadamard_step<16>(a, c, l);
    a *= 0.125f;
    c *= 0.125f;
}

__device__ __forceinline__ int k_row(int t) { return 64 * (t / 64) + 16 * ((t % 64) % 4) + (t % 64) / 4; }

__device__ __forceinline__ void load_q_pair(const DecodeParams& p, int b, int hq, float& a, float& c) {
    const int l = lane_id();
    const size_t off = ((size_t)b * p.Hq + hq) * kDim;
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

// 3-bit TurboQuant code of channel j from a 48-byte K row: group j/32 holds three bit-plane
// words, value e of a word at bit 16*(e%2) + e/2.
__device__ __forceinline__ uint32_t turbo_k_code(const uint8_t* row, int j) {
    const int g = j >> 5, e = j & 31;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(row + 12 * g);
    const int b = 16 * (e & 1) + (e >> 1);
    return ((w[0] >> b) & 1u) | (((w[1] >> b) & 1u) << 1) | (((w[2] >> b) & 1u) << 2);
}

// nb-bit TurboQuant code of (token t, channel d) from the V plane's 32-token blocks (nb = 3 or
// 4 planes; word 2 nb (16 o + n) + 2 k + N / 4 of block t / 32).
__device__ __forceinline__ uint32_t turbo_v_code(const uint8_t* codes, int t, int d, int nb) {
    const int o = (t & 31) >> 3, i = t & 7, n = d & 15, N = d >> 4;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(codes + (size_t)(t >> 5) * (512 * nb)) +
                        2 * nb * (16 * o + n) + (N >> 2);
    const int b = 16 * (i & 1) + 4 * (N & 3) + (i >> 1);
    uint32_t c = 0;
    for (int k = 0; k < nb; ++k) c |= ((w[2 * k] >> b) & 1u) << k;
    return c;
}

// Split key (b = 3 or 4): code of position j from a row of per-group plane words (group
// g = j / 32 has b - 1 planes if g < 2, else b - 2, from word split_k_group_word(g, b)).
__device__ __forceinline__ uint32_t split_k_code(const uint8_t* row, int j, int b) {
    const int g = j >> 5, e = j & 31, nb = g < 2 ? b - 1 : b - 2;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(row) + split_k_group_word(g, b);
    const int bit = 16 * (e & 1) + (e >> 1);
    uint32_t c = 0;
    for (int k = 0; k < nb; ++k) c |= ((w[k] >> bit) & 1u) << k;
    return c;
}

// Split V (bo outlier bits, W = 2 bo - 1 words per (octet, column)): code of position d of token
// t; the outlier half (d < 64) has bo planes at words W (16 o + n) + k, the rest bo - 1 at + bo + k.
__device__ __forceinline__ uint32_t split_v_code(const uint8_t* codes, int t, int d, int bo) {
    const int W = 2 * bo - 1, o = (t & 31) >> 3, i = t & 7, n = d & 15, N = d >> 4;
    const int rest = d >= 64, nb = rest ? bo - 1 : bo;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(codes + (size_t)(t >> 5) * (256 * W)) +
                        W * (16 * o + n) + (rest ? bo : 0);
    const int b = 16 * (i & 1) + 4 * (N & 3) + (i >> 1);
    uint32_t c = 0;
    for (int k = 0; k < nb; ++k) c |= ((w[k] >> b) & 1u) << k;
    return c;
}

__global__ __launch_bounds__(256) void decode_vec_kernel(DecodeParams p) {
    __shared__ float qp[kMaxGroupHeads][kDim];
    __shared__ float sp[kMaxGroupHeads][kDim];
    __shared__ float qsum[kMaxGroupHeads][4];
    __shared__ float spsum[kMaxGroupHeads];
    __shared__ float pbuf[4][kMaxGroupHeads][64];
    __shared__ float wm[4][kMaxGroupHeads], wl[4][kMaxGroupHeads];
    __shared__ float wacc[4][kMaxGroupHeads][kDim];

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, l = lane_id();
    const int G = p.G, W = p.window;
    const int n = p.len[b];
    const int nq = (W > 0) ? max(0, n - W) : n;
    const bool wsplit = (W > 0) && (split == p.n_splits);
    int t0, t1;
    if (wsplit) {
        t0 = nq;
        t1 = n;
    } else {
        t0 = split * p.split_tokens;
        t1 = min(nq, t0 + p.split_tokens);
    }
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

    // ---- query preparation: q' = (R_K q .* c_K) * scale * log2(e) (plain q for the window)
    for (int h = wave; h < G; h += 4) {
        float a, c;
        load_q_pair(p, b, kvh * G + h, a, c);
        if (!wsplit && KG.scheme == kTurboSplit) {
            const int2 pm = reinterpret_cast<const int2*>(p.perm_k + (size_t)kvh * kDim)[l];
            const float2 sg = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 0) * kDim)[l];
            split_rotate(a, c, pm, sg);
        } else if (!wsplit && KG.rotate) {
            const float* sg = p.signs + (size_t)(kvh * 2 + 0) * kDim;
            if (sg[2 * l] < 0.0f) a = -a;
            if (sg[2 * l + 1] < 0.0f) c = -c;
            hadamard_wave(a, c);
            a *= c0f();
            c *= c0f();
        }
        if (!wsplit && KG.sinkhorn) {
            const float* cs = p.cs + (size_t)(kvh * 2 + 0) * kDim;
            a *= cs[2 * l];
            c *= cs[2 * l + 1];
        }
        qp[h][2 * l] = a * p.qscale;
        qp[h][2 * l + 1] = c * p.qscale;
    }
    __syncthreads();
    const bool turbo_k = !wsplit && (KG.scheme == kTurboQjl || KG.scheme == kTurboSplit);
    if (turbo_k) {
        for (int idx = threadIdx.x; idx < G * kDim; idx += 256) {
            const int h = idx / kDim, i = idx % kDim;
            float s = 0.0f;
            for (int j = 0; j < kDim; ++j) s += p.qjl_st[j * kDim + i] * qp[h][j];
            sp[h][i] = s;
        }
    }
    if (threadIdx.x < G * 4) {
        const int h = threadIdx.x / 4, g = threadIdx.x % 4;
        float s = 0.0f;
        for (int j = 0; j < 32; ++j) s += qp[h][32 * g + j];
        qsum[h][g] = s;
    }
    __syncthreads();
    if (turbo_k && threadIdx.x < G) {
        float s = 0.0f;
        for (int i = 0; i < kDim; ++i) s += sp[threadIdx.x][i];
        spsum[threadIdx.x] = s;
    }
    __syncthreads();

    float m[kMaxGroupHeads], lsum[kMaxGroupHeads], acc0[kMaxGroupHeads], acc1[kMaxGroupHeads];
#pragma unroll
    for (int h = 0; h < kMaxGroupHeads; ++h) {
        m[h] = kNegInf;
        lsum[h] = 0.0f;
        acc0[h] = 0.0f;
        acc1[h] = 0.0f;
    }

    const float kappa = 0.0097915166977774f; // sqrt(pi/2) / 128
    for (int cs0 = t0 + 64 * wave; cs0 < t1; cs0 += 256) {
        const int t = cs0 + l;
        const bool valid = t < t1;
        float s[kMaxGroupHeads];
#pragma unroll
        for (int h = 0; h < kMaxGroupHeads; ++h) s[h] = 0.0f;
        if (valid) {
            if (wsplit) {
                const float* kr = kring + (size_t)(t % W) * kDim;
                for (int j = 0; j < kDim; j += 4) {
                    const float4 kv = *reinterpret_cast<const float4*>(kr + j);
#pragma unroll
                    for (int h = 0; h < kMaxGroupHeads; ++h)
                        if (h < G)
                            s[h] += kv.x * qp[h][j] + kv.y * qp[h][j + 1] + kv.z * qp[h][j + 2] +
                                    kv.w * qp[h][j + 3];
                }
            } else if (KG.scheme == kUniform) {
                const int row = k_row(t);
                const uint16_t* mt = reinterpret_cast<const uint16_t*>(kmeta + (size_t)row * 16);
                float dot[kMaxGroupHeads][4];
#pragma unroll
                for (int h = 0; h < kMaxGroupHeads; ++h)
#pragma unroll
                    for (int g = 0; g < 4; ++g) dot[h][g] = 0.0f;
                if (KG.bits == 3) { // three bit planes per group in a 48-byte row
                    const uint8_t* r = kcodes + (size_t)row * 48;
                    for (int j = 0; j < kDim; ++j) {
                        const float cv = (float)turbo_k_code(r, j);
#pragma unroll
                        for (int h = 0; h < kMaxGroupHeads; ++h)
                            if (h < G) dot[h][j >> 5] += cv * qp[h][j];
                    }
                } else if (KG.bits == 4) {
                    const uint32_t* r = reinterpret_cast<const uint32_t*>(kcodes + (size_t)row * 64);
#pragma unroll
                    for (int w = 0; w < 16; ++w) {
                        const uint32_t word = r[w];
                        const int kb = w >> 2, g = w & 3;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const float cv = (float)((word >> (16 * (i & 1) + 4 * (i >> 1))) & 15u);
                            const int j = 32 * g + 8 * kb + i;
#pragma unroll
                            for (int h = 0; h < kMaxGroupHeads; ++h)
                                if (h < G) dot[h][g] += cv * qp[h][j];
                        }
                    }
                } else {
                    const uint8_t* r = kcodes + (size_t)row * 128;
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        const int kb = u >> 2, g = u & 3;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const float cv = (float)r[8 * u + i];
                            const int j = 32 * g + 8 * kb + i;
#pragma unroll
                            for (int h = 0; h < kMaxGroupHeads; ++h)
                                if (h < G) dot[h][g] += cv * qp[h][j];
                        }
                    }
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float sc = h2f(mt[g]), zc = h2f(mt[4 + g]);
#pragma unroll
                    for (int h = 0; h < kMaxGroupHeads; ++h)
                        if (h < G) s[h] += sc * dot[h][g] + zc * qsum[h][g];
                }
            } else if (KG.scheme == kTurboSplit) { // split key: two halves, then the QJL term
                const int krow = k_row(t), kb = KG.bits;
                const uint8_t* row = kcodes + (size_t)krow * split_k_row_bytes(kb);
                const uint16_t* mt = reinterpret_cast<const uint16_t*>(kmeta + (size_t)krow * 8);
                const float nO = h2f(mt[0]), nR = h2f(mt[1]), gam = h2f(mt[2]);
                const float* muO = p.mu64 + split_table_off(1 << (kb - 1));
                const float* muR = p.mu64 + split_table_off(1 << (kb - 2));
                float aO[kMaxGroupHeads], aR[kMaxGroupHeads], a2[kMaxGroupHeads];
#pragma unroll
                for (int h = 0; h < kMaxGroupHeads; ++h) aO[h] = aR[h] = a2[h] = 0.0f;
                for (int j = 0; j < 64; ++j) {
                    const float mv = muO[split_k_code(row, j, kb)];
#pragma unroll
                    for (int h = 0; h < kMaxGroupHeads; ++h)
                        if (h < G) aO[h] += mv * qp[h][j];
                }
                for (int j = 64; j < kDim; ++j) {
                    const float mv = muR[split_k_code(row, j, kb)];
#pragma unroll
                    for (int h = 0; h < kMaxGroupHeads; ++h)
                        if (h < G) aR[h] += mv * qp[h][j];
                }
                const uint32_t* qb = reinterpret_cast<const uint32_t*>(kqjl + (size_t)krow * 16);
                for (int w = 0; w < 4; ++w) {
                    const uint32_t bits = qb[w];
                    for (int i = 0; i < 32; ++i)
                        if ((bits >> i) & 1u) {
                            const int idx = 32 * w + 2 * (i & 15) + (i >> 4);
#pragma unroll
                            for (int h = 0; h < kMaxGroupHeads; ++h)
                                if (h < G) a2[h] += sp[h][idx];
                        }
                }
#pragma unroll
                for (int h = 0; h < kMaxGroupHeads; ++h)
                    if (h < G) s[h] = nO * aO[h] + nR * aR[h] + gam * kappa * (2.0f * a2[h] - spsum[h]);
            } else { // TurboQuant key
                const int krow = k_row(t);
                const uint8_t* row = kcodes + (size_t)krow * 48;
                const uint16_t* mt = reinterpret_cast<const uint16_t*>(kmeta + (size_t)krow * 4);
                const float nrm = h2f(mt[0]), gam = h2f(mt[1]);
                float a1[kMaxGroupHeads], a2[kMaxGroupHeads];
#pragma unroll
                for (int h = 0; h < kMaxGroupHeads; ++h) a1[h] = a2[h] = 0.0f;
                for (int j = 0; j < kDim; ++j) {
                    const float mv = p.mu[turbo_k_code(row, j)];
#pragma unroll
                    for (int h = 0; h < kMaxGroupHeads; ++h)
                        if (h < G) a1[h] += mv * qp[h][j];
                }
                const uint32_t* qb = reinterpret_cast<const uint32_t*>(kqjl + (size_t)krow * 16);
                for (int w = 0; w < 4; ++w) {
                    const uint32_t bits = qb[w];
                    for (int i = 0; i < 32; ++i)
                        if ((bits >> i) & 1u) {
                            const int idx = 32 * w + 2 * (i & 15) + (i >> 4);
#pragma unroll
                            for (int h = 0; h < kMaxGroupHeads; ++h)
                                if (h < G) a2[h] += sp[h][idx];
                        }
                }
#pragma unroll
                for (int h = 0; h < kMaxGroupHeads; ++h)
                    if (h < G) s[h] = nrm * a1[h] + gam * kappa * (2.0f * a2[h] - spsum[h]);
            }
        }
        // online softmax over this 64-token chunk
        float alpha[kMaxGroupHeads];
#pragma unroll
        for (int h = 0; h < kMaxGroupHeads; ++h) {
            if (h < G) {
                const float cm = wave_max(valid ? s[h] : kNegInf);
                const float mn = fmaxf(m[h], cm);
                const float al = (mn == kNegInf) ? 1.0f : exp2f(m[h] - mn);
                const float pr = valid ? exp2f(s[h] - mn) : 0.0f;
                lsum[h] = lsum[h] * al + wave_sum(pr);
                m[h] = mn;
                alpha[h] = al;
                pbuf[wave][h][l] = pr;
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int h = 0; h < kMaxGroupHeads; ++h)
            if (h < G) {
                acc0[h] *= alpha[h];
                acc1[h] *= alpha[h];
            }
        const int nv = min(64, t1 - cs0);
        const int d0 = 2 * l;
        for (int tau = 0; tau < nv; ++tau) {
            const int tok = cs0 + tau;
            float v0, v1;
            if (wsplit) {
                const float2 vv = reinterpret_cast<const float2*>(vring + (size_t)(tok % W) * kDim)[l];
                v0 = vv.x;
                v1 = vv.y;
            } else if (VG.scheme == kUniform) {
                const int blk = tok >> 5, kb = (tok & 31) >> 3, i = tok & 7;
                const int w0 = 8 * (16 * kb + (d0 & 15)) + (d0 >> 4);
                const uint16_t* mt = reinterpret_cast<const uint16_t*>(vmeta + (size_t)tok * 16);
                const int g = d0 >> 5;
                const float sc = h2f(mt[g]), zc = h2f(mt[4 + g]);
                uint32_t q0, q1;
                if (VG.bits == 3) { // bit planes in the TurboQuant-MSE V layout
                    q0 = turbo_v_code(vcodes, tok, d0, 3);
                    q1 = turbo_v_code(vcodes, tok, d0 + 1, 3);
                } else if (VG.bits == 4) {
                    const uint32_t* bp = reinterpret_cast<const uint32_t*>(vcodes + (size_t)blk * 2048);
                    const int sh = 16 * (i & 1) + 4 * (i >> 1);
                    q0 = (bp[w0] >> sh) & 15u;
                    q1 = (bp[w0 + 8] >> sh) & 15u;
                } else {
                    const uint8_t* bp = vcodes + (size_t)blk * 4096;
                    q0 = bp[8 * w0 + i];
                    q1 = bp[8 * (w0 + 8) + i];
                }
                v0 = zc + sc * (float)q0;
                v1 = zc + sc * (float)q1;
            } else if (VG.scheme == kTurboSplit) { // split: positions 2l, 2l + 1 of one half
                const int rest = d0 >= 64, levels = rest ? (1 << (VG.bits - 1)) : (1 << VG.bits);
                const float* mu = p.mu64 + (levels - 4);
                const float nrm = h2f(reinterpret_cast<const uint16_t*>(vmeta)[2 * tok + rest]);
                v0 = nrm * mu[split_v_code(vcodes, tok, d0, VG.bits)];
                v1 = nrm * mu[split_v_code(vcodes, tok, d0 + 1, VG.bits)];
            } else { // TurboQuant-MSE value (rotated domain), 3- or 4-bit codes
                const float* mu = VG.bits == 4 ? p.mu16 : p.mu;
                const float nrm = h2f(reinterpret_cast<const uint16_t*>(vmeta)[tok]);
                v0 = nrm * mu[turbo_v_code(vcodes, tok, d0, VG.bits)];
                v1 = nrm * mu[turbo_v_code(vcodes, tok, d0 + 1, VG.bits)];
            }
#pragma unroll
            for (int h = 0; h < kMaxGroupHeads; ++h)
                if (h < G) {
                    const float pr = pbuf[wave][h][tau];
                    acc0[h] += pr * v0;
                    acc1[h] += pr * v1;
                }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- combine the four waves, then write this split's partial per query head
#pragma unroll
    for (int h = 0; h < kMaxGroupHeads; ++h)
        if (h < G) {
            if (l == 0) {
                wm[wave][h] = m[h];
                wl[wave][h] = lsum[h];
            }
            wacc[wave][h][2 * l] = acc0[h];
            wacc[wave][h][2 * l + 1] = acc1[h];
        }
    // the value plane's output map tables for the lane's channel pair
    const bool vsplit = VG.scheme == kTurboSplit;
    const size_t vtab = (size_t)(kvh * 2 + 1) * kDim;
    float2 cs2 = make_float2(1.0f, 1.0f), sg2 = cs2;
    int2 pm2 = make_int2(2 * l, 2 * l + 1);
    if (!wsplit) {
        if (VG.sinkhorn) cs2 = reinterpret_cast<const float2*>(p.cs + vtab)[l];
        if (VG.rotate || vsplit) sg2 = reinterpret_cast<const float2*>(p.signs + vtab)[l];
        if (vsplit) pm2 = reinterpret_cast<const int2*>(p.perm + (size_t)kvh * kDim)[l];
    }
    __syncthreads();
    // partial of this split per query head in the plain channel domain: one wave per head, lane l
    // the channel pair 2l, 2l + 1, mapped back by the value plane's output map
    for (int h = wave; h < G; h += 4) {
        float M = kNegInf;
        for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][h]);
        float A0 = 0.0f, A1 = 0.0f, L = 0.0f;
        if (M != kNegInf) {
            for (int w = 0; w < 4; ++w) {
                if (wm[w][h] == kNegInf) continue;
                const float f = exp2f(wm[w][h] - M);
                A0 += wacc[w][h][2 * l] * f;
                A1 += wacc[w][h][2 * l + 1] * f;
                L += wl[w][h] * f;
            }
        }
        if (!wsplit) value_out_map(A0, A1, vsplit, VG.sinkhorn, VG.rotate, cs2, sg2);
        float* part = p.partials +
                      (((size_t)b * p.Hq + kvh * G + h) * p.n_splits_total + split) * kPartialFloats;
        if (l == 0) {
            part[0] = M;
            part[1] = L;
        }
        part[4 + pm2.x] = A0;
        part[4 + pm2.y] = A1;
    }
}

// Fixed-order merge of the splits of one (sequence, query head): the partials arrive in the plain
// channel domain (the split kernels apply the value plane's output map), so
// out = (sum_s 2^(m_s - M) acc_s) / (sum_s 2^(m_s - M) l_s).  256 threads: thread t owns channels
// 4 (t / 8) .. 4 (t / 8) + 3 of splits t % 8, t % 8 + 8, ..., combined in ascending order; the
// eight threads of a channel group (consecutive lanes) then combine over a fixed xor tree, so the
// result depends only on the split count, with no shared memory and no barrier.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
    const int hq = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int c4 = t >> 3, part = t & 7;
    float4* out = reinterpret_cast<float4*>(p.out + ((size_t)b * p.Hq + hq) * kDim) + c4;
    // Every split wrote its partial (an empty split: m = -inf, l = 0, acc = 0), so all loads are
    // issued before anything is tested, and the combine has no branch that the compiler could
    // turn into a second round trip; an empty sequence (l = 0) is resolved at the store.
    const float* base = p.partials + ((size_t)b * p.Hq + hq) * p.n_splits_total * kPartialFloats;
    float m = kNegInf, l = 0.0f;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto merge_round = [&](int s0) __attribute__((always_inline)) {
        float ms[8], ls[8];
        float4 as[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // a split past the last re-reads the last one and is given weight 0
            const int s = s0 + 8 * i;
            const float* ps = base + (size_t)min(s, p.n_splits_total - 1) * kPartialFloats;
            const float2 ml = *reinterpret_cast<const float2*>(ps);
            ms[i] = s < p.n_splits_total ? ml.x : kNegInf;
            ls[i] = ml.y;
            as[i] = *reinterpret_cast<const float4*>(ps + 4 + 4 * c4);
        }
        // all of the round's loads in flight before the first is consumed
#pragma unroll
        for (int i = 0; i < 8; ++i)
            asm volatile("" ::"v"(ms[i]), "v"(ls[i]), "v"(as[i].x), "v"(as[i].y), "v"(as[i].z), "v"(as[i].w));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // weights exp2(m - mn) and exp2(ms - mn) are 0 for a -inf side; both sides -inf
            // leaves the state as it is
            const float mn = fmaxf(m, ms[i]);
            const bool none = (mn == kNegInf);
            const float fo = none ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
            const float fn = none ? 0.0f : __builtin_amdgcn_exp2f(ms[i] - mn);
            m = mn;
            l = fmaf(ls[i], fn, l * fo);
            a.x = fmaf(as[i].x, fn, a.x * fo);
            a.y = fmaf(as[i].y, fn, a.y * fo);
            a.z = fmaf(as[i].z, fn, a.z * fo);
            a.w = fmaf(as[i].w, fn, a.w * fo);
        }
    };
    // the first round of up to 64 splits unconditionally (no branch ahead of its loads)
    merge_round(part);
    for (int s0 = part + 64; s0 < p.n_splits_total; s0 += 64) merge_round(s0);
    // the eight split classes of the channel group: pairs at xor distance 1, 2, 4 (a fixed tree;
    // lane part == 0 holds the result)
    auto pair = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float mo = xor_lane<h>(m), lo = xor_lane<h>(l);
        const float ax = xor_lane<h>(a.x), ay = xor_lane<h>(a.y), az = xor_lane<h>(a.z), aw = xor_lane<h>(a.w);
        const float mn = fmaxf(m, mo);
        const float f = (m == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        const float g = (mo == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
        m = mn;
        l = l * f + lo * g;
        a.x = a.x * f + ax * g;
        a.y = a.y * f + ay * g;
        a.z = a.z * f + az * g;
        a.w = a.w * f + aw * g;
    };
    pair(std::integral_constant<int, 1>{});
    pair(std::integral_constant<int, 2>{});
    pair(std::integral_constant<int, 4>{});
    if (part == 0) {
        // l = 0 only for an empty sequence (a non-empty one has a weight-1 token in some split)
        const float inv_l = 1.0f / l;
        *out = (l == 0.0f) ? make_float4(0.0f, 0.0f, 0.0f, 0.0f) : make_float4(a.x * inv_l, a.y * inv_l, a.z * inv_l, a.w * inv_l);
    }
}

} // namespace

// Library-held scratch for the split partials of kvq_attn_decode_static (callers that cannot
// allocate).  Each GPU the library runs on holds one copy until the process ends; in host code the
// name is only a stand-in, so kernels receive the per-device address taken below.
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};
} // namespace

hipError_t static_scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device]) return hipSuccess;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice; // the device must be current
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = static_cast<float*>(ptr);
    return hipSuccess;
}

float* static_scratch(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    return g_scratch_ptr[device];
}

hipError_t launch_decode_vec(const DecodeParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    dim3 grid(p.n_splits_total, p.Hkv, p.batch);
    hipExtLaunchKernelGGL(decode_vec_kernel, grid, dim3(256), 0, s, ev0, ev1, 0, p);
    return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t s) {
    hipLaunchKernelGGL(decode_merge_kernel, dim3(p.Hq, p.batch), dim3(256), 0, s, p);
    return hipGetLastError();
}

} // namespace kvq
