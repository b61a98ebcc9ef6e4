// Matrix-core (MFMA) split-K decode attention over uniform 4/8-bit caches, gfx950.
//
// What it computes (pages by title and section): the quantcpp article's progressive cache
// (4-bit codes with fp16 scale/zero per 32 channels, newest 128 tokens read in FP32) and the
// KVarN post's Walsh-Hadamard + Sinkhorn-balanced 4-bit cache: out = softmax(q k^T * scale) v,
// with k, v the dequantized tokens, scores in the rotated/balanced domain via q' = R(q) .* c and
// the output un-rotated at the end: R^-1(c .* sum_t p_t yhat_t).
//
// How (one workgroup = NW waves per (sequence, kv head, token split); each wave streams 64-token
// chunks):
//  * Scores: v_mfma_f32_16x16x32_f16 with A = the G query rows split into fp16 hi + lo parts and
//    laid out as (head, group) rows, B = the raw 4-bit / 8-bit codes.  4-bit codes enter the
//    B operand as fp16 subnormal bit patterns (code * 2^-24, or 16 * code * 2^-24 for the odd
//    nibbles, compensated in A), 8-bit codes as zero-extended bytes (code * 2^-24): no
//    int->float conversion, and products are exact.  The per-group fp16 scale and zero fold in
//    afterwards: s_t = sum_g scale_g,t * dot_g + zero_g,t * sum_{j in g} q'_j.
//  * Online softmax in the log2 domain (q' carries softmax_scale * log2(e) and a per-head power
//    of two that keeps 16 q' inside fp16 range).
//  * PV: A = p * scale_g (fp16 hi + lo) staged through LDS into matrix-operand order, B = raw V
//    codes from the token-blocked V plane (dense over tokens), plus a vector-ALU sum of
//    p * zero_g.
//  * Each split writes one partial (running max, sum, acc[128]) per query head; the separate
//    merge kernel combines them in a fixed order and applies c_V and R_V^-1.
//  * The FP32 window (progressive mode) is one extra split computed on the vector ALU.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kPRow = 72;                       // halves per staged P row: 64 tokens + 8 pad
constexpr int kPWave = 4 * 2 * 8 * kPRow;       // halves per wave: [group][hi/lo][row][token]

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h8 as_h8(u4 v) { return __builtin_bit_cast(h8, v); }
__device__ __forceinline__ float c0f() { return __uint_as_float(0x3DB504F3u); }
__device__ __forceinline__ float lo_h(uint32_t w) { return (float)__builtin_bit_cast(h2v, w)[0]; }
__device__ __forceinline__ float hi_h(uint32_t w) { return (float)__builtin_bit_cast(h2v, w)[1]; }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 4-bit word (channel/token i at bit 16*(i%2) + 4*(i/2)) -> 8 fp16 subnormal operands in
// natural order, slots 2,3,6,7 carry an extra factor 16.
__device__ __forceinline__ u4 unpack4(uint32_t x) {
    u4 r;
    r.x = x & 0x000F000Fu;
    r.y = x & 0x00F000F0u;
    const uint32_t y = x >> 8;
    r.z = y & 0x000F000Fu;
    r.w = y & 0x00F000F0u;
    return r;
}

// 8 bytes (value i at byte i) -> 8 zero-extended 16-bit operands in natural order.
__device__ __forceinline__ u4 unpack8(uint32_t x0, uint32_t x1) {
    u4 r;
    r.x = __builtin_amdgcn_perm(0u, x0, 0x0c010c00u);
    r.y = __builtin_amdgcn_perm(0u, x0, 0x0c030c02u);
    r.z = __builtin_amdgcn_perm(0u, x1, 0x0c010c00u);
    r.w = __builtin_amdgcn_perm(0u, x1, 0x0c030c02u);
    return r;
}

// Reductions across the 16 lanes of a DPP row (lanes 16r .. 16r+15): swap within pairs, within
// quads, mirror within half-rows, mirror within the row; every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));  // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));  // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v)); // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v)); // row_mirror
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ void hadamard_wave(float& a, float& b, int l) {
    const float s = a + b, d = a - b;
    a = s;
    b = d;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float pa = __shfl_xor(a, m), pb = __shfl_xor(b, m);
        const bool lower = (l & m) == 0;
        a = lower ? (a + pa) : (pa - a);
        b = lower ? (b + pb) : (pb - b);
    }
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Loads of one 64-token chunk, split so that the next chunk's K can be requested as soon as the
// scores are done and its V as soon as PV is done.  Per lane: K codes and meta of rows
// 16j + (lane % 16) of the 64-token block; V codes of the two 32-token blocks (32 * VB / 4 bytes
// at lane * 32 * VB / 4); V meta of tokens 4 * (lane % 16) + 0..3.
template <int KB>
struct KRegs {
    u4 kc[4][KB / 4], km[4];
};
template <int VB>
struct VRegs {
    u4 vc[2][VB / 2], vm[4];
};

template <int KB>
__device__ __forceinline__ void load_k(KRegs<KB>& r, const uint8_t* kc, const uint8_t* km) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int u = 0; u < KB / 4; ++u)
            r.kc[j][u] = *reinterpret_cast<const u4*>(kc + j * 16 * 16 * KB + 16 * u);
        r.km[j] = *reinterpret_cast<const u4*>(km + j * 16 * 16);
    }
}
template <int VB>
__device__ __forceinline__ void load_v(VRegs<VB>& r, const uint8_t* vc, const uint8_t* vm) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int u = 0; u < VB / 2; ++u) r.vc[k][u] = *reinterpret_cast<const u4*>(vc + k * 512 * VB + 16 * u);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.vm[j] = *reinterpret_cast<const u4*>(vm + 16 * j);
}

template <int KB, int VB, int MB, int kNW>
__global__ __launch_bounds__(kNW * 64) void decode_mfma_kernel(DecodeParams p) {
    __shared__ float s_q[kMaxGroupHeads][kDim];   // q' in the rotated/balanced domain, scaled
    __shared__ float s_qw[kMaxGroupHeads][kDim];  // plain q * scale * log2e (FP32 window)
    __shared__ float s_qsum[kMaxGroupHeads][4];
    __shared__ float s_qfac[kMaxGroupHeads];
    __shared__ __align__(16) _Float16 s_p[kNW * kPWave];
    __shared__ float s_wm[kNW][kMaxGroupHeads], s_wl[kNW][kMaxGroupHeads];
    __shared__ float s_wz[kNW][kMaxGroupHeads][4];

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
    const float* kring = reinterpret_cast<const float*>(slot + p.plane_off[0] + KG.ring_off);
    const uint8_t* vcodes = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.codes_off);
    const uint8_t* vmeta = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.meta_off);
    const float* vring = reinterpret_cast<const float*>(slot + p.plane_off[1] + VG.ring_off);
    const float UK = (KB == 4) ? 1048576.0f : 16777216.0f; // 2^20 / 2^24: unit of a code product
    const float UV = (VB == 4) ? 1048576.0f : 16777216.0f;

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
                qa[i] = bf2f((uint16_t)(v & 0xffff));
                qc[i] = bf2f((uint16_t)(v >> 16));
            }
        }
    }
    const float2 sgn = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 0) * kDim)[l];
    const float2 csk = reinterpret_cast<const float2*>(p.cs + (size_t)(kvh * 2 + 0) * kDim)[l];
    const int lr = l & 15, lq = l >> 4; // column / quarter of the 16x16 tiles
    const int tok_begin = split * p.split_tokens;
    const int tok_end = wsplit ? tok_begin : min(nq, tok_begin + p.split_tokens);
    const int nch = (tok_end > tok_begin) ? (tok_end - tok_begin + 63) / 64 : 0;
    // chunk ci of this split starts at token tok_begin + 64 ci; a lane's addresses in it:
    auto kc_at = [&](int ci) { return kcodes + ((size_t)tok_begin + 64 * ci + lr) * (16 * KB) + (16 * KB / 4) * lq; };
    auto km_at = [&](int ci) { return kmeta + ((size_t)tok_begin + 64 * ci + lr) * 16; };
    auto vc_at = [&](int ci) {
        return vcodes + (size_t)((tok_begin + 64 * ci) / 32) * (512 * VB) + (size_t)(32 * VB / 4) * l;
    };
    auto vm_at = [&](int ci) { return vmeta + ((size_t)tok_begin + 64 * ci + 4 * lr) * 16; };
    // The wave's first chunk is requested right away; each later chunk is requested as soon as
    // the registers it goes into have been consumed (K after the scores, V after PV).
    KRegs<KB> kr;
    VRegs<VB> vr;
    if (wave < nch) {
        load_k(kr, kc_at(wave), km_at(wave));
        load_v(vr, vc_at(wave), vm_at(wave));
    }

    // ---------------- query preparation (once per workgroup) ----------------
#pragma unroll
    for (int i = 0; i < kHPW; ++i) {
        const int h = wave + i * kNW;
        if (h >= G) break;
        float a = qa[i], c = qc[i];
        s_qw[h][2 * l] = a * p.qscale;
        s_qw[h][2 * l + 1] = c * p.qscale;
        if (KG.rotate) {
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

    // per-wave softmax state, in the score layout (lane: head 4*mb + lq, column lr)
    float m_run[MB], l_run[MB], z_run[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        m_run[mb] = kNegInf;
        l_run[mb] = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) z_run[mb][g] = 0.0f;
    }
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

    _Float16* my_p = s_p + wave * kPWave;

    if (!wsplit) {
        // ---------------- A operands: (head, group) rows of q' split into fp16 hi + lo -------
        h8 Ahi[MB][4], Alo[MB][4];
        float qs_l[MB][4], F[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int h = 4 * mb + (lr >> 2), gq = lr & 3;
            const int hc = min(h, G - 1);
            h8 hi, lo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float w = (KB == 4 && (i == 0 || i == 1 || i == 4 || i == 5)) ? 16.0f : 1.0f;
                const float x = (h < G) ? s_q[hc][32 * gq + 8 * lq + i] * w : 0.0f;
                const _Float16 xh = (_Float16)x;
                hi[i] = xh;
                lo[i] = (_Float16)(x - (float)xh);
            }
            const h8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                Ahi[mb][g] = (g == gq) ? hi : zero;
                Alo[mb][g] = (g == gq) ? lo : zero;
            }
            const int hs = min(4 * mb + lq, G - 1);
#pragma unroll
            for (int g = 0; g < 4; ++g) qs_l[mb][g] = s_qsum[hs][g] * (1.0f / UK);
            F[mb] = UK * s_qfac[hs];
        }

        for (int ci = wave; ci < nch; ci += kNW) {
            const int c0 = tok_begin + 64 * ci;
            const int nci = ci + kNW; // the chunk the registers are refilled with
            const bool more = nci < nch;
            const auto& kc = kr.kc;
            const auto& km = kr.km;
            const auto& vc = vr.vc;
            const auto& vm = vr.vm;

            // ---- scores
            float raw[MB][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h8 B[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if (KB == 4)
                        B[g] = as_h8(unpack4(kc[j][0][g]));
                    else
                        B[g] = as_h8(unpack8(kc[j][g >> 1][2 * (g & 1)], kc[j][g >> 1][2 * (g & 1) + 1]));
                }
                const bool valid = (c0 + 4 * lr + j) < tok_end;
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
            }

            // the next chunk's K is requested as soon as this chunk's scores are formed
            if (more) load_k(kr, kc_at(nci), km_at(nci));

            // ---- online softmax
            float pj[MB][4], alpha[MB];
            bool grew = false;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float t = fmaxf(fmaxf(raw[mb][0], raw[mb][1]), fmaxf(raw[mb][2], raw[mb][3]));
                t = row_max16(t);
                const float mnew = fmaxf(m_run[mb], t * F[mb]);
                const bool inf = (mnew == kNegInf);
                alpha[mb] = inf ? 1.0f : exp2f(m_run[mb] - mnew);
                grew |= (mnew > m_run[mb]);
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pj[mb][j] = inf ? 0.0f : exp2f(fmaf(raw[mb][j], F[mb], -mnew));
                    s += pj[mb][j];
                }
                l_run[mb] = l_run[mb] * alpha[mb] + s;
                m_run[mb] = mnew;
#pragma unroll
                for (int g = 0; g < 4; ++g) z_run[mb][g] *= alpha[mb];
            }
            if (__ballot(grew) != 0) {
                // rescale the PV accumulators: row 4*lq + v of the 16x16 tiles is head 4*lq + v
                float av[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float a0 = readlane_f(alpha[0], 16 * v);
                    float a1 = 1.0f;
                    if (MB == 2) a1 = readlane_f(alpha[MB - 1], 16 * v);
                    av[v] = (lq == 0) ? a0 : ((lq == 1) ? a1 : 1.0f);
                }
#pragma unroll
                for (int N = 0; N < 8; ++N)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[N][v] *= av[v];
            }

            // ---- zero-point term, and P * scale staged into matrix-operand order
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    z_run[mb][0] = fmaf(pj[mb][j], lo_h(vm[j].z), z_run[mb][0]);
                    z_run[mb][1] = fmaf(pj[mb][j], hi_h(vm[j].z), z_run[mb][1]);
                    z_run[mb][2] = fmaf(pj[mb][j], lo_h(vm[j].w), z_run[mb][2]);
                    z_run[mb][3] = fmaf(pj[mb][j], hi_h(vm[j].w), z_run[mb][3]);
                }
                const int row = 4 * mb + lq;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    h4 hv, lv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float w = (VB == 4 && j < 2) ? 16.0f : 1.0f;
                        const uint32_t sw = (g < 2) ? vm[j].x : vm[j].y;
                        const float sc = (g & 1) ? hi_h(sw) : lo_h(sw);
                        const float P = (pj[mb][j] * w) * sc;
                        const _Float16 ph = (_Float16)P;
                        hv[j] = ph;
                        lv[j] = (_Float16)(P - (float)ph);
                    }
                    *reinterpret_cast<h4*>(my_p + ((g * 2 + 0) * 8 + row) * kPRow + 4 * lr) = hv;
                    *reinterpret_cast<h4*>(my_p + ((g * 2 + 1) * 8 + row) * kPRow + 4 * lr) = lv;
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

            // ---- PV over the two 32-token blocks of the chunk
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                h8 Ph[4], Pl[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    Ph[g] = *reinterpret_cast<const h8*>(my_p + ((g * 2 + 0) * 8 + (lr & 7)) * kPRow + 32 * k + 8 * lq);
                    Pl[g] = *reinterpret_cast<const h8*>(my_p + ((g * 2 + 1) * 8 + (lr & 7)) * kPRow + 32 * k + 8 * lq);
                }
#pragma unroll
                for (int N = 0; N < 8; ++N) {
                    h8 Bv;
                    if (VB == 4)
                        Bv = as_h8(unpack4(vc[k][N >> 2][N & 3]));
                    else
                        Bv = as_h8(unpack8(vc[k][N >> 1][2 * (N & 1)], vc[k][N >> 1][2 * (N & 1) + 1]));
                    acc[N] = mfma16(Ph[N >> 1], Bv, acc[N]);
                    acc[N] = mfma16(Pl[N >> 1], Bv, acc[N]);
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            if (more) load_v(vr, vc_at(nci), vm_at(nci));
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
                const float al = (mnew == kNegInf) ? 1.0f : exp2f(wm[h] - mnew);
                const float p0 = (s0 == kNegInf) ? 0.0f : exp2f(s0 - mnew);
                const float p1 = (s1 == kNegInf) ? 0.0f : exp2f(s1 - mnew);
                const float p2 = (s2 == kNegInf) ? 0.0f : exp2f(s2 - mnew);
                const float p3 = (s3 == kNegInf) ? 0.0f : exp2f(s3 - mnew);
                wl[h] = wl[h] * al + ((p0 + p1) + (p2 + p3));
                wm[h] = mnew;
                wacc0[h] = fmaf(p3, vv[3].x, fmaf(p2, vv[2].x, fmaf(p1, vv[1].x, fmaf(p0, vv[0].x, wacc0[h] * al))));
                wacc1[h] = fmaf(p3, vv[3].y, fmaf(p2, vv[2].y, fmaf(p1, vv[1].y, fmaf(p0, vv[0].y, wacc1[h] * al))));
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
                for (int g = 0; g < 4; ++g) s_wz[wave][h][g] = z_run[mb][g];
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
    float* s_acc = reinterpret_cast<float*>(s_p); // [kNW][8][128]
    if (!wsplit) {
#pragma unroll
        for (int N = 0; N < 8; ++N)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int h = 4 * lq + v;
                if (h < G) s_acc[(wave * 8 + h) * kDim + 16 * N + lr] = acc[N][v] * UV;
            }
    } else {
        for (int h = 0; h < G; ++h) {
            s_acc[(wave * 8 + h) * kDim + 2 * l] = wacc0[h];
            s_acc[(wave * 8 + h) * kDim + 2 * l + 1] = wacc1[h];
        }
    }
    __syncthreads();
    // partial of this split for each of its query heads: [b][hq][split][m, l, -, -, acc[128]]
    for (int idx = tid; idx < G * kDim; idx += kNW * 64) {
        const int h = idx >> 7, d = idx & 127;
        float M = kNegInf;
        for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_wm[w][h]);
        float A = 0.0f, L = 0.0f;
        if (M != kNegInf) {
            for (int w = 0; w < kNW; ++w) {
                if (s_wm[w][h] == kNegInf) continue;
                const float f = exp2f(s_wm[w][h] - M);
                A = fmaf(f, s_acc[(w * 8 + h) * kDim + d] + s_wz[w][h][d >> 5], A);
                L = fmaf(f, s_wl[w][h], L);
            }
        }
        float* part = p.partials + (((size_t)b * p.Hq + kvh * G + h) * p.n_splits_total + split) * kPartialFloats;
        part[4 + d] = A;
        if (d == 0) {
            part[0] = M;
            part[1] = L;
        }
    }
}

template <int KB, int VB, int MB>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
    constexpr int NW = (KB == 4 && VB == 4 && MB == 1) ? 8 : 4;
    dim3 grid(p.n_splits_total, p.Hkv, p.batch);
    hipLaunchKernelGGL((decode_mfma_kernel<KB, VB, MB, NW>), grid, dim3(NW * 64), 0, s, p);
    return hipGetLastError();
}

} // namespace

bool mfma_path_supported(const DecodeParams& p) {
    return p.geom[0].scheme == kUniform && p.geom[1].scheme == kUniform &&
           (p.geom[0].bits == 4 || p.geom[0].bits == 8) && (p.geom[1].bits == 4 || p.geom[1].bits == 8) &&
           p.G <= kMaxGroupHeads;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s) {
    const int kb = p.geom[0].bits, vb = p.geom[1].bits;
    const bool two = p.G > 4;
    if (kb == 4 && vb == 4) return two ? launch_t<4, 4, 2>(p, s) : launch_t<4, 4, 1>(p, s);
    if (kb == 4 && vb == 8) return two ? launch_t<4, 8, 2>(p, s) : launch_t<4, 8, 1>(p, s);
    if (kb == 8 && vb == 4) return two ? launch_t<8, 4, 2>(p, s) : launch_t<8, 4, 1>(p, s);
    return two ? launch_t<8, 8, 2>(p, s) : launch_t<8, 8, 1>(p, s);
}

} // namespace kvq
