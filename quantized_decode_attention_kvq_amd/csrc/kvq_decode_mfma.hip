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
//  * Split partials are merged by the last workgroup to finish for each (sequence, kv head)
//    (device-scope arrival counter, fixed merge order), which also applies R_V^-1 and c_V.
//    Partials travel through write-through stores/loads, so no cache flush is needed.
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

// Write-through (agent-scope) accesses for the split partials and the arrival counter: they
// reach the device-coherent level directly, so no L2 writeback/invalidate is needed to hand
// data between workgroups on different dies.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    __shared__ float s_M[kMaxGroupHeads], s_L[kMaxGroupHeads];
    __shared__ int s_last;

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
    const int G = p.G, W = p.window;
    const int n = p.len[b];
    const int nq = (W > 0) ? max(0, n - W) : n;
    const bool wsplit = (W > 0) && (split == p.n_splits);
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

    // ---------------- query preparation (once per workgroup) ----------------
    for (int h = wave; h < G; h += kNW) {
        const size_t off = ((size_t)b * p.Hq + kvh * G + h) * kDim;
        float a, c;
        if (p.dtype == 0) {
            const float2 v = reinterpret_cast<const float2*>(static_cast<const float*>(p.q) + off)[l];
            a = v.x;
            c = v.y;
        } else {
            const uint32_t v = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + off)[l];
            a = bf2f((uint16_t)(v & 0xffff));
            c = bf2f((uint16_t)(v >> 16));
        }
        s_qw[h][2 * l] = a * p.qscale;
        s_qw[h][2 * l + 1] = c * p.qscale;
        if (KG.rotate) {
            const float* sg = p.signs + (size_t)(kvh * 2 + 0) * kDim;
            if (sg[2 * l] < 0.0f) a = -a;
            if (sg[2 * l + 1] < 0.0f) c = -c;
            hadamard_wave(a, c, l);
            a *= c0f();
            c *= c0f();
        }
        if (KG.sinkhorn) {
            const float* cs = p.cs + (size_t)(kvh * 2 + 0) * kDim;
            a *= cs[2 * l];
            c *= cs[2 * l + 1];
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

    const int lr = l & 15, lq = l >> 4; // column / quarter of the 16x16 tiles

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

        const int tok_begin = split * p.split_tokens;
        const int tok_end = min(nq, tok_begin + p.split_tokens);
        const int nch = (tok_end > tok_begin) ? (tok_end - tok_begin + 63) / 64 : 0;
        // per-wave streams (advanced by kNW chunks per iteration)
        const int t0w = tok_begin + 64 * wave;
        const uint8_t* kc_p = kcodes + ((size_t)t0w + lr) * (16 * KB) + (16 * KB / 4) * lq;
        const uint8_t* km_p = kmeta + ((size_t)t0w + lr) * 16;
        const uint8_t* vc_p = vcodes + (size_t)(t0w / 32) * (512 * VB) + (size_t)(32 * VB / 4) * l;
        const uint8_t* vm_p = vmeta + ((size_t)t0w + 4 * lr) * 16;
        constexpr size_t kc_step = (size_t)64 * kNW * 16 * KB, km_step = (size_t)64 * kNW * 16;
        constexpr size_t vc_step = (size_t)2 * kNW * 512 * VB, vm_step = (size_t)64 * kNW * 16;
        KRegs<KB> kr;
        VRegs<VB> vr;
        if (wave < nch) {
            load_k(kr, kc_p, km_p);
            load_v(vr, vc_p, vm_p);
        }
        for (int ci = wave; ci < nch; ci += kNW) {
            const int c0 = tok_begin + 64 * ci;
            const bool more = ci + kNW < nch;
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
            if (more) {
                kc_p += kc_step;
                km_p += km_step;
                load_k(kr, kc_p, km_p);
            }

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
            if (more) {
                vc_p += vc_step;
                vm_p += vm_step;
                load_v(vr, vc_p, vm_p);
            }
        }
        // reduce the per-lane softmax sums over each row of 16 lanes
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            l_run[mb] = row_sum16(l_run[mb]);
#pragma unroll
            for (int g = 0; g < 4; ++g) z_run[mb][g] = row_sum16(z_run[mb][g]);
        }
    } else {
        // ---------------- FP32 window split (vector ALU): tokens nq .. n-1 ----------------
        // kWinPW tokens per wave: lanes 0..kWinPW-1 score one token each, then every lane
        // accumulates two channels over those tokens.
        constexpr int kWinPW = kWindowMax / kNW;
        float* pb = reinterpret_cast<float*>(my_p); // [8 heads][kWinPW] probabilities
        const int base = nq + kWinPW * wave;
        if (base < n) {
            const int t = base + l;
            const bool valid = (l < kWinPW) && (t < n);
            float sc[kMaxGroupHeads];
#pragma unroll
            for (int h = 0; h < kMaxGroupHeads; ++h) sc[h] = 0.0f;
            if (valid) {
                const float* kr = kring + (size_t)(t % W) * kDim;
#pragma unroll 4
                for (int j = 0; j < kDim; j += 4) {
                    const float4 kv = *reinterpret_cast<const float4*>(kr + j);
#pragma unroll
                    for (int h = 0; h < kMaxGroupHeads; ++h)
                        if (h < G)
                            sc[h] += kv.x * s_qw[h][j] + kv.y * s_qw[h][j + 1] + kv.z * s_qw[h][j + 2] +
                                     kv.w * s_qw[h][j + 3];
                }
            }
#pragma unroll
            for (int h = 0; h < kMaxGroupHeads; ++h) {
                if (h < G) {
                    const float mh = wave_max(valid ? sc[h] : kNegInf);
                    const float pr = valid ? exp2f(sc[h] - mh) : 0.0f;
                    wm[h] = mh;
                    wl[h] = wave_sum(pr);
                    if (l < kWinPW) pb[h * kWinPW + l] = pr;
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            float2 vv[kWinPW];
#pragma unroll
            for (int tau = 0; tau < kWinPW; ++tau) {
                const int tt = min(base + tau, n - 1);
                vv[tau] = reinterpret_cast<const float2*>(vring + (size_t)(tt % W) * kDim)[l];
            }
#pragma unroll
            for (int tau = 0; tau < kWinPW; ++tau) {
                if (base + tau < n) {
#pragma unroll
                    for (int h = 0; h < kMaxGroupHeads; ++h)
                        if (h < G) {
                            const float pr = pb[h * kWinPW + tau];
                            wacc0[h] = fmaf(pr, vv[tau].x, wacc0[h]);
                            wacc1[h] = fmaf(pr, vv[tau].y, wacc1[h]);
                        }
                }
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
    const int S_total = p.n_splits_total;
    float* part_kvh = p.partials + (((size_t)b * p.Hkv + kvh) * S_total) * G * kPartialFloats;
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
        float* part = part_kvh + ((size_t)split * G + h) * kPartialFloats;
        st_agent(part + 4 + d, A);
        if (d == 0) {
            st_agent(part + 0, M);
            st_agent(part + 1, L);
        }
    }

    // ---------------- the last workgroup of this (sequence, kv head) merges ----------------
    // Every partial store above is write-through and has completed once the barrier's wait on
    // outstanding memory operations returns; only then is the arrival counted.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[b * p.Hkv + kvh], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (unsigned)(S_total - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;

    float* s_wgt = s_acc;                         // [8][S_total] split weights
    float* s_fin = s_acc + kMaxGroupHeads * (kMaxSplits + 1);  // [8][128] code-domain sums
    float* s_finw = s_fin + kMaxGroupHeads * kDim;             // [8][128] window sums
    for (int h = wave; h < G; h += kNW) {
        float M = kNegInf;
        for (int s = l; s < S_total; s += 64) M = fmaxf(M, ld_agent(part_kvh + ((size_t)s * G + h) * kPartialFloats));
        M = wave_max(M);
        float L = 0.0f;
        for (int s = l; s < S_total; s += 64) {
            const float* ps = part_kvh + ((size_t)s * G + h) * kPartialFloats;
            const float ms = ld_agent(ps);
            const float w = (ms == kNegInf) ? 0.0f : exp2f(ms - M);
            s_wgt[h * (kMaxSplits + 1) + s] = w;
            L = fmaf(w, ld_agent(ps + 1), L);
        }
        L = wave_sum(L);
        if (l == 0) {
            s_M[h] = M;
            s_L[h] = L;
        }
    }
    __syncthreads();
    {
        // code-domain splits: every thread sums a strided subset of splits for one (head, 4
        // channels); loads are issued in batches of 4 so their latencies overlap.  The subsets
        // and their final sum run in a fixed order.
        const int items = G * 32;
        const int nparts = max(1, (kNW * 64) / items);
        const int nqs = p.n_splits;
        float4* s_red = reinterpret_cast<float4*>(s_finw + kMaxGroupHeads * kDim); // [nparts][items]
        if (tid < items * nparts) {
            const int item = tid % items, part = tid / items;
            const int h = item >> 5, d4 = item & 31;
            float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (int s0 = part; s0 < nqs; s0 += 4 * nparts) {
                float4 v[4];
                float w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s = s0 + u * nparts;
                    if (s < nqs) {
                        w[u] = s_wgt[h * (kMaxSplits + 1) + s];
                        const float* ps = part_kvh + ((size_t)s * G + h) * kPartialFloats + 4 + 4 * d4;
                        v[u] = make_float4(ld_agent(ps), ld_agent(ps + 1), ld_agent(ps + 2), ld_agent(ps + 3));
                    } else {
                        w[u] = 0.0f;
                        v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    a.x = fmaf(w[u], v[u].x, a.x);
                    a.y = fmaf(w[u], v[u].y, a.y);
                    a.z = fmaf(w[u], v[u].z, a.z);
                    a.w = fmaf(w[u], v[u].w, a.w);
                }
            }
            s_red[part * items + item] = a;
        }
        // the FP32 window split
        if (tid < items) {
            const int h = tid >> 5, d4 = tid & 31;
            float4 aw = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (W > 0) {
                const float w = s_wgt[h * (kMaxSplits + 1) + nqs];
                const float* ps = part_kvh + ((size_t)nqs * G + h) * kPartialFloats + 4 + 4 * d4;
                const float4 v = make_float4(ld_agent(ps), ld_agent(ps + 1), ld_agent(ps + 2), ld_agent(ps + 3));
                aw = make_float4(w * v.x, w * v.y, w * v.z, w * v.w);
            }
            *reinterpret_cast<float4*>(s_finw + h * kDim + 4 * d4) = aw;
        }
        __syncthreads();
        if (tid < items) {
            float4 a = s_red[tid];
            for (int q = 1; q < nparts; ++q) {
                const float4 b2 = s_red[q * items + tid];
                a.x += b2.x;
                a.y += b2.y;
                a.z += b2.z;
                a.w += b2.w;
            }
            const int h = tid >> 5, d4 = tid & 31;
            *reinterpret_cast<float4*>(s_fin + h * kDim + 4 * d4) = a;
        }
    }
    __syncthreads();
    for (int h = wave; h < G; h += kNW) {
        float a = s_fin[h * kDim + 2 * l], c = s_fin[h * kDim + 2 * l + 1];
        if (VG.sinkhorn) {
            const float* cs = p.cs + (size_t)(kvh * 2 + 1) * kDim;
            a *= cs[2 * l];
            c *= cs[2 * l + 1];
        }
        if (VG.rotate) {
            hadamard_wave(a, c, l);
            a *= c0f();
            c *= c0f();
            const float* sg = p.signs + (size_t)(kvh * 2 + 1) * kDim;
            if (sg[2 * l] < 0.0f) a = -a;
            if (sg[2 * l + 1] < 0.0f) c = -c;
        }
        const float L = s_L[h];
        const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
        float2 o;
        o.x = (a + s_finw[h * kDim + 2 * l]) * inv;
        o.y = (c + s_finw[h * kDim + 2 * l + 1]) * inv;
        reinterpret_cast<float2*>(p.out + ((size_t)b * p.Hq + kvh * G + h) * kDim)[l] = o;
    }
    if (tid == 0) __hip_atomic_store(&p.counters[b * p.Hkv + kvh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 8 waves (2 per SIMD, <= 256 registers each) for the 4-bit / 4-bit, <= 4 heads-per-group
// variant; 4 waves (1 per SIMD, up to 512 registers) for the variants with more operand state.
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
