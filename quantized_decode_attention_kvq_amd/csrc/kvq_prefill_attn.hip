// Multi-query attention of a prefill chunk over the compressed cache, gfx950 matrix cores.
//
// What it computes (pages by title and section):
//  * quantcpp article "Beyond RAG...", v3.2 batched prefill: a prompt is processed as whole
//    chunks.  Here the n_q newest tokens of each sequence (already appended to the cache) are the
//    chunk's queries; query i, at position pos_i = len - n_q + i, attends to the cache as it
//    stands, up to its own position: out_i = softmax(q_i k_t^T * scale | t <= pos_i) v.
//  * quantcpp article, progressive table and "how it works" (4-bit codes with fp16 scale and
//    zero per 32 channels), and the KVarN post, TL;DR (Walsh-Hadamard + Sinkhorn-balanced
//    cache): keys and values are the dequantized uniform codes; scores are taken in the
//    rotated / balanced domain with q' = R(q) .* c, and the output is mapped back with c_V and
//    R_V^-1.
//
// How: one workgroup per (sequence, query head, 64-query tile), one wave per 16 queries; each
// wave walks the cache in 64-token chunks up to its last query's position.
//  * Scores: per 32-channel group g, D_g = Q'_g C_g on v_mfma_f32_16x16x32_f16 with A = the 16
//    query rows of q' (fp16 hi and a 2^11-scaled lo part) and B = the raw codes as exact fp16
//    operands (the decode kernel's operand forms).  The token's fp16 scale and zero fold in
//    afterwards: s = sum_g scale_g D_g + zero_g sum_{j in g} q'_j.
//  * Online softmax per query row in the log2 domain; tokens after a row's position are masked.
//  * PV: A = p * scale_g in fp16 (p in [0, 1]: a relative rounding of 2^-12 per weight, which
//    averages out over the tokens) staged through LDS, B = centred V codes c - 8 (c - 128) as
//    exact fp16 integers; the zero-point term sum p (zero + 8 scale) on the vector ALU in fp32.
//  * Each row's output is divided by its softmax sum and mapped back with c_V and R_V^-1.
// Planes with an FP32 window, or TurboQuant planes, are refused by the host (not supported by
// this kernel).
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_lanes.h"
#include "kvq_mfma_ops.h"
#include "kvq_quant_dev.h"

namespace kvq {
namespace {

using namespace mops;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kWaves = 4;              // waves per workgroup (16 query rows each)
constexpr int kPR = 72;                // halves per staged P row: 64 tokens + 8 pad
constexpr int kStage = 4 * 16 * kPR;   // halves per wave: [group][16 rows][token], and the
                                       // [16][128] float rows before and after the loop
static_assert(kStage * 2 >= 16 * kDim * 4, "row scratch fits the staging area");

__device__ __forceinline__ float wave_max(float v) {
    return xor_reduce<64>(v, [](float x, float y) { return fmaxf(x, y); });
}

template <int KB, int VB>
__global__ __launch_bounds__(kWaves * 64) void prefill_attn_kernel(PrefillParams p) {
    __shared__ __align__(16) _Float16 s_stage[kWaves * kStage];
    __shared__ float s_qsum[kWaves][16][4];
    __shared__ float s_qfac[kWaves][16];

    const int tile = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
    const int G = p.G, kvh = hq / G;
    const int N = p.len[b], P0 = N - p.n_q;
    const int i0 = tile * 64 + wave * 16; // first query row of this wave
    if (i0 >= p.n_q) return;              // the waves share no barrier
    const int rows = min(16, p.n_q - i0);
    const PlaneGeom& KG = p.geom[0];
    const PlaneGeom& VG = p.geom[1];
    const char* slot = p.layer_base + (size_t)b * p.seq_stride + (size_t)kvh * p.head_stride;
    const uint8_t* kcodes = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.codes_off);
    const uint8_t* kmeta = reinterpret_cast<const uint8_t*>(slot + p.plane_off[0] + KG.meta_off);
    const uint8_t* vcodes = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.codes_off);
    const uint8_t* vmeta = reinterpret_cast<const uint8_t*>(slot + p.plane_off[1] + VG.meta_off);
    _Float16* my_stage = s_stage + wave * kStage;
    float* s_row = reinterpret_cast<float*>(my_stage); // [16][128] floats, before and after the loop

    // ---------------- q' of the 16 rows: R_K(q) .* c_K * scale * log2(e), a power of two per
    // row keeping 16 max|q'| in [2^10, 2^11), and the row's four group sums
    const float2 sgn = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 0) * kDim)[l];
    const float2 csk = reinterpret_cast<const float2*>(p.cs + (size_t)(kvh * 2 + 0) * kDim)[l];
    for (int r = 0; r < 16; ++r) {
        float a = 0.0f, c = 0.0f;
        if (r < rows) {
            const size_t off = (((size_t)b * p.n_q + i0 + r) * p.Hq + hq) * kDim;
            if (p.dtype == 0) {
                const float2 v = reinterpret_cast<const float2*>(static_cast<const float*>(p.q) + off)[l];
                a = v.x;
                c = v.y;
            } else {
                const uint32_t v = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + off)[l];
                a = bf2f((uint16_t)(v & 0xffff));
                c = bf2f((uint16_t)(v >> 16));
            }
        }
        if (KG.rotate) {
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
        const float mx = wave_max(fmaxf(fabsf(a), fabsf(c)));
        int e2 = 0;
        if (mx > 0.0f) frexpf(mx, &e2);
        const int e = (mx > 0.0f) ? min(max(7 - e2, -100), 100) : 0;
        const float f = ldexpf(1.0f, e);
        a *= f;
        c *= f;
        s_row[r * kDim + 2 * l] = a;
        s_row[r * kDim + 2 * l + 1] = c;
        const float gs = row_sum16(a + c);
        if (lr == 0) s_qsum[wave][r][lq] = gs;
        if (l == 0) s_qfac[wave][r] = ldexpf(1.0f, -e);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---------------- A operands: row lr = query, k-slice = channels 32g + 8 lq + 0..7
    const float UK = (KB == 4) ? 1048576.0f : 16777216.0f; // unit of a code product
    const float UV = (VB == 4) ? 0.0625f : 1.0f;
    h8 Ahi[4], Alo[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float w = (KB == 4 && (i == 0 || i == 1 || i == 4 || i == 5)) ? 16.0f : 1.0f;
            const float x = s_row[lr * kDim + 32 * g + 8 * lq + i] * w;
            const _Float16 xh = (_Float16)x;
            Ahi[g][i] = xh;
            Alo[g][i] = (_Float16)((x - (float)xh) * kLoScale);
        }
    }
    // score layout: lane holds rows 4 lq + v, token column lr
    float qs_l[4][4], F[4];
    int pos[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int r = 4 * lq + v;
#pragma unroll
        for (int g = 0; g < 4; ++g) qs_l[v][g] = s_qsum[wave][r][g] * (1.0f / UK);
        F[v] = UK * s_qfac[wave][r];
        pos[v] = (r < rows) ? P0 + i0 + r : -1; // -1: no token is visible to an absent row
    }
    __builtin_amdgcn_wave_barrier();

    float m_run[4], l_run[4], z_run[4][4];
    f4 acc[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        m_run[v] = kNegInf;
        l_run[v] = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) z_run[v][g] = 0.0f;
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    const int kend = min(N, P0 + i0 + rows); // keys this wave needs: 0 .. kend - 1
    const int nch = (kend + 63) / 64;
    u4 kc[4][KB / 4], km[4], vc[2][VB / 2], vm[4];
    auto load_k = [&](int ci) {
        const size_t r0 = (size_t)64 * ci + lr; // row of sub-tile 0: token 4 lr + j in row 16 j + lr
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint8_t* c = kcodes + (r0 + 16 * j) * (16 * KB) + (16 * KB / 4) * lq;
#pragma unroll
            for (int u = 0; u < KB / 4; ++u) kc[j][u] = *reinterpret_cast<const u4*>(c + 16 * u);
            km[j] = *reinterpret_cast<const u4*>(kmeta + (r0 + 16 * j) * 16);
        }
    };
    auto load_v = [&](int ci) {
        const size_t t0 = (size_t)64 * ci;
        const uint8_t* c = vcodes + (t0 / 32) * (512 * VB) + (size_t)(32 * VB / 4) * l;
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int u = 0; u < VB / 2; ++u) vc[k][u] = *reinterpret_cast<const u4*>(c + k * 512 * VB + 16 * u);
#pragma unroll
        for (int j = 0; j < 4; ++j) vm[j] = *reinterpret_cast<const u4*>(vmeta + (t0 + 4 * lr + j) * 16);
    };
    if (nch > 0) {
        load_k(0);
        load_v(0);
    }

    for (int ci = 0; ci < nch; ++ci) {
        // ---- scores of sub-tile j: token t = 64 ci + 4 lr + j
        float raw[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 64 * ci + 4 * lr + j;
            h8 B[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (KB == 4)
                    B[g] = as_h8(unpack4(kc[j][0][g]));
                else
                    B[g] = as_h8(unpack8(kc[j][g >> 1][2 * (g & 1)], kc[j][g >> 1][2 * (g & 1) + 1]));
            }
            const float sc[4] = {lo_h(km[j].x), hi_h(km[j].x), lo_h(km[j].y), hi_h(km[j].y)};
            const float zr[4] = {lo_h(km[j].z), hi_h(km[j].z), lo_h(km[j].w), hi_h(km[j].w)};
            float r[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
                const f4 D = mfma16(Ahi[g], B[g], zero4);
                const f4 E = mfma16(Alo[g], B[g], zero4);
#pragma unroll
                for (int v = 0; v < 4; ++v) r[v] = fmaf(sc[g], fmaf(E[v], kLoInv, D[v]), r[v]);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float s = r[v];
#pragma unroll
                for (int g = 0; g < 4; ++g) s = fmaf(zr[g], qs_l[v][g], s);
                raw[j][v] = (t <= pos[v] && t < N) ? s : kNegInf;
            }
        }
        if (ci + 1 < nch) load_k(ci + 1);

        // ---- online softmax per row (state per lane: its 4 tokens; the row max over the
        // row's 16 lanes)
        float pj[4][4], al[4];
        bool grew = false;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float t = fmaxf(fmaxf(raw[0][v], raw[1][v]), fmaxf(raw[2][v], raw[3][v]));
            t = row_max16(t);
            const float mnew = fmaxf(m_run[v], t * F[v]);
            const bool inf = (mnew == kNegInf);
            const float alpha = inf ? 1.0f : exp2f(m_run[v] - mnew);
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pj[j][v] = inf ? 0.0f : exp2f(fmaf(raw[j][v], F[v], -mnew));
                s += pj[j][v];
            }
            l_run[v] = l_run[v] * alpha + s;
            grew |= mnew > m_run[v];
            m_run[v] = mnew;
            al[v] = alpha;
        }
        if (__ballot(grew) != 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
#pragma unroll
                for (int g = 0; g < 4; ++g) z_run[v][g] *= al[v];
#pragma unroll
                for (int n = 0; n < 8; ++n) acc[n][v] *= al[v];
            }
        }

        // ---- zero-point term and the PV A operands: p * scale_g in fp16, [g][row][token 4 lr + j]
        constexpr float mid = (VB == 4) ? 8.0f : 128.0f; // codes enter as c - mid
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float vs[4] = {lo_h(vm[j].x), hi_h(vm[j].x), lo_h(vm[j].y), hi_h(vm[j].y)};
            const float vz[4] = {lo_h(vm[j].z), hi_h(vm[j].z), lo_h(vm[j].w), hi_h(vm[j].w)};
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int g = 0; g < 4; ++g) z_run[v][g] = fmaf(pj[j][v], fmaf(mid, vs[g], vz[g]), z_run[v][g]);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                h4 hv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = (g < 2) ? vm[j].x : vm[j].y;
                    const float sg = (g & 1) ? hi_h(w) : lo_h(w);
                    const float wt = (VB == 4 && j < 2) ? 16.0f : 1.0f;
                    hv[j] = (_Float16)(pj[j][v] * sg * wt);
                }
                const int row = 4 * lq + v;
                *reinterpret_cast<h4*>(my_stage + g * 16 * kPR + row * kPR + 4 * lr) = hv;
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- PV over the chunk's two 32-token blocks
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            h8 Ph[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                Ph[g] = *reinterpret_cast<const h8*>(my_stage + g * 16 * kPR + lr * kPR + 32 * k + 8 * lq);
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                h8 Bv;
                if (VB == 4)
                    Bv = as_h8(centred4(vc[k][n >> 2][n & 3]));
                else
                    Bv = as_h8(centred8(vc[k][n >> 1][2 * (n & 1)], vc[k][n >> 1][2 * (n & 1) + 1]));
                acc[n] = mfma16(Ph[n >> 1], Bv, acc[n]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (ci + 1 < nch) load_v(ci + 1);
    }

    // ---------------- rows: softmax sum and zero-point term over the row's 16 lanes, then
    // out = R_V^-1(c_V .* acc) / l
    float lt[4], zt[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        lt[v] = row_sum16(l_run[v]);
#pragma unroll
        for (int g = 0; g < 4; ++g) zt[v][g] = row_sum16(z_run[v][g]);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float a = acc[n][v] * UV + zt[v][n >> 1];
            s_row[(4 * lq + v) * kDim + 16 * n + lr] = (lt[v] > 0.0f) ? a / lt[v] : 0.0f;
        }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float2 csv = reinterpret_cast<const float2*>(p.cs + (size_t)(kvh * 2 + 1) * kDim)[l];
    const float2 sgv = reinterpret_cast<const float2*>(p.signs + (size_t)(kvh * 2 + 1) * kDim)[l];
    for (int r = 0; r < rows; ++r) {
        float a = s_row[r * kDim + 2 * l], c = s_row[r * kDim + 2 * l + 1];
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
        float2* o = reinterpret_cast<float2*>(p.out + (((size_t)b * p.n_q + i0 + r) * p.Hq + hq) * kDim);
        o[l] = make_float2(a, c);
    }
}

template <int KB, int VB>
hipError_t launch_t(const PrefillParams& p, hipStream_t s) {
    const dim3 grid((p.n_q + 63) / 64, p.Hq, p.batch);
    hipLaunchKernelGGL((prefill_attn_kernel<KB, VB>), grid, dim3(kWaves * 64), 0, s, p);
    return hipGetLastError();
}

} // namespace

bool prefill_attn_supported(const PrefillParams& p) {
    const PlaneGeom& K = p.geom[0];
    const PlaneGeom& V = p.geom[1];
    auto ok = [](const PlaneGeom& g) { return g.scheme == kUniform && (g.bits == 4 || g.bits == 8); };
    return ok(K) && ok(V) && p.window == 0;
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
    const int kb = p.geom[0].bits, vb = p.geom[1].bits;
    if (kb == 4) return vb == 4 ? launch_t<4, 4>(p, s) : launch_t<4, 8>(p, s);
    return vb == 4 ? launch_t<8, 4>(p, s) : launch_t<8, 8>(p, s);
}

} // namespace kvq
