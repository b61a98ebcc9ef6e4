// Quantize-on-append, Sinkhorn calibration and Lloyd-Max codebook kernels for gfx950.
//
// Built with -ffp-contract=off: every binary32 operation below rounds separately, in the order
// written, so packed codes and fp16 scales are bit-identical to any other implementation of the
// same format.  fmaf() is used only where the format fuses (the QJL projection).
//
// Method sources (pages by title and section):
//  - quantcpp article "Beyond RAG...", progressive table + "how it works": 4-bit codes with fp16
//    scale and zero per 32 channels (6.4x), newest 128 tokens kept in FP32.
//  - KVarN-on-Bonsai post, TL;DR: Walsh-Hadamard transform and Sinkhorn variance balancing
//    before 4-bit quantization.
//  - "LLM memory saving ... 2026", TurboQuant row of the method table: random rotation,
//    per-coordinate optimal scalar quantizer, 1-bit QJL of the residual.
#include <algorithm>

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_quant_dev.h"
#include "kvq_quant_bulk.h"

namespace kvq {
namespace {

using qdev::lane_id;
using qdev::f16_rn;
using qdev::f16_val;
using qdev::rotate_wave;
using qdev::c0f;

// One wave per (tensor, sequence, kv head, 8-token octet) of the appended tokens.
__global__ __launch_bounds__(256) void quantize_kernel(QuantParams p) {
    __shared__ float rbuf[4][kDim];
    const int wave = threadIdx.x >> 6;
    qdev::quantize_wave(p, blockIdx.z & 1, blockIdx.z >> 1, blockIdx.y, blockIdx.x * 4 + wave, rbuf[wave]);
}

// The same for one tensor only: bulk prefill of planes that have no lane-dense quantizer (the
// split key).
__global__ __launch_bounds__(256) void quantize_tensor_kernel(QuantParams p, int tensor) {
    __shared__ float rbuf[4][kDim];
    const int wave = threadIdx.x >> 6;
    qdev::quantize_wave(p, tensor, blockIdx.z, blockIdx.y, blockIdx.x * 4 + wave, rbuf[wave]);
}

// Bulk quantizer of a split TurboQuant V plane (BO outlier bits): waves 2u and 2u + 1 of a
// workgroup take the outlier and the rest half (NB = BO or BO - 1 code bits) of the same octets
// (2x + u, then every 2 * gridDim.x-th after it), requesting the next octet's source before
// coding the current one.
template <int BO, int NB>
__device__ __forceinline__ void splitv_loop(const QuantParams& p, const qbulk::WavePlane& w, int hv, const int* pm,
                                            const uint32_t* sgm, float* wl) {
    constexpr int levels = 1 << NB;
    const float* t = p.theta64 + (levels - 4); // levels - 1 ascending thresholds
    auto at = [&](int k) { return k < levels - 1 ? t[k] : 0.0f; };
    const qbulk::TurboTabs4 th{at(0), at(1), at(2), at(3), at(4), at(5), at(6), at(7),
                               at(8), at(9), at(10), at(11), at(12), at(13), at(14)};
    const int g_first = w.start / 8, step = gridDim.x * 2;
    int u = blockIdx.x * 2 + ((threadIdx.x >> 6) >> 1);
    qbulk::SplitIn cur;
    qbulk::load_split(w, g_first + u, pm, cur);
    for (; u < p.groups8; u += step) {
        qbulk::SplitIn nxt;
        qbulk::load_split(w, g_first + u + step, pm, nxt);
        qbulk::split_v_octet<BO, NB>(w, g_first + u, hv, cur, pm, sgm, th, wl);
        cur = nxt;
    }
}

template <int BO>
__global__ __launch_bounds__(256) void quantize_splitv_bulk_kernel(QuantParams p) {
    constexpr int kW = 4, tensor = 1;
    __shared__ __align__(16) float wl[kW][128]; // 8 tokens x 64 positions of code bytes per wave
    const int b = blockIdx.z, head = blockIdx.y, wave = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int hv = wave & 1;
    const qbulk::WavePlane w = qbulk::wave_plane(p, tensor, b, head);
    // the lane's 8 positions 64 hv + 8 (L % 8) + i: their channels and sign bits
    const int pos0 = 64 * hv + 8 * (L & 7);
    int pm[8];
    uint32_t sgm[8];
    const float* sg = p.signs[tensor] + (size_t)(head * 2 + tensor) * kDim + pos0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        pm[i] = p.perm[(size_t)head * kDim + pos0 + i];
        sgm[i] = sg[i] < 0.0f ? 0x80000000u : 0u;
    }
    if (hv) splitv_loop<BO, BO - 1>(p, w, 1, pm, sgm, wl[wave]);
    else splitv_loop<BO, BO>(p, w, 0, pm, sgm, wl[wave]);
}

// Bulk quantizer of one TurboQuant tensor (QJL: TurboQuant-QJL K, else TurboQuant-MSE).  Wave
// w of workgroup x takes octets 4x + w, then every 4 * gridDim.x-th after it, of one (sequence,
// kv head), requesting the next octet's source before quantizing the current one.  QJL
// workgroups first stage S^T (64 KiB) in LDS for all of their octets.
template <bool QJL>
__global__ __launch_bounds__(QJL ? 1024 : 256) void quantize_turbo_bulk_kernel(QuantParams p, int tensor) {
    constexpr int kW = QJL ? 16 : 4; // waves per workgroup: QJL workgroups share one copy of S^T
    __shared__ __align__(16) float wl[kW][qbulk::kTurboWaveLds / 4];
    __shared__ __align__(16) float st[QJL ? kDim * kDim : 4];
    const int b = blockIdx.z, head = blockIdx.y, wave = threadIdx.x >> 6, j = threadIdx.x & 15;
    if constexpr (QJL) {
        const float4* src = reinterpret_cast<const float4*>(p.qjl_st);
        float4* dst = reinterpret_cast<float4*>(st);
        for (int i = threadIdx.x; i < kDim * kDim / 4; i += blockDim.x) dst[i] = src[i];
        __syncthreads();
    }
    const qbulk::WavePlane w = qbulk::wave_plane(p, tensor, b, head);
    uint8_t* qjl_base = reinterpret_cast<uint8_t*>(p.layer_base + (size_t)b * p.seq_stride +
                                                   (size_t)head * p.head_stride + p.plane_off[tensor] +
                                                   p.geom[tensor].qjl_off);
    uint32_t sgm[8], kbit[8];
    const float* sg = p.signs[tensor] + (size_t)(head * 2 + tensor) * kDim + 8 * j;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sgm[i] = sg[i] < 0.0f ? 0x80000000u : 0u;
        const int v = 8 * (j & 3) + i; // value index of channel 8j + i in its 32-channel group
        kbit[i] = 1u << (16 * (v & 1) + (v >> 1));
    }
    const float* th = p.theta;
    const float* mu = p.mu;
    const qbulk::TurboTabs T{th[0], th[1], th[2], th[3], th[4], th[5], th[6],
                             mu[0], mu[1], mu[2], mu[3], mu[4], mu[5], mu[6], mu[7]};
    const bool is_v = tensor == 1;
    const int g_first = w.start / 8, step = gridDim.x * kW;
    int u = blockIdx.x * kW + wave;
    qbulk::OctetIn cur;
    qbulk::load_octet(w, g_first + u, cur);
    for (; u < p.groups8; u += step) {
        qbulk::OctetIn nxt;
        qbulk::load_octet(w, g_first + u + step, nxt);
        qbulk::turbo_octet<QJL>(w, is_v, g_first + u, cur, sgm, T, kbit, wl[wave], st, qjl_base);
        cur = nxt;
    }
}

// Bulk quantizer of uniform planes (BITS-bit codes, ROT: rotated, SINK: Sinkhorn-balanced); the
// launch covers tensors tensor0 .. tensor0 + n_tensors - 1, which share that format.  Wave w of
// workgroup x takes octets 4x + w, then every 4 * gridDim.x-th after it, of one (tensor,
// sequence, kv head), requesting the next octet's source before quantizing the current one.
// Bulk quantizer of a 4-bit TurboQuant-MSE V plane: the same schedule as the MSE kernel above.
__global__ __launch_bounds__(256) void quantize_turbo4v_bulk_kernel(QuantParams p) {
    constexpr int kW = 4, tensor = 1;
    __shared__ __align__(16) float wl[kW][qbulk::kTurboWaveLds / 4];
    const int b = blockIdx.z, head = blockIdx.y, wave = threadIdx.x >> 6, j = threadIdx.x & 15;
    const qbulk::WavePlane w = qbulk::wave_plane(p, tensor, b, head);
    uint32_t sgm[8];
    const float* sg = p.signs[tensor] + (size_t)(head * 2 + tensor) * kDim + 8 * j;
#pragma unroll
    for (int i = 0; i < 8; ++i) sgm[i] = sg[i] < 0.0f ? 0x80000000u : 0u;
    const float* th = p.theta16;
    const qbulk::TurboTabs4 T{th[0], th[1], th[2], th[3], th[4], th[5], th[6], th[7],
                              th[8], th[9], th[10], th[11], th[12], th[13], th[14]};
    const int g_first = w.start / 8, step = gridDim.x * kW;
    int u = blockIdx.x * kW + wave;
    qbulk::OctetIn cur;
    qbulk::load_octet(w, g_first + u, cur);
    for (; u < p.groups8; u += step) {
        qbulk::OctetIn nxt;
        qbulk::load_octet(w, g_first + u + step, nxt);
        qbulk::turbo4_v_octet(w, g_first + u, cur, sgm, T, wl[wave]);
        cur = nxt;
    }
}

template <int BITS, bool ROT, bool SINK, bool SYM>
__global__ __launch_bounds__(256) void quantize_uniform_bulk_kernel(QuantParams p, int tensor0,
                                                                    int n_tensors) {
    __shared__ __align__(16) uint8_t wv[4][8 * kDim];
    const int tensor = tensor0 + (int)blockIdx.z % n_tensors, b = (int)blockIdx.z / n_tensors;
    const int head = blockIdx.y, wave = threadIdx.x >> 6, j = threadIdx.x & 15;
    const qbulk::WavePlane w = qbulk::wave_plane(p, tensor, b, head);
    uint32_t sgm[8];
    float ic[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sgm[i] = 0u;
        ic[i] = 1.0f;
    }
    if (ROT) {
        const float* sg = p.signs[tensor] + (size_t)(head * 2 + tensor) * kDim + 8 * j;
#pragma unroll
        for (int i = 0; i < 8; ++i) sgm[i] = sg[i] < 0.0f ? 0x80000000u : 0u;
    }
    if (SINK) {
        const float* c = p.inv_c[tensor] + (size_t)(head * 2 + tensor) * kDim + 8 * j;
#pragma unroll
        for (int i = 0; i < 8; ++i) ic[i] = c[i];
    }
    const bool is_v = tensor == 1;
    const int g_first = w.start / 8, step = gridDim.x * 4;
    int u = blockIdx.x * 4 + wave;
    qbulk::OctetIn cur;
    qbulk::load_octet(w, g_first + u, cur);
    for (; u < p.groups8; u += step) {
        qbulk::OctetIn nxt;
        qbulk::load_octet(w, g_first + u + step, nxt);
        qbulk::uniform_octet<BITS, ROT, SINK, SYM>(w, is_v, g_first + u, cur, sgm, ic, wv[wave]);
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------------------------
// Sinkhorn calibration (fp64, sequential sums in index order)
// ---------------------------------------------------------------------------------------------

// Work layout: A [2][Hkv][n][128], then the current sweep's column scales sdc [2][Hkv][128],
// then the accumulated column scales C [2][Hkv][128] (all binary64).
__device__ __forceinline__ double* calib_A(const CalibParams& p, int tensor, int head) {
    return p.work + ((size_t)tensor * p.Hkv + head) * (size_t)p.n * kDim;
}
__device__ __forceinline__ double* calib_sdc(const CalibParams& p, int tensor, int head) {
    return p.work + (size_t)2 * p.Hkv * p.n * kDim + ((size_t)tensor * p.Hkv + head) * kDim;
}
__device__ __forceinline__ double* calib_C(const CalibParams& p, int tensor, int head) {
    return calib_sdc(p, tensor, head) + (size_t)2 * p.Hkv * kDim;
}

// A = R(x) (binary32 butterflies, as the quantizer rotates) widened to binary64, or x; C = 1.
// One thread per (token, kv head, tensor).
__global__ __launch_bounds__(64) void calib_init_kernel(CalibParams p) {
    const int t = blockIdx.x * 64 + threadIdx.x, head = blockIdx.y, tensor = blockIdx.z;
    if (!p.do_tensor[tensor]) return;
    if (blockIdx.x == 0)
        for (int j = threadIdx.x; j < kDim; j += 64) calib_C(p, tensor, head)[j] = 1.0;
    if (t >= p.n) return;
    const float* signs = p.signs + (size_t)(head * 2 + tensor) * kDim;
    float y[kDim];
    const size_t off = ((size_t)t * p.Hkv + head) * kDim;
#pragma unroll
    for (int j = 0; j < kDim; ++j) {
        float v = (p.dtype == 0) ? static_cast<const float*>(p.src[tensor])[off + j]
                                 : in16_to_f32(static_cast<const uint16_t*>(p.src[tensor])[off + j], p.dtype);
        if (p.rotate[tensor] && signs[j] < 0.0f) v = -v;
        y[j] = v;
    }
    if (p.rotate[tensor]) {
#pragma unroll
        for (int h = 1; h < kDim; h <<= 1)
#pragma unroll
            for (int i = 0; i < kDim; ++i)
                if (!(i & h)) {
                    const float u = y[i], w = y[i + h];
                    y[i] = u + w;
                    y[i + h] = u - w;
                }
#pragma unroll
        for (int j = 0; j < kDim; ++j) y[j] = y[j] * c0f();
    }
    double* A = calib_A(p, tensor, head) + (size_t)t * kDim;
#pragma unroll
    for (int j = 0; j < kDim; ++j) A[j] = (double)y[j];
}

// Row sweep, one wave per row: (when `divide`) the previous sweep's column scales are applied
// first, A[t][j] / sdc[j]; then mean and variance of the row, each a sum in index order taken by
// lane 0 from LDS, and A[t][j] / sd_row by every lane.
__global__ __launch_bounds__(256) void calib_rows_kernel(CalibParams p, int divide) {
    __shared__ double s_row[4][kDim];
    __shared__ double s_sd[4];
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave, head = blockIdx.y, tensor = blockIdx.z;
    if (!p.do_tensor[tensor] || t >= p.n) return;
    double* A = calib_A(p, tensor, head) + (size_t)t * kDim;
    const double* sdc = calib_sdc(p, tensor, head);
    double2 a = reinterpret_cast<const double2*>(A)[l];
    if (divide) {
        a.x = a.x / sdc[2 * l];
        a.y = a.y / sdc[2 * l + 1];
    }
    s_row[wave][2 * l] = a.x;
    s_row[wave][2 * l + 1] = a.y;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (l == 0) {
        const double* r = s_row[wave];
        double s = 0.0;
#pragma unroll 16
        for (int j = 0; j < kDim; ++j) s = s + r[j];
        const double mean = s / 128.0;
        double v = 0.0;
#pragma unroll 16
        for (int j = 0; j < kDim; ++j) {
            const double dv = r[j] - mean;
            v = v + dv * dv;
        }
        double sd = sqrt(v / 128.0);
        if (sd < 1e-30) sd = 1e-30;
        s_sd[wave] = sd;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const double sd = s_sd[wave];
    reinterpret_cast<double2*>(A)[l] = make_double2(a.x / sd, a.y / sd);
}

// Column sweep: lane l of wave w of (kv head, tensor) takes column 64 w + l; mean and variance
// over the n rows, each a sum in index order; sdc = sd, C *= sd.  `last`: also write c = C and
// 1 / c as binary32.
__global__ __launch_bounds__(128) void calib_cols_kernel(CalibParams p, int last) {
    const int head = blockIdx.x, tensor = blockIdx.y, j = threadIdx.x;
    if (!p.do_tensor[tensor]) return;
    const int n = p.n;
    const double* A = calib_A(p, tensor, head) + j;
    double s = 0.0;
#pragma unroll 16
    for (int t = 0; t < n; ++t) s = s + A[(size_t)t * kDim];
    const double mean = s / (double)n;
    double v = 0.0;
#pragma unroll 16
    for (int t = 0; t < n; ++t) {
        const double dv = A[(size_t)t * kDim] - mean;
        v = v + dv * dv;
    }
    double sd = sqrt(v / (double)n);
    if (sd < 1e-30) sd = 1e-30;
    calib_sdc(p, tensor, head)[j] = sd;
    double* C = calib_C(p, tensor, head);
    const double c = C[j] * sd;
    C[j] = c;
    if (last) {
        const float cf = (float)c;
        p.cs[(size_t)(head * 2 + tensor) * kDim + j] = cf;
        p.inv_c[(size_t)(head * 2 + tensor) * kDim + j] = (float)(1.0 / (double)cf);
    }
}

// ---------------------------------------------------------------------------------------------
// Lloyd-Max quantizer of N(0,1) with `levels` = 8 or 16 levels (positive half line, mirrored),
// scaled by 1/sqrt(128); the half line starts evenly spaced at 2 (k + 1) / (levels / 2)
// ---------------------------------------------------------------------------------------------

__device__ double phi_d(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846); }

__device__ double mass_d(double a, double b, bool b_inf) {
    const double eb = b_inf ? 0.0 : erfc(b / sqrt(2.0));
    return 0.5 * (erfc(a / sqrt(2.0)) - eb);
}

// One lane per centroid k < levels / 2 of the upper half: each iteration, lane k takes its
// neighbours' centroids by shuffle, forms the cell bounds b_k = (m_{k-1} + m_k) / 2 (b_0 = 0) and
// b_{k+1}, and moves m_k to the cell's conditional mean (phi(b_k) - phi(b_{k+1})) / P(b_k < x <
// b_{k+1}); the last cell is open above. Every value is the same binary64 expression, in the same
// order, as in a one-thread loop over k, so the tables do not depend on the lane count.
__global__ __launch_bounds__(64) void codebook_kernel(float* mu, float* theta, int iters, int levels, int dim) {
    const int h = levels / 2, k = threadIdx.x;
    const bool last = (k == h - 1);
    double m = 2.0 * (double)(min(k, h - 1) + 1) / (double)h;
    for (int it = 0; it < iters; ++it) {
        const double ml = __shfl(m, max(k - 1, 0)), mr = __shfl(m, min(k + 1, 63));
        const double b0 = (k == 0) ? 0.0 : (ml + m) * 0.5;
        const double b1 = last ? 0.0 : (m + mr) * 0.5;
        const double pb = last ? 0.0 : phi_d(b1);
        const double nm = (phi_d(b0) - pb) / mass_d(b0, b1, last);
        m = (k < h) ? nm : m;
    }
    const double r = sqrt((double)dim);
    const double ml = __shfl(m, max(k - 1, 0));
    if (k < h) {
        const float f = (float)(m / r);
        mu[h + k] = f;
        mu[h - 1 - k] = -f;
        if (k == 0) {
            theta[h - 1] = 0.0f;
            theta[levels - 1] = 0.0f;
        } else {
            const double t = (ml + m) * 0.5;
            const float ft = (float)(t / r);
            theta[h - 1 + k] = ft;
            theta[h - 1 - k] = -ft;
        }
    }
}

// Outlier channels of one kv head's calibration tokens (TurboQuant split): thread d sums
// x[t][d]^2 in binary64 in token order (each square is exact), then ranks its channel against
// the others (larger energy first, ties to the smaller index); the top 64 go to positions
// 0..63 in ascending channel order, the rest to 64..127.
__global__ __launch_bounds__(128) void select_outliers_kernel(OutlierParams p) {
    __shared__ double s_e[kDim];
    __shared__ int s_out[kDim];
    const int head = blockIdx.x, d = threadIdx.x;
    double acc = 0.0;
    for (int t = 0; t < p.n; ++t) {
        const size_t i = ((size_t)t * p.Hkv + head) * kDim + d;
        const double v = p.dtype == 0 ? (double)static_cast<const float*>(p.src)[i]
                                      : (double)in16_to_f32(static_cast<const uint16_t*>(p.src)[i], p.dtype);
        acc = acc + v * v;
    }
    s_e[d] = acc;
    __syncthreads();
    int rank = 0;
    for (int i = 0; i < kDim; ++i) {
        const double e = s_e[i];
        rank += (e > acc || (e == acc && i < d)) ? 1 : 0;
    }
    const int out = rank < kDim / 2 ? 1 : 0;
    s_out[d] = out;
    __syncthreads();
    int pos = out ? 0 : kDim / 2;
    for (int i = 0; i < d; ++i) pos += (s_out[i] == out) ? 1 : 0;
    p.perm[(size_t)head * kDim + pos] = d;
}

__global__ void fill_kernel(float* p, size_t n, float v) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void transpose128_kernel(const float* in, float* out) {
    const int i = blockIdx.x, j = threadIdx.x;
    out[j * kDim + i] = in[i * kDim + j];
}

} // namespace

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
    dim3 grid((p.groups8 + 3) / 4, p.Hkv, 2 * p.batch);
    hipLaunchKernelGGL(quantize_kernel, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

namespace {

template <bool QJL>
hipError_t launch_turbo_bulk(const QuantParams& p, hipStream_t s, int tensor) {
    // QJL K planes: about two workgroups per compute unit (LDS holds two), each staging S^T once
    constexpr int kW = QJL ? 16 : 4;
    const int planes = p.Hkv * p.batch;
    const int target = QJL ? kQuantBulkQjlBlocks : kQuantBulkBlocks;
    const int gx = std::max(1, std::min((p.groups8 + kW - 1) / kW, (target + planes - 1) / planes));
    hipLaunchKernelGGL(quantize_turbo_bulk_kernel<QJL>, dim3(gx, p.Hkv, p.batch), dim3(kW * 64), 0, s, p, tensor);
    return hipGetLastError();
}

template <int BITS, bool ROT, bool SINK, bool SYM = false>
hipError_t launch_uniform_bulk(const QuantParams& p, hipStream_t s, int tensor0, int n_tensors) {
    const int planes = p.Hkv * p.batch * n_tensors;
    const int gx = std::max(1, std::min((p.groups8 + 3) / 4, (kQuantBulkBlocks + planes - 1) / planes));
    hipLaunchKernelGGL((quantize_uniform_bulk_kernel<BITS, ROT, SINK, SYM>), dim3(gx, p.Hkv, n_tensors * p.batch),
                       dim3(256), 0, s, p, tensor0, n_tensors);
    return hipGetLastError();
}

hipError_t launch_uniform_bulk_for(const PlaneGeom& G, const QuantParams& p, hipStream_t s,
                                   int tensor0, int n_tensors) {
    if (G.bits == 3) {
        switch ((G.rotate ? 2 : 0) | (G.sinkhorn ? 1 : 0)) {
        case 0: return launch_uniform_bulk<3, false, false>(p, s, tensor0, n_tensors);
        case 1: return launch_uniform_bulk<3, false, true>(p, s, tensor0, n_tensors);
        case 2: return launch_uniform_bulk<3, true, false>(p, s, tensor0, n_tensors);
        default: return launch_uniform_bulk<3, true, true>(p, s, tensor0, n_tensors);
        }
    }
    const int key = (G.symmetric ? 8 : 0) | (G.bits == 8 ? 4 : 0) | (G.rotate ? 2 : 0) | (G.sinkhorn ? 1 : 0);
    switch (key) {
    case 12: return launch_uniform_bulk<8, false, false, true>(p, s, tensor0, n_tensors);
    case 13: return launch_uniform_bulk<8, false, true, true>(p, s, tensor0, n_tensors);
    case 14: return launch_uniform_bulk<8, true, false, true>(p, s, tensor0, n_tensors);
    case 15: return launch_uniform_bulk<8, true, true, true>(p, s, tensor0, n_tensors);
    case 0: return launch_uniform_bulk<4, false, false>(p, s, tensor0, n_tensors);
    case 1: return launch_uniform_bulk<4, false, true>(p, s, tensor0, n_tensors);
    case 2: return launch_uniform_bulk<4, true, false>(p, s, tensor0, n_tensors);
    case 3: return launch_uniform_bulk<4, true, true>(p, s, tensor0, n_tensors);
    case 4: return launch_uniform_bulk<8, false, false>(p, s, tensor0, n_tensors);
    case 5: return launch_uniform_bulk<8, false, true>(p, s, tensor0, n_tensors);
    case 6: return launch_uniform_bulk<8, true, false>(p, s, tensor0, n_tensors);
    default: return launch_uniform_bulk<8, true, true>(p, s, tensor0, n_tensors);
    }
}

hipError_t launch_turbo4v_bulk(const QuantParams& p, hipStream_t s) {
    constexpr int kW = 4;
    const int planes = p.Hkv * p.batch;
    const int gx = std::max(1, std::min((p.groups8 + kW - 1) / kW, (kQuantBulkBlocks + planes - 1) / planes));
    hipLaunchKernelGGL(quantize_turbo4v_bulk_kernel, dim3(gx, p.Hkv, p.batch), dim3(kW * 64), 0, s, p);
    return hipGetLastError();
}

// One launch for tensors tensor0 .. tensor0 + n_tensors - 1 (TurboQuant: one tensor).
hipError_t launch_bulk_scheme(int scheme, const QuantParams& p, hipStream_t s, int tensor0,
                              int n_tensors) {
    switch (scheme) {
    case kUniform: return launch_uniform_bulk_for(p.geom[tensor0], p, s, tensor0, n_tensors);
    case kTurboQjl: return launch_turbo_bulk<true>(p, s, tensor0);
    case kTurboSplit: {
        if (tensor0 == 0) { // split key: the per-token quantizer, one wave per octet
            hipLaunchKernelGGL(quantize_tensor_kernel, dim3((p.groups8 + 3) / 4, p.Hkv, p.batch), dim3(256), 0, s, p,
                               0);
            return hipGetLastError();
        }
        const int planes = p.Hkv * p.batch;
        const int gx = std::max(1, std::min((p.groups8 + 1) / 2, (kQuantBulkBlocks + planes - 1) / planes));
        if (p.geom[tensor0].bits == 4)
            hipLaunchKernelGGL(quantize_splitv_bulk_kernel<4>, dim3(gx, p.Hkv, p.batch), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(quantize_splitv_bulk_kernel<3>, dim3(gx, p.Hkv, p.batch), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    default:
        if (p.geom[tensor0].bits == 4) return launch_turbo4v_bulk(p, s); // V only
        return launch_turbo_bulk<false>(p, s, tensor0);
    }
}

} // namespace

hipError_t launch_quantize_bulk(const QuantParams& p, hipStream_t s) {
    const PlaneGeom &g0 = p.geom[0], &g1 = p.geom[1];
    const int s0 = g0.scheme, s1 = g1.scheme;
    const bool same = s0 == kUniform && s1 == kUniform && g0.bits == g1.bits &&
                      g0.rotate == g1.rotate && g0.sinkhorn == g1.sinkhorn && g0.symmetric == g1.symmetric;
    if (same) return launch_bulk_scheme(s0, p, s, 0, 2);
    const hipError_t e = launch_bulk_scheme(s0, p, s, 0, 1);
    if (e != hipSuccess) return e;
    return launch_bulk_scheme(s1, p, s, 1, 1);
}

hipError_t launch_calibrate(const CalibParams& p, hipStream_t s) {
    hipLaunchKernelGGL(calib_init_kernel, dim3((p.n + 63) / 64, p.Hkv, 2), dim3(64), 0, s, p);
    hipError_t e = hipGetLastError();
    for (int it = 0; it < p.iters && e == hipSuccess; ++it) {
        hipLaunchKernelGGL(calib_rows_kernel, dim3((p.n + 3) / 4, p.Hkv, 2), dim3(256), 0, s, p, it > 0 ? 1 : 0);
        e = hipGetLastError();
        if (e != hipSuccess) break;
        hipLaunchKernelGGL(calib_cols_kernel, dim3(p.Hkv, 2), dim3(kDim), 0, s, p, it == p.iters - 1 ? 1 : 0);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_codebook(float* mu, float* theta, int iters, int levels, int dim, hipStream_t s) {
    hipLaunchKernelGGL(codebook_kernel, dim3(1), dim3(64), 0, s, mu, theta, iters, levels, dim);
    return hipGetLastError();
}

hipError_t launch_select_outliers(const OutlierParams& p, hipStream_t s) {
    hipLaunchKernelGGL(select_outliers_kernel, dim3(p.Hkv), dim3(kDim), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fill(float* p, size_t n, float v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_transpose128(const float* in, float* out, hipStream_t s) {
    hipLaunchKernelGGL(transpose128_kernel, dim3(kDim), dim3(kDim), 0, s, in, out);
    return hipGetLastError();
}

} // namespace kvq
