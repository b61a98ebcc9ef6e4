// Cross-lane exchange within a 64-lane wavefront on gfx950: lane l receives the value of lane
// l ^ M.  Same result as __shfl_xor(v, M), but without the LDS address round trip for M = 1, 2, 8
// (DPP quad_perm [1,0,3,2] / [2,3,0,1], row_ror:8 over rows of 16 lanes) and M = 32
// (v_permlane32_swap), and as a single ds_swizzle (xor mask inside 32 lanes) for M = 4, 16.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace kvq {

// A 16-bit input element as fp32, exactly: bf16 (dtype 1) by widening its bits, fp16 (dtype 2) by
// conversion.
__device__ __forceinline__ float in16_to_f32(uint32_t b16, int dtype) {
    return dtype == 2 ? (float)__builtin_bit_cast(_Float16, (uint16_t)b16) : __uint_as_float(b16 << 16);
}

template <int M>
__device__ __forceinline__ int xor_lane_i(int x) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "xor distance");
    if constexpr (M == 1) {
        return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);
    } else if constexpr (M == 2) {
        return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);
    } else if constexpr (M == 8) {
        return __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false);
    } else if constexpr (M == 4 || M == 16) {
        return __builtin_amdgcn_ds_swizzle(x, 0x1F | (M << 10));
    } else {
        const auto pr = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (__lane_id() < 32) ? (int)pr[1] : (int)pr[0];
    }
}

template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    return __int_as_float(xor_lane_i<M>(__float_as_int(v)));
}

template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    return (uint32_t)xor_lane_i<M>((int)v);
}

// Butterfly over the xor distances 1, 2, ..., W/2 (ascending): v = op(v, partner) each step.
template <int W, typename T, typename Op>
__device__ __forceinline__ T xor_reduce(T v, Op op) {
    if constexpr (W > 1) v = op(v, xor_lane<1>(v));
    if constexpr (W > 2) v = op(v, xor_lane<2>(v));
    if constexpr (W > 4) v = op(v, xor_lane<4>(v));
    if constexpr (W > 8) v = op(v, xor_lane<8>(v));
    if constexpr (W > 16) v = op(v, xor_lane<16>(v));
    if constexpr (W > 32) v = op(v, xor_lane<32>(v));
    return v;
}

// The value plane's output map on one head's accumulator held as channel pairs (lane l: code-
// domain positions 2l, 2l + 1), so that split partials leave in the plain channel domain:
//  - outlier split (split): each 64-position half's inverse rotation (1/8) d .* H64 y (the
//    butterflies of spans 1 .. 32, then the signs by position); the caller stores position p at
//    channel perm[p];
//  - otherwise y .* c (Sinkhorn, when sink) and, for a rotated plane (rot), d .* (c0 H y) with
//    c0 = fp32(2^-3.5).
// cs and sg hold the lane's two entries of c_V and of the plane's signs.
__device__ __forceinline__ void value_out_map(float& a, float& b, bool split, bool sink, bool rot, float2 cs,
                                              float2 sg) {
    const int l = threadIdx.x & 63;
    auto step = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float pa = xor_lane<h>(a), pb = xor_lane<h>(b);
        const bool lower = (l & h) == 0;
        a = lower ? (a + pa) : (pa - a);
        b = lower ? (b + pb) : (pb - b);
    };
    if (split || rot) {
        if (!split && sink) {
            a *= cs.x;
            b *= cs.y;
        }
        const float s = a + b, d = a - b;
        a = s;
        b = d;
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 4>{});
        step(std::integral_constant<int, 8>{});
        step(std::integral_constant<int, 16>{});
        if (!split) step(std::integral_constant<int, 32>{});
        const float f = split ? 0.125f : __uint_as_float(0x3DB504F3u);
        a *= f;
        b *= f;
        if (sg.x < 0.0f) a = -a;
        if (sg.y < 0.0f) b = -b;
    } else if (sink) {
        a *= cs.x;
        b *= cs.y;
    }
}

} // namespace kvq
