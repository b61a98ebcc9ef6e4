// Internal declarations shared by the host code and the HIP kernels of libkvq.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace kvq {

constexpr int kDim = 128;
constexpr int kGroup = 32;
constexpr int kMaxBatch = 64;
constexpr int kMaxGroupHeads = 8;   // query heads per kv head
constexpr int kMaxSplits = 256;     // splits per (sequence, kv head), window splits included
constexpr int kPartialFloats = 132; // m, l, pad, pad, acc[128] per (sequence, q head, split)
constexpr int kWindowMax = 128;
constexpr int kWinSplitsMatrix = 1; // FP32-window workgroups per (sequence, kv head), matrix path

// kTurboSplit: the outlier-channel split (the public KVQ_TURBO_SPLIT).  V: TurboQuant-MSE codes,
// bits = the outlier subset's code bits (3 or 4), the other 64 channels take one bit fewer.
// K: bits = b (3 or 4), the TurboQuant key coder at b - 0.5 bits per channel -- MSE codes of
// b - 1 bits on the outliers and b - 2 on the rest, plus the 1-bit QJL sketch of the residual.
enum Scheme { kUniform = 0, kTurboQjl = 1, kTurboMse = 2, kTurboSplit = 4 };
// Split-coder codebooks for N(0, 1/64) with L = 4, 8, 16 levels start at float L - 4 of the
// 30-float tables, the 2-level one at float 28 (centroids; thresholds likewise, L - 1 of L used)
constexpr int kSplitTable = 30;
__host__ __device__ constexpr int split_table_off(int levels) { return levels == 2 ? 28 : levels - 4; }
// Bytes of a split key row's code planes (b - 1 planes on each outlier group, b - 2 on each
// other group, 4 bytes per plane word) and the word at which position group g's planes start.
__host__ __device__ constexpr int split_k_row_bytes(int b) { return 4 * (4 * b - 6); }
__host__ __device__ constexpr int split_k_group_word(int g, int b) {
    return g < 2 ? g * (b - 1) : 2 * (b - 1) + (g - 2) * (b - 2);
}

// Geometry of one tensor's plane inside a (layer, seq, head) slot.
struct PlaneGeom {
    int scheme, bits, rotate, sinkhorn;
    int symmetric; // uniform 8-bit plane written by the symmetric (q8_0-style) quantizer
    size_t codes_off, meta_off, qjl_off, ring_off; // byte offsets from the slot base
    size_t codes_bytes, meta_bytes, qjl_bytes, ring_bytes;
};

// Parameters of the quantize-on-append kernel (K and V in one launch).
struct QuantParams {
    const void* src[2];       // [batch][T][Hkv][128] of dtype
    char* layer_base;         // slot of (layer, seq 0, head 0)
    size_t seq_stride;        // bytes between sequences
    size_t head_stride;       // bytes between kv heads (= slot bytes)
    size_t plane_off[2];      // offset of the K / V plane inside a slot
    PlaneGeom geom[2];
    const float* signs[2];    // layer base of [Hkv][2][128]; index (head*2 + tensor)*128
    const float* inv_c[2];    // same indexing
    const float* qjl_st;      // [128 j][128 i] = S[i][j]
    const float* mu;          // [8]
    const float* theta;       // [8], 7 used
    const float* mu16;        // [16]: 4-bit TurboQuant-MSE V codebook
    const float* theta16;     // [16], 15 used
    const int* perm;          // layer base [Hkv][128]: channel at each position (split V)
    const int* perm_k;        // layer base [Hkv][128]: the same for a split K
    const float* mu64;        // [kSplitTable] split codebooks
    const float* theta64;     // [kSplitTable]
    int dtype, T, batch, Hkv, window;
    int groups8;              // 8-token groups per (sequence) unit range (max over sequences)
    int start[kMaxBatch];     // length before this append, per sequence
};

// Parameters of the decode kernels.
struct DecodeParams {
    const void* q;            // [batch][Hq][128] of dtype
    float* out;               // [batch][Hq][128]
    char* layer_base;
    size_t seq_stride, head_stride;
    size_t plane_off[2];
    PlaneGeom geom[2];
    const float* signs;       // layer base [Hkv][2][128]
    const float* cs;          // layer base [Hkv][2][128] Sinkhorn c
    const float* qjl_st;      // [128 j][128 i]
    const float* mu;
    const float* mu16;        // [16]: 4-bit TurboQuant-MSE V codebook
    const int* perm;          // layer base [Hkv][128] (split V)
    const int* perm_k;        // layer base [Hkv][128] (split K)
    const float* mu64;        // [kSplitTable] split codebooks
    float* partials;          // [batch][Hq][n_splits_total][kPartialFloats]
    int dtype, batch, Hq, Hkv, G, window;
    float qscale;             // softmax scale * log2(e)
    int split_tokens, n_splits, n_win_splits, n_splits_total; // window splits come last
    int len[kMaxBatch];
    // Fused append (kvq_append_attn_decode, matrix path): when set, the workgroup whose split
    // holds token len[b] - 1 of (b, kv head) first appends that token with `append` (T = 1).
    int fuse;
    QuantParams append;
};

// Parameters of the prefill-chunk attention kernel: the n_q newest tokens of each sequence are
// the queries, each attending to the cache up to its own position.
constexpr int kPrefillRowsPerBlock = 128; // (query, head) rows per prefill-attention workgroup

struct PrefillParams {
    const void* q;            // [batch][n_q][Hq][128] of dtype
    float* out;               // [batch][n_q][Hq][128]
    float* partials;          // [batch][n_q][Hq][n_splits][kPartialFloats] when n_splits > 1
    float* wring;             // [batch][Hkv][2][kWindowMax][128]: the window mapped into the code
                              // domain (window_in_code_domain), else null
    char* layer_base;
    size_t seq_stride, head_stride;
    size_t plane_off[2];
    PlaneGeom geom[2];
    const float* signs;       // layer base [Hkv][2][128]
    const float* cs;          // layer base [Hkv][2][128] Sinkhorn c
    const float* inv_c;       // layer base [Hkv][2][128] 1 / c (window originals into the code domain)
    const float* qjl_st;      // [128 j][128 i] = S[i][j] (TurboQuant-QJL keys)
    const float* mu;          // [8]: 3-bit TurboQuant codebook (QJL K, MSE V)
    const float* mu16;        // [16]: 4-bit TurboQuant-MSE V codebook
    const int* perm;          // layer base [Hkv][128] (split V)
    const int* perm_k;        // layer base [Hkv][128] (split K)
    const float* mu64;        // [kSplitTable] split codebooks
    int dtype, batch, n_q, Hq, Hkv, G, window;
    int n_splits;             // key splits per row (1: the attention kernel writes out itself)
    float qscale;             // softmax scale * log2(e)
    int len[kMaxBatch];
};

// An FP32 window beside rotated or balanced codes (TurboQuant planes are rotated): prefill
// attention reads the window's originals from a copy mapped into the code domain.
inline bool window_in_code_domain(const PlaneGeom& K, const PlaneGeom& V, int window) {
    return window > 0 && (K.rotate || K.sinkhorn || V.rotate || V.sinkhorn || V.scheme == kTurboSplit);
}
inline size_t prefill_window_bytes(int batch, int Hkv) {
    return (size_t)batch * Hkv * 2 * kWindowMax * kDim * sizeof(float);
}

struct CalibParams {
    const void* src[2];       // [n][Hkv][128] of dtype
    double* work;             // [2][Hkv][n][128], then [2][Hkv][128] twice (column scales)
    const float* signs;       // layer base [Hkv][2][128]
    float* cs;                // layer base
    float* inv_c;             // layer base
    int do_tensor[2], rotate[2];
    int dtype, n, Hkv, iters;
};

// Outlier selection of a split V plane: per kv head, the 64 channels of largest energy over the
// n calibration tokens ([n][Hkv][128] of dtype), written as perm [Hkv][128].
struct OutlierParams {
    const void* src;
    int* perm;                // layer base
    int dtype, n, Hkv;
};

// Launchers (defined in the .hip files); return the launch's hipError_t.
hipError_t launch_quantize(const QuantParams& p, hipStream_t s);
// Lane-dense quantizer for many tokens per call (same bytes as launch_quantize).
hipError_t launch_quantize_bulk(const QuantParams& p, hipStream_t s);
// Workgroups a bulk-quantizer launch aims for (its waves loop over octets beyond that), and the
// same for TurboQuant-QJL K planes (one 16-wave workgroup per CU, holding S^T in 64 KiB of LDS).
constexpr int kQuantBulkBlocks = 4096;
constexpr int kQuantBulkQjlBlocks = 256;
// Smallest append the bulk quantizer takes.
constexpr int kQuantBulkMinTokens = 16;
hipError_t launch_calibrate(const CalibParams& p, hipStream_t s);
hipError_t launch_select_outliers(const OutlierParams& p, hipStream_t s);
// Lloyd-Max codebook with `levels` levels for coordinates of unit vectors in `dim` dimensions.
hipError_t launch_codebook(float* mu, float* theta, int iters, int levels, int dim, hipStream_t s);
hipError_t launch_transpose128(const float* in, float* out, hipStream_t s);
hipError_t launch_fill(float* p, size_t n, float v, hipStream_t s);
// The split-K launchers take optional events bound to the kernel's dispatch (measurement).
hipError_t launch_decode_vec(const DecodeParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t s);
bool mfma_path_supported(const DecodeParams& p);
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// Static scratch of kvq_attn_decode_static: its size, the one-time per-device address lookup
// (hipGetSymbolAddress, with that device current) and the address it found (null before).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch_setup(int device);
float* static_scratch(int device);
bool prefill_attn_supported(const PrefillParams& p);
hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s);

} // namespace kvq
