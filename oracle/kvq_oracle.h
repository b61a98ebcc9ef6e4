/*
 * kvq_oracle.h -- plain C CPU oracle for the compressed-KV decode-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py may load this library.  It shares no code, header, table or generator with the HIP
 * library under quantized_decode_attention_kvq_amd/.
 *
 * What it follows (pages, by title and section):
 *  - quantcpp article ("Beyond RAG: load whole documents on your laptop"), the progressive table
 *    and its "how it works" paragraph: 4-bit KV with the most recent 128 tokens kept in FP32,
 *    6.4x compression (4-bit codes + fp16 scale + fp16 zero per 32 values).
 *  - KVarN-on-Bonsai post, TL;DR paragraph: Walsh-Hadamard transform plus Sinkhorn variance
 *    balancing before 4-bit quantization.
 *  - "LLM memory saving: weights vs KV-cache quantization 2026", method comparison table
 *    (TurboQuant row "core idea"): random rotation, per-coordinate optimal scalar quantizer,
 *    1-bit QJL on the residual for an unbiased inner product.
 *  - the same page, method comparison table (the row of re-checked figures: 2.5 and 3.5 bits) and
 *    its verification notes (non-integer bit widths come from splitting off outlier channels;
 *    the printed example is garbled): the outlier-channel split of the value coder, and of the
 *    key coder's MSE stage in front of its 1-bit QJL sketch (keys at 2.5 / 3.5 bits).
 * Every step the pages leave open is fixed by a stated reading (see the .c file's comments).
 *
 * Arithmetic conventions: binary32 round-to-nearest-even with no FMA contraction (the library is
 * built with -ffp-contract=off; fmaf is called only where the format says "fused"), denormals
 * preserved, binary16 converted by integer manipulation, attention in binary64.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_D 128
#define ORC_GROUP 32
#define ORC_NGROUPS 4

enum { ORC_UNIFORM = 0, ORC_TURBO_QJL = 1, ORC_TURBO_MSE = 2, ORC_Q8_0 = 3, ORC_TURBO_SPLIT = 4 };
enum { ORC_TENSOR_K = 0, ORC_TENSOR_V = 1 };

/* One (layer, sequence, kv head, tensor) plane description. */
typedef struct {
    int scheme;    /* ORC_UNIFORM / ORC_TURBO_QJL / ORC_TURBO_MSE / ORC_Q8_0 / ORC_TURBO_SPLIT */
    int bits;      /* uniform: 3, 4 or 8; turbo: 3 (MSE V also 4); split: outlier bits 3 or 4 */
    int rotate;    /* random-sign WHT before coding (always on for turbo) */
    int sinkhorn;  /* fold 1/c before uniform coding */
    int window;    /* FP32 window W: 0 (flat) or 128 (progressive) */
    int tensor;    /* ORC_TENSOR_K or ORC_TENSOR_V: selects the code layout */
    int capacity;  /* tokens the plane can hold */
} orc_plane_cfg;

/* Tables for one (layer, kv head, tensor) plus the per-cache turbo tables. */
typedef struct {
    const float* signs;  /* [128] +-1, used when rotate */
    const float* c;      /* [128] Sinkhorn channel scale (NULL = all ones) */
    const float* inv_c;  /* [128] fp32(1/c) (NULL = all ones) */
    const float* S;      /* [128*128] QJL projection, row-major S[i][j] */
    const float* mu;     /* [8] Lloyd-Max centroids for N(0,1/128), fp32 */
    const float* theta;  /* [7] decision thresholds, fp32 */
    /* outlier split (ORC_TURBO_SPLIT): mu / theta above are the outlier subset's codebook, these
     * the other subset's (one bit fewer), both for N(0, 1/64); perm[j] = channel at position j */
    const float* mu2;
    const float* theta2;
    const int* perm;
} orc_tables;

/* ---- binary16 ---- */
uint16_t orc_f32_to_f16_rn(float x);
uint16_t orc_f32_to_f16_rd(float x);
float orc_f16_to_f32(uint16_t h);

/* ---- rotation R(x) = c0 * H (d .* x) ---- */
void orc_rotate_f32(const float* x, const float* signs, float* y);
void orc_rotate_f64(const double* x, const float* signs, double* y);
void orc_unrotate_f64(const double* y, const float* signs, double* x);

/* ---- Sinkhorn variance balancing (calibration) ---- */
void orc_sinkhorn(const float* X, int n, const float* signs_or_null, int iters, float* c,
                  float* inv_c, double* A_out /* [n*128] or NULL */, double* C_out /* [128] or NULL */);

/* ---- uniform asymmetric group quantizer ---- */
void orc_quant_group(const float* y, int bits, uint8_t* codes, uint16_t* s16, uint16_t* z16);

/* ---- symmetric 8-bit group quantizer (reading of "q8_0", named as a cache type by the KVarN
 * post's comparison and as "K = Q8" by the application rules of the 2026 survey page; neither
 * page defines it): d = fp16 round-to-nearest of max|y| / 127, q = rint(y * fp32(1/d)) clamped
 * to [-127, 127] (d = 0: q = 0).  Stored in the 8-bit uniform layout as code q + 128 with scale
 * field d and zero field fp16(-128 d), so that zero + scale * code = d q. ---- */
void orc_quant_group_sym8(const float* y, uint8_t* codes, uint16_t* d16, uint16_t* z16);

/* ---- Lloyd-Max codebook ---- */
void orc_lloyd_max(int iters, double* mu_star, float* mu, float* theta, double* last_change);
/* The same for `levels` = 8 or 16 (4-bit codes): mu[levels], theta[levels - 1]. */
void orc_lloyd_max_levels(int levels, int iters, double* mu_star, float* mu, float* theta,
                          double* last_change);

/* The same for coordinates of a unit vector in `dim` dimensions: centroids mu* / sqrt(dim). */
void orc_lloyd_max_dim(int levels, int dim, int iters, double* mu_star, float* mu, float* theta,
                       double* last_change);

/* ---- TurboQuant token code ---- */
void orc_turbo_encode(const float* x, const orc_tables* tb, int with_qjl, float* rho_out,
                      uint8_t* codes, uint16_t* n16, uint16_t* g16, uint8_t* bits,
                      float* resid_out);
/* The same with b-bit codes (b = 3: theta[7]; b = 4: theta[15] of the 16-level codebook). */
void orc_turbo_encode_bits(const float* x, const orc_tables* tb, int code_bits, int with_qjl,
                           float* rho_out, uint8_t* codes, uint16_t* n16o, uint16_t* g16o,
                           uint8_t* bits, float* resid_out);
float orc_tree_sum_sq(const float* v);

/* ---- outlier-channel split (fractional bit widths) ---- */
/* 64-point random-sign rotation (1/8) H64 (d .* x), and its inverse in binary64. */
void orc_rotate64_f32(const float* x, const float* signs, float* y);
void orc_unrotate64_f64(const double* y, const float* signs, double* x);
float orc_tree_sum_sq64(const float* v);
/* perm[128]: the 64 outlier channels of the calibration tokens X [n][128] ascending, then the
 * other 64 ascending. */
void orc_select_outliers(const float* X, int n, int* perm);
/* Token code of the split: codes[j] for position j (channel perm[j]), n16[2] = subset norms. */
void orc_split_encode(const float* x, const orc_tables* tb, int bits_o, uint8_t* codes, uint16_t* n16);
/* Split key at b = 3 or 4: the split codes with b - 1 / b - 2 bits (tb->mu/theta: outlier
 * codebook, mu2/theta2: the rest), n16[2], then gamma and the 128 QJL bits of the residual. */
void orc_split_qjl_encode(const float* x, const orc_tables* tb, int b, uint8_t* codes, uint16_t* n16,
                          uint16_t* g16, uint8_t* bits);
/* y[128] = the split domain of q (binary64): position 64h + j = R64(q[perm[64h + .]])_j. */
void orc_split_rotate_f64(const double* q, const orc_tables* tb, double* y);

/* ---- planes ---- */
size_t orc_codes_bytes(const orc_plane_cfg* pc);
size_t orc_meta_bytes(const orc_plane_cfg* pc);
size_t orc_qjl_bytes(const orc_plane_cfg* pc);
size_t orc_ring_floats(const orc_plane_cfg* pc);

/* Append tokens t0..t0+n-1 (X: [n][128] fp32 originals) to one plane, one token at a time. */
void orc_plane_append(const orc_plane_cfg* pc, const orc_tables* tb, const float* X, int t0, int n,
                      uint8_t* codes, uint8_t* meta, uint8_t* qjl, float* ring);

/* Read back token t's unpacked code fields. */
void orc_plane_read(const orc_plane_cfg* pc, const uint8_t* codes, const uint8_t* meta,
                    const uint8_t* qjl, int t, uint8_t* code128, uint16_t* meta8, uint8_t* bits128);

/* Dequantized token in the ORIGINAL domain (uniform / turbo-MSE; fp64). */
void orc_dequant_token(const orc_plane_cfg* pc, const orc_tables* tb, const uint8_t* codes,
                       const uint8_t* meta, int t, double* out);

/* Turbo-QJL score estimate of <q, k_t> (fp64, unscaled). */
double orc_turbo_score(const orc_tables* tb, const uint8_t* codes, const uint8_t* meta,
                       const uint8_t* qjl, int t, const double* rho_q, const double* s_rho_q);
/* Split-key score estimate (rho_q = split domain of q, s_rho_q = S rho_q). */
double orc_split_score(const orc_plane_cfg* pc, const orc_tables* tb, const uint8_t* codes,
                       const uint8_t* meta, const uint8_t* qjl, int t, const double* rho_q,
                       const double* s_rho_q);

/* Attention of one kv head's G query heads over tokens 0 .. n_vis - 1 of a cache of n tokens
 * (window tokens chosen by n), fp64. */
void orc_attention_prefix(const orc_plane_cfg* kc, const orc_plane_cfg* vc,
                          const orc_tables* ktb, const orc_tables* vtb, const uint8_t* kcodes,
                          const uint8_t* kmeta, const uint8_t* kqjl, const float* kring,
                          const uint8_t* vcodes, const uint8_t* vmeta, const float* vring, int n,
                          int n_vis, int G, const float* q, double scale, double* out);

/* Decode attention for one kv head and its G query heads, fp64. */
void orc_attention(const orc_plane_cfg* kc, const orc_plane_cfg* vc, const orc_tables* ktb,
                   const orc_tables* vtb, const uint8_t* kcodes, const uint8_t* kmeta,
                   const uint8_t* kqjl, const float* kring, const uint8_t* vcodes,
                   const uint8_t* vmeta, const float* vring, int n, int G, const float* q,
                   double scale, double* out);

/* Seeded random tables (the pages draw a random-sign rotation and a Gaussian QJL projection but
 * name no generator; this is the stated reading).  Parity unpinned in part: no published
 * SplitMix64 output is at hand to pin the exact bit stream; the counter structure, the
 * Box-Muller closed forms and the distributions of the draws are pinned.  Counter-based SplitMix64: a stream key chains
 * the SplitMix64 output function over (seed, tag, layer, head, tensor); draw i of a stream is
 * the (i + 1)-th output of a SplitMix64 generator started at the key. */
uint64_t orc_stream_key(uint64_t seed, int tag, int layer, int head, int tensor);
uint64_t orc_stream_draw(uint64_t key, uint64_t i);
/* Box-Muller in binary64 from two 64-bit draws: u1 = ((x1 >> 11) + 1) 2^-53 in (0, 1],
 * u2 = (x2 >> 11) 2^-53 in [0, 1), z = sqrt(-2 ln u1) cos(2 pi u2). */
double orc_box_muller(uint64_t x1, uint64_t x2);
/* signs [n_layers][n_kv_heads][2][128] = +-1 (tag 1, bit 63 of draw j set -> -1) and
 * S [128][128] = fp32 of Box-Muller over draws 2k, 2k + 1 of the tag-2 stream, k = 128 i + j. */
void orc_derive_tables(uint64_t seed, int n_layers, int n_kv_heads, float* signs, float* S);

#ifdef __cplusplus
}
#endif
#endif
