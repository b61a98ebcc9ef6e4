/*
 * kvq.h -- C ABI of the MI355X (gfx950) compressed KV cache and decode-attention library.
 *
 * The library keeps, per (layer, sequence, kv head), a K plane and a V plane of quantized tokens
 * inside ONE device buffer that the caller allocates and owns.  It never allocates device memory.
 * All device pointers are caller-owned and stream-ordered: they must stay valid until the given
 * stream has passed the call.  Streams are hipStream_t handles passed as void* (NULL = the
 * default stream).  Every argument check runs on the host before anything is enqueued; on any
 * error nothing is enqueued and no length changes.  A handle is not thread-safe, and calls on one
 * handle must be issued on one stream (they share one workspace inside the buffer).
 *
 * What each call computes follows these pages (cited by title and section):
 *  [P1] quantcpp article "Beyond RAG: load whole documents on your laptop": progressive table
 *       and "how it works" paragraph (4-bit KV, 128 most recent tokens in FP32, 6.4x
 *       compression = 4-bit codes + fp16 scale + fp16 zero per group of 32), the Python API line
 *       with progressive=True and context_length=131072.
 *  [P2] KVarN-on-Bonsai post, TL;DR and caveats: Walsh-Hadamard transform plus Sinkhorn variance
 *       balancing before 4-bit quantization; cache types chosen separately for K and V
 *       (--cache-type-k / --cache-type-v).
 *  [P3] "LLM memory saving: weights vs KV-cache quantization 2026", method table (TurboQuant
 *       row: random rotation, per-coordinate optimal scalar quantizer, 1-bit QJL on the residual
 *       for an unbiased inner product; online and training-free) and the application rules
 *       (asymmetric K = 8-bit, V = 3/4-bit).
 *
 * Data conventions: head_dim = 128; groups of 32 consecutive channels; GQA maps query head h to
 * kv head h / (n_q_heads / n_kv_heads); fp32 outputs; inputs fp32 or bf16; all input/output
 * pointers 16-byte aligned and contiguous in the shapes stated.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = 1,      /* null pointer, index out of range, bad count            */
    KVQ_ERR_UNSUPPORTED = 2,      /* configuration outside what the kernels implement       */
    KVQ_ERR_CAPACITY = 3,         /* append would exceed max_context; nothing is written    */
    KVQ_ERR_NOT_READY = 4,        /* rotation/QJL tables not set, or layer not calibrated   */
    KVQ_ERR_BUFFER_TOO_SMALL = 5, /* dev_buf smaller than kvq_cache_required_bytes()        */
    KVQ_ERR_MISALIGNED = 6,       /* a pointer is not 16-byte (dev_buf: 256-byte) aligned   */
    KVQ_ERR_HOST_ALLOC = 7,       /* host memory for the handle could not be allocated      */
    KVQ_ERR_DEVICE = 8,           /* a HIP call failed; kvq_last_hip_error() has its code   */
    KVQ_ERR_SCRATCH = 9           /* kvq_attn_decode_static: the call's split partials need
                                     more than KVQ_STATIC_SCRATCH_BYTES                     */
} kvq_status;

/* Bytes of the library-held device scratch that kvq_attn_decode_static uses (one per GPU). */
#define KVQ_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* Element type of the inputs (K, V, q, calibration blocks).  16-bit inputs are widened to fp32
 * exactly on load; every computation is the same as for fp32 inputs of those values. */
typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1, KVQ_F16 = 2 } kvq_dtype;

typedef enum {
    KVQ_UNIFORM = 0,   /* b-bit asymmetric groups of 32, fp16 scale + fp16 zero [P1], b = 3|4|8 */
    KVQ_TURBO_QJL = 1, /* K only: rotation + 3-bit Lloyd-Max code + 1-bit QJL residual [P3]  */
    KVQ_TURBO_MSE = 2, /* rotation + 3-bit (or, for V, 4-bit) Lloyd-Max code, no residual
                          sketch [P3]                                                      */
    KVQ_Q8_0 = 3,      /* symmetric 8-bit groups of 32, one fp16 scale d ("q8_0", [P2]'s
                          baseline; K = Q8 of [P3]'s application rules): q = rint(y / d) in
                          [-127, 127] with d = fp16(max|y| / 127); stored in the UNIFORM 8-bit
                          layout as code q + 128 with zero = -128 d, so y = d q exactly       */
    KVQ_TURBO_SPLIT = 4 /* the outlier-channel split that gives the fractional bit widths of
                          [P3] (2.5 and 3.5 bits, method table and verification notes).
                          kvq_calibrate picks per (layer, kv head, tensor) the 64 channels of
                          largest energy (sum of squares over the calibration tokens, binary64
                          in token order; ties to the smaller index); each 64-channel subset
                          gets its own 64-point random-sign Walsh-Hadamard rotation (signs
                          0..63 / 64..127 of the tensor's sign vector, scale 1/8), fp16 norm
                          and Lloyd-Max code for N(0, 1/64).  V: TurboQuant-MSE, v_bits (3 or
                          4) bits on the outliers, v_bits - 1 on the rest.  K (k_bits = b = 3
                          or 4): the TurboQuant key coder at b - 0.5 bits per channel, MSE
                          codes of b - 1 bits on the outliers and b - 2 on the rest, then the
                          1-bit QJL sketch of the whole residual with the cache's S          */
} kvq_scheme;

typedef struct {
    int n_layers, n_q_heads, n_kv_heads; /* n_q_heads % n_kv_heads == 0, group <= 8          */
    int head_dim;                        /* must be 128                                      */
    int max_batch, max_context;          /* sequences per call (<= 64); tokens per sequence
                                            ("context_length" of [P1])                       */
    int k_scheme, v_scheme;              /* kvq_scheme, chosen separately for K and V [P2]   */
    int k_bits, v_bits;                  /* UNIFORM: 3, 4 or 8; TURBO_QJL: 3; TURBO_MSE: 3, or 4
                                            for V ("Turbo4", [P3] rules); Q8_0: 8;
                                            TURBO_SPLIT: 3 (2.5 bits) or 4 (3.5 bits), K or V */
    int group_size;                      /* must be 32                                       */
    int fp32_window;                     /* 0 = flat, 128 = progressive [P1]                 */
    int rotate_k, rotate_v;              /* random-sign Walsh-Hadamard before coding [P2];
                                            implied by the TURBO schemes                      */
    int sinkhorn_iters, calib_tokens;    /* Sinkhorn balancing of UNIFORM planes [P2]; 0 = off;
                                            calib_tokens bounds kvq_calibrate's n_tokens (also
                                            needed, 2..65536, by a TURBO_SPLIT V)             */
} kvq_config;

typedef struct kvq_cache kvq_cache; /* opaque host-side handle */

/* Device view of one (layer, sequence, kv head, tensor) plane, for inspection and tests.
 * Byte layouts:
 *  UNIFORM K (token-major rows, blocks of 64 tokens): token t at row
 *      64*(t/64) + 16*((t%64)%4) + (t%64)/4 of the code and meta planes.  4-bit row = 16 u32
 *      words, word 4*kb+g holds channels 32g+8kb+i (i=0..7) with channel i at bit
 *      16*(i%2) + 4*(i/2); 8-bit row = 16 units of 8 B, unit 4*kb+g, channel i at byte i.
 *  UNIFORM planes of both tensors hold whole 64-token blocks.
 *  UNIFORM V (blocks of 32 tokens): token t -> block t/32, kb = (t%32)/8, i = t%8; channel d
 *      -> word (4-bit) or 8-byte unit (8-bit) index 8*(16*kb + d%16) + d/16; token i at bit
 *      16*(i%2) + 4*(i/2) (4-bit) or byte i (8-bit).
 *  UNIFORM meta: 16 B per token: u16 fp16 scale[4], then u16 fp16 zero[4] (K: row order,
 *      V: token order).
 *  UNIFORM 3-bit codes: three bit planes laid out exactly as the TURBO 3-bit planes below (K:
 *      48-byte rows in the UNIFORM K row order; V: 1536-byte blocks of 32 tokens), with the
 *      UNIFORM meta: 64 B per token-head.
 *  TURBO planes keep the three bits of each 3-bit code in three bit planes of "half-interleaved"
 *      u32 words: value e (0..31) of a word at bit 16*(e%2) + e/2.  Every plane holds whole
 *      64-token blocks.
 *  TURBO_QJL K: rows in the UNIFORM K order; 48 B per row, group g at byte 12g = words P0, P1,
 *      P2 with value e of Pk = bit k of the code of channel 32g+e.  QJL plane: 16 B per row,
 *      word w value e = sign bit of projection 32w+e.  Meta per row: u16 fp16 norm, u16 fp16
 *      residual norm.
 *  TURBO_MSE V (b = v_bits = 3 or 4 bit planes): blocks of 32 tokens, 512*b B each; token t
 *      (tau = t%32, o = tau/8, i = tau%8), channel d (n = d%16, N = d/16): bit k of its code is
 *      in u32 word 2b*(16o + n) + 2k + N/4 of block t/32, at bit 16*(i%2) + 4*(N%4) + i/2.
 *      Meta: u16 fp16 norm per token.  4-bit codes index the 16-level Lloyd-Max codebook.
 *  TURBO_SPLIT V (bo = v_bits, W = 2 bo - 1): blocks of 32 tokens, 256 W B each; position j
 *      (channel perm[j], n = j%16, N = j/16): bit k of its code is in u32 word
 *      W*(16o + n) + k (j < 64, k < bo) or W*(16o + n) + bo + k (j >= 64, k < bo - 1) of block
 *      t/32, at bit 16*(i%2) + 4*(N%4) + i/2.  Meta: u16 fp16 outlier norm, u16 fp16 rest norm
 *      per token.
 *  TURBO_SPLIT K (b = k_bits): rows in the UNIFORM K row order; position group g (positions
 *      32g .. 32g+31; groups 0, 1 are the outliers with b - 1 code planes, groups 2, 3 the rest
 *      with b - 2) keeps plane k as the u32 word g(b-1) + k (g < 2) or 2(b-1) + (g-2)(b-2) + k
 *      (g >= 2) of its row, value e of the group at bit 16*(e%2) + e/2: 4(4b - 6) B per row
 *      (24 or 40).  QJL plane: 16 B per row as for TURBO_QJL.  Meta: 8 B per row, u16 fp16
 *      outlier norm, rest norm, residual norm, 0.
 *  Window ring: [fp32_window][128] fp32, token t at slot t % fp32_window.               */
typedef struct {
    void *codes, *meta, *qjl, *window;
    size_t codes_bytes, meta_bytes, qjl_bytes, window_bytes;
    int length;
} kvq_layout;

/* Device pointers of the cache's tables (see kvq_set_random_tables / kvq_calibrate). */
typedef struct {
    const float* signs;  /* [n_layers][n_kv_heads][2][128] rotation signs (+-1)          */
    const float* c;      /* [n_layers][n_kv_heads][2][128] Sinkhorn channel scales       */
    const float* inv_c;  /* [n_layers][n_kv_heads][2][128] fp32(1/c)                     */
    const float* qjl_S;  /* [128][128] QJL projection, row-major                         */
    const float* mu;     /* [8] Lloyd-Max centroids for N(0, 1/128)                      */
    const float* theta;  /* [7] Lloyd-Max decision thresholds                            */
    const float* mu16;   /* [16] 16-level centroids (4-bit TurboQuant-MSE V), if present */
    const float* theta16; /* [15] their thresholds                                       */
    const int* perm;     /* [n_layers][n_kv_heads][128] TURBO_SPLIT V position -> channel  */
    const float* mu64;   /* [30] TURBO_SPLIT codebooks of N(0, 1/64): 4, 8, 16 levels at 0,
                            4, 12; 2 levels at 28                                       */
    const float* theta64; /* [30] their thresholds, same offsets (levels - 1 used)       */
    const int* perm_k;   /* [n_layers][n_kv_heads][128] TURBO_SPLIT K position -> channel  */
} kvq_tables;

enum {
    KVQ_OPT_SPLIT_TOKENS = 1, /* tokens per decode split (multiple of 64); 0 = automatic     */
    KVQ_OPT_DECODE_PATH = 2   /* 0 = automatic, 1 = vector-ALU kernel, 2 = matrix-core kernel
                                 (every scheme has both except a TURBO_SPLIT K, which decodes
                                 on the vector ALU: 2 gives KVQ_ERR_UNSUPPORTED for it)      */
};

/* Bytes of device memory a cache with this configuration needs (planes for every layer,
 * sequence and kv head at max_context, tables and workspace).  Pure host computation. */
kvq_status kvq_cache_required_bytes(const kvq_config* cfg, size_t* bytes);

/* Bind a cache to the caller's device buffer (256-byte aligned, >= required bytes) on the
 * current HIP device.  Zero-fills the buffer on `stream` and, when a TURBO scheme is used,
 * computes the Lloyd-Max codebook on the device ([P3], TurboQuant row).  The handle is
 * host memory owned by the library until kvq_cache_destroy. */
kvq_status kvq_cache_create(const kvq_config* cfg, void* dev_buf, size_t bytes, void* stream,
                            kvq_cache** out);

/* Free the host handle.  The device buffer stays the caller's. */
kvq_status kvq_cache_destroy(kvq_cache* cache);

/* Install the random tables the method draws ([P2] random-sign rotation, [P3] random rotation
 * and QJL projection): signs [n_layers][n_kv_heads][2][128] of +-1.0f and S [128][128] of
 * N(0,1) fp32, both device pointers, copied on `stream`.  Either may be NULL when no plane
 * uses it.  Required before appending to a rotated or TURBO plane (else KVQ_ERR_NOT_READY).
 * Entries are not checked on the device. */
kvq_status kvq_set_random_tables(kvq_cache* cache, const float* signs, const float* qjl_S,
                                 void* stream);

/* Draw those tables from a 64-bit seed, on the host (no device work, no handle): signs
 * [n_layers][n_kv_heads][2][128] of +-1.0f and S [128][128] of N(0,1) rounded to fp32, into
 * caller-owned host arrays (either may be NULL).  The pages ask for random signs and a Gaussian
 * projection ([P2] TL;DR; [P3] method comparison table, TurboQuant row) but name no generator;
 * this one is counter-based SplitMix64 (Steele, Lea and Flood, 2014): a stream key chains the
 * SplitMix64 output function over (seed, tag, layer, head, tensor), draw i of a stream is the
 * (i + 1)-th output of the generator started at the key.  Sign j of (layer, head, tensor) is -1
 * when bit 63 of draw j of the tag-1 stream is set.  S[i][j] = fp32 of the binary64 Box-Muller
 * value sqrt(-2 ln u1) cos(2 pi u2) with u1 = ((x1 >> 11) + 1) 2^-53, u2 = (x2 >> 11) 2^-53 from
 * draws 2k and 2k + 1 (k = 128 i + j) of the tag-2 stream (key fields 0, 0, 0).  The same seed
 * gives the same tables on every host with the same C math library.  KVQ_ERR_INVALID_ARG when
 * n_layers or n_kv_heads < 1 and signs is not NULL. */
kvq_status kvq_derive_random_tables(unsigned long long seed, int n_layers, int n_kv_heads, float* signs,
                                    float* qjl_S);

/* kvq_set_random_tables with the tables kvq_derive_random_tables draws from `seed` for this
 * cache's n_layers and n_kv_heads.  Synchronous: the draw is staged in host memory the call
 * allocates (KVQ_ERR_HOST_ALLOC if it cannot), copied on `stream`, and the call returns after
 * the copy has completed. */
kvq_status kvq_set_random_tables_seeded(kvq_cache* cache, unsigned long long seed, void* stream);

/* Sinkhorn variance balancing of one layer ([P2] TL;DR): for every kv head and every UNIFORM
 * tensor with sinkhorn_iters > 0, rotate the calibration tokens (device, [n_tokens][n_kv_heads]
 * [128] of dtype for K and V; a tensor's pointer may be NULL when it is not balanced), then
 * alternately divide rows and columns by their population standard deviation sinkhorn_iters
 * times in fp64 on the device, and store c = product of the column divisors and fp32(1/c).
 * 2 <= n_tokens <= calib_tokens.  A TURBO_SPLIT V (K) takes its 64 outlier channels per kv
 * head from Vc (Kc), required then, in the same call.  Required once per layer before appending
 * to it. */
kvq_status kvq_calibrate(kvq_cache* cache, int layer, const void* Kc, const void* Vc, int dtype,
                         int n_tokens, void* stream);

/* Quantize and append n_tokens new tokens of every sequence b < batch of `layer` ([P1]
 * progressive window, [P2] rotation + balancing, [P3] online TurboQuant code).
 * K, V: device [batch][n_tokens][n_kv_heads][128] of dtype.  Token k of sequence b becomes
 * token len[b] + k.  Bit-identical to n_tokens calls of kvq_append.  KVQ_ERR_CAPACITY if
 * len[b] + n_tokens > max_context for any b. */
kvq_status kvq_prefill_quantize(kvq_cache* cache, int layer, const void* K, const void* V,
                                int dtype, int n_tokens, int batch, void* stream);

/* kvq_prefill_quantize with n_tokens = 1; k, v: device [batch][n_kv_heads][128]. */
kvq_status kvq_append(kvq_cache* cache, int layer, const void* k, const void* v, int dtype,
                      int batch, void* stream);

/* Decode attention of one new query token per sequence over everything cached for `layer`
 * ([P1], [P3] method row): out[b][h] = sum_t softmax_t(scale <q[b][h], k_t>) v_t, where k_t, v_t
 * are the FP32 originals for the last fp32_window tokens and the dequantized codes (or the
 * TurboQuant estimate for K) before that.  q: device [batch][n_q_heads][128] of dtype;
 * out: device [batch][n_q_heads][128] fp32.  softmax_scale <= 0 means 1/sqrt(128).  A sequence
 * with no tokens gets zeros. */
kvq_status kvq_attn_decode(kvq_cache* cache, int layer, const void* q, int dtype, float* out,
                           int batch, float softmax_scale, void* stream);

/* kvq_attn_decode for callers that cannot allocate device memory or touch the cache's own work
 * area per call (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, checks, kernels and split plan as kvq_attn_decode, hence the same
 * output bit for bit; the split partials (batch x n_q_heads x splits x 528 B) go to a static
 * device array of KVQ_STATIC_SCRATCH_BYTES that the library holds on each GPU until the process
 * ends (its address is taken once per device by kvq_cache_create).  Nothing is allocated: no
 * hipMalloc, hipFree or allocating library routine.  KVQ_ERR_SCRATCH (nothing enqueued) when the
 * partials would exceed the scratch.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents (every partial is written before it is read, so nothing needs to start
 * at zero): calls that overlap on one GPU (other streams, other threads) race. */
kvq_status kvq_attn_decode_static(kvq_cache* cache, int layer, const void* q, int dtype, float* out,
                                  int batch, float softmax_scale, void* stream);

/* One decode step of one layer: kvq_append(k, v) followed by kvq_attn_decode(q) over the cache
 * that now includes the new token, in one call ([P1], [P2], [P3] as for those two calls).  Same
 * arguments, layouts, checks and results: the packed planes are bit-identical to the two calls,
 * and so is the output.  On the matrix-core path the append runs inside the decode kernel: the
 * workgroup whose token range holds the new token quantizes it before reading.  The lengths grow
 * by one only when the call is accepted. */
kvq_status kvq_append_attn_decode(kvq_cache* cache, int layer, const void* k, const void* v,
                                  const void* q, int dtype, float* out, int batch,
                                  float softmax_scale, void* stream);

/* Attention of a prefill chunk ([P1] v3.2 batched prefill: the prompt goes through in whole
 * chunks; keys and values as for kvq_attn_decode).  The n_q newest tokens of each of the first
 * `batch` sequences are the queries: they must already be in the cache (kvq_prefill_quantize),
 * and query i of sequence b, at position pos = len[b] - n_q + i, attends to tokens 0 .. pos of
 * the cache as it stands: out[b][i][h] = sum_{t <= pos} softmax_t(scale <q[b][i][h], k_t>) v_t.
 * q: device [batch][n_q][n_q_heads][128] of dtype; out: device [batch][n_q][n_q_heads][128]
 * fp32 (row-major, 16-byte aligned).  softmax_scale <= 0 means 1/sqrt(128).
 * Every key and value scheme of kvq_config is read, with or without the FP32 window; TurboQuant-
 * QJL keys score as in kvq_attn_decode ([P3] method table, TurboQuant row: n <R q, mu[code]>
 * plus the 1-bit QJL estimate of the residual's inner product).
 * workspace: optional caller-owned device memory (16-byte aligned, workspace_bytes long).  It
 * holds, first, when fp32_window > 0 beside rotated, balanced or TurboQuant codes, the window's
 * originals mapped into the code domain (batch x n_kv_heads x 2 x 128 x 128 fp32), then the
 * partial results when the keys of each query are split over several workgroups; NULL uses the
 * cache's own workspace.  kvq_attn_prefill_workspace() gives the bytes the fastest split plan
 * needs; with less, the call uses fewer splits (the result agrees to rounding), and with less
 * than the window copy it fails with KVQ_ERR_BUFFER_TOO_SMALL.  Like the cache's own workspace,
 * it must not be in use by another call at the same time.
 * Errors (nothing enqueued): KVQ_ERR_INVALID_ARG for a bad handle, layer, pointer, dtype, batch
 * outside 1 .. max_batch, n_q < 1, or n_q above some sequence's length; KVQ_ERR_MISALIGNED;
 * KVQ_ERR_NOT_READY before the layer's tables / calibration are set; KVQ_ERR_BUFFER_TOO_SMALL as
 * above. */
kvq_status kvq_attn_prefill(kvq_cache* cache, int layer, const void* q, int dtype, float* out,
                            int n_q, int batch, float softmax_scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Device workspace bytes for kvq_attn_prefill(cache, layer, ..., n_q, batch, ...) with the
 * layer's current lengths: the mapped window copy (if the cache needs one) plus the partials of
 * the fastest split plan (none when one split per query fills the GPU).  Pure host computation;
 * KVQ_ERR_INVALID_ARG as for kvq_attn_prefill. */
kvq_status kvq_attn_prefill_workspace(const kvq_cache* cache, int layer, int n_q, int batch,
                                      size_t* bytes);

/* Plane pointers and sizes of (layer, seq, kv_head, tensor 0 = K / 1 = V). */
kvq_status kvq_get_layout(const kvq_cache* cache, int layer, int seq, int kv_head, int tensor,
                          kvq_layout* out);

/* Device pointers of the tables. */
kvq_status kvq_get_tables(const kvq_cache* cache, kvq_tables* out);

/* Set a tuning option (KVQ_OPT_*). Results do not depend on it beyond float rounding order. */
kvq_status kvq_set_option(kvq_cache* cache, int option, int value);

/* Measurement hook: while set, every kvq_attn_decode launches its split-K decode kernel with
 * ev_start / ev_stop attached to the kernel's own dispatch (hipExtLaunchKernelGGL), so the pair
 * times exactly that kernel on the call's stream.  hipEvent_t handles passed as void*, created
 * (with timing) and owned by the caller, who keeps them alive while set.  Both NULL clears the
 * hook; exactly one NULL is KVQ_ERR_INVALID_ARG.  Results do not depend on it. */
kvq_status kvq_set_timing_events(kvq_cache* cache, void* ev_start, void* ev_stop);

/* Tokens cached for (layer, seq); -1 on a bad argument. */
int kvq_get_length(const kvq_cache* cache, int layer, int seq);

/* Static description of a status code. */
const char* kvq_status_str(kvq_status status);

/* hipError_t of the last failed HIP call on this handle (0 if none). */
int kvq_last_hip_error(const kvq_cache* cache);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
