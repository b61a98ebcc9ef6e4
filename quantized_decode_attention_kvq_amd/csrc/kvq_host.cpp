// Host side of libkvq: configuration checks, the device-buffer layout planner, table setup and
// kernel launches behind the C ABI declared in include/kvq.h.  No call allocates device memory;
// every argument is checked before anything is enqueued.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

using namespace kvq;

namespace {

constexpr size_t kAlign = 256;
constexpr int kLloydIters = 2000;

size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
size_t ceil_to(size_t x, size_t m) { return (x + m - 1) / m * m; }

struct Plan {
    PlaneGeom geom[2];
    size_t plane_bytes[2];
    size_t slot_bytes;
    size_t off_signs, off_c, off_inv_c, off_S, off_ST, off_mu, off_theta, off_mu16, off_theta16;
    size_t off_perm, off_perm_k, off_mu64, off_theta64;
    size_t off_work, work_bytes;
    size_t off_planes, total;
};

kvq_status check_config(const kvq_config* c) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (c->n_layers < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->max_batch < 1 ||
        c->max_context < 1 || c->head_dim < 1 || c->group_size < 1 || c->sinkhorn_iters < 0 ||
        c->calib_tokens < 0 || c->fp32_window < 0)
        return KVQ_ERR_INVALID_ARG;
    if (c->n_q_heads % c->n_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
    if (c->head_dim != kDim || c->group_size != kGroup) return KVQ_ERR_UNSUPPORTED;
    if (c->n_q_heads / c->n_kv_heads > kMaxGroupHeads) return KVQ_ERR_UNSUPPORTED;
    if (c->max_batch > kMaxBatch) return KVQ_ERR_UNSUPPORTED;
    if (c->max_context > (1 << 26)) return KVQ_ERR_UNSUPPORTED;
    if (c->fp32_window != 0 && c->fp32_window != kWindowMax) return KVQ_ERR_UNSUPPORTED;
    if (c->k_scheme != KVQ_UNIFORM && c->k_scheme != KVQ_TURBO_QJL && c->k_scheme != KVQ_Q8_0 &&
        c->k_scheme != KVQ_TURBO_SPLIT)
        return KVQ_ERR_UNSUPPORTED;
    if (c->v_scheme != KVQ_UNIFORM && c->v_scheme != KVQ_TURBO_MSE && c->v_scheme != KVQ_Q8_0 &&
        c->v_scheme != KVQ_TURBO_SPLIT)
        return KVQ_ERR_UNSUPPORTED;
    for (int t = 0; t < 2; ++t) {
        const int scheme = t == 0 ? c->k_scheme : c->v_scheme, bits = t == 0 ? c->k_bits : c->v_bits;
        if (scheme == KVQ_UNIFORM && bits != 3 && bits != 4 && bits != 8) return KVQ_ERR_UNSUPPORTED;
        if (scheme == KVQ_Q8_0 && bits != 8) return KVQ_ERR_UNSUPPORTED;
        if (scheme == KVQ_TURBO_QJL && bits != 3) return KVQ_ERR_UNSUPPORTED;
        // TurboQuant-MSE: 3-bit codes, or 4-bit codes for V ("Turbo4")
        if (scheme == KVQ_TURBO_MSE && bits != 3 && !(bits == 4 && t == 1)) return KVQ_ERR_UNSUPPORTED;
        // outlier split: V with 3 or 4 bits on the outlier half and one fewer on the rest; K at
        // b = 3 or 4 (b - 1 / b - 2 MSE bits plus the QJL bit: 2.5 or 3.5 bits per channel)
        if (scheme == KVQ_TURBO_SPLIT && bits != 3 && bits != 4) return KVQ_ERR_UNSUPPORTED;
    }
    if ((c->rotate_k != 0 && c->rotate_k != 1) || (c->rotate_v != 0 && c->rotate_v != 1))
        return KVQ_ERR_INVALID_ARG;
    if (c->sinkhorn_iters > 1000) return KVQ_ERR_UNSUPPORTED;
    if ((c->sinkhorn_iters > 0 || c->v_scheme == KVQ_TURBO_SPLIT || c->k_scheme == KVQ_TURBO_SPLIT) &&
        (c->calib_tokens < 2 || c->calib_tokens > 65536))
        return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

PlaneGeom make_geom(const kvq_config* c, int tensor) {
    PlaneGeom g{};
    const int cfg_scheme = tensor == 0 ? c->k_scheme : c->v_scheme;
    // a q8_0 plane is an 8-bit uniform plane to every kernel that reads it; only its quantizer
    // differs (symmetric codes, zero field = -128 * scale)
    const int scheme = cfg_scheme == KVQ_Q8_0 ? KVQ_UNIFORM : cfg_scheme;
    g.scheme = scheme;
    g.symmetric = cfg_scheme == KVQ_Q8_0 ? 1 : 0;
    g.bits = tensor == 0 ? c->k_bits : c->v_bits;
    g.rotate = (scheme != KVQ_UNIFORM) ? 1 : (tensor == 0 ? c->rotate_k : c->rotate_v);
    g.sinkhorn = (scheme == KVQ_UNIFORM && c->sinkhorn_iters > 0) ? 1 : 0;
    // whole 64-token blocks for every plane: decode reads 64 tokens at a time
    const size_t rows = ceil_to((size_t)c->max_context, 64);
    if (scheme == KVQ_UNIFORM) {
        g.codes_bytes = rows * 16 * (size_t)g.bits;
        g.meta_bytes = rows * 16;
        g.qjl_bytes = 0;
    } else if (scheme == KVQ_TURBO_SPLIT && tensor == 0) {
        g.codes_bytes = rows * (size_t)split_k_row_bytes(g.bits); // per-group plane words per row
        g.meta_bytes = rows * 8;                                  // fp16 n_outlier, n_rest, gamma, 0
        g.qjl_bytes = rows * 16;
    } else if (scheme == KVQ_TURBO_SPLIT) {
        g.codes_bytes = rows * 8 * (size_t)(2 * g.bits - 1); // bits + (bits - 1) planes of 8 B
        g.meta_bytes = rows * 4;                             // two fp16 norms per token
        g.qjl_bytes = 0;
    } else {
        g.codes_bytes = rows * 16 * (size_t)g.bits; // b bit planes of 16 B per token-head
        g.meta_bytes = rows * (scheme == KVQ_TURBO_QJL ? 4 : 2);
        g.qjl_bytes = scheme == KVQ_TURBO_QJL ? rows * 16 : 0;
    }
    g.ring_bytes = (size_t)c->fp32_window * kDim * sizeof(float);
    size_t off = 0;
    g.codes_off = off;
    off = align_up(off + g.codes_bytes);
    g.meta_off = off;
    off = align_up(off + g.meta_bytes);
    g.qjl_off = off;
    off = align_up(off + g.qjl_bytes);
    g.ring_off = off;
    return g;
}

Plan make_plan(const kvq_config* c) {
    Plan p{};
    for (int t = 0; t < 2; ++t) {
        p.geom[t] = make_geom(c, t);
        p.plane_bytes[t] = align_up(p.geom[t].ring_off + p.geom[t].ring_bytes);
    }
    p.slot_bytes = p.plane_bytes[0] + p.plane_bytes[1];
    const size_t tab = (size_t)c->n_layers * c->n_kv_heads * 2 * kDim * sizeof(float);
    size_t off = 0;
    p.off_signs = off;
    off = align_up(off + tab);
    p.off_c = off;
    off = align_up(off + tab);
    p.off_inv_c = off;
    off = align_up(off + tab);
    p.off_S = off;
    off = align_up(off + kDim * kDim * sizeof(float));
    p.off_ST = off;
    off = align_up(off + kDim * kDim * sizeof(float));
    p.off_mu = off;
    off = align_up(off + 8 * sizeof(float));
    p.off_theta = off;
    off = align_up(off + 8 * sizeof(float));
    p.off_mu16 = off;
    off = align_up(off + 16 * sizeof(float));
    p.off_theta16 = off;
    off = align_up(off + 16 * sizeof(float));
    p.off_perm = off;
    off = align_up(off + (size_t)c->n_layers * c->n_kv_heads * kDim * sizeof(int));
    p.off_perm_k = off;
    off = align_up(off + (size_t)c->n_layers * c->n_kv_heads * kDim * sizeof(int));
    p.off_mu64 = off;
    off = align_up(off + kSplitTable * sizeof(float));
    p.off_theta64 = off;
    off = align_up(off + kSplitTable * sizeof(float));
    const size_t partial = (size_t)c->max_batch * c->n_q_heads * kMaxSplits * kPartialFloats *
                           sizeof(float);
    // Sinkhorn work: the calibration block [2][Hkv][n][128], then two [2][Hkv][128] scale rows
    const size_t calib = c->sinkhorn_iters > 0
                             ? (size_t)2 * c->n_kv_heads * (c->calib_tokens + 2) * kDim * sizeof(double)
                             : 0;
    // prefill attention beside rotated or balanced codes also keeps the mapped window there
    const size_t win = window_in_code_domain(p.geom[0], p.geom[1], c->fp32_window)
                           ? align_up(prefill_window_bytes(c->max_batch, c->n_kv_heads))
                           : 0;
    p.work_bytes = align_up(std::max(partial + win, calib));
    p.off_work = off;
    off += p.work_bytes;
    p.off_planes = off;
    off += (size_t)c->n_layers * c->max_batch * c->n_kv_heads * p.slot_bytes;
    p.total = off;
    return p;
}

// Seeded tables: SplitMix64 (Steele, Lea and Flood, 2014) used counter-style.  Its generator
// steps a 64-bit state by the odd constant 0x9E3779B97F4A7C15 and outputs the state through a
// fixed mixing function, so the (i + 1)-th output from a state k is mix(k + (i + 1) * step).
constexpr uint64_t kSeedStep = 0x9E3779B97F4A7C15ull;
inline uint64_t splitmix_out(uint64_t x) {
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}
// One stream of draws: key = the output function chained over (seed, tag, layer, head, tensor).
struct SeedStream {
    uint64_t key;
    SeedStream(uint64_t seed, int tag, int layer, int head, int tensor) {
        const int fields[4] = {tag, layer, head, tensor};
        key = seed;
        for (int f : fields) key = splitmix_out(key + kSeedStep * (uint64_t)(f + 1));
    }
    uint64_t draw(uint64_t i) const { return splitmix_out(key + kSeedStep * (i + 1)); }
};
// Box-Muller: radius from u1 in (0, 1], angle from u2 in [0, 1), binary64, rounded to fp32 once.
inline float gaussian_from(uint64_t a, uint64_t b) {
    const double scale = 0x1p-53;
    const double u1 = static_cast<double>((a >> 11) + 1) * scale;
    const double u2 = static_cast<double>(b >> 11) * scale;
    const double radius = std::sqrt(-2.0 * std::log(u1));
    const double angle = 6.283185307179586 * u2;
    const double value = radius * std::cos(angle);
    return static_cast<float>(value);
}

} // namespace

struct kvq_cache {
    kvq_config cfg;
    Plan plan;
    char* base;
    size_t bytes;
    std::vector<int> len;              // [n_layers][max_batch]
    std::vector<unsigned char> calibrated;
    bool tables_set;
    int last_hip_error;
    int split_tokens_opt;
    int decode_path;
    int num_cus;
    int device;
    hipEvent_t ev[2]; // measurement hook of kvq_set_timing_events (caller-owned), or both null

    float* signs() const { return reinterpret_cast<float*>(base + plan.off_signs); }
    float* cs() const { return reinterpret_cast<float*>(base + plan.off_c); }
    float* inv_c() const { return reinterpret_cast<float*>(base + plan.off_inv_c); }
    float* S() const { return reinterpret_cast<float*>(base + plan.off_S); }
    float* ST() const { return reinterpret_cast<float*>(base + plan.off_ST); }
    float* mu() const { return reinterpret_cast<float*>(base + plan.off_mu); }
    float* theta() const { return reinterpret_cast<float*>(base + plan.off_theta); }
    float* mu16() const { return reinterpret_cast<float*>(base + plan.off_mu16); }
    float* theta16() const { return reinterpret_cast<float*>(base + plan.off_theta16); }
    bool turbo4() const { return cfg.v_scheme == KVQ_TURBO_MSE && cfg.v_bits == 4; }
    bool split() const { return cfg.v_scheme == KVQ_TURBO_SPLIT; }
    bool split_k() const { return cfg.k_scheme == KVQ_TURBO_SPLIT; }
    int* perm() const { return reinterpret_cast<int*>(base + plan.off_perm); }
    int* perm_k() const { return reinterpret_cast<int*>(base + plan.off_perm_k); }
    float* mu64() const { return reinterpret_cast<float*>(base + plan.off_mu64); }
    float* theta64() const { return reinterpret_cast<float*>(base + plan.off_theta64); }
    size_t perm_off(int layer) const { return (size_t)layer * cfg.n_kv_heads * kDim; }
    char* layer_base(int layer) const {
        return base + plan.off_planes + (size_t)layer * cfg.max_batch * cfg.n_kv_heads * plan.slot_bytes;
    }
    size_t table_off(int layer) const { return (size_t)layer * cfg.n_kv_heads * 2 * kDim; }
    bool needs_signs() const { return plan.geom[0].rotate || plan.geom[1].rotate; }
    bool needs_S() const { return cfg.k_scheme == KVQ_TURBO_QJL || cfg.k_scheme == KVQ_TURBO_SPLIT; }
    bool needs_sinkhorn() const { return plan.geom[0].sinkhorn || plan.geom[1].sinkhorn; }
    bool needs_calib() const { return needs_sinkhorn() || split() || split_k(); }
    bool turbo() const { return cfg.k_scheme == KVQ_TURBO_QJL || cfg.v_scheme == KVQ_TURBO_MSE; }
};

namespace {

kvq_status dev_fail(kvq_cache* c, hipError_t e) {
    if (c) c->last_hip_error = (int)e;
    return KVQ_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void fill_params_common(const kvq_cache* c, int layer, char*& lb, size_t& seq_stride,
                        size_t& head_stride, size_t plane_off[2], PlaneGeom geom[2]) {
    lb = c->layer_base(layer);
    head_stride = c->plan.slot_bytes;
    seq_stride = (size_t)c->cfg.n_kv_heads * c->plan.slot_bytes;
    plane_off[0] = 0;
    plane_off[1] = c->plan.plane_bytes[0];
    geom[0] = c->plan.geom[0];
    geom[1] = c->plan.geom[1];
}

} // namespace

extern "C" {

kvq_status kvq_cache_required_bytes(const kvq_config* cfg, size_t* bytes) {
    if (!bytes) return KVQ_ERR_INVALID_ARG;
    const kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    *bytes = make_plan(cfg).total;
    return KVQ_OK;
}

kvq_status kvq_cache_create(const kvq_config* cfg, void* dev_buf, size_t bytes, void* stream,
                            kvq_cache** out) {
    if (!out) return KVQ_ERR_INVALID_ARG;
    *out = nullptr;
    const kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    if (!dev_buf) return KVQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(dev_buf) & (kAlign - 1)) != 0) return KVQ_ERR_MISALIGNED;
    const Plan plan = make_plan(cfg);
    if (bytes < plan.total) return KVQ_ERR_BUFFER_TOO_SMALL;
    kvq_cache* c = new (std::nothrow) kvq_cache();
    if (!c) return KVQ_ERR_HOST_ALLOC;
    try {
        c->len.assign((size_t)cfg->n_layers * cfg->max_batch, 0);
        c->calibrated.assign((size_t)cfg->n_layers, 0);
    } catch (...) {
        delete c;
        return KVQ_ERR_HOST_ALLOC;
    }
    c->cfg = *cfg;
    c->plan = plan;
    c->base = static_cast<char*>(dev_buf);
    c->bytes = bytes;
    c->tables_set = false;
    c->last_hip_error = 0;
    c->split_tokens_opt = 0;
    c->decode_path = 0;
    c->ev[0] = c->ev[1] = nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipGetDevice(&c->device);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, c->device);
    if (e == hipSuccess) e = hipMemsetAsync(dev_buf, 0, plan.total, s);
    if (e == hipSuccess) {
        const size_t n = (size_t)cfg->n_layers * cfg->n_kv_heads * 2 * kDim;
        e = launch_fill(c->cs(), n, 1.0f, s);
        if (e == hipSuccess) e = launch_fill(c->inv_c(), n, 1.0f, s);
        if (e == hipSuccess) e = launch_fill(c->signs(), n, 1.0f, s);
    }
    // the static scratch of kvq_attn_decode_static: its address on this device, once per device
    if (e == hipSuccess) e = static_scratch_setup(c->device);
    if (e == hipSuccess && c->turbo()) e = launch_codebook(c->mu(), c->theta(), kLloydIters, 8, 128, s);
    if (e == hipSuccess && c->turbo4()) e = launch_codebook(c->mu16(), c->theta16(), kLloydIters, 16, 128, s);
    // split V / K: the 2-, 4-, 8- and 16-level codebooks of N(0, 1/64) (split_table_off)
    for (int levels = 2; levels <= 16 && e == hipSuccess && (c->split() || c->split_k()); levels *= 2)
        e = launch_codebook(c->mu64() + split_table_off(levels), c->theta64() + split_table_off(levels), kLloydIters,
                            levels, 64, s);
    if (e != hipSuccess) {
        delete c;
        return KVQ_ERR_DEVICE;
    }
    *out = c;
    return KVQ_OK;
}

kvq_status kvq_cache_destroy(kvq_cache* cache) {
    if (!cache) return KVQ_ERR_INVALID_ARG;
    delete cache;
    return KVQ_OK;
}

kvq_status kvq_set_random_tables(kvq_cache* c, const float* signs, const float* qjl_S, void* stream) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (c->needs_signs() && !signs) return KVQ_ERR_INVALID_ARG;
    if (c->needs_S() && !qjl_S) return KVQ_ERR_INVALID_ARG;
    if ((signs && !aligned16(signs)) || (qjl_S && !aligned16(qjl_S))) return KVQ_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (signs)
        e = hipMemcpyAsync(c->signs(), signs,
                           (size_t)c->cfg.n_layers * c->cfg.n_kv_heads * 2 * kDim * sizeof(float),
                           hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && qjl_S) {
        e = hipMemcpyAsync(c->S(), qjl_S, kDim * kDim * sizeof(float), hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess) e = launch_transpose128(c->S(), c->ST(), s);
    }
    if (e != hipSuccess) return dev_fail(c, e);
    c->tables_set = true;
    return KVQ_OK;
}

kvq_status kvq_derive_random_tables(unsigned long long seed, int n_layers, int n_kv_heads, float* signs,
                                    float* qjl_S) {
    if (signs && (n_layers < 1 || n_kv_heads < 1)) return KVQ_ERR_INVALID_ARG;
    if (signs) {
        for (int layer = 0; layer < n_layers; ++layer)
            for (int head = 0; head < n_kv_heads; ++head)
                for (int tensor = 0; tensor < 2; ++tensor) {
                    const SeedStream st(seed, 1, layer, head, tensor);
                    float* row = signs + (((size_t)layer * n_kv_heads + head) * 2 + tensor) * kDim;
                    for (int j = 0; j < kDim; ++j) row[j] = (st.draw((uint64_t)j) >> 63) != 0 ? -1.0f : 1.0f;
                }
    }
    if (qjl_S) {
        const SeedStream st(seed, 2, 0, 0, 0);
        for (int e = 0; e < kDim * kDim; ++e) qjl_S[e] = gaussian_from(st.draw(2 * (uint64_t)e), st.draw(2 * (uint64_t)e + 1));
    }
    return KVQ_OK;
}

kvq_status kvq_set_random_tables_seeded(kvq_cache* c, unsigned long long seed, void* stream) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    const size_t n_signs = (size_t)c->cfg.n_layers * c->cfg.n_kv_heads * 2 * kDim;
    std::vector<float> staging;
    try {
        staging.resize(n_signs + (size_t)kDim * kDim);
    } catch (const std::bad_alloc&) {
        return KVQ_ERR_HOST_ALLOC;
    }
    kvq_derive_random_tables(seed, c->cfg.n_layers, c->cfg.n_kv_heads, staging.data(), staging.data() + n_signs);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(c->signs(), staging.data(), n_signs * sizeof(float), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->S(), staging.data() + n_signs, (size_t)kDim * kDim * sizeof(float), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_transpose128(c->S(), c->ST(), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s); // the staging vector goes out of scope below
    if (e != hipSuccess) return dev_fail(c, e);
    c->tables_set = true;
    return KVQ_OK;
}

kvq_status kvq_calibrate(kvq_cache* c, int layer, const void* Kc, const void* Vc, int dtype,
                         int n_tokens, void* stream) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (layer < 0 || layer >= c->cfg.n_layers) return KVQ_ERR_INVALID_ARG;
    if (dtype != KVQ_F32 && dtype != KVQ_BF16 && dtype != KVQ_F16) return KVQ_ERR_INVALID_ARG;
    if (!c->needs_calib()) return KVQ_ERR_INVALID_ARG;
    if (n_tokens < 2 || n_tokens > c->cfg.calib_tokens) return KVQ_ERR_INVALID_ARG;
    CalibParams p{};
    const void* src[2] = {Kc, Vc};
    for (int t = 0; t < 2; ++t) {
        p.do_tensor[t] = c->plan.geom[t].sinkhorn;
        p.rotate[t] = c->plan.geom[t].rotate;
        if (p.do_tensor[t] && !src[t]) return KVQ_ERR_INVALID_ARG;
        if (src[t] && !aligned16(src[t])) return KVQ_ERR_MISALIGNED;
        p.src[t] = src[t];
    }
    if ((c->split() && !Vc) || (c->split_k() && !Kc)) return KVQ_ERR_INVALID_ARG;
    if (c->needs_signs() && !c->tables_set) return KVQ_ERR_NOT_READY;
    p.work = reinterpret_cast<double*>(c->base + c->plan.off_work);
    p.signs = c->signs() + c->table_off(layer);
    p.cs = c->cs() + c->table_off(layer);
    p.inv_c = c->inv_c() + c->table_off(layer);
    p.dtype = dtype;
    p.n = n_tokens;
    p.Hkv = c->cfg.n_kv_heads;
    p.iters = c->cfg.sinkhorn_iters;
    hipError_t e = hipSuccess;
    if (c->needs_sinkhorn()) e = launch_calibrate(p, static_cast<hipStream_t>(stream));
    for (int t = 0; t < 2 && e == hipSuccess; ++t) {
        if (!(t == 0 ? c->split_k() : c->split())) continue;
        OutlierParams op{};
        op.src = t == 0 ? Kc : Vc;
        op.perm = (t == 0 ? c->perm_k() : c->perm()) + c->perm_off(layer);
        op.dtype = dtype;
        op.n = n_tokens;
        op.Hkv = c->cfg.n_kv_heads;
        e = launch_select_outliers(op, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return dev_fail(c, e);
    c->calibrated[(size_t)layer] = 1;
    return KVQ_OK;
}

namespace {

// Checks of an append / prefill of n_tokens and its kernel parameters (nothing is enqueued and
// no length changes here).
kvq_status make_quant(kvq_cache* c, int layer, const void* K, const void* V, int dtype, int n_tokens,
                      int batch, QuantParams& p) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (layer < 0 || layer >= c->cfg.n_layers) return KVQ_ERR_INVALID_ARG;
    if (batch < 1 || batch > c->cfg.max_batch || n_tokens < 0) return KVQ_ERR_INVALID_ARG;
    if (dtype != KVQ_F32 && dtype != KVQ_BF16 && dtype != KVQ_F16) return KVQ_ERR_INVALID_ARG;
    if (!K || !V) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(K) || !aligned16(V)) return KVQ_ERR_MISALIGNED;
    const int* len = &c->len[(size_t)layer * c->cfg.max_batch];
    for (int b = 0; b < batch; ++b)
        if ((long long)len[b] + n_tokens > c->cfg.max_context) return KVQ_ERR_CAPACITY;
    if ((c->needs_signs() || c->needs_S()) && !c->tables_set) return KVQ_ERR_NOT_READY;
    if (c->needs_calib() && !c->calibrated[(size_t)layer]) return KVQ_ERR_NOT_READY;

    p = QuantParams{};
    p.src[0] = K;
    p.src[1] = V;
    fill_params_common(c, layer, p.layer_base, p.seq_stride, p.head_stride, p.plane_off, p.geom);
    for (int t = 0; t < 2; ++t) {
        p.signs[t] = c->signs() + c->table_off(layer);
        p.inv_c[t] = c->inv_c() + c->table_off(layer);
    }
    p.qjl_st = c->ST();
    p.mu = c->mu();
    p.theta = c->theta();
    p.mu16 = c->mu16();
    p.theta16 = c->theta16();
    p.perm = c->perm() + c->perm_off(layer);
    p.perm_k = c->perm_k() + c->perm_off(layer);
    p.mu64 = c->mu64();
    p.theta64 = c->theta64();
    p.dtype = dtype;
    p.T = n_tokens;
    p.batch = batch;
    p.Hkv = c->cfg.n_kv_heads;
    p.window = c->cfg.fp32_window;
    int groups = 0;
    for (int b = 0; b < batch; ++b) {
        p.start[b] = len[b];
        groups = std::max(groups, (len[b] + n_tokens - 1) / 8 - len[b] / 8 + 1);
    }
    p.groups8 = groups;
    return KVQ_OK;
}

// Argument checks of a decode call.
kvq_status check_decode(const kvq_cache* c, int layer, const void* q, int dtype, const float* out,
                        int batch, float softmax_scale) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (layer < 0 || layer >= c->cfg.n_layers) return KVQ_ERR_INVALID_ARG;
    if (batch < 1 || batch > c->cfg.max_batch) return KVQ_ERR_INVALID_ARG;
    if (dtype != KVQ_F32 && dtype != KVQ_BF16 && dtype != KVQ_F16) return KVQ_ERR_INVALID_ARG;
    if (!q || !out) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_MISALIGNED;
    if (!std::isfinite(softmax_scale)) return KVQ_ERR_INVALID_ARG;
    if ((c->needs_signs() || c->needs_S()) && !c->tables_set) return KVQ_ERR_NOT_READY;
    return KVQ_OK;
}

// Decode parameters and split plan over the current lengths; `matrix` = matrix-core path.
kvq_status make_decode(const kvq_cache* c, int layer, const void* q, int dtype, float* out, int batch,
                       float softmax_scale, DecodeParams& p, bool& matrix) {
    p = DecodeParams{};
    p.q = q;
    p.out = out;
    fill_params_common(c, layer, p.layer_base, p.seq_stride, p.head_stride, p.plane_off, p.geom);
    p.signs = c->signs() + c->table_off(layer);
    p.cs = c->cs() + c->table_off(layer);
    p.qjl_st = c->ST();
    p.mu = c->mu();
    p.mu16 = c->mu16();
    p.perm = c->perm() + c->perm_off(layer);
    p.perm_k = c->perm_k() + c->perm_off(layer);
    p.mu64 = c->mu64();
    p.partials = reinterpret_cast<float*>(c->base + c->plan.off_work);
    p.dtype = dtype;
    p.batch = batch;
    p.Hq = c->cfg.n_q_heads;
    p.Hkv = c->cfg.n_kv_heads;
    p.G = p.Hq / p.Hkv;
    p.window = c->cfg.fp32_window;
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(128.0f);
    p.qscale = scale * 1.4426950408889634f;
    const int* len = &c->len[(size_t)layer * c->cfg.max_batch];
    int nq_max = 0;
    for (int b = 0; b < batch; ++b) {
        p.len[b] = len[b];
        const int nq = p.window > 0 ? std::max(0, len[b] - p.window) : len[b];
        nq_max = std::max(nq_max, nq);
    }
    matrix = c->decode_path != 1 && mfma_path_supported(p);
    if (c->decode_path == 2 && !matrix) return KVQ_ERR_UNSUPPORTED;
    int st;
    if (c->split_tokens_opt > 0) {
        st = c->split_tokens_opt;
    } else if (matrix) {
        // one workgroup per compute unit across all (sequence, kv head) pairs, the FP32-window
        // workgroup included, so that no workgroup waits for a free compute unit
        const int per = std::max(1, c->num_cus / (p.Hkv * batch));
        const int target = std::max(1, per - (p.window > 0 ? kWinSplitsMatrix : 0));
        st = (int)ceil_to((size_t)std::max(1, (nq_max + target - 1) / target), 64);
        st = std::max(st, 128);
    } else {
        const int target = std::max(1, (2 * c->num_cus + p.Hkv * batch - 1) / (p.Hkv * batch));
        st = (int)ceil_to((size_t)std::max(1, (nq_max + target - 1) / target), 64);
        st = std::max(st, 256);
    }
    const int nwin = p.window > 0 ? (matrix ? kWinSplitsMatrix : 1) : 0;
    const int max_code_splits = kMaxSplits - nwin;
    int ns = std::max(1, (nq_max + st - 1) / st);
    if (ns > max_code_splits) {
        st = (int)ceil_to((size_t)((nq_max + max_code_splits - 1) / max_code_splits), 64);
        ns = std::max(1, (nq_max + st - 1) / st);
    }
    p.split_tokens = st;
    p.n_splits = ns;
    p.n_win_splits = nwin;
    p.n_splits_total = ns + nwin;
    return KVQ_OK;
}

hipError_t launch_decode(const kvq_cache* c, const DecodeParams& p, bool matrix, hipStream_t s) {
    hipError_t e = matrix ? launch_decode_mfma(p, s, c->ev[0], c->ev[1])
                          : launch_decode_vec(p, s, c->ev[0], c->ev[1]);
    if (e == hipSuccess) e = launch_decode_merge(p, s);
    return e;
}

} // namespace

kvq_status kvq_prefill_quantize(kvq_cache* c, int layer, const void* K, const void* V, int dtype,
                                int n_tokens, int batch, void* stream) {
    QuantParams p;
    const kvq_status st = make_quant(c, layer, K, V, dtype, n_tokens, batch, p);
    if (st != KVQ_OK || n_tokens == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = n_tokens >= kQuantBulkMinTokens ? launch_quantize_bulk(p, s) : launch_quantize(p, s);
    if (e != hipSuccess) return dev_fail(c, e);
    int* len = &c->len[(size_t)layer * c->cfg.max_batch];
    for (int b = 0; b < batch; ++b) len[b] += n_tokens;
    return KVQ_OK;
}

kvq_status kvq_append(kvq_cache* c, int layer, const void* k, const void* v, int dtype, int batch,
                      void* stream) {
    return kvq_prefill_quantize(c, layer, k, v, dtype, 1, batch, stream);
}

kvq_status kvq_attn_decode(kvq_cache* c, int layer, const void* q, int dtype, float* out, int batch,
                           float softmax_scale, void* stream) {
    kvq_status st = check_decode(c, layer, q, dtype, out, batch, softmax_scale);
    if (st != KVQ_OK) return st;
    DecodeParams p;
    bool matrix = false;
    st = make_decode(c, layer, q, dtype, out, batch, softmax_scale, p, matrix);
    if (st != KVQ_OK) return st;
    const hipError_t e = launch_decode(c, p, matrix, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return dev_fail(c, e);
    return KVQ_OK;
}

kvq_status kvq_attn_decode_static(kvq_cache* c, int layer, const void* q, int dtype, float* out, int batch,
                                  float softmax_scale, void* stream) {
    kvq_status st = check_decode(c, layer, q, dtype, out, batch, softmax_scale);
    if (st != KVQ_OK) return st;
    DecodeParams p;
    bool matrix = false;
    st = make_decode(c, layer, q, dtype, out, batch, softmax_scale, p, matrix);
    if (st != KVQ_OK) return st;
    const size_t need = (size_t)batch * p.Hq * p.n_splits_total * kPartialFloats * sizeof(float);
    if (need > kStaticScratchBytes) return KVQ_ERR_SCRATCH;
    float* ptr = static_scratch(c->device);
    if (!ptr) return dev_fail(c, hipErrorNotInitialized);
    p.partials = ptr; // every split writes its partial before the merge reads it: nothing to clear
    const hipError_t e = launch_decode(c, p, matrix, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return dev_fail(c, e);
    return KVQ_OK;
}

kvq_status kvq_append_attn_decode(kvq_cache* c, int layer, const void* k, const void* v, const void* q,
                                  int dtype, float* out, int batch, float softmax_scale, void* stream) {
    QuantParams qp;
    kvq_status st = make_quant(c, layer, k, v, dtype, 1, batch, qp);
    if (st != KVQ_OK) return st;
    st = check_decode(c, layer, q, dtype, out, batch, softmax_scale);
    if (st != KVQ_OK) return st;
    // plan the decode over the lengths after the append; undone if the plan is refused
    int* len = &c->len[(size_t)layer * c->cfg.max_batch];
    for (int b = 0; b < batch; ++b) len[b] += 1;
    DecodeParams p;
    bool matrix = false;
    st = make_decode(c, layer, q, dtype, out, batch, softmax_scale, p, matrix);
    if (st != KVQ_OK) {
        for (int b = 0; b < batch; ++b) len[b] -= 1;
        return st;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (matrix) {
        p.fuse = 1;
        p.append = qp;
        e = launch_decode_mfma(p, s, c->ev[0], c->ev[1]);
        if (e != hipSuccess) { // nothing was enqueued: the append did not happen
            for (int b = 0; b < batch; ++b) len[b] -= 1;
            return dev_fail(c, e);
        }
        e = launch_decode_merge(p, s);
    } else {
        e = launch_quantize(qp, s);
        if (e != hipSuccess) { // nothing was enqueued: the append did not happen
            for (int b = 0; b < batch; ++b) len[b] -= 1;
            return dev_fail(c, e);
        }
        e = launch_decode(c, p, false, s);
    }
    if (e != hipSuccess) return dev_fail(c, e);
    return KVQ_OK;
}

namespace {

// Key splits per (query, head) row for a prefill-attention call.  A workgroup owns
// kPrefillRowsPerBlock rows of one (sequence, kv head) and streams its keys in 64-token chunks;
// with `base` workgroups per split, S splits take ceil(base S / CUs) rounds of ceil(chunks / S)
// chunks each, and every split adds one partial row (kPartialFloats floats) per row, written and
// read once by the merge.  The plan minimises that modelled time over S (at most `cap_bytes` of
// partials).
int prefill_splits(const kvq_cache* c, int n_q, int batch, int max_len, size_t cap_bytes) {
    const int G = c->cfg.n_q_heads / c->cfg.n_kv_heads;
    const long tiles = (static_cast<long>(n_q) * G + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock;
    const long base = tiles * c->cfg.n_kv_heads * batch;
    const long chunks = (max_len + 63) / 64;
    const double rows = static_cast<double>(batch) * n_q * c->cfg.n_q_heads;
    const double chunk_s = 3.4e-6, merge_launch_s = 4e-6, hbm_Bps = 4e12; // measured on MI355X
    const long cus = std::max(1, c->num_cus);
    int best = 1;
    double best_t = 0.0;
    for (int S = 1; S <= 64 && S <= chunks; ++S) {
        const double bytes = rows * S * kPartialFloats * sizeof(float);
        if (S > 1 && bytes > static_cast<double>(cap_bytes)) break;
        const long rounds = (base * S + cus - 1) / cus;
        double t = static_cast<double>(rounds) * ((chunks + S - 1) / S) * chunk_s;
        if (S > 1) t += merge_launch_s + 2.0 * bytes / hbm_Bps;
        if (S == 1 || t < 0.97 * best_t) {
            best = S;
            best_t = t;
        }
    }
    return best;
}

// Workspace bytes ahead of the partials: the window mapped into the code domain, if the planes
// need it (256-byte aligned, so the partials stay aligned).
size_t prefill_window_area(const kvq_cache* c, int batch) {
    return window_in_code_domain(c->plan.geom[0], c->plan.geom[1], c->cfg.fp32_window)
               ? align_up(prefill_window_bytes(batch, c->cfg.n_kv_heads))
               : 0;
}

kvq_status check_prefill(const kvq_cache* c, int layer, int n_q, int batch, int* max_len) {
    if (!c || layer < 0 || layer >= c->cfg.n_layers || batch < 1 || batch > c->cfg.max_batch || n_q < 1)
        return KVQ_ERR_INVALID_ARG;
    const int* len = &c->len[(size_t)layer * c->cfg.max_batch];
    int mx = 0;
    for (int b = 0; b < batch; ++b) {
        if (n_q > len[b]) return KVQ_ERR_INVALID_ARG;
        mx = std::max(mx, len[b]);
    }
    *max_len = mx;
    return KVQ_OK;
}

} // namespace

kvq_status kvq_attn_prefill_workspace(const kvq_cache* c, int layer, int n_q, int batch, size_t* bytes) {
    int max_len = 0;
    const kvq_status st = check_prefill(c, layer, n_q, batch, &max_len);
    if (st != KVQ_OK) return st;
    if (!bytes) return KVQ_ERR_INVALID_ARG;
    const int S = prefill_splits(c, n_q, batch, max_len, static_cast<size_t>(-1));
    *bytes = prefill_window_area(c, batch) +
             (S > 1 ? (size_t)batch * n_q * c->cfg.n_q_heads * S * kPartialFloats * sizeof(float) : 0);
    return KVQ_OK;
}

kvq_status kvq_attn_prefill(kvq_cache* c, int layer, const void* q, int dtype, float* out, int n_q,
                            int batch, float softmax_scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
    kvq_status st = check_decode(c, layer, q, dtype, out, batch, softmax_scale);
    if (st != KVQ_OK) return st;
    int max_len = 0;
    st = check_prefill(c, layer, n_q, batch, &max_len);
    if (st != KVQ_OK) return st;
    if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return KVQ_ERR_MISALIGNED;
    PrefillParams p{};
    p.q = q;
    p.out = out;
    fill_params_common(c, layer, p.layer_base, p.seq_stride, p.head_stride, p.plane_off, p.geom);
    p.signs = c->signs() + c->table_off(layer);
    p.cs = c->cs() + c->table_off(layer);
    p.inv_c = c->inv_c() + c->table_off(layer);
    p.qjl_st = c->ST();
    p.mu = c->mu();
    p.mu16 = c->mu16();
    p.perm = c->perm() + c->perm_off(layer);
    p.perm_k = c->perm_k() + c->perm_off(layer);
    p.mu64 = c->mu64();
    p.dtype = dtype;
    p.batch = batch;
    p.n_q = n_q;
    p.Hq = c->cfg.n_q_heads;
    p.Hkv = c->cfg.n_kv_heads;
    p.G = p.Hq / p.Hkv;
    p.window = c->cfg.fp32_window;
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(128.0f);
    p.qscale = scale * 1.4426950408889634f;
    const int* len = &c->len[(size_t)layer * c->cfg.max_batch];
    for (int b = 0; b < batch; ++b) p.len[b] = len[b];
    if (!prefill_attn_supported(p)) return KVQ_ERR_UNSUPPORTED;
    // workspace: [mapped window (if any)][partials]
    char* ws = workspace ? static_cast<char*>(workspace) : c->base + c->plan.off_work;
    const size_t ws_bytes = workspace ? workspace_bytes : c->plan.work_bytes;
    const size_t win = prefill_window_area(c, batch);
    if (ws_bytes < win) return KVQ_ERR_BUFFER_TOO_SMALL;
    p.wring = win ? reinterpret_cast<float*>(ws) : nullptr;
    p.partials = reinterpret_cast<float*>(ws + win);
    p.n_splits = prefill_splits(c, n_q, batch, max_len, ws_bytes - win);
    const hipError_t e = launch_prefill_attn(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return dev_fail(c, e);
    return KVQ_OK;
}

kvq_status kvq_get_layout(const kvq_cache* c, int layer, int seq, int kv_head, int tensor,
                          kvq_layout* out) {
    if (!c || !out) return KVQ_ERR_INVALID_ARG;
    if (layer < 0 || layer >= c->cfg.n_layers || seq < 0 || seq >= c->cfg.max_batch ||
        kv_head < 0 || kv_head >= c->cfg.n_kv_heads || (tensor != 0 && tensor != 1))
        return KVQ_ERR_INVALID_ARG;
    char* slot = c->layer_base(layer) + (size_t)seq * c->cfg.n_kv_heads * c->plan.slot_bytes +
                 (size_t)kv_head * c->plan.slot_bytes + (tensor ? c->plan.plane_bytes[0] : 0);
    const PlaneGeom& g = c->plan.geom[tensor];
    out->codes = slot + g.codes_off;
    out->meta = slot + g.meta_off;
    out->qjl = g.qjl_bytes ? slot + g.qjl_off : nullptr;
    out->window = g.ring_bytes ? slot + g.ring_off : nullptr;
    out->codes_bytes = g.codes_bytes;
    out->meta_bytes = g.meta_bytes;
    out->qjl_bytes = g.qjl_bytes;
    out->window_bytes = g.ring_bytes;
    out->length = c->len[(size_t)layer * c->cfg.max_batch + seq];
    return KVQ_OK;
}

kvq_status kvq_get_tables(const kvq_cache* c, kvq_tables* out) {
    if (!c || !out) return KVQ_ERR_INVALID_ARG;
    out->signs = c->signs();
    out->c = c->cs();
    out->inv_c = c->inv_c();
    out->qjl_S = c->S();
    out->mu = c->mu();
    out->theta = c->theta();
    out->mu16 = c->mu16();
    out->theta16 = c->theta16();
    out->perm = c->perm();
    out->perm_k = c->perm_k();
    out->mu64 = c->mu64();
    out->theta64 = c->theta64();
    return KVQ_OK;
}

kvq_status kvq_set_option(kvq_cache* c, int option, int value) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    switch (option) {
    case KVQ_OPT_SPLIT_TOKENS:
        if (value < 0 || value % 64 != 0) return KVQ_ERR_INVALID_ARG;
        c->split_tokens_opt = value;
        return KVQ_OK;
    case KVQ_OPT_DECODE_PATH:
        if (value < 0 || value > 2) return KVQ_ERR_INVALID_ARG;
        c->decode_path = value;
        return KVQ_OK;
    default:
        return KVQ_ERR_INVALID_ARG;
    }
}

kvq_status kvq_set_timing_events(kvq_cache* c, void* ev_start, void* ev_stop) {
    if (!c || (!ev_start) != (!ev_stop)) return KVQ_ERR_INVALID_ARG;
    c->ev[0] = static_cast<hipEvent_t>(ev_start);
    c->ev[1] = static_cast<hipEvent_t>(ev_stop);
    return KVQ_OK;
}

int kvq_get_length(const kvq_cache* c, int layer, int seq) {
    if (!c || layer < 0 || layer >= c->cfg.n_layers || seq < 0 || seq >= c->cfg.max_batch) return -1;
    return c->len[(size_t)layer * c->cfg.max_batch + seq];
}

const char* kvq_status_str(kvq_status s) {
    switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "context capacity exceeded";
    case KVQ_ERR_NOT_READY: return "tables not set or layer not calibrated";
    case KVQ_ERR_BUFFER_TOO_SMALL: return "device buffer too small";
    case KVQ_ERR_MISALIGNED: return "misaligned pointer";
    case KVQ_ERR_HOST_ALLOC: return "host allocation failed";
    case KVQ_ERR_DEVICE: return "HIP error";
    case KVQ_ERR_SCRATCH: return "decode partials exceed the library's static scratch";
    }
    return "unknown status";
}

int kvq_last_hip_error(const kvq_cache* c) { return c ? c->last_hip_error : 0; }

} // extern "C"
