// Native driver of the decode-step loop used by bench.py: the same C ABI calls a serving loop
// makes per generated token (kvq_append then kvq_attn_decode for every layer), issued from C++ so
// that host-side call overhead of the interpreter does not starve the GPU.  Part of the
// measurement harness, not of libkvq's ABI.
#include "kvq.h"

extern "C" {

// steps x layers: kvq_append(layer, k[s % pool][layer], v[...]) then kvq_attn_decode(layer,
// q[s % pool][layer], out[layer]), or the same as one kvq_append_attn_decode call when `fused`.
// Inputs are [pool][n_layers] arrays of device pointers.  When ev_start / ev_stop are non-NULL ([steps][n_layers] hipEvent_t handles) each decode call's
// split-K kernel is timed with the pair (kvq_set_timing_events).  Returns the first non-OK status
// (with the failing step * n_layers + layer in *where), else KVQ_OK.
int kvq_bench_steps(kvq_cache* cache, int n_layers, int steps, int pool, const void* const* k,
                    const void* const* v, const void* const* q, float* const* out, int dtype,
                    int batch, void* stream, void* const* ev_start, void* const* ev_stop,
                    int fused, int* where) {
    if (!cache || n_layers <= 0 || steps < 0 || pool <= 0 || !k || !v || !q || !out || !where)
        return KVQ_ERR_INVALID_ARG;
    for (int s = 0; s < steps; ++s) {
        for (int layer = 0; layer < n_layers; ++layer) {
            const int i = (s % pool) * n_layers + layer;
            *where = s * n_layers + layer;
            kvq_status st = KVQ_OK;
            if (ev_start && ev_stop) {
                const int e = s * n_layers + layer;
                st = kvq_set_timing_events(cache, ev_start[e], ev_stop[e]);
                if (st != KVQ_OK) return st;
            }
            if (fused) {
                st = kvq_append_attn_decode(cache, layer, k[i], v[i], q[i], dtype, out[layer], batch,
                                            0.0f, stream);
            } else {
                st = kvq_append(cache, layer, k[i], v[i], dtype, batch, stream);
                if (st == KVQ_OK)
                    st = kvq_attn_decode(cache, layer, q[i], dtype, out[layer], batch, 0.0f, stream);
            }
            if (st != KVQ_OK) return st;
        }
    }
    if (ev_start && ev_stop) return kvq_set_timing_events(cache, nullptr, nullptr);
    return KVQ_OK;
}

} // extern "C"
