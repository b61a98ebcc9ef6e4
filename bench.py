"""Decode-step benchmark of the compressed-KV path on one MI355X.

One step = for every layer: kvq_append of the new token's K and V (rotation, Sinkhorn fold,
4-bit group quantization) then kvq_attn_decode of the new query over the whole cache.  Inputs are
seeded synthetic tensors of the workload's shape, generated on the device before timing.

Prints one JSON line: queries/s (one query = one (sequence, layer) decode attention over all
query heads), ms per step, the split-K decode kernel's achieved HBM bandwidth against the 8 TB/s
MI355X peak (algorithmic compressed bytes / the kernel's average duration, from HIP events bound
to that kernel's dispatch on the launch stream inside the timed region; the time of one layer's
append + decode + merge is reported beside it), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "decode-attn queries/s + achieved HBM GB/s (% peak) at 32K/128K, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak (no sparsity)


def token_head_bytes(scheme, bits):
    """Compressed bytes per token-head read by decode (codes + scale/zero or norms + QJL bits)."""
    if not W.is_turbo(scheme):
        return 16 * bits + 16
    if scheme == W.TURBO_QJL:
        return 48 + 4 + 16
    if scheme == W.TURBO_SPLIT:
        return 8 * (2 * bits - 1) + 4  # bits + (bits - 1) planes of 8 B + two fp16 norms
    return 16 * bits + 2  # TurboQuant-MSE: b bit planes + fp16 norm


def query_bytes(wl: W.Workload, n: int) -> int:
    """Algorithmic HBM bytes of one (sequence, layer) decode query at context n."""
    W_ = wl.window
    nq = max(0, n - W_) if W_ else n
    nw = n - nq
    per = token_head_bytes(wl.k_scheme, wl.k_bits) + token_head_bytes(wl.v_scheme, wl.v_bits)
    return wl.n_kv_heads * (nq * per + nw * 2 * 512)


def step_driver(cache, wl: W.Workload, step_in, qs, out, stream, fused=True):
    """run(n, events=None): n decode steps (append + decode for every layer) issued by the native
    loop in libkvq_bench.so through the C ABI (kvq_append_attn_decode per layer when fused, else
    kvq_append then kvq_attn_decode); inputs cycle through the pool."""
    import ctypes

    import quantized_decode_attention_kvq_amd as K
    lib = ctypes.CDLL(os.path.join(os.path.dirname(K.__file__), "libkvq_bench.so"))
    fn = lib.kvq_bench_steps
    vp = ctypes.c_void_p
    fn.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, ctypes.c_int,
                   ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    fn.restype = ctypes.c_int
    L, pool = wl.n_layers, len(step_in)
    arr = lambda xs: (vp * len(xs))(*[vp(x) for x in xs])  # noqa: E731
    kp = arr([step_in[s][l][0].data_ptr() for s in range(pool) for l in range(L)])
    vptr = arr([step_in[s][l][1].data_ptr() for s in range(pool) for l in range(L)])
    qp = arr([qs[s][l].data_ptr() for s in range(pool) for l in range(L)])
    op = arr([out[l].data_ptr() for l in range(L)])
    dtype = 1 if qs[0][0].dtype == torch.bfloat16 else 0

    def run(n, events=None):
        e0 = e1 = None
        if events is not None:
            e0 = arr([pair[0].cuda_event for pair in events])
            e1 = arr([pair[1].cuda_event for pair in events])
        where = ctypes.c_int(-1)
        st = fn(cache.handle, L, n, pool, kp, vptr, qp, op, dtype, wl.batch, vp(stream.cuda_stream),
                e0, e1, int(fused), ctypes.byref(where))
        if st != 0:
            raise RuntimeError(f"kvq_bench_steps failed with status {st} at call {where.value}")

    return run


# The sources the split-K decode kernel is compiled from (its unit and the headers it includes).
DECODE_SOURCES = ["kvq_decode_mfma.hip", "kvq_internal.h", "kvq_lanes.h", "kvq_mfma_ops.h", "kvq_quant_dev.h"]


def decode_source_sha() -> str:
    """sha256 over the decode kernel's sources, concatenated in DECODE_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "quantized_decode_attention_kvq_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record(wl: W.Workload):
    """HBM bytes per launch of the split-K kernel measured with rocprofv3 --pmc (FETCH_SIZE and
    WRITE_SIZE, scaled by the copy-probe factors) and recorded under profiles/, valid only while
    the kernel's sources have the recorded sha256 (decode_source_sha); None otherwise."""
    import glob
    sha = decode_source_sha()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if line.startswith("traffic_record "):
                rec = json.loads(line[len("traffic_record "):])
                if rec["workload"] == wl.name and rec.get("batch", 1) == wl.batch and \
                        rec["kernel_sha256"] == sha:
                    return rec
    return None


def prefill_report(wl: W.Workload, prefill_s):
    """Bulk kvq_prefill_quantize of the whole context, one call per layer (HIP events around
    each call on the launch stream): source bytes read + packed bytes written per second."""
    n, B = wl.context, wl.batch
    src = B * n * wl.n_kv_heads * 128 * 2 * (2 if wl.dtype == "bf16" else 4)
    per = token_head_bytes(wl.k_scheme, wl.k_bits) + token_head_bytes(wl.v_scheme, wl.v_bits)
    packed = B * wl.n_kv_heads * (n * per + min(n, wl.window) * 2 * 512)
    t = float(np.mean(prefill_s))
    return {"tokens_per_call": B * n, "calls": len(prefill_s), "us_per_call": 1e6 * t,
            "tokens_per_s": B * n / t, "bytes_per_call": src + packed,
            "achieved_GBps": (src + packed) / t / 1e9}


def split_kernel_name(wl: W.Workload) -> str:
    """The split-K decode kernel the library launches for this cache (matrix-core path)."""
    kind = lambda scheme, bits, t: ((f"Sk{bits}" if t == 0 else f"Ts{bits}") if scheme == W.TURBO_SPLIT else  # noqa: E731
                                    ("Tb4" if bits == 4 else "Tb") if W.is_turbo(scheme) else f"U{bits}")
    return (f"decode_mfma_kernel (K {kind(wl.k_scheme, wl.k_bits, 0)}, V {kind(wl.v_scheme, wl.v_bits, 1)}, "
            f"{wl.group} query heads per kv head)")


def build_cache(wl: W.Workload, extra: int, log, keep_first: bool = True):
    import quantized_decode_attention_kvq_amd as K
    cfg = wl.kvq_config(max_context=wl.context + extra)
    cache = K.KvCache(device="cuda", **cfg)
    signs = torch.from_numpy(np.ascontiguousarray(W.rotation_signs(wl))).cuda()
    S = torch.from_numpy(W.qjl_projection(wl)).cuda()
    cache.set_random_tables(signs, S)
    keep = None
    stream = torch.cuda.current_stream()
    pre = []  # (start, end) events around each layer's bulk prefill on the launch stream
    for layer in range(wl.n_layers):
        if wl.sinkhorn_iters > 0 or wl.v_scheme == W.TURBO_SPLIT or wl.k_scheme == W.TURBO_SPLIT:
            cache.calibrate(layer, W.gen_calib(wl, layer, 0, device="cuda"),
                            W.gen_calib(wl, layer, 1, device="cuda"))
        k = W.gen_kv(wl, layer, 0, device="cuda")
        v = W.gen_kv(wl, layer, 1, device="cuda")
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record(stream)
        cache.prefill_quantize(layer, k, v)
        ev[1].record(stream)
        pre.append(ev)
        if layer == 0 and keep_first:
            keep = (k[:1].cpu(), v[:1].cpu())
        del k, v
        if layer % 8 == 7:
            log(f"prefilled {layer + 1}/{wl.n_layers} layers")
    torch.cuda.synchronize()
    prefill_s = np.array([a.elapsed_time(b) for a, b in pre]) / 1e3
    return cache, keep, prefill_s


def _cpu_share():
    """Host threads this process may use: its CPU affinity, capped at the 16 cores a one-GPU machine
    grants a job."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl: W.Workload, kv0, budget_s: float):
    """The oracle (plain C, fp64 attention) on a bounded sample of the same workload: layer 0 /
    sequence 0, every kv head at the full context.

    - quantize: building the oracle's planes (rotation, balancing, group codes, packing) of the
      sample, on one thread for two token-head streams and on all host threads for all of them;
      source fp32 bytes per second;
    - decode: full decode queries (all kv heads) on one thread, then on all host threads (one kv
      head of one query per task; ctypes releases the interpreter lock inside the C calls)."""
    import concurrent.futures as cf

    import oracle
    k0, v0 = (t[0].float().numpy() for t in kv0)  # [n][Hkv][128]
    n = k0.shape[0]
    signs = W.rotation_signs(wl)[0]
    S = W.qjl_projection(wl)
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    threads = _cpu_share()

    def tables(h, tensor):
        scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
        bits = wl.k_bits if tensor == 0 else wl.v_bits
        rot = (wl.rotate_k if tensor == 0 else wl.rotate_v) or W.is_turbo(scheme)
        sink = wl.sinkhorn_iters > 0 and not W.is_turbo(scheme)
        kw = dict(mu=mu, theta=theta, S=S)
        if rot:
            kw["signs"] = signs[h, tensor]
        if sink:
            cal = W.gen_calib(wl, 0, tensor)[:, h].float().numpy()
            kw["c"], kw["inv_c"] = oracle.sinkhorn(cal, kw.get("signs"), wl.sinkhorn_iters)
        if scheme == W.TURBO_SPLIT:
            kw["perm"] = oracle.select_outliers(W.gen_calib(wl, 0, 1)[:, h].float().numpy())
            _, kw["mu"], kw["theta"], _ = oracle.lloyd_max(oracle.LLOYD_ITERS, 1 << bits, 64)
            _, kw["mu2"], kw["theta2"], _ = oracle.lloyd_max(oracle.LLOYD_ITERS, 1 << (bits - 1), 64)
        return oracle.TableSet(**kw), scheme, bits, rot, sink

    units = [(h, tensor) for h in range(wl.n_kv_heads) for tensor in (0, 1)]
    tabs = {u: tables(*u) for u in units}

    def build(u):
        h, tensor = u
        tb, scheme, bits, rot, sink = tabs[u]
        p = oracle.Plane(scheme, bits, rot, sink, wl.window, tensor, n)
        p.append((k0 if tensor == 0 else v0)[:, h], tb)
        return p

    src_bytes = n * 128 * 4  # one token-head stream of fp32 source
    t0 = time.perf_counter()
    for u in units[:2]:
        build(u)
    q1 = 2 * src_bytes / (time.perf_counter() - t0)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        built = dict(zip(units, ex.map(build, units)))
    qall = len(units) * src_bytes / (time.perf_counter() - t0)
    planes = [(built[(h, 0)], tabs[(h, 0)][0], built[(h, 1)], tabs[(h, 1)][0]) for h in range(wl.n_kv_heads)]

    q = W.gen_q(wl, 0, 0)[0].float().numpy()
    G = wl.group

    def head(h):
        pk, tk, pv, tv = planes[h]
        oracle.attention(pk, pv, tk, tv, q[h * G:(h + 1) * G])

    half = budget_s / 2
    n1 = 0
    t0 = time.perf_counter()
    while True:
        for h in range(wl.n_kv_heads):
            head(h)
        n1 += 1
        if time.perf_counter() - t0 > half:
            break
    dt1 = time.perf_counter() - t0
    nall = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        while time.perf_counter() - t0 <= half:
            list(ex.map(head, [h for _ in range(threads) for h in range(wl.n_kv_heads)]))
            nall += threads
    dtall = time.perf_counter() - t0
    qb = query_bytes(wl, n)
    return {"value": n1 / dt1, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0, sequence 0, {n} tokens, all {wl.n_kv_heads} kv heads x {G} query "
                      f"heads; {n1} full decode queries in {dt1:.1f} s on one thread (fp64 attention "
                      f"over the oracle's own planes; plane building timed separately)",
            "compressed_GBps": n1 / dt1 * qb / 1e9,
            "all_cores": {"value": nall / dtall, "unit": "queries/s", "cores": threads,
                          "nproc": os.cpu_count(), "compressed_GBps": nall / dtall * qb / 1e9,
                          "sample": f"{nall} queries in {dtall:.1f} s, one kv head per task"},
            "quantize": {"GBps_1_core": q1 / 1e9, "GBps_all_cores": qall / 1e9, "cores": threads,
                         "unit": "GB/s of fp32 source",
                         "sample": f"oracle planes of layer 0 / sequence 0: 2 of the {len(units)} "
                                   f"token-head streams ({n} tokens each) on one thread, all "
                                   f"{len(units)} on {threads} threads"}}


def copy_probe():
    """Three plain device copies of exactly 1 GiB: the reference for scaling rocprofv3's
    FETCH_SIZE / WRITE_SIZE counters to HBM bytes."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": "torch copy_", "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "launches": 3}), flush=True)


def copy_bandwidth():
    """Device-to-device copy rate on this machine (read + written bytes / time, three 1 GiB copies
    after one warm-up): what a plain streaming kernel reaches here, beside the 8 TB/s peak."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 3 * 2 * 4 * n / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def prefill_attention_report(cache, wl: W.Workload, n_q: int = 512, reps: int = 5):
    """kvq_attn_prefill of an n_q-token chunk at the end of layer 0's cache (the chunk's queries
    see the cache up to their own positions), timed with events on the launch stream.  Bound:
    the fp16 matrix cores; algorithmic flops = 4 * 128 * Hq * sum_i (visible tokens of query i)
    per sequence (QK^T and PV, multiply-adds counted as two)."""
    import quantized_decode_attention_kvq_amd as K
    B = wl.batch
    n = cache.length(0)
    if n < n_q:
        return None
    g = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn((B, n_q, wl.n_q_heads, 128), generator=g, device="cuda")
    if wl.dtype == "bf16":
        q = q.to(torch.bfloat16)
    out = torch.empty((B, n_q, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    try:
        ws_bytes = cache.attn_prefill_workspace(0, n_q, B)
        cache.attn_prefill(0, q, out)
    except K.KvqError as e:
        return {"supported": False, "status": e.name}
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        cache.attn_prefill(0, q, out)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    visible = sum(n - n_q + i + 1 for i in range(n_q))
    flops = 4.0 * 128 * wl.n_q_heads * visible * B
    tflops = flops / sec / 1e12
    return {"supported": True, "n_q": n_q, "context": n, "us_per_call": 1e6 * sec,
            "workspace_bytes": ws_bytes,
            "query_tokens_per_s": B * n_q / sec,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / MFMA_F16_PEAK_TFLOPS,
                         "flops_per_call": flops}}


def measure(wl: W.Workload, cache, prefill_s, steps: int, warmup: int, fused: bool = True):
    """Decode steps over a built cache: `warmup` untimed steps, then `steps` timed steps (events
    on the launch stream around them, nothing else inside), then the same steps again with
    events bound to each split-K dispatch for the kernel's own duration."""
    L, B = wl.n_layers, wl.batch
    pool = 4
    step_in = [[W.gen_step_kv(wl, layer, s, device="cuda") for layer in range(L)] for s in range(pool)]
    qs = [[W.gen_q(wl, layer, s, device="cuda") for layer in range(L)] for s in range(pool)]
    out = torch.empty((L, B, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    run = step_driver(cache, wl, step_in, qs, out, stream, fused=fused)

    run(warmup)
    torch.cuda.synchronize()
    n_start = cache.length(0)
    # timed region: `steps` decode steps, nothing but the library's own launches inside
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record(stream)
    run(steps)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    elapsed = t0.elapsed_time(t1) / 1e3
    # kernel pass: the same steps again with start / stop events bound by the library to each
    # split-K kernel's own dispatch on the launch stream (each recorded once here so it exists)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps * L)]
    for pair in evs:
        for e in pair:
            e.record(stream)
    torch.cuda.synchronize()
    run(steps, evs)
    torch.cuda.synchronize()
    split = np.array([pair[0].elapsed_time(pair[1]) for pair in evs]) / 1e3
    assert torch.isfinite(out).all()

    queries = L * B * steps
    qps = queries / elapsed
    n_mean = 0.5 * (n_start + 1 + cache.length(0))  # mean context over both passes
    bytes_per_launch = B * query_bytes(wl, int(round(n_mean)))
    split_mean = float(split.mean())
    achieved = bytes_per_launch / split_mean / 1e9
    rec = traffic_record(wl)
    traffic = None if rec is None else rec["fetch_bytes"] + rec["write_bytes"]
    return {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": 1e3 * elapsed / steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "batch": B, "context": wl.context,
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "k_cache": [wl.k_scheme, wl.k_bits, bool(wl.rotate_k)],
                   "v_cache": [wl.v_scheme, wl.v_bits, bool(wl.rotate_v)],
                   "fp32_window": wl.window, "sinkhorn_iters": wl.sinkhorn_iters,
                   "source_dtype": wl.dtype,
                   "step": ("kvq_append_attn_decode" if fused
                            else "kvq_append + kvq_attn_decode") + " per layer"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_unit": "bytes/launch",
                     "traffic_vs_algorithmic": None if traffic is None else traffic / bytes_per_launch,
                     "kernel": split_kernel_name(wl),
                     "bytes_per_launch": bytes_per_launch, "avg_launch_us": 1e6 * split_mean,
                     "p10_us": 1e6 * float(np.percentile(split, 10)),
                     "p90_us": 1e6 * float(np.percentile(split, 90)),
                     "layer_step_us": 1e6 * elapsed / (steps * L),
                     "step_GBps": B * query_bytes(wl, int(round(n_mean))) * L * steps / elapsed / 1e9},
        "wall_s": wall,
        "prefill": prefill_report(wl, prefill_s),
    }


# The other half of the metric: the long-context workloads, each measured on its own cache (built,
# measured, freed) after the headline, in the same JSON line.
LONG_CONTEXT = [W.LLAMA3B_128K_PROGRESSIVE, W.LLAMA3B_128K_PROGRESSIVE.with_(batch=8),
                W.DENSE27B_120K_KVARN, W.DENSE27B_120K_U8]
# The other 32K caches: the TurboQuant cache (QJL keys, 4-bit values) and its asymmetric variants
# (8-bit keys with TurboQuant-MSE or uniform 3-bit values), and the whole cache at 2.5 / 3.5 bits
# by the outlier split on both tensors.
OTHER_32K = [W.LLAMA3B_32K_TURBO, W.LLAMA3B_32K_TURBO_ASYM, W.LLAMA3B_32K_U8_K_U3_V,
             W.LLAMA8B_32K_TURBO25_KV, W.LLAMA8B_32K_TURBO35_KV]


def gpu_info():
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2**30, 1)}
    arch = getattr(p, "gcnArchName", None)
    if arch:
        info["arch"] = arch
    return info


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.LLAMA3B_32K_KVARN.name, choices=sorted(W.BY_NAME))
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true",
                    help="only the headline workload (skip the 128K / 120K and other 32K lines)")
    ap.add_argument("--separate", action="store_true",
                    help="kvq_append + kvq_attn_decode per layer instead of kvq_append_attn_decode")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device-to-device (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no cross-GPU step in this build "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    if args.copy_probe:
        copy_probe()
        return
    import quantized_decode_attention_kvq_amd  # noqa: F401  (fails loudly without libkvq.so)
    wl = W.BY_NAME[args.workload]
    if args.batch:
        wl = wl.with_(batch=args.batch)
    torch.cuda.init()
    log(f"workload {wl.name}: building cache")
    t_build = time.perf_counter()
    cache, kv0, prefill_s = build_cache(wl, args.warmup + 2 * args.steps, log)
    log(f"cache built in {time.perf_counter() - t_build:.1f} s")

    res = measure(wl, cache, prefill_s, args.steps, args.warmup, not args.separate)
    res["prefill_attention"] = prefill_attention_report(cache, wl)
    res["gpu"] = gpu_info()
    res["gpu"]["copy_GBps"] = copy_bandwidth()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(wl, kv0, args.cpu_budget)
    if not args.no_long_context and args.workload == W.LLAMA3B_32K_KVARN.name and not args.batch:
        del cache, kv0
        torch.cuda.empty_cache()
        res["long_context"] = []
        res["other_32k"] = []
        for lwl in LONG_CONTEXT + OTHER_32K:
            st, wu = min(args.steps, 20), min(args.warmup, 3)
            log(f"workload {lwl.name} batch {lwl.batch}: building cache")
            lcache, _, lpre = build_cache(lwl, wu + 2 * st, log, keep_first=False)
            r = measure(lwl, lcache, lpre, st, wu, not args.separate)
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data"):
                r.pop(k)
            res["long_context" if lwl in LONG_CONTEXT else "other_32k"].append(r)
            log(f"  {lwl.name} B{lwl.batch}: {r['value']:.0f} queries/s, {r['ms_per_step']:.3f} ms/step, "
                f"split-K {r['roofline']['avg_launch_us']:.1f} us = {r['roofline']['frac']:.3f} of peak")
            del lcache
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
