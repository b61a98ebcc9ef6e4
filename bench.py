"""Decode-step benchmark of the compressed-KV path on one MI355X.

One step = for every layer: kvq_append of the new token's K and V (rotation, Sinkhorn fold,
4-bit group quantization) then kvq_attn_decode of the new query over the whole cache.  Inputs are
seeded synthetic tensors of the workload's shape, generated on the device before timing.

Prints one JSON line: queries/s (one query = one (sequence, layer) decode attention over all
query heads), ms per step, the decode kernel's achieved HBM bandwidth against the 8 TB/s MI355X
peak (algorithmic compressed bytes / average decode-call duration from HIP events recorded on
the launch stream inside the timed region), and the CPU oracle timed on a bounded sample.
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


def token_head_bytes(scheme, bits):
    """Compressed bytes per token-head read by decode (codes + scale/zero or norms + QJL bits)."""
    if scheme == W.UNIFORM:
        return 16 * bits + 16
    if scheme == W.TURBO_QJL:
        return 48 + 4 + 16
    return 48 + 2


def query_bytes(wl: W.Workload, n: int) -> int:
    """Algorithmic HBM bytes of one (sequence, layer) decode query at context n."""
    W_ = wl.window
    nq = max(0, n - W_) if W_ else n
    nw = n - nq
    per = token_head_bytes(wl.k_scheme, wl.k_bits) + token_head_bytes(wl.v_scheme, wl.v_bits)
    return wl.n_kv_heads * (nq * per + nw * 2 * 512)


def build_cache(wl: W.Workload, extra: int, log):
    import quantized_decode_attention_kvq_amd as K
    cfg = wl.kvq_config(max_context=wl.context + extra)
    cache = K.KvCache(device="cuda", **cfg)
    signs = torch.from_numpy(np.ascontiguousarray(W.rotation_signs(wl))).cuda()
    S = torch.from_numpy(W.qjl_projection(wl)).cuda()
    cache.set_random_tables(signs, S)
    keep = None
    for layer in range(wl.n_layers):
        if wl.sinkhorn_iters > 0:
            cache.calibrate(layer, W.gen_calib(wl, layer, 0, device="cuda"),
                            W.gen_calib(wl, layer, 1, device="cuda"))
        k = W.gen_kv(wl, layer, 0, device="cuda")
        v = W.gen_kv(wl, layer, 1, device="cuda")
        cache.prefill_quantize(layer, k, v)
        if layer == 0:
            keep = (k[:1].cpu(), v[:1].cpu())
        del k, v
        if layer % 8 == 7:
            log(f"prefilled {layer + 1}/{wl.n_layers} layers")
    torch.cuda.synchronize()
    return cache, keep


def cpu_baseline(wl: W.Workload, kv0, budget_s: float):
    """The oracle (single-threaded C) on a bounded sample: layer 0 / sequence 0 of the same
    workload, planes built once, then full decode queries timed until the budget is spent."""
    import oracle
    k0, v0 = (t[0].float().numpy() for t in kv0)  # [n][Hkv][128]
    signs = W.rotation_signs(wl)[0]
    S = W.qjl_projection(wl)
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    planes = []
    for h in range(wl.n_kv_heads):
        row = []
        for tensor, X in ((0, k0), (1, v0)):
            scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
            bits = wl.k_bits if tensor == 0 else wl.v_bits
            rot = (wl.rotate_k if tensor == 0 else wl.rotate_v) or scheme != W.UNIFORM
            sink = wl.sinkhorn_iters > 0 and scheme == W.UNIFORM
            kw = dict(mu=mu, theta=theta, S=S)
            if rot:
                kw["signs"] = signs[h, tensor]
            if sink:
                cal = W.gen_calib(wl, 0, tensor)[:, h].float().numpy()
                kw["c"], kw["inv_c"] = oracle.sinkhorn(cal, kw.get("signs"), wl.sinkhorn_iters)
            tb = oracle.TableSet(**kw)
            p = oracle.Plane(scheme, bits, rot, sink, wl.window, tensor, X.shape[0])
            p.append(X[:, h], tb)
            row += [p, tb]
        planes.append(row)
    q = W.gen_q(wl, 0, 0)[0].float().numpy()
    G = wl.group
    n_q = 0
    t0 = time.perf_counter()
    while True:
        for h in range(wl.n_kv_heads):
            pk, tk, pv, tv = planes[h]
            oracle.attention(pk, pv, tk, tv, q[h * G:(h + 1) * G])
        n_q += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n_q / dt, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0, sequence 0, {k0.shape[0]} tokens, all {wl.n_kv_heads} kv heads "
                      f"x {G} query heads; {n_q} full decode queries in {dt:.1f} s "
                      f"(fp64 attention over the oracle's own planes; plane building not timed)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.LLAMA3B_32K_KVARN.name, choices=sorted(W.BY_NAME))
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no cross-GPU step in this build "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    import quantized_decode_attention_kvq_amd  # noqa: F401  (fails loudly without libkvq.so)
    wl = W.BY_NAME[args.workload]
    if args.batch:
        wl = wl.with_(batch=args.batch)
    torch.cuda.init()
    total_steps = args.warmup + args.steps
    log(f"workload {wl.name}: building cache")
    t_build = time.perf_counter()
    cache, kv0 = build_cache(wl, total_steps, log)
    log(f"cache built in {time.perf_counter() - t_build:.1f} s")

    L, B = wl.n_layers, wl.batch
    pool = 4
    step_in = [[W.gen_step_kv(wl, layer, s, device="cuda") for layer in range(L)] for s in range(pool)]
    qs = [[W.gen_q(wl, layer, s, device="cuda") for layer in range(L)] for s in range(pool)]
    out = torch.empty((L, B, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(s, evs=None):
        for layer in range(L):
            k, v = step_in[s % pool][layer]
            cache.append(layer, k, v)
            if evs is not None:
                evs[2 * layer].record(stream)
            cache.attn_decode(layer, qs[s % pool][layer], out[layer])
            if evs is not None:
                evs[2 * layer + 1].record(stream)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    n_start = cache.length(0)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * L)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record(stream)
    for s in range(args.steps):
        step(args.warmup + s, evs[s])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    elapsed = t0.elapsed_time(t1) / 1e3
    dec = np.array([[e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(L)] for e in evs]) / 1e3
    n_end = cache.length(0)
    assert torch.isfinite(out).all()

    queries = L * B * args.steps
    qps = queries / elapsed
    n_mean = 0.5 * (n_start + 1 + n_end)
    bytes_per_launch = B * query_bytes(wl, int(round(n_mean)))
    dec_mean = float(dec.mean())
    achieved = bytes_per_launch / dec_mean / 1e9
    res = {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "batch": B, "context": wl.context,
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "k_cache": [wl.k_scheme, wl.k_bits, bool(wl.rotate_k)],
                   "v_cache": [wl.v_scheme, wl.v_bits, bool(wl.rotate_v)],
                   "fp32_window": wl.window, "sinkhorn_iters": wl.sinkhorn_iters,
                   "step": "append + decode per layer"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kvq_attn_decode (split-K + merge)",
                     "bytes_per_launch": bytes_per_launch, "avg_launch_us": 1e6 * dec_mean,
                     "p10_us": 1e6 * float(np.percentile(dec, 10)),
                     "p90_us": 1e6 * float(np.percentile(dec, 90))},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(wl, kv0, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
