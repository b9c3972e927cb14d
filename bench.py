#!/usr/bin/env python3
"""Benchmark of the INT8 paged decode-attention path on one MI355X.

One step = every layer of the workload, each layer being: kv_write of the step's new token
(quantize-on-write into the paged INT8 cache), decode_split (split-KV GQA attention over the
cache) and decode_merge (log-sum-exp merge).  Each layer has its own cache, so a step streams
the whole multi-layer cache from HBM (1.06 GiB of INT8 K/V at 32K context, far above the
256 MB Infinity Cache).  Inputs are seeded synthetic tensors with the workload's shapes and
value distribution, resident in HBM before the timed region.

Timing: the step is captured once into a HIP graph and replayed; HIP events bracket the
timed replays.  The decode_split kernel is also timed on its own stream with HIP events
around each launch (the host is made to run ahead of the GPU so that no host gap is
counted), which gives the roofline figure.  The BF16-cache variant of the same step runs
alongside for comparison, and the CPU oracle is timed on a bounded sample of the workload.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "INT8 paged decode-attn µs/step + achieved HBM GB/s (% of peak) at 32K ctx"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=3, help="workload id (3 = 32K context, 16 layers)")
    p.add_argument("--splits", type=int, default=0, help="split count (0 = the library's choice)")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's)")
    p.add_argument("--no-bf16", action="store_true", help="skip the BF16-cache comparison")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=12.0, help="CPU seconds for the oracle sample")
    p.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    return p.parse_args()


def algorithmic_bytes(lens, Hkv, D, dtype):
    """K and V bytes every step must read from HBM: codes + fp16 scales (INT8), or bf16 values."""
    per_token_head = (2 * D + 2 * (D // 32) * 2) if dtype == "int8" else 4 * D
    return int(np.sum(lens, dtype=np.int64)) * Hkv * per_token_head


class LayerState:
    pass


def prepare(cid, n_layers, dtypes, keep_host_layers):
    import torch

    import decode_attention_quantized_amd as K
    import workloads as W

    states = {d: [] for d in dtypes}
    host = []
    for li in range(n_layers):
        lay, t = W.make_layer_device(cid, li)
        cfg = lay.cfg
        pre = torch.from_numpy(lay.prefill_rows()).cuda()
        stp = torch.from_numpy(lay.step_rows()).cuda()
        slots = torch.from_numpy(lay.slots).cuda()
        k_new, v_new, slot_new = t["k"][stp].contiguous(), t["v"][stp].contiguous(), slots[stp].contiguous()
        k_pre, v_pre, slot_pre = t["k"][pre].contiguous(), t["v"][pre].contiguous(), slots[pre].contiguous()
        bt = torch.from_numpy(lay.block_tables).cuda()
        lens = torch.from_numpy(lay.context_lens).cuda()
        for d in dtypes:
            L = LayerState()
            L.cache = K.Cache(d, lay.num_blocks, cfg.num_kv_heads, cfg.head_dim).fill()
            K.write(L.cache, k_pre, v_pre, slot_pre)
            L.k_new, L.v_new, L.slot_new = k_new, v_new, slot_new
            L.q, L.bt, L.lens = t["q"], bt, lens
            L.out = torch.empty((lay.S, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
            L.lse = torch.empty((lay.S, cfg.num_q_heads), dtype=torch.float32, device="cuda")
            states[d].append(L)
        if li < keep_host_layers:
            host.append((lay, t["k"].view(torch.int16).cpu().numpy().view(np.uint16),
                         t["v"].view(torch.int16).cpu().numpy().view(np.uint16),
                         t["q"].view(torch.int16).cpu().numpy().view(np.uint16)))
        del t, k_pre, v_pre, slot_pre
        torch.cuda.synchronize()
        log(f"prepared layer {li + 1}/{n_layers}")
    return states, host, lay


def make_step(K, layers, S, Hq, mcl, ns, ws):
    def step():
        for L in layers:
            K.write(L.cache, L.k_new, L.v_new, L.slot_new)
            K.decode_partials(L.cache, L.q, L.bt, L.lens, mcl, ns, ws)
            K.decode_merge(L.cache, L.lens, mcl, S, Hq, ns, ws, L.out, L.lse)
    return step


def time_step(torch, step, steps, warmup, eager):
    """Average ms per step over `steps` timed repetitions (graph replay unless eager)."""
    if eager:
        run = step
    else:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run = graph.replay
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def sleep_cycles_for(torch, ms):
    """torch.cuda._sleep spin length that takes about `ms` milliseconds on this GPU."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1_000_000
    e0.record()
    torch.cuda._sleep(n)
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1), 1e-3) / n
    return int(ms / per)


def time_split_kernel(torch, K, layers, mcl, ns, ws, passes):
    """Average duration (us) of one decode_split launch, HIP events around each launch on the
    launch stream; a GPU-side spin lets the host enqueue a whole pass ahead of the GPU."""
    cycles = sleep_cycles_for(torch, 3.0)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
    durs = []
    for _ in range(passes):
        torch.cuda._sleep(cycles)
        for (a, b), L in zip(pairs, layers):
            a.record()
            K.decode_partials(L.cache, L.q, L.bt, L.lens, mcl, ns, ws)
            b.record()
        torch.cuda.synchronize()
        durs.extend(a.elapsed_time(b) * 1e3 for a, b in pairs)
    return float(np.mean(durs)), float(np.median(durs))


def cpu_baseline(host, states_int8, budget_s):
    """The oracle (as it stands) on the first layers of the workload until ~budget_s CPU seconds:
    kv_write of the step token plus decode of every query row of the layer.  Also returns the
    largest deviation of the GPU's output for those layers from the oracle."""
    import oracle as O

    O.lib()
    elapsed, nbytes, layers_done, max_err, within = 0.0, 0, 0, 0.0, True
    for (lay, k, v, q), L in zip(host, states_int8):
        cfg = lay.cfg
        oc = O.OracleCache.empty("int8", lay.num_blocks, cfg.num_kv_heads, cfg.head_dim)
        pre, stp = lay.prefill_rows(), lay.step_rows()
        O.kv_write(oc, k[pre], v[pre], lay.slots[pre])
        t0 = time.perf_counter()
        O.kv_write(oc, k[stp], v[stp], lay.slots[stp])
        out, lse = O.decode(oc, q, lay.block_tables, lay.context_lens)
        elapsed += time.perf_counter() - t0
        nbytes += algorithmic_bytes(lay.context_lens, cfg.num_kv_heads, cfg.head_dim, "int8")
        layers_done += 1
        g = L.out.cpu().numpy().astype(np.float64)
        err = np.abs(g - out)
        max_err = max(max_err, float(err.max()))
        within = within and bool(np.all(err <= 2e-3 + 1e-3 * np.abs(out)))
        log(f"oracle layer {layers_done}: {elapsed:.2f}s so far, gpu max abs err {err.max():.2e}")
        if elapsed >= budget_s:
            break
    return elapsed, nbytes, layers_done, max_err, within


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this decode-attention path runs on a single MI355X "
              "(see the sharding notes); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_quantized_amd as K
    import workloads as W

    torch.cuda.set_device(0)
    cfg = W.CONFIGS[args.config]
    n_layers = args.layers or cfg.layers
    dtypes = ["int8"] if args.no_bf16 else ["int8", "bf16"]
    keep = 0 if args.no_cpu_baseline else n_layers
    log(f"workload {cfg.name}: {n_layers} layers, preparing caches ({', '.join(dtypes)})")
    states, host, lay = prepare(args.config, n_layers, dtypes, keep)
    S, Hq, Hkv, D = lay.S, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    mcl = int(lay.context_lens.max())
    lens = lay.context_lens

    results = {}
    for d in dtypes:
        layers = states[d]
        ns = args.splits or K.choose_num_splits(layers[0].cache, S, Hq, mcl)
        ws = torch.empty(K.workspace_bytes(layers[0].cache, S, Hq, ns), dtype=torch.uint8, device="cuda")
        step = make_step(K, layers, S, Hq, mcl, ns, ws)
        ms, wall_ms = time_step(torch, step, args.steps, args.warmup, args.eager)
        step_bytes = algorithmic_bytes(lens, Hkv, D, d) * n_layers
        kern_mean, kern_med = time_split_kernel(torch, K, layers, mcl, ns, ws, passes=min(args.steps, 20))
        results[d] = dict(ms=ms, wall_ms=wall_ms, ns=ns, step_bytes=step_bytes, kern_us=kern_mean,
                          kern_med_us=kern_med, layer_bytes=algorithmic_bytes(lens, Hkv, D, d))
        log(f"{d}: {ms * 1e3:.1f} us/step (wall {wall_ms * 1e3:.1f}), {step_bytes / ms / 1e6:.0f} GB/s, "
            f"decode_split {kern_mean:.2f} us/launch (median {kern_med:.2f}), splits {ns}")

    r = results["int8"]
    value = r["step_bytes"] / (r["ms"] * 1e-3) / 1e9
    achieved = r["layer_bytes"] / (r["kern_us"] * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "us_per_step": round(r["ms"] * 1e3, 1),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) K/V/Q with x20 outlier channels, bf16; random block-table permutation)",
        "config": {
            "workload": f"{cfg.name}: {n_layers} layers x (kv_write 1 token/seq + decode_split + decode_merge), "
                        f"batch {S}, context {mcl}, {Hq} Q / {Hkv} KV heads, head_dim {D}, INT8 q8_0 16-token pages",
            "layers": n_layers, "batch": S, "context": mcl, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "num_splits": r["ns"], "timing": "eager" if args.eager else "hip-graph replay",
            "algorithmic_bytes_per_step": r["step_bytes"],
        },
        "roofline": {
            "kernel": "decode_split_kernel<256,4,int8>" if D == 256 else "decode_split_kernel<128,4,int8>",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None,
            "bytes_per_launch": r["layer_bytes"],
            "avg_launch_us": round(r["kern_us"], 3),
        },
    }
    if "bf16" in results:
        b = results["bf16"]
        out["bf16_variant"] = {
            "us_per_step": round(b["ms"] * 1e3, 1),
            "GB_per_s": round(b["step_bytes"] / (b["ms"] * 1e-3) / 1e9, 1),
            "decode_split_us": round(b["kern_us"], 3),
            "int8_speedup_step": round(b["ms"] / r["ms"], 3),
        }
    if not args.no_cpu_baseline:
        el, nb, nl, max_err, within = cpu_baseline(host, states["int8"], args.cpu_budget_s)
        import oracle as O
        out["cpu_baseline"] = {
            "value": round(nb / el / 1e9, 4),
            "unit": "GB/s",
            "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{nl} of {n_layers} layers: kv_write of the step token + fp64 decode of all {S * Hq} "
                      f"query rows per layer ({el:.1f} s)",
        }
        out["parity_sample"] = {"layers": nl, "max_abs_err": max_err, "within_tolerance": within}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
