#!/usr/bin/env python3
"""Benchmark of the INT8 paged decode-attention path on one MI355X.

One step = every layer of the workload, each layer being: kv_write of the step's new token
(quantize-on-write into the paged INT8 cache), decode_split (split-KV GQA attention over the
cache) and decode_merge (log-sum-exp merge).  The timed step uses kvq_decode_step, where the
split kernel writes the new token itself (two launches per layer); the same work as three
launches per layer (kvq_write, then the split and merge kernels) is timed beside it.  Each layer has its own cache, so a step streams
the whole multi-layer cache from HBM (1.06 GiB of INT8 K/V at 32K context, far above the
256 MB Infinity Cache).  Inputs are seeded synthetic tensors with the workload's shapes and
value distribution, resident in HBM before the timed region.

Timing: the step is captured once into a HIP graph and replayed; HIP events bracket the
timed replays.  The decode_split kernel is also timed on its own: the split launches of all
layers back to back in a HIP graph, events around the replays, which gives the roofline
figure.  The roofline's `traffic` (HBM bytes per split launch) comes from a committed counter
summary (FETCH_SIZE and WRITE_SIZE runs of `--pmc-workload`, scaled by a copy kernel of known
size) and is reported only while the kernel source matches the one it was measured on.  The
BF16-cache variant of the same step runs alongside for comparison, and the CPU oracle is timed
on a bounded sample of the workload.

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
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=3, help="workload id (3 = 32K context, 16 layers)")
    p.add_argument("--splits", type=int, default=0, help="split count (0 = the library's choice)")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's)")
    p.add_argument("--no-bf16", action="store_true", help="skip the BF16-cache comparison")
    p.add_argument("--no-head-format", action="store_true", help="skip the per-head INT8 format comparison")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-multi-token", action="store_true", help="skip the several-query-token decode timings")
    p.add_argument("--no-int-qk", action="store_true", help="skip the integer Q.K timing")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the fused step of the tiny 512-token, 4K, mixed-batch and dense-8B workloads")
    p.add_argument("--cpu-budget-s", type=float, default=12.0, help="CPU seconds for the oracle sample")
    p.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    p.add_argument("--sweep", action="store_true",
                   help="time the step at each of the workload's split counts and the automatic one")
    p.add_argument("--sweep-out", default="", help="also write the sweep table (markdown) to this path")
    p.add_argument("--context-lens", default="",
                   help="with --sweep: comma-separated context lengths replacing the workload's (same heads, "
                        "head dim and layers), e.g. 32768,32768,32768,32768 for a uniform batch")
    p.add_argument("--pmc-workload", action="store_true",
                   help="run only the calibration copy and the decode_split launches (under rocprofv3 --pmc)")
    p.add_argument("--pmc-summarize", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CMD_FETCH", "CMD_WRITE"),
                   help="write the HBM-traffic summary from the two counter runs of --pmc-workload")
    return p.parse_args()


def algorithmic_bytes(lens, Hkv, D, dtype):
    """K and V bytes every step must read from HBM: codes + fp16 scales per 32 values (INT8 q8_0),
    codes + one fp32 scale per row (INT8 per head), or bf16 values."""
    per_token_head = {"int8": 2 * D + 2 * (D // 32) * 2, "int8_head": 2 * D + 2 * 4, "bf16": 4 * D}[dtype]
    return int(np.sum(lens, dtype=np.int64)) * Hkv * per_token_head


class LayerState:
    pass


def prepare(cid, n_layers, dtypes, keep_host_layers):
    import torch

    import decode_attention_quantized_amd as K
    import workloads as W

    states = {d: [] for d in dtypes}
    host = []
    fill = None
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
        if li == 0:
            fill = (k_pre, v_pre, slot_pre)
        if li < keep_host_layers:
            host.append((lay, t["k"].view(torch.int16).cpu().numpy().view(np.uint16),
                         t["v"].view(torch.int16).cpu().numpy().view(np.uint16),
                         t["q"].view(torch.int16).cpu().numpy().view(np.uint16)))
        del t, k_pre, v_pre, slot_pre
        torch.cuda.synchronize()
        log(f"prepared layer {li + 1}/{n_layers}")
    return states, host, lay, fill


def fill_bytes(T, Hkv, D, dtype):
    """Algorithmic bytes of a kv_write of T tokens: the bf16 K and V rows and the slot mapping
    read, the cache entries written (codes and scales, or bf16 values)."""
    written = {"int8": 2 * D + 2 * (D // 32) * 2, "bf16": 4 * D, "int8_head": 2 * D + 8}[dtype]
    return T * Hkv * (4 * D + written) + 4 * T


def time_fill(torch, K, states, fill, Hkv, D, steps, warmup):
    """The bulk kv_write of a prefill (every token of the context but the step's), rewritten into
    layer 1's cache: average launch time over HIP events on the launch stream."""
    k_pre, v_pre, slot_pre = fill
    T = int(slot_pre.shape[0])
    res = {"tokens": T, "what": f"kvq_write of {T} prefill tokens x {Hkv} KV heads (K and V), one launch"}
    for d, layers in states.items():
        cache = layers[0].cache
        for _ in range(max(warmup, 3)):
            K.write(cache, k_pre, v_pre, slot_pre)
        torch.cuda.synchronize()
        n = max(steps, 20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            K.write(cache, k_pre, v_pre, slot_pre)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        gbs = fill_bytes(T, Hkv, D, d) / (us * 1e-6) / 1e9
        res[d] = {"us": round(us, 2), "GB_per_s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                  "bytes": fill_bytes(T, Hkv, D, d)}
        log(f"kv_write fill {d}: {T} tokens, {us:.1f} us, {gbs:.0f} GB/s")
    return res


def make_step(K, layers, S, Hq, mcl, ns, ws, fused=True):
    """One step over every layer.  fused: kvq_decode_step (the new token's write inside the split
    kernel, then the merge); else three launches per layer: kv_write, decode_split, decode_merge."""
    def step_fused():
        for L in layers:
            K.decode_step(L.cache, L.k_new, L.v_new, L.q, L.bt, L.lens, mcl, ns, out=L.out, lse=L.lse, workspace=ws)

    def step_unfused():
        for L in layers:
            K.write(L.cache, L.k_new, L.v_new, L.slot_new)
            K.decode_partials(L.cache, L.q, L.bt, L.lens, mcl, ns, ws)
            K.decode_merge(L.cache, L.lens, mcl, S, Hq, ns, ws, L.out, L.lse)
    return step_fused if fused else step_unfused


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


def time_int_qk(torch, K, layers, S, Hq, mcl, ns, n_layers, steps, warmup):
    """us per step of attention alone (split + merge for every layer, no cache write) with the
    exact f16 Q.K and with integer Q.K, at the same split count; graph replay."""
    res = {}
    ws = torch.empty(K.workspace_bytes(layers[0].cache, S, Hq, ns), dtype=torch.uint8, device="cuda")
    # outputs of their own: each layer's out / lse keep the fused step's result, which the parity
    # sample compares with the oracle
    outs = [(torch.empty_like(L.out), torch.empty_like(L.lse)) for L in layers]
    for name, iq in (("f16_qk", False), ("int8_qk", True)):
        def step():
            for L, (o, l) in zip(layers, outs):
                K.decode(L.cache, L.q, L.bt, L.lens, mcl, ns, out=o, lse=l, workspace=ws, int_qk=iq)
        ms, _ = time_step(torch, step, steps, warmup, False)
        res[name + "_us_per_step"] = round(ms * 1e3, 1)
        log(f"attention only ({name}): {ms * 1e3:.1f} us/step")
    return res


def time_multi_token(torch, K, layers, S, Hq, D, mcl, lens, Hkv, n_layers, steps, warmup, keep=None):
    """us per step (every layer: split + merge) of decode with n_q query tokens per sequence,
    causal among them, at the library's split count; graph replay as for the main step.  keep (a
    dict), if given, receives layer 1's queries and outputs of the 8-token decode and of the
    prompt section, for the parity sample."""
    res = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    for nq in (2, 4, 8):
        q = torch.randn((S, nq, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
        ns = K.choose_num_splits_mq(layers[0].cache, S, nq, Hq, mcl)
        ws = torch.empty(K.workspace_bytes(layers[0].cache, S * nq, Hq, ns), dtype=torch.uint8, device="cuda")
        outs = [(torch.empty((S, nq, Hq, D), dtype=torch.float32, device="cuda"),
                 torch.empty((S, nq, Hq), dtype=torch.float32, device="cuda")) for _ in layers]

        def step():
            for L, (o, l) in zip(layers, outs):
                K.decode_mq(L.cache, q, L.bt, L.lens, mcl, ns, out=o, lse=l, workspace=ws)
        ms, _ = time_step(torch, step, steps, warmup, False)
        if keep is not None and nq == 8:
            keep["mq8"] = (q.view(torch.int16).cpu().numpy().view(np.uint16), outs[0][0].cpu().numpy(), ns)
        res[str(nq)] = {"us_per_step": round(ms * 1e3, 1), "num_splits": ns,
                        "GB_per_s": round(algorithmic_bytes(lens, Hkv, D, "int8") * n_layers / (ms * 1e-3) / 1e9, 1)}
        log(f"int8 decode with {nq} query tokens: {ms * 1e3:.1f} us/step, splits {ns}")
    # a prompt section: the last 2048 positions of the context attend over the cache, causally among
    # themselves (one layer; flops 4 * Hq * D * sum of the visible keys of every query)
    nq, L = 2048, int(mcl)
    q = torch.randn((S, nq, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    ns = K.choose_num_splits_mq(layers[0].cache, S, nq, Hq, mcl)
    ws = torch.empty(K.workspace_bytes(layers[0].cache, S * nq, Hq, ns), dtype=torch.uint8, device="cuda")
    o = torch.empty((S, nq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((S, nq, Hq), dtype=torch.float32, device="cuda")

    def section():
        K.decode_mq(layers[0].cache, q, layers[0].bt, layers[0].lens, mcl, ns, out=o, lse=lse, workspace=ws)
    ms, _ = time_step(torch, section, max(steps // 10, 3), 1, False)
    if keep is not None:
        keep["section"] = (q.view(torch.int16).cpu().numpy().view(np.uint16), o.cpu().numpy(), ns)
    flops = 4.0 * Hq * D * S * sum(L - nq + i + 1 for i in range(nq))
    res["prompt_section_2048"] = {"us_per_layer": round(ms * 1e3, 1), "num_splits": ns,
                                  "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 1)}
    log(f"prompt section of {nq} tokens: {ms * 1e3:.1f} us per layer, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    return res


def time_split_kernel(torch, K, layers, mcl, ns, ws, passes):
    """Average duration (us) of one decode_split launch: the launches of all layers back to back
    (the same kernels the step runs, without the write and merge between them), captured once
    into a HIP graph and replayed; HIP events on the replay stream bracket `passes` replays."""
    def split_only():
        for L in layers:
            K.decode_partials(L.cache, L.q, L.bt, L.lens, mcl, ns, ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        split_only()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            split_only()
        graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(passes):
            graph.replay()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (passes * len(layers))


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_split_i8_long32k_hbm_traffic.md")
FILL_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "kv_write_i8_long32k_fill_hbm_traffic.md")
SECTION_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "section_i8_2048_long32k_hbm_traffic.md")
EIGHT_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "section_i8_8tok_long32k_hbm_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "decode_attention_quantized_amd", "csrc", "kvq_kernels.hip")


def kernel_source_digest():
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(path=None):
    """HBM bytes per launch from a committed counter summary (the decode_split one by default),
    or None when that summary is missing or was taken on a different kernel source."""
    try:
        with open(path or TRAFFIC_SUMMARY) as f:
            for line in f:
                if line.startswith("{"):
                    rec = json.loads(line)
                    if rec.get("kernel_source_sha256") == kernel_source_digest():
                        return rec
    except (OSError, ValueError):
        pass
    return None


COPY_BYTES = 512 << 20  # calibration copy: reads and writes this many bytes


SECTION_TOKENS = 2048  # the prompt section bench.py times (the last 2048 tokens of the 32K context)


def pmc_workload(args):
    """Runs what the HBM-traffic counters are taken on: the prefill fill of every layer's cache
    (one kvq_write each, at set-up), a plain copy kernel of known size (the calibration), the
    decode_split launches of every layer, a few times each, then decodes of 4 and 8 query tokens
    (three each) and one 2048-token prompt section over the first layer."""
    import torch

    import decode_attention_quantized_amd as K
    import workloads as W

    torch.cuda.set_device(0)
    cfg = W.CONFIGS[args.config]
    n_layers = args.layers or cfg.layers
    states, _, lay, _ = prepare(args.config, n_layers, ["int8"], 0)
    S, Hq = lay.S, cfg.num_q_heads
    mcl = int(lay.context_lens.max())
    layers = states["int8"]
    ns = args.splits or K.choose_num_splits_lengths(layers[0].cache, lay.context_lens, Hq)
    ws = torch.empty(K.workspace_bytes(layers[0].cache, S, Hq, ns), dtype=torch.uint8, device="cuda")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)  # one elementwise kernel: COPY_BYTES read, COPY_BYTES written
    torch.cuda.synchronize()
    for _ in range(3):
        for L in layers:
            K.decode_partials(L.cache, L.q, L.bt, L.lens, mcl, ns, ws)
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    L0 = layers[0]
    for nq in (4, 8):
        qm = torch.randn((S, nq, Hq, cfg.head_dim), generator=g, device="cuda").to(torch.bfloat16)
        for _ in range(3):
            K.decode_mq(L0.cache, qm, L0.bt, L0.lens, mcl, 0)
    qs = torch.randn((S, SECTION_TOKENS, Hq, cfg.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    K.decode_mq(L0.cache, qs, L0.bt, L0.lens, mcl, 0)
    torch.cuda.synchronize()
    log(f"pmc workload done: splits {ns}, decodes of 4 and 8 query tokens, and a {SECTION_TOKENS}-token section")


def _traffic_summary(fetch_csv, write_csv, cmd_fetch, cmd_write, kernel, tag, algorithmic, title, path,
                     workload="long-32k layer: batch 1, context 32768, 24/4 heads, head_dim 256", note=""):
    """Per-dispatch medians of FETCH_SIZE and WRITE_SIZE for the kernel whose name (with its
    template arguments) starts `tag`, scaled by what the same counters read for the calibration
    copy; written to `path`."""
    import csv

    def per_dispatch(path_, counter):
        mine, copy = [], []
        with open(path_) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"]) * 1024.0  # KiB -> bytes
                name = r["Kernel_Name"]
                if name.startswith("void kvq::"):
                    name = name[len("void kvq::"):]
                if name.startswith(tag):
                    mine.append(v)
                elif "bitwise_not" in r["Kernel_Name"]:
                    copy.append(v)
        med = lambda x: float(np.median(x)) if x else 0.0
        return med(mine), med(copy), len(mine), len(copy)

    fs, fc, nfs, nfc = per_dispatch(fetch_csv, "FETCH_SIZE")
    ws_, wc, nws, nwc = per_dispatch(write_csv, "WRITE_SIZE")
    if min(nfs, nws, nfc, nwc) == 0:
        log(f"no {tag} or calibration dispatches in the counter runs: {os.path.relpath(path, ROOT)} not written")
        return None
    kf, kw = COPY_BYTES / fc, COPY_BYTES / wc
    rec = {
        "kernel": kernel,
        "workload": workload,
        "kernel_source_sha256": kernel_source_digest(),
        "fetch_kib_per_launch_raw": round(fs / 1024, 1), "write_kib_per_launch_raw": round(ws_ / 1024, 1),
        "copy_fetch_kib_raw": round(fc / 1024, 1), "copy_write_kib_raw": round(wc / 1024, 1),
        "copy_bytes": COPY_BYTES, "fetch_factor": round(kf, 4), "write_factor": round(kw, 4),
        "fetch_bytes_per_launch": int(fs * kf), "write_bytes_per_launch": int(ws_ * kw),
        "traffic_bytes_per_launch": int(fs * kf + ws_ * kw), "algorithmic_bytes_per_launch": algorithmic,
        "dispatches": {"kernel_fetch": nfs, "kernel_write": nws, "copy_fetch": nfc, "copy_write": nwc},
    }
    text = [
        title,
        "",
        "Two counter runs of the same program, one counter each (commands from the repository root",
        "on one MI355X; `$REPO` is the repository root):",
        "",
        "```", cmd_fetch, cmd_write, "```",
        "",
        "Per dispatch, medians.  Each counter is scaled by what it reads for a plain copy kernel of",
        f"{COPY_BYTES} bytes (torch bitwise_not of an int32 tensor: {COPY_BYTES} read, {COPY_BYTES} written).",
        "",
        "| | raw KiB | factor | bytes |",
        "|---|---|---|---|",
        f"| kernel FETCH_SIZE | {fs / 1024:.1f} | {kf:.4f} | {int(fs * kf)} |",
        f"| kernel WRITE_SIZE | {ws_ / 1024:.1f} | {kw:.4f} | {int(ws_ * kw)} |",
        f"| copy FETCH_SIZE | {fc / 1024:.1f} | | {COPY_BYTES} |",
        f"| copy WRITE_SIZE | {wc / 1024:.1f} | | {COPY_BYTES} |",
        "",
        *([note, ""] if note else []),
        f"Algorithmic bytes per launch: {algorithmic}; measured / algorithmic = "
        f"{(fs * kf + ws_ * kw) / algorithmic:.3f}.  The record below holds the digest of the kernel source",
        "it was taken on (bench.py reports a record only while the source still has that digest):",
        "",
        json.dumps(rec),
        "",
    ]
    with open(path, "w") as f:
        f.write("\n".join(text))
    print("\n".join(text))
    return rec


def pmc_summarize(fetch_csv, write_csv, cmd_fetch, cmd_write):
    """Turns the two counter runs of pmc_workload into the traffic summaries: the decode_split
    launches and the prefill fill's kvq_write launches (one 32767-token write per layer at set-up),
    which bench.py reads, and the 2048-token prompt section and the 8-token decode."""
    import workloads as W
    cfg = W.CONFIGS[3]
    lens = np.array(cfg.context_lens)
    _traffic_summary(fetch_csv, write_csv, cmd_fetch, cmd_write, "decode_split_i8_kernel<256, 4, 0, 0>",
                     "decode_split_i8_kernel<256, 4, 0, 0>", algorithmic_bytes(lens, cfg.num_kv_heads, cfg.head_dim, "int8"),
                     "# HBM traffic: decode_split_i8_kernel<256, 4, 0, 0> (q8_0), long-32k layer (context 32768, "
                     "24/4 heads, D 256)", TRAFFIC_SUMMARY)
    T = int(lens[0]) - 1
    _traffic_summary(fetch_csv, write_csv, cmd_fetch, cmd_write, "kv_write_i8_kernel<256, 0>",
                     "kv_write_i8_kernel<256, 0>", fill_bytes(T, cfg.num_kv_heads, cfg.head_dim, "int8"),
                     f"# HBM traffic: kv_write_i8_kernel<256, 0> (q8_0), prefill fill of a long-32k layer ({T} tokens, "
                     "4 KV heads, D 256)", FILL_TRAFFIC_SUMMARY)
    # The prompt section: every chunk of 10 query tokens reads the cache up to its own last token,
    # so the kernel requests the prefix once per chunk (205 times).  Its algorithmic bytes count
    # each input once (cache, Q) and the partials written once: what HBM must carry if the repeated
    # reads are served from the caches.
    Hq, D, Hkv = cfg.num_q_heads, cfg.head_dim, cfg.num_kv_heads
    ns = 4
    sec_alg = int(algorithmic_bytes(lens, Hkv, D, "int8") + SECTION_TOKENS * Hq * D * 2
                  + SECTION_TOKENS * Hq * ns * (D * 4 + 8))
    _traffic_summary(fetch_csv, write_csv, cmd_fetch, cmd_write, "section_i8_kernel<256, 2, 3, 1>",
                     "section_i8_kernel<256, 2, 3, 1>", sec_alg,
                     f"# HBM traffic: section_i8_kernel<256, 2, 3, 1> (q8_0), a {SECTION_TOKENS}-token prompt section "
                     "over a long-32k layer", SECTION_TRAFFIC_SUMMARY,
                     workload=f"long-32k layer: the last {SECTION_TOKENS} of 32768 tokens as query tokens, "
                              f"24/4 heads, head_dim 256, {ns} splits",
                     note=(f"Algorithmic bytes count the cache ({int(algorithmic_bytes(lens, Hkv, D, 'int8'))} B), "
                           f"the query block ({SECTION_TOKENS * Hq * D * 2} B) and the partials "
                           f"({SECTION_TOKENS * Hq * ns * (D * 4 + 8)} B) once each; the kernel requests the "
                           "cache once per 10-token chunk, 205 times."))
    # The decode of 8 query tokens per sequence (one chunk, 64 splits of the two-page-group form):
    # the cache and Q read once, the partials written once.
    nq8, ns8 = 8, 64
    dec8_alg = int(algorithmic_bytes(lens, Hkv, D, "int8") + nq8 * Hq * D * 2 + nq8 * Hq * ns8 * (D * 4 + 8))
    _traffic_summary(fetch_csv, write_csv, cmd_fetch, cmd_write, "section_i8_kernel<256, 2, 2, 2>",
                     "section_i8_kernel<256, 2, 2, 2>", dec8_alg,
                     "# HBM traffic: section_i8_kernel<256, 2, 2, 2> (q8_0), a decode of 8 query tokens over a "
                     "long-32k layer", EIGHT_TRAFFIC_SUMMARY,
                     workload=f"long-32k layer: the last {nq8} of 32768 tokens as query tokens, 24/4 heads, "
                              f"head_dim 256, {ns8} splits",
                     note=(f"Algorithmic bytes count the cache ({int(algorithmic_bytes(lens, Hkv, D, 'int8'))} B), "
                           f"the query block ({nq8 * Hq * D * 2} B) and the partials "
                           f"({nq8 * Hq * ns8 * (D * 4 + 8)} B) once each."))


def oracle_cache_for(O, lay, k, v):
    """The oracle's cache of one layer after the prefill and the step's token (what the GPU cache
    holds after the fused step)."""
    cfg = lay.cfg
    oc = O.OracleCache.empty("int8", lay.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    pre, stp = lay.prefill_rows(), lay.step_rows()
    O.kv_write(oc, k[pre], v[pre], lay.slots[pre])
    O.kv_write(oc, k[stp], v[stp], lay.slots[stp])
    return oc


def cpu_baseline(host, states_int8, budget_s):
    """The oracle (as it stands) on the first layers of the workload until ~budget_s CPU seconds:
    kv_write of the step token plus decode of every query row of the layer.  Also returns the
    largest deviation of the GPU's output for those layers from the oracle, and layer 1's oracle
    cache (for the several-query-token parity sample)."""
    import oracle as O

    O.lib()
    elapsed, nbytes, layers_done, max_err, within = 0.0, 0, 0, 0.0, True
    first = None
    for (lay, k, v, q), L in zip(host, states_int8):
        cfg = lay.cfg
        oc = O.OracleCache.empty("int8", lay.num_blocks, cfg.num_kv_heads, cfg.head_dim)
        pre, stp = lay.prefill_rows(), lay.step_rows()
        O.kv_write(oc, k[pre], v[pre], lay.slots[pre])
        t0 = time.perf_counter()
        O.kv_write(oc, k[stp], v[stp], lay.slots[stp])
        out, lse = O.decode(oc, q, lay.block_tables, lay.context_lens)
        elapsed += time.perf_counter() - t0
        if first is None:
            first = oc
        nbytes += algorithmic_bytes(lay.context_lens, cfg.num_kv_heads, cfg.head_dim, "int8")
        layers_done += 1
        g = L.out.cpu().numpy().astype(np.float64)
        err = np.abs(g - out)
        max_err = max(max_err, float(err.max()))
        within = within and bool(np.all(err <= 2e-3 + 1e-3 * np.abs(out)))
        log(f"oracle layer {layers_done}: {elapsed:.2f}s so far, gpu max abs err {err.max():.2e}")
        if elapsed >= budget_s:
            break
    return elapsed, nbytes, layers_done, max_err, within, first


def multi_token_parity(O, oc, lay, keep, n_section_tokens=16, seed=7):
    """The several-query-token outputs the bench timed (layer 1, at the bench's launch
    configuration) against the oracle: every row of the 8-token decode, and every head of a seeded
    sample of the prompt section's query tokens (its first and last included).  Query token i of n
    attends to the first L - n + i + 1 keys: the oracle's decode over that prefix."""
    res = {}
    L = int(lay.context_lens[0])
    bt = lay.block_tables[:1]
    for name, sel in (("decode_8_tokens", None), ("prompt_section_2048", n_section_tokens)):
        key = "mq8" if name == "decode_8_tokens" else "section"
        if key not in keep:
            continue
        q, out, ns = keep[key]                  # q [1][n][Hq][D] bits, out [1][n][Hq][D]
        n = q.shape[1]
        if sel is None:
            toks = np.arange(n)
        else:
            rng = np.random.default_rng(seed)
            toks = np.unique(np.concatenate([[0, n - 1], rng.choice(n, sel - 2, replace=False)]))
        lens = (L - n + 1 + toks).astype(np.int32)
        ref, ref_lse = O.decode(oc, np.ascontiguousarray(q[0, toks]), np.repeat(bt, len(toks), axis=0), lens)
        g = out[0, toks].astype(np.float64)
        err = np.abs(g - ref)
        ok = bool(np.all(err <= 2e-3 + 1e-3 * np.abs(ref)))
        res[name] = {"query_tokens_checked": int(len(toks)), "rows": int(len(toks) * q.shape[2]),
                     "num_splits": int(ns), "max_abs_err": float(err.max()), "within_tolerance": ok}
        log(f"parity sample {name}: {len(toks)} query tokens, max abs err {err.max():.3e}"
            + ("" if ok else " OUT OF TOLERANCE"))
    return res


def cpu_baseline_one_thread(host):
    """The same oracle work for the first layer on one host thread: (seconds, algorithmic bytes)."""
    import oracle as O

    lay, k, v, q = host[0]
    cfg = lay.cfg
    oc = O.OracleCache.empty("int8", lay.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    pre, stp = lay.prefill_rows(), lay.step_rows()
    O.kv_write(oc, k[pre], v[pre], lay.slots[pre])
    n0 = O.num_threads()
    O.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        O.kv_write(oc, k[stp], v[stp], lay.slots[stp])
        O.decode(oc, q, lay.block_tables, lay.context_lens)
        el = time.perf_counter() - t0
    finally:
        O.set_num_threads(n0)
    log(f"oracle layer 1 on one thread: {el:.2f}s")
    return el, algorithmic_bytes(lay.context_lens, cfg.num_kv_heads, cfg.head_dim, "int8")


FLUSH_BYTES = 512 << 20  # written between steps when the whole cache fits in the 256 MB MALL


def time_graph_median(torch, step, steps, warmup, flush=None):
    """Median us of one graph replay of `step` over `steps` replays (HIP events on the replay
    stream around each replay); with `flush`, a fill of that buffer before every replay (outside
    the timed region) evicts the caches from the MALL."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step()
        times = []
        for i in range(warmup + steps):
            if flush is not None:
                flush.fill_(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            graph.replay()
            e1.record(s)
            if i >= warmup:
                times.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in times])) * 1e3


def other_workloads(torch, K, W, cids, steps, warmup, parity):
    """The fused step (every layer: decode_split with the new token's write, then decode_merge) of
    the other workloads at the library's split count, each prepared, timed and freed in turn: us
    per step, algorithmic GB/s and % of 8 TB/s.  Workloads whose caches would fit in the 256 MB
    MALL get a 512 MiB fill between replays.  With `parity`, layer 1's output is compared with the
    oracle."""
    res = {}
    for cid in cids:
        cfg = W.CONFIGS[cid]
        states, host, lay, _ = prepare(cid, cfg.layers, ["int8"], 1 if parity else 0)
        layers = states["int8"]
        S, Hq, Hkv, D = lay.S, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
        mcl = int(lay.context_lens.max())
        ns = K.choose_num_splits_lengths(layers[0].cache, lay.context_lens, Hq)
        ws = torch.empty(K.workspace_bytes(layers[0].cache, S, Hq, ns), dtype=torch.uint8, device="cuda")
        step_bytes = sum(algorithmic_bytes(L_.lens.cpu().numpy(), Hkv, D, "int8") for L_ in layers)
        flush = None
        if algorithmic_bytes(lay.context_lens, Hkv, D, "bf16") * cfg.layers < 2 * FLUSH_BYTES:
            flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        us = time_graph_median(torch, make_step(K, layers, S, Hq, mcl, ns, ws), steps, warmup, flush)
        gbs = step_bytes / (us * 1e-6) / 1e9
        r = {"us_per_step": round(us, 1), "GB_per_s": round(gbs, 1), "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 1),
             "num_splits": ns, "layers": cfg.layers, "batch": S,
             "context": f"{int(lay.context_lens.min())}..{mcl}" if S > 1 else mcl,
             "heads": f"{Hq}/{Hkv}", "head_dim": D, "algorithmic_bytes_per_step": int(step_bytes),
             "mall_flushed": flush is not None}
        log(f"{cfg.name}: {us:.1f} us/step, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of peak), splits {ns}")
        if parity:
            import oracle as O
            lay0, k, v, q = host[0]
            oc = oracle_cache_for(O, lay0, k, v)
            ref, _ = O.decode(oc, q, lay0.block_tables, lay0.context_lens)
            g = layers[0].out.cpu().numpy().astype(np.float64)
            err = np.abs(g - ref)
            r["parity_layer1"] = {"max_abs_err": float(err.max()),
                                  "within_tolerance": bool(np.all(err <= 2e-3 + 1e-3 * np.abs(ref)))}
            log(f"{cfg.name} layer 1 against the oracle: max abs err {err.max():.3e}")
        res[cfg.name] = r
        del states, host, layers, ws, flush
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def cpu_info():
    """The host CPU's model name (from /proc/cpuinfo) and os.cpu_count()."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def sweep(args):
    """Per dtype and split count: us per step (graph replay of the fused step, one replay per
    timing, the MALL flushed between replays when the workload's caches would fit in it)."""
    import torch

    import decode_attention_quantized_amd as K
    import workloads as W

    torch.cuda.set_device(0)
    if args.context_lens:
        import dataclasses
        lens = tuple(int(x) for x in args.context_lens.split(","))
        base = W.CONFIGS[args.config]
        name = f"{base.name} with lengths {args.context_lens}"
        W.CONFIGS[args.config] = base._replace(name=name, context_lens=lens, seeded_lens=None) \
            if hasattr(base, "_replace") else dataclasses.replace(base, name=name, context_lens=lens, seeded_lens=None)
    cfg = W.CONFIGS[args.config]
    n_layers = args.layers or cfg.layers
    dtypes = ["int8"] if args.no_bf16 else ["int8", "bf16"]
    states, _, lay, _ = prepare(args.config, n_layers, dtypes, 0)
    S, Hq, Hkv, D = lay.S, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    mcl = int(lay.context_lens.max())
    flush = None
    if algorithmic_bytes(lay.context_lens, Hkv, D, "bf16") * n_layers < 2 * FLUSH_BYTES:
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    rows = []
    for d in dtypes:
        layers = states[d]
        # the library's choice from the batch's lengths, and from the maximum length alone
        auto = K.choose_num_splits_lengths(layers[0].cache, lay.context_lens, Hq)
        auto_max = K.choose_num_splits(layers[0].cache, S, Hq, mcl)
        counts = sorted(set(list(cfg.splits) + [auto, auto_max]))
        step_bytes = algorithmic_bytes(lay.context_lens, Hkv, D, d) * n_layers
        for ns in counts:
            ws = torch.empty(K.workspace_bytes(layers[0].cache, S, Hq, ns), dtype=torch.uint8, device="cuda")
            step = make_step(K, layers, S, Hq, mcl, ns, ws)
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step()
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=s):
                    step()
                times = []
                for i in range(args.warmup + args.steps):
                    if flush is not None:
                        flush.fill_(i)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(s)
                    graph.replay()
                    e1.record(s)
                    if i >= args.warmup:
                        times.append((e0, e1))
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) for a, b in times])) * 1e3
            mark = "/".join(m for m, x in (("lengths", auto), ("max only", auto_max)) if ns == x)
            rows.append((d, ns, mark, us, step_bytes / (us * 1e-6) / 1e9))
            log(f"{d} splits {ns}{f' (auto: {mark})' if mark else ''}: {us:.1f} us/step, {rows[-1][4]:.0f} GB/s")
            del graph, ws
    text = [f"# Split-count sweep: {cfg.name} ({n_layers} layers, batch {S}, context "
            f"{'/'.join(str(int(x)) for x in np.unique(lay.context_lens)) if S <= 8 else f'{int(lay.context_lens.min())}..{mcl}'}, "
            f"{Hq}/{Hkv} heads, D {D})", "",
            "Command (run from the repository root on one MI355X):", "", "```",
            f"python3 bench.py --sweep --config {args.config} --steps {args.steps} --warmup {args.warmup}"
            + (f" --context-lens {args.context_lens}" if args.context_lens else "")
            + (" --no-bf16" if args.no_bf16 else "") + (f" --sweep-out {args.sweep_out}" if args.sweep_out else ""),
            "```", "",
            "Median over the timed steps of one graph replay of the fused step (every layer: decode_split with "
            "the new token's write, then decode_merge), HIP events on the replay stream."
            + (f"  A {FLUSH_BYTES >> 20} MiB fill between replays evicts the caches from the 256 MB MALL "
               "(outside the timed region)." if flush is not None else ""), "",
            "", "auto: the library's choice from the batch's lengths (kvq_choose_num_splits_lengths, what the "
            "benchmark uses) and from the maximum length alone (kvq_choose_num_splits, num_splits = 0).", "",
            "| cache | splits | auto | us per step | GB/s (algorithmic) |", "|---|---|---|---|---|"]
    for d, ns, a, us, gbs in rows:
        text.append(f"| {d} | {ns} | {a} | {us:.1f} | {gbs:.0f} |")
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            f.write("\n".join(text) + "\n")
    print("\n".join(text), flush=True)


def main():
    args = parse()
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this decode-attention path runs on a single MI355X "
              "(see the sharding notes); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_quantized_amd as K
    import workloads as W

    if args.pmc_workload:
        pmc_workload(args)
        return
    if args.sweep:
        sweep(args)
        return
    torch.cuda.set_device(0)
    cfg = W.CONFIGS[args.config]
    n_layers = args.layers or cfg.layers
    dtypes = ["int8"] + ([] if args.no_bf16 else ["bf16"]) + ([] if args.no_head_format else ["int8_head"])
    keep = 0 if args.no_cpu_baseline else n_layers
    log(f"workload {cfg.name}: {n_layers} layers, preparing caches ({', '.join(dtypes)})")
    states, host, lay, fill = prepare(args.config, n_layers, dtypes, keep)
    S, Hq, Hkv, D = lay.S, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    mcl = int(lay.context_lens.max())
    lens = lay.context_lens

    results = {}
    for d in dtypes:
        layers = states[d]
        ns = args.splits or K.choose_num_splits_lengths(layers[0].cache, lay.context_lens, Hq)
        ws = torch.empty(K.workspace_bytes(layers[0].cache, S, Hq, ns), dtype=torch.uint8, device="cuda")
        ms_unfused, _ = time_step(torch, make_step(K, layers, S, Hq, mcl, ns, ws, fused=False), args.steps,
                                  args.warmup, args.eager)
        ms, wall_ms = time_step(torch, make_step(K, layers, S, Hq, mcl, ns, ws), args.steps, args.warmup,
                                args.eager)
        # noise control: the same step captured and timed again (auto split count both times)
        ms_rep, _ = time_step(torch, make_step(K, layers, S, Hq, mcl, ns, ws), args.steps, args.warmup,
                              args.eager)
        step_bytes = algorithmic_bytes(lens, Hkv, D, d) * n_layers
        kern_us = time_split_kernel(torch, K, layers, mcl, ns, ws, passes=max(args.steps, 20))
        results[d] = dict(ms=ms, wall_ms=wall_ms, ms_unfused=ms_unfused, ns=ns, step_bytes=step_bytes,
                          kern_us=kern_us, layer_bytes=algorithmic_bytes(lens, Hkv, D, d), ms_rep=ms_rep)
        log(f"{d}: {ms * 1e3:.1f} us/step (wall {wall_ms * 1e3:.1f}; three kernels per layer "
            f"{ms_unfused * 1e3:.1f}), {step_bytes / ms / 1e6:.0f} GB/s, decode_split {kern_us:.2f} us/launch, "
            f"splits {ns}")

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
        "us_per_step_unfused": round(r["ms_unfused"] * 1e3, 1),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 1),
        "noise_control": {"what": "the same fused step (auto split count) captured and timed a second time",
                          "us_per_step_repeat": round(r["ms_rep"] * 1e3, 1),
                          "spread_pct": round(100 * abs(r["ms_rep"] - r["ms"]) / r["ms"], 2)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) K/V/Q with x20 outlier channels, bf16; random block-table permutation)",
        "config": {
            "workload": f"{cfg.name}: {n_layers} layers x (decode_split with the new token's kv_write fused in "
                        f"+ decode_merge), "
                        f"batch {S}, context {mcl}, {Hq} Q / {Hkv} KV heads, head_dim {D}, INT8 q8_0 16-token pages",
            "layers": n_layers, "batch": S, "context": mcl, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "num_splits": r["ns"], "timing": "eager" if args.eager else "hip-graph replay",
            "algorithmic_bytes_per_step": r["step_bytes"],
        },
        "roofline": {
            "kernel": "decode_split_i8_kernel<256, 4, 0, 0>" if D == 256 else "decode_split_i8_kernel<128, 4, 0, 0>",
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
    tr = measured_traffic() if (args.config == 3 and D == 256) else None
    if tr is not None:
        out["roofline"]["traffic"] = tr["traffic_bytes_per_launch"]
        out["roofline"]["traffic_source"] = os.path.relpath(TRAFFIC_SUMMARY, ROOT)
    if "int8_head" in results:
        hres = results["int8_head"]
        out["int8_head_variant"] = {
            "format": "int8 codes + one fp32 scale per (token, KV head): 520 B per token per head at D 256",
            "us_per_step": round(hres["ms"] * 1e3, 1),
            "GB_per_s": round(hres["step_bytes"] / (hres["ms"] * 1e-3) / 1e9, 1),
            "decode_split_us": round(hres["kern_us"], 3),
            "split_GB_per_s": round(hres["layer_bytes"] / (hres["kern_us"] * 1e-6) / 1e9, 1),
        }
    if "bf16" in results:
        b = results["bf16"]
        out["bf16_variant"] = {
            "us_per_step": round(b["ms"] * 1e3, 1),
            "us_per_step_unfused": round(b["ms_unfused"] * 1e3, 1),
            "GB_per_s": round(b["step_bytes"] / (b["ms"] * 1e-3) / 1e9, 1),
            "decode_split_us": round(b["kern_us"], 3),
            "int8_speedup_step": round(b["ms"] / r["ms"], 3),
        }
    out["kv_write_fill"] = time_fill(torch, K, states, fill, Hkv, D, args.steps, args.warmup)
    ftr = measured_traffic(FILL_TRAFFIC_SUMMARY) if (args.config == 3 and D == 256) else None
    if ftr is not None and "int8" in out["kv_write_fill"]:
        out["kv_write_fill"]["int8"]["traffic"] = ftr["traffic_bytes_per_launch"]
        out["kv_write_fill"]["int8"]["traffic_source"] = os.path.relpath(FILL_TRAFFIC_SUMMARY, ROOT)
    if not args.no_int_qk:
        out["int8_qk_variant"] = time_int_qk(torch, K, states["int8"], S, Hq, mcl, r["ns"], n_layers,
                                             args.steps, args.warmup)
    keep = {}
    if not args.no_multi_token:
        out["multi_token"] = time_multi_token(torch, K, states["int8"], S, Hq, D, mcl, lens, Hkv, n_layers,
                                              args.steps, args.warmup, keep)
    if not args.no_cpu_baseline:
        el, nb, nl, max_err, within, oc1 = cpu_baseline(host, states["int8"], args.cpu_budget_s)
        import oracle as O
        model, ncpu = cpu_info()
        out["cpu_baseline"] = {
            "value": round(nb / el / 1e9, 4),
            "unit": "GB/s",
            "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{nl} of {n_layers} layers: kv_write of the step token + fp64 decode of all {S * Hq} "
                      f"query rows per layer ({el:.1f} s)",
            "cpu_model": model,
            "os_cpu_count": ncpu,
        }
        el1, nb1 = cpu_baseline_one_thread(host)
        out["cpu_baseline"]["one_thread"] = {"value": round(nb1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                             "sample": f"layer 1 of {n_layers} ({el1:.1f} s)"}
        out["parity_sample"] = {"layers": nl, "max_abs_err": max_err, "within_tolerance": within}
        log(f"parity sample ({nl} layers, fused step against the oracle): max abs err {max_err:.3e}, "
            + ("within tolerance" if within else "OUT OF TOLERANCE"))
        if keep:
            out["parity_sample"]["several_query_tokens"] = multi_token_parity(O, oc1, host[0][0], keep)
    if not args.no_other_workloads and args.config == 3 and not args.layers:
        # free the 32K workload first: the others are prepared one at a time
        del states, host
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["other_workloads"] = other_workloads(torch, K, W, [1, 2, 4, 5], max(args.steps // 2, 20), args.warmup,
                                                 not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
