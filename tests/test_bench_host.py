"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte counts the
roofline divides by, and the HBM-traffic summary (counter scaling by the calibration copy, and
the digest check that stops a summary taken on other kernels from being reported)."""
import csv
import os
import subprocess
import sys

import numpy as np

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and "--gpus 1" in r.stderr


def test_algorithmic_bytes_per_layer():
    # q8_0: per (token, KV head) 2 D code bytes + 2 (D / 32) fp16 scales; at D 256 that is 544 B
    assert bench.algorithmic_bytes(np.array([32768]), 4, 256, "int8") == 32768 * 4 * 544 == 71303168
    assert bench.algorithmic_bytes(np.array([512]), 4, 256, "int8") == 1114112
    # bf16: 4 D bytes; per-head INT8: 2 D codes + two fp32 scales
    assert bench.algorithmic_bytes(np.array([32768]), 4, 256, "bf16") == 134217728
    assert bench.algorithmic_bytes(np.array([32768]), 4, 256, "int8_head") == 32768 * 4 * 520
    # a batch sums its sequences; D 128 has 272 B per (token, KV head)
    lens = np.array([2048, 8192, 16384, 32768])
    assert bench.algorithmic_bytes(lens, 4, 256, "int8") == int(lens.sum()) * 4 * 544
    assert bench.algorithmic_bytes(np.array([1000]), 8, 128, "int8") == 1000 * 8 * 272
    # the long-32k workload's step: 16 layers
    cfg = W.CONFIGS[3]
    assert bench.algorithmic_bytes(np.array(cfg.context_lens), cfg.num_kv_heads, cfg.head_dim, "int8") * 16 == 1140850688


def test_fill_bytes():
    # a prefill kv_write reads 2 bf16 rows (K, V) of D values and the slot, and writes the entries:
    # q8_0 codes 2 D + scales 2 (D / 32) fp16 = 544 B at D 256; BF16 4 D; per-head 2 D + 2 fp32
    T = 32767
    assert bench.fill_bytes(T, 4, 256, "int8") == T * 4 * (1024 + 544) + 4 * T == 205645692
    assert bench.fill_bytes(T, 4, 256, "bf16") == T * 4 * (1024 + 1024) + 4 * T
    assert bench.fill_bytes(T, 4, 256, "int8_head") == T * 4 * (1024 + 520) + 4 * T
    assert bench.fill_bytes(10, 8, 128, "int8") == 10 * 8 * (512 + 272) + 40


def _counter_csv(path, counter, split_kib, copy_kib, fill_kib=()):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        d = 0
        for v in fill_kib:
            d += 1
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "void kvq::kv_write_i8_kernel<256, 0>(kvq::WriteArgs)",
                        "Counter_Name": counter, "Counter_Value": v})
        for v in copy_kib:
            d += 1
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "void at::native::bitwise_not_kernel(...)",
                        "Counter_Name": counter, "Counter_Value": v})
        for v in split_kib:
            d += 1
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "void kvq::decode_split_i8_kernel<256, 4, 0, 0>(...)",
                        "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    # FETCH_SIZE reads half the copy's bytes (factor 2), WRITE_SIZE all of them (factor 1)
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [35000.0, 34990.0, 35010.0], [copy_kib / 2] * 3)
    _counter_csv(write, "WRITE_SIZE", [1584.0] * 3, [copy_kib] * 3)
    out = tmp_path / "summary.md"
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(out))
    monkeypatch.setattr(bench, "FILL_TRAFFIC_SUMMARY", str(tmp_path / "fill.md"))
    bench.pmc_summarize(str(fetch), str(write), "cmd fetch", "cmd write")
    rec = bench.measured_traffic()
    assert rec is not None
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["fetch_bytes_per_launch"] == int(35000.0 * 1024 * 2)  # the median dispatch
    assert rec["write_bytes_per_launch"] == 1584 * 1024
    assert rec["traffic_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == 71303168
    assert "cmd fetch" in out.read_text() and "cmd write" in out.read_text()


def test_traffic_summary_of_other_kernels_is_not_reported(tmp_path, monkeypatch):
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [35000.0], [copy_kib / 2])
    _counter_csv(write, "WRITE_SIZE", [1584.0], [copy_kib])
    out = tmp_path / "summary.md"
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(out))
    monkeypatch.setattr(bench, "FILL_TRAFFIC_SUMMARY", str(tmp_path / "fill.md"))
    bench.pmc_summarize(str(fetch), str(write), "a", "b")
    assert bench.measured_traffic() is not None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.measured_traffic() is None


def test_fill_traffic_summary(tmp_path, monkeypatch):
    # the prefill fill's kvq_write dispatches in the same counter runs get a record of their own
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [35000.0], [copy_kib / 2], fill_kib=[67000.0, 67200.0, 67100.0])
    _counter_csv(write, "WRITE_SIZE", [1584.0], [copy_kib], fill_kib=[69600.0] * 3)
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "split.md"))
    monkeypatch.setattr(bench, "FILL_TRAFFIC_SUMMARY", str(tmp_path / "fill.md"))
    bench.pmc_summarize(str(fetch), str(write), "a", "b")
    rec = bench.measured_traffic(str(tmp_path / "fill.md"))
    assert rec["kernel"] == "kv_write_i8_kernel<256, 0>"
    assert rec["fetch_bytes_per_launch"] == int(67100.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == 69600 * 1024
    assert rec["algorithmic_bytes_per_launch"] == bench.fill_bytes(32767, 4, 256, "int8")
    # the decode_split record is unaffected by the writer's dispatches
    assert bench.measured_traffic()["fetch_bytes_per_launch"] == int(35000.0 * 1024 * 2)


def test_cpu_info_names_the_host():
    model, n = bench.cpu_info()
    assert n == os.cpu_count()
    assert model is None or isinstance(model, str)


def test_multi_token_parity_sample_uses_each_query_tokens_prefix():
    # the sample compares query token i of n with the oracle's decode over the first L - n + i + 1
    # keys: fed the oracle's own causal result it passes, and a row computed over one key too many
    # (the whole context for every token) fails
    import oracle as O
    lay = W.make_layer(1, 0)
    cfg = lay.cfg
    oc = bench.oracle_cache_for(O, lay, lay.k, lay.v)
    n = 8
    rng = np.random.default_rng(3)
    q = W.f32_to_bf16_bits(rng.standard_normal((1, n, cfg.num_q_heads, cfg.head_dim)).astype(np.float32))
    good, _ = O.decode_mq(oc, q, lay.block_tables, lay.context_lens)
    res = bench.multi_token_parity(O, oc, lay, {"mq8": (q, good.astype(np.float32), 4)})
    assert res["decode_8_tokens"]["within_tolerance"] and res["decode_8_tokens"]["rows"] == n * cfg.num_q_heads
    full, _ = O.decode(oc, q.reshape(n, cfg.num_q_heads, cfg.head_dim), np.repeat(lay.block_tables, n, axis=0),
                       np.repeat(lay.context_lens, n))
    bad = full.reshape(good.shape).astype(np.float32)
    res = bench.multi_token_parity(O, oc, lay, {"mq8": (q, bad, 4)})
    assert not res["decode_8_tokens"]["within_tolerance"]
