"""bench.py's host logic on the CPU: the algorithmic byte and flop counts behind the roofline,
the counter-file arithmetic behind `traffic` (calibration scaling, per-call sums), the kernel
labels, the source-hash guard on the committed traffic, and the refusal of more than one GPU."""

import csv
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)

FWD_STORE = "_ZN3kda12_GLOBAL__N_116chunk_fwd_kernelINS_6bf16_tEDF16_Li64ELi128ELi128ELi8ELb1ELi0EEEvNS_9ChunkArgsE"
REPLAY_X = "_ZN3kda12_GLOBAL__N_113replay_kernelIDF16_Li64ELi128ELi128ELi8ELb1ELb0EEEvNS_9ChunkArgsE"
REPLAY_O = "_ZN3kda12_GLOBAL__N_113replay_kernelIDF16_Li64ELi128ELi128ELi8ELb0ELb0EEEvNS_9ChunkArgsE"
COMBINE = "void kda::(anonymous namespace)::split_combine_kernel<128, 128>(kda::ChunkArgs)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"


def test_algorithmic_counts():
    # bf16 q, k, v; float32 g, beta, o (per token and head, K = V = 128)
    assert bench.prefill_bytes_per_token_head(128, 128) == 2 * 128 * 2 + 128 * 2 + 128 * 4 + 4 + 128 * 4 == 1796
    assert bench.fused_prefill_bytes_per_token_head(128, 128) == 1540
    # state read and written in float32 dominates: 2 * 256 * 32 * 128 * 128 * 4 bytes
    assert bench.decode_bytes_per_step(256, 32, 128, 128) == 1_088_454_656
    assert bench.decode_bytes_per_step(256, 32, 128, 128) - 2 * 256 * 32 * 128 * 128 * 4 == 256 * 32 * (1284 + 512)
    # 6KV + 3CK + 2CV + C^2/3 per token-head at C = 64
    assert abs(bench.prefill_flops_per_token_head(128, 128, 64) - (6 * 128 * 128 + 3 * 64 * 128 + 2 * 64 * 128 + 64 * 64 / 3)) < 1e-9
    assert round(bench.prefill_flops_per_token_head(128, 128, 64)) == 140_629
    # backward: 9CK + 5CV + 16KV + C^2 per token-head at C = 64, K = V = 128
    assert bench.bwd_flops_per_token_head(128, 128, 64) == 9 * 64 * 128 + 5 * 64 * 128 + 16 * 128 * 128 + 64 * 64 == 380_928


def test_kernel_labels():
    assert bench.kernel_label(FWD_STORE) == "chunk_fwd_kernel (split forward, records)"
    assert bench.kernel_label(REPLAY_X) == "replay_kernel (segment maps X)"
    assert bench.kernel_label(REPLAY_O) == "replay_kernel (outputs)"
    assert bench.kernel_label(COMBINE) == "split_combine_kernel"
    demangled = "void kda::(anonymous namespace)::chunk_fwd_kernel<kda::bf16_t, _Float16, 64, 128, 128, 8, true, 1>(kda::ChunkArgs)"
    assert bench.kernel_label(demangled) == "chunk_fwd_kernel (split forward, records, fused gate and q/k norm)"


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"])
        for name, disp, val in rows:
            w.writerow([name, disp, counter, val])


def test_traffic_from_counters(tmp_path):
    """FETCH_SIZE counting half the calibration copy's bytes gives scale 2, WRITE_SIZE
    counting them exactly scale 1; the prefill kernels of each call are summed."""
    gib_kib = (1 << 30) / 1024
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # two calls of four dispatches each, and the calibration copy
    _counter_csv(fetch, "FETCH_SIZE", [(NEG, 1, gib_kib / 2),
                                      (FWD_STORE, 2, 1000), (REPLAY_X, 3, 300), (COMBINE, 4, 100), (REPLAY_O, 5, 600),
                                      (FWD_STORE, 6, 1000), (REPLAY_X, 7, 300), (COMBINE, 8, 100), (REPLAY_O, 9, 600)])
    _counter_csv(write, "WRITE_SIZE", [(NEG, 1, gib_kib),
                                      (FWD_STORE, 2, 800), (REPLAY_X, 3, 10), (COMBINE, 4, 20), (REPLAY_O, 5, 400),
                                      (FWD_STORE, 6, 800), (REPLAY_X, 7, 10), (COMBINE, 8, 20), (REPLAY_O, 9, 400)])
    t = bench.traffic_from(str(fetch), str(write))
    assert t["fetch"]["calls"] == 2 and t["write"]["calls"] == 2
    assert abs(t["fetch"]["scale"] - 2.0) < 1e-12 and abs(t["write"]["scale"] - 1.0) < 1e-12
    assert t["fetch"]["bytes_per_call"] == (1000 + 300 + 100 + 600) * 1024 * 2.0
    assert t["write"]["bytes_per_call"] == (800 + 10 + 20 + 400) * 1024 * 1.0
    assert t["fetch"]["per_kernel_kib_per_dispatch"]["replay_kernel (outputs)"] == 600


def test_traffic_is_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({"kernel_source_sha": bench.kernel_sha(), "hbm_bytes_per_launch": 12345}))
    assert bench.load_traffic(1.0) == 12345
    f.write_text(json.dumps({"kernel_source_sha": "0" * 16, "hbm_bytes_per_launch": 12345}))
    assert bench.load_traffic(1.0) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic(1.0) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and r.stdout == ""
