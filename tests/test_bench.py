"""CPU checks of bench.py's measurement arithmetic (no GPU): the algorithmic
FLOP and byte counts against a brute-force enumeration over the oracle's
attended positions, the counter summariser on a synthetic rocprofv3 CSV, and
the one-GPU guard."""
import csv
import importlib.util
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

import oracle.ref as ref
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def test_prefill_flop_brute_force():
    """4 * D * H per (query row, attended key) pair, the keys of each row
    enumerated from the oracle's attended positions (causal and window)."""
    for window in (0, 9):
        w = wl.make_prefill(prefix_len=32, chunk_lens=[20, 7, 1], num_heads=4, num_kv_heads=2, head_dim=64,
                            block_size=16, dtype="bf16", seed=1, window=window)
        pairs = 0
        for s in range(w.num_seqs):
            C = int(w.q_start[s + 1] - w.q_start[s])
            L = int(w.context_lens[s])
            for i in range(C):
                pairs += len(ref.attended_positions(L - C + i + 1, window))
        assert bench.prefill_flop(w) == 4 * w.head_dim * w.num_heads * pairs


def test_prefill_flop_config5_closed_form():
    """Chunked prefill over a shared prefix: 8 sequences, rows 2048..2559 of
    each attend 2049..2560 keys; 4 * 128 * 32 per pair."""
    pairs = 8 * sum(2048 + i + 1 for i in range(512))
    assert bench.prefill_flop(wl.config(5)) == 4 * 128 * 32 * pairs == 154652377088


def test_decode_bytes_brute_force():
    """K and V rows of every attended position once per kv head, q in its
    dtype, fp32 out, lse, one 4-byte table entry per attended block, one
    4-byte length per sequence."""
    for window in (0, 40):
        w = wl.make_decode(lens=[1, 17, 100, 0, 64], num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                           dtype="f16", seed=3, window=window)
        eb = 2
        rows = blocks = 0
        for s in range(w.num_seqs):
            pos = ref.attended_positions(int(w.context_lens[s]), window)
            rows += len(pos)
            blocks += len(np.unique(pos // w.block_size))
        S, H, D = w.num_seqs, w.num_heads, w.head_dim
        want = (rows * w.num_kv_heads * D * 2 * eb + S * H * D * eb + S * H * D * 4 + S * H * 4 + blocks * 4
                + S * 4)
        got = bench.decode_bytes(w)
        assert got["attend"] == want
        assert got["kv"] == rows * w.num_kv_heads * D * 2 * eb
        # 8-bit pools: D code bytes plus a 4-byte scale per row
        assert bench.decode_bytes(w, "i8")["kv"] == rows * w.num_kv_heads * (D + 4) * 2


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                           "Grid_Size"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_summarize_pmc_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """Per-call bytes = the call's raw KiB x 1024 x (copy bytes / the copy's
    raw bytes), averaged over calls; the record round-trips through
    traffic_for under its source hash."""
    copy = "__amd_rocclr_copyBuffer"
    kern = "void pkv::prefill_kernel<pkv::BF16T, 128, 16, 4>(pkv::PrefillArgs, float)"
    small = "void at::native::elementwise_kernel<...>"
    fetch = [
        {"Dispatch_Id": 1, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 10, "Grid_Size": 64},
        {"Dispatch_Id": 2, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 131072,
         "Grid_Size": 1 << 20},
        {"Dispatch_Id": 3, "Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 600, "Grid_Size": 512},
        {"Dispatch_Id": 3, "Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 400, "Grid_Size": 512},
        {"Dispatch_Id": 4, "Kernel_Name": small, "Counter_Name": "FETCH_SIZE", "Counter_Value": 9999,
         "Grid_Size": 64},
        {"Dispatch_Id": 5, "Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1200,
         "Grid_Size": 512},
    ]
    write = [
        {"Dispatch_Id": 2, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 262144,
         "Grid_Size": 1 << 20},
        {"Dispatch_Id": 3, "Kernel_Name": kern, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500, "Grid_Size": 512},
        {"Dispatch_Id": 5, "Kernel_Name": kern, "Counter_Name": "WRITE_SIZE", "Counter_Value": 700, "Grid_Size": 512},
    ]
    _counter_csv(str(tmp_path / "f" / "x"), fetch)
    _counter_csv(str(tmp_path / "w" / "x"), write)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda *names: "h")
    args = SimpleNamespace(config=5, seed=None, kv="native")
    assert bench.summarize_pmc(args, str(tmp_path / "f"), str(tmp_path / "w"), 256) == 0
    key = "paged_attn_prefill|" + wl.config(5).name
    # FETCH: scale 256 MiB / (131072 KiB) = 2; calls of 1000 and 1200 KiB
    # (the two counter rows of dispatch 3 are one dispatch's instances)
    fetch_bytes = round((1000 + 1200) / 2 * 1024 * 2.0)
    write_bytes = round((500 + 700) / 2 * 1024 * 1.0)
    assert bench.traffic_for(key, "h") == fetch_bytes + write_bytes
    assert bench.traffic_for(key, "other source") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
