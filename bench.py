#!/usr/bin/env python3
"""Throughput of the paged-KV attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic,
seeded input already resident in HBM: write the step's new tokens' K/V into
their pool slots through the block table (``paged_kv_write``), then attend
(``paged_attn_decode`` for the decode workloads, ``paged_attn_prefill`` for
the chunked-prefill one, ``paged_attn_decode_compressed`` for the
compressed-slot tier, whose step first compresses as many groups as a steady
state averages per step with ``paged_kv_compress``).  W untimed warm-up steps, then exactly K timed
steps between two device synchronisations; HIP events on the launch stream
also time the write and the attention call of every step (called eagerly:
the host enqueues ahead of the GPU; ``--graph`` replays them as HIP graphs).

Prints one JSON line.  ``value`` is the algorithmic bytes one step must move
(decode: every attended K/V row once per kv head, queries, outputs, table
entries; plus the write's read and store) per second, or the algorithmic
FLOP of the prefill (4 * head_dim per unmasked query/key pair and head) per
second.  ``roofline`` relates the attention call alone to MI355X's peak (HBM
8 TB/s; dense bf16/fp16 MFMA 2.5 PFLOP/s).  ``cpu_baseline`` times the fp64
oracle on the host on a bounded sample of the same workload.

By default the line is the long-context GQA decode workload (64 sequences,
32 query / 8 kv heads, head_dim 128, block_size 32, bf16, contexts
log-uniform in [1024, 32768]), the largest that fits one GPU, with the
chunked prefill over a shared prefix (8 sequences x 512-row chunks after a
2048-position prefix, 32 / 8 heads, bf16) timed on the same GPU in the same
run and reported under "prefill" (its own steps, roofline and oracle
baseline).

    python bench.py [--gpus 1] [--steps 20] [--warmup 100] [--config 3] [--prefill-config 5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-read GB/s (% of HBM peak); prefill TFLOP/s (% MFMA)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}


def decode_bytes(w, kv: str = "native") -> dict:
    """Algorithmic bytes of one decode call and of the step's write.  With
    8-bit pools (kv "i8" / "fp8") a K or V row is D code bytes plus its
    4-byte scale."""
    import numpy as np
    eb = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    S, H, D, B = w.num_seqs, w.num_heads, w.head_dim, w.block_size
    L = w.context_lens.astype(np.int64)
    lo = np.maximum(0, L - w.window) if w.window > 0 else np.zeros_like(L)
    slot_blocks = 0
    if w.full_start is not None:
        lo = np.maximum(lo, np.minimum(w.full_start.astype(np.int64), L))
        slot_blocks = int(((w.num_slots.astype(np.int64) + B - 1) // B).sum())
    blocks = np.where(L > 0, (L + B - 1) // B - lo // B, 0)
    kv_bytes = w.kv_bytes_attended()
    if kv != "native":
        kv_bytes = kv_bytes // (D * eb) * (D + 4)
    attend = (kv_bytes + S * H * D * eb + S * H * D * 4 + S * H * 4 + (int(blocks.sum()) + slot_blocks) * 4 +
              S * 4 * (1 if w.full_start is None else 3))
    T = int((L > 0).sum())
    stored = D * eb if kv == "native" else D + 4
    write = T * w.num_kv_heads * 2 * (D * eb + stored) + T * 8 + T * 4
    return {"attend": attend, "write": write, "kv": kv_bytes}


def prefill_flop(w) -> int:
    """4 * D per unmasked (query, key) pair, per query head."""
    total = 0
    for s in range(w.num_seqs):
        C = int(w.q_start[s + 1] - w.q_start[s])
        L = int(w.context_lens[s])
        for i in range(C):
            p = L - C + i
            n = p + 1 if w.window <= 0 else min(p + 1, w.window)
            total += n
    return 4 * w.head_dim * w.num_heads * total


def steady_compressions(w):
    """Compressions of a step of the tier workload in its steady state: a
    sequence compresses once every window/2 = 128 appended positions, so a
    step of S sequences averages S / 128 of them. Op i averages the group
    [full_start, full_start + 128) of sequence i (8 blocks, always inside its
    full tier) into ring row 0 of its slot table: the same bytes as a real
    compression, and idempotent, so repeated steps see the same state."""
    import numpy as np
    B, half = w.block_size, 128
    n = max(1, round(w.num_seqs / half))
    src = np.stack([w.block_tables[i, w.full_start[i] // B:w.full_start[i] // B + half // B] for i in range(n)])
    return src.astype(np.int32), w.slot_tables[:n, 0].astype(np.int32), np.zeros(n, np.int32)


def pkv_workers(d) -> int:
    from paged_kv_cache_30_amd import paged_attn_decode_workers
    w = d.w
    return paged_attn_decode_workers(d.k_pool, w.num_heads, w.num_seqs, w.max_context_len, w.window, w.sinks)


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_30_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key: str, src: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, target_s: float):
    """fp64 oracle on the host cores (NumPy, its BLAS free to use every
    visible core), on the first sequences of the workload until about
    target_s seconds of work (whole workload if less)."""
    import os
    import numpy as np
    import oracle.compressed as oc
    import oracle.ref as ref
    cores = len(os.sched_getaffinity(0))
    threads = cores
    try:
        from threadpoolctl import threadpool_info
        blas = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if blas:
            threads = max(blas)
    except ImportError:  # pragma: no cover
        pass
    kp, vp = ref.build_pools(w)
    eb = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    done, elapsed, units = 0, 0.0, 0.0
    while done < w.num_seqs and elapsed < target_s:
        t = time.perf_counter()
        if w.kind == "decode" and w.full_start is not None:
            s = [done]
            oc.decode_compressed(w.q[s], kp, vp, w.block_tables[s], w.context_lens[s], w.full_start[s],
                                 w.slot_tables[s], w.num_slots[s], block_size=w.block_size,
                                 num_kv_heads=w.num_kv_heads, window=w.window, scale=w.scale, dtype=w.dtype)
            L = int(w.context_lens[done])
            n = L - max(int(w.full_start[done]), L - w.window if w.window > 0 else 0) + int(w.num_slots[done])
            units += n * w.num_kv_heads * w.head_dim * 2 * eb
        elif w.kind == "decode":
            ref.decode(w.q, kp, vp, w.block_tables, w.context_lens, block_size=w.block_size,
                       num_kv_heads=w.num_kv_heads, window=w.window, scale=w.scale, dtype=w.dtype,
                       seqs=[done])
            L = int(w.context_lens[done])
            n = min(L, w.window) if w.window > 0 else L
            units += n * w.num_kv_heads * w.head_dim * 2 * eb
        else:
            ref.prefill(w.q, w.q_start, kp, vp, w.block_tables, w.context_lens, block_size=w.block_size,
                        num_kv_heads=w.num_kv_heads, window=w.window, scale=w.scale, dtype=w.dtype,
                        seqs=[done])
            C = int(w.q_start[done + 1] - w.q_start[done])
            L = int(w.context_lens[done])
            pairs = sum((L - C + i + 1) if w.window <= 0 else min(L - C + i + 1, w.window) for i in range(C))
            units += 4 * w.head_dim * w.num_heads * pairs
        elapsed += time.perf_counter() - t
        done += 1
    if w.kind == "decode":
        value, unit = units / elapsed / 1e9, "GB/s"
    else:
        value, unit = units / elapsed / 1e12, "TFLOP/s"
    return {"value": round(value, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"first {done} of {w.num_seqs} sequences (all heads), fp64 NumPy oracle, "
                      f"{elapsed:.2f} s, BLAS threads {threads} of {cores} visible cores"}


KERNELS = {"decode": ("decode_split_kernel", "decode_mma_kernel", "decode_merge_kernel", "decode_plan_kernel"),
           "prefill": ("prefill_kernel",)}
# The kernel that starts an attention call (its split kernel, either kind).
CALL_START = {"decode": ("decode_split_kernel", "decode_mma_kernel"), "prefill": ("prefill_kernel",)}


def attend_sources(kind: str, kv: str):
    """Source files of the kernels one attention call launches."""
    if kind == "decode":
        return ("decode.hip", "common.h")
    return ("prefill.hip", "common.h")


def summarize_pmc(args, fetch_dir, write_dir, copy_mib) -> int:
    """HBM bytes per attention call from rocprofv3 counter runs.

    Each run's counter CSV has one row per dispatch with FETCH_SIZE or
    WRITE_SIZE (KiB). The calibration copy (a torch elementwise copy of
    COPY_MIB MiB) gives the scale of each counter: bytes it should read or
    write / what the counter reports for it. The attention call's kernels are
    summed per launch and averaged over launches."""
    import csv
    import glob
    import workloads as wl
    w = wl.config(args.config, args.seed)
    kind = w.kind
    copy_bytes = int(copy_mib) << 20

    def per_dispatch(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals, grids = {}, {}
        for row in csv.DictReader(open(files[0])):
            if row.get("Counter_Name") != counter:
                continue
            key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
            grids[key] = int(row["Grid_Size"])
        return vals, grids

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, grids = per_dispatch(d, counter)
        # The calibration copy is the device-to-device copy-buffer dispatch
        # with the largest grid (torch's copy_ of COPY_MIB MiB).
        copies = [(grids[k], v) for k, v in vals.items() if "copyBuffer" in k[1]]
        copy_val = max(copies)[1] if copies else None
        scale = copy_bytes / (copy_val * 1024.0) if copy_val else 1.0
        ours = sorted((i, k, v) for (i, k), v in vals.items() if any(n in k for n in KERNELS[kind]))
        # group consecutive dispatches of one call: the split/prefill kernel
        # starts a call
        calls, cur = [], None
        for i, k, v in ours:
            if any(f in k for f in CALL_START[kind]):
                cur = [v]
                calls.append(cur)
            elif cur is not None:
                cur.append(v)
        per_call = [sum(c) * 1024.0 * scale for c in calls]
        out[counter] = {"kib_per_call_raw": round(sum(sum(c) for c in calls) / max(len(calls), 1), 1),
                        "calls": len(calls), "copy_kib_raw": copy_val, "scale": round(scale, 4),
                        "bytes_per_call": round(sum(per_call) / max(len(per_call), 1))}
    src = source_hash(*attend_sources(kind, args.kv))
    key = f"paged_attn_{kind}|{w.name}" + ("" if args.kv == "native" else f"|{args.kv}")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        db = json.load(open(path))
    except (OSError, ValueError):
        db = {}
    db[key] = {"source_hash": src, "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"],
               "bytes_per_launch": out["FETCH_SIZE"]["bytes_per_call"] + out["WRITE_SIZE"]["bytes_per_call"]}
    os.makedirs(os.path.dirname(path), exist_ok=True)
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)
    print(json.dumps({key: db[key]}))
    return 0


def run_leg(w, args, warmup: int, steps: int, settle_s: float = 0.0) -> dict:
    """Stage workload w on the GPU, run `warmup` untimed steps (then more
    until `settle_s` seconds of steps have run, if asked), time exactly
    `steps` steps and return the leg's figures."""
    import torch
    from paged_kv_cache_30_amd import session

    d = session.DeviceWorkload(w, num_workers=args.workers, kv_format=args.kv)
    comp_bytes = 0
    if w.full_start is not None:
        src_b, dst_b, dst_s = steady_compressions(w)
        d.set_compress_ops(src_b, dst_b, dst_s)
        row = w.num_kv_heads * w.head_dim * {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
        comp_bytes = src_b.size * w.block_size * row * 2 + len(dst_b) * row * 2 + src_b.size * 4 + len(dst_b) * 8
    torch.cuda.synchronize()
    if args.calibration_copy_mib:
        # A plain device copy of known size, for scaling HBM byte counters.
        n = args.calibration_copy_mib << 20
        src_t = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst_t = torch.empty_like(src_t)
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t

    for _ in range(warmup):
        d.step()
    torch.cuda.synchronize()
    n_settle = 0
    if settle_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            for _ in range(50):
                d.step()
            n_settle += 50
            torch.cuda.synchronize()

    # The step's two calls, replayed as HIP graphs (no host launch gaps) or
    # called eagerly.
    def prep():  # compressions (tier workload only), then the write
        d.compress_step()
        d.write_step()

    if not args.graph:
        do_write, do_attend = prep, d.attend
    else:
        g_write, g_attend = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_write):
            prep()
        with torch.cuda.graph(g_attend):
            d.attend()
        torch.cuda.synchronize()
        for _ in range(2):
            g_write.replay()
            g_attend.replay()
        torch.cuda.synchronize()
        do_write, do_attend = g_write.replay, g_attend.replay

    K = steps
    flush_buf = (torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda")
                 if args.flush_mib > 0 else None)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        if flush_buf is not None:
            flush_buf.fill_(i & 0xFF)
        ev[i][0].record()
        do_write()
        ev[i][1].record()
        do_attend()
        ev[i][2].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / K
    if flush_buf is not None:
        ms_step = sum(e[0].elapsed_time(e[2]) for e in ev) / K
    write_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    attend_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    att_mean = sum(attend_ms) / K
    att_med = attend_ms[K // 2]

    if w.kind == "decode":
        by = decode_bytes(w, args.kv)
        step_units = by["attend"] + by["write"] + comp_bytes
        value = step_units / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = by["attend"] / (att_mean * 1e-3) / 1e9
        src = source_hash(*attend_sources("decode", args.kv))
        key = f"paged_attn_decode|{w.name}" + ("" if args.kv == "native" else f"|{args.kv}")
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(key, src)}
        extra = {"decode_workers": d.num_workers or pkv_workers(d), "kv_pool": args.kv}
        if w.full_start is not None:
            extra.update(compressions_per_step=int(len(d.compress_ops[1])), tier_window=256, max_slots=16)
    else:
        flop = prefill_flop(w)
        value = flop / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = flop / (att_mean * 1e-3) / 1e12
        src = source_hash(*attend_sources("prefill", args.kv))
        key = f"paged_attn_prefill|{w.name}" + ("" if args.kv == "native" else f"|{args.kv}")
        peak = MFMA_PEAK_TFLOPS[w.dtype]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_for(key, src)}
        extra = {"kv_pool": args.kv} if args.kv != "native" else {}
    del d
    return {
        "value": round(value, 3), "unit": unit, "ms_per_step": round(ms_step, 5), "steps": K,
        "warmup": warmup + n_settle,
        "dtype": w.dtype if args.kv == "native" else f"{args.kv}+{w.dtype}",
        "config": {"workload": w.name, "kind": w.kind, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "window": w.window, "max_context_len": w.max_context_len,
                   "total_context": int(w.context_lens.sum()), "seed": w.seed, **extra},
        "roofline": roof,
        "timing": {"attend_ms_mean": round(att_mean, 5), "attend_ms_median": round(att_med, 5),
                   "attend_ms_min": round(attend_ms[0], 5), "write_ms_mean": round(sum(write_ms) / K, 5),
                   "wall_s_timed": round(wall, 4), "mode": "hip_graph" if args.graph else "eager",
                   "flush_mib": args.flush_mib, "source_hash": src},
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before the timed ones")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5, 6, 7],
                    help="workload: 1 tiny fp32 decode, 2 batched MHA decode, 3 long GQA decode (default: the "
                         "largest), 4 sliding-window decode, 5 chunked prefill over a shared prefix, 6 decode over "
                         "a compressed-slot tier (window 256, 16 slots), 7 long decode with 8 query heads per "
                         "kv head")
    ap.add_argument("--prefill-config", type=int, default=5, choices=[0, 5],
                    help="with a decode --config, also time this chunked-prefill workload on the same GPU and "
                         "report it under \"prefill\" (0 = skip)")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of back-to-back prefill steps run before the prefill leg's timed steps, after "
                         "its warm-up steps (the MFMA-bound call runs ~20 %% slower until the clocks settle "
                         "under load)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--workers", type=int, default=0, help="decode wavefront workers (0 = automatic)")
    ap.add_argument("--kv", choices=["native", "i8", "fp8"], default="native",
                    help="pools: the workload's dtype (default) or 8-bit INT8 / FP8 E4M3 codes with row "
                         "scales, encoded from the workload's rows on write (decode and prefill workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step's two calls as HIP graphs instead of calling the library per step")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="before every step, overwrite a buffer of this many MiB (evicts L2 and the 256 MiB "
                         "MALL); ms_per_step then sums the per-step events, which exclude the flush")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="copy this many MiB once before the timed steps (scale for HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_MIB"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this command into "
                         "profiles/traffic.json entries and exit")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        return summarize_pmc(args, *args.summarize_pmc)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode and prefill paths "
              "shard by sequence or kv head with no exchange, which this build does not launch.",
              file=sys.stderr)
        return 2

    import torch
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    w = wl.config(args.config, args.seed)
    if args.kv != "native" and w.kind not in ("decode", "prefill"):
        print("8-bit pools (--kv) serve decode and prefill workloads", file=sys.stderr)
        return 2
    settle = args.settle_s if w.kind == "prefill" else 0.0
    leg = run_leg(w, args, args.warmup, args.steps, settle)
    print(f"leg {w.name}: {leg['value']} {leg['unit']} per step, call frac {leg['roofline']['frac']}",
          file=sys.stderr, flush=True)
    pw = None
    pleg = None
    if w.kind == "decode" and args.prefill_config:
        pw = wl.config(args.prefill_config, None)
        pleg = run_leg(pw, args, args.warmup, args.steps, args.settle_s)
        print(f"leg {pw.name}: {pleg['value']} {pleg['unit']} per step, call frac {pleg['roofline']['frac']}",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    rec = {
        "metric": METRIC,
        "value": leg["value"],
        "unit": leg["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": leg["dtype"],
        "data": "synthetic (seeded, shapes and distributions of the workload)",
        "config": leg["config"],
        "roofline": leg["roofline"],
        "timing": leg["timing"],
    }
    if leg["warmup"] != args.warmup:
        rec["timing"]["settle_steps"] = leg["warmup"] - args.warmup
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    if pleg is not None:
        prec = {k: pleg[k] for k in ("value", "unit", "ms_per_step", "steps", "dtype", "config", "roofline",
                                      "timing")}
        prec["warmup"] = args.warmup
        prec["timing"]["settle_steps"] = pleg["warmup"] - args.warmup
        if not args.no_cpu_baseline:
            prec["cpu_baseline"] = cpu_baseline(pw, args.cpu_seconds)
        rec["prefill"] = prec
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
