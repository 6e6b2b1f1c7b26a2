"""Benchmark of the paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step = the whole hot path over one batch: copy_blocks (CoW pairs, if the
workload has any) -> reshape_and_cache (each sequence's new token) ->
paged_attention_decode (partition launch + merge launch). The default workload
is the LLaMA-7B-shape decode batch: 64 sequences, 32 heads x 128, fp16, block
size 16, context lengths uniform in [128, 2048].

Inputs are resident in HBM before timing starts. The pools are replicated R
times at different addresses and the steps rotate through the replicas, so no
step finds the previous step's K/V in the 256 MB last-level cache.

Printed: one JSON line with the step throughput (algorithmic K+V bytes per
second), the decode kernel's roofline fraction from HIP events recorded around
every partition launch inside the timed region, and the CPU oracle timed on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak, 8 TB/s
METRIC = "paged decode attention KV GB/s + seqs/s, % of MI355X HBM peak (LLaMA-7B shape)"
# Sources of the kernels a timed decode launch runs, per path; committed
# counter traffic is used only while their digest matches.
DECODE_SOURCES = ["paged_kv_cache_159_amd/csrc/pkv_decode.hip",
                  "paged_kv_cache_159_amd/csrc/pkv_partition.h",
                  "paged_kv_cache_159_amd/csrc/pkv_launch.h",
                  "paged_kv_cache_159_amd/csrc/pkv_device.h"]
GROUPED_SOURCES = DECODE_SOURCES + ["paged_kv_cache_159_amd/csrc/pkv_grouped.hip",
                                    "paged_kv_cache_159_amd/csrc/pkv_mfma.h"]
# Kernels whose dispatches make up one timed decode launch, per mode.
TIMED_KERNELS = {"plain": ("decode_partition_kernel",),
                 "grouped": ("decode_grouped_kernel", "decode_merge")}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, help="workload index 1..5 (default 2)")
    ap.add_argument("--block-size", type=int, default=16, choices=(8, 16, 32),
                    help="tokens per KV block (default 16; 8 and 32 rebuild the same "
                         "workload's pools and tables at that size)")
    ap.add_argument("--replicas", type=int, default=0, help="pool copies to rotate (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ungrouped", action="store_true",
                    help="shared-prefix workload: use the plain decode instead of the grouped one")
    ap.add_argument("--traffic-summary", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="turn rocprofv3 counter_collection.csv files (FETCH_SIZE and WRITE_SIZE "
                         "runs of this bench, then of --calibrate-copy) into "
                         "profiles/traffic_<workload>.json and .md, and exit (no GPU needed)")
    ap.add_argument("--swap", action="store_true",
                    help="measure swap_blocks instead: half of the workload's sequences "
                         "swapped out to pinned host pools and back (one launch each way), "
                         "next to a contiguous pinned copy of the same bytes; prints its own "
                         "JSON line")
    ap.add_argument("--beam", action="store_true",
                    help="measure beam-search decoding instead: 16 prompts x 8 beams at the "
                         "LLaMA-7B shape, 32 steps of CoW copy + cache write + decode (grouped "
                         "by prompt, grouped by parent, and plain); prints its own JSON line")
    ap.add_argument("--prefill", action="store_true",
                    help="measure paged_attention_prefill instead: whole prompts (8 x "
                         "1024..4096 tokens) and chunks (16 x 512 after 1024..3072 cached), "
                         "LLaMA-7B shape; prints its own JSON line")
    ap.add_argument("--dtype", default="f16", choices=("f16", "bf16"),
                    help="element type of the --prefill workloads")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the fp16 prefill records of the default run")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-workload records (workloads 2-5, 5 warm-up + 50 timed "
                         "decode calls each) that the default run adds to its JSON line")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="turn a rocprofv3 --stats kernel_stats.csv of `bench.py --workload N "
                         "--no-per-config --no-prefill --no-cpu-baseline` into profiles/kernels_<workload>.md "
                         "and exit (no GPU needed)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 plain device copies of 1 GiB (the known-size reference for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_dispatch": n,
                      "bytes_written_per_dispatch": n, "dispatches": 5}), flush=True)


def unique_kv_tokens(w):
    """Distinct (physical block, row) token slots the decode reads: a block
    shared by several sequences (a common prefix) is counted once, with the
    most rows any of its readers uses."""
    rows = np.zeros(w.num_blocks, dtype=np.int64)
    for s in range(w.num_seqs):
        ctx = int(w.context_lens[s])
        n = (ctx + w.block_size - 1) // w.block_size
        r = np.minimum(w.block_size, ctx - w.block_size * np.arange(n))
        np.maximum.at(rows, w.block_tables[s, :n].astype(np.int64), r)
    return int(rows.sum())


def algorithmic_bytes(w):
    """Bytes the method must move, per launch, stated per unit:
    decode: K+V of every distinct valid token slot (num_heads*head_dim*2 B
    each for K and V: 16 KiB per token at 32 x 128 fp16; a shared prefix block
    counts once), the query and output rows, the block-table entries of the
    valid blocks and the context lengths;
    write: each new token's K+V read once and written once, plus its slot;
    copy: each CoW block read once and written once, K and V.
    Also returns the logical decode bytes (every sequence's tokens counted)."""
    kvt = w.kv_bytes_per_token
    rowb = w.num_heads * w.head_dim * 2
    nblocks = int(((w.context_lens.astype(np.int64) + w.block_size - 1) // w.block_size).sum())
    meta = 2 * w.num_seqs * rowb + 4 * nblocks + 4 * w.num_seqs
    decode = unique_kv_tokens(w) * kvt + meta
    logical = w.total_context * kvt + meta
    T = len(w.slot_mapping)
    write = 2 * T * kvt + 8 * T
    copy = len(w.copy_pairs) * (2 * 2 * w.block_size * rowb + 8)
    return decode, write, copy, logical


def _code_only(text):
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that the digest follows the code and not its commentary. String and
    character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(grouped=False):
    """Digest of the code (comments and layout excluded) of the kernels one
    timed decode launch runs."""
    h = hashlib.sha256()
    for p in (GROUPED_SOURCES if grouped else DECODE_SOURCES):
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_key(w, grouped):
    return (w.name + ("" if w.block_size == 16 else f"_bs{w.block_size}") +
            ("_grouped" if grouped else ""))


def _counter_per_dispatch(path):
    """{dispatch id: (kernel name, summed counter value in KiB)} of one
    rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            d = int(row["Dispatch_Id"])
            short = row["Kernel_Name"].split("(")[0].replace("void ", "")
            name, v = out.get(d, (short, 0.0))
            out[d] = (name, v + float(row["Counter_Value"]))
    return out


def traffic_summary(paths, w, grouped):
    """HBM bytes per timed decode launch from FETCH_SIZE / WRITE_SIZE counters,
    each scaled by what the same counter reads for a plain 1 GiB device copy."""
    fetch, write, cal_f, cal_w = (_counter_per_dispatch(p) for p in paths)
    kib = float(1 << 20)                         # 1 GiB in KiB

    def copy_value(c):
        vals = sorted(v for n, v in c.values() if "copy" in n.lower())
        if not vals:
            raise SystemExit("no copy kernel in the calibration counters")
        return float(np.median(vals[-5:]))       # the five 1 GiB copies are the largest

    cf, cw = copy_value(cal_f), copy_value(cal_w)
    ff, fw = kib / cf, kib / cw
    names = TIMED_KERNELS["grouped" if grouped else "plain"]

    def per_launch(c):
        per_kernel = {}
        for n, v in c.values():
            for k in names:
                if k in n:
                    per_kernel.setdefault(n, []).append(v)
        if not per_kernel:
            raise SystemExit(f"no {names} dispatch in the counters")
        return {n: float(np.mean(v)) for n, v in per_kernel.items()}, \
            {n: len(v) for n, v in per_kernel.items()}

    fk, nf = per_launch(fetch)
    wk, _ = per_launch(write)
    fetch_b = sum(fk.values()) * 1024 * ff
    write_b = sum(wk.values()) * 1024 * fw
    dec_b = algorithmic_bytes(w)[0]
    res = {
        "kernels": sorted(fk),
        "workload": f"{w.name} ({w.num_seqs} seqs x {w.num_heads} heads x {w.head_dim}, {w.dtype}, "
                    f"bs {w.block_size}, sum ctx {w.total_context})",
        "mode": "grouped" if grouped else "plain",
        "decode_source_digest": source_digest(grouped),
        "fetch_size_kib_per_dispatch": {n: round(v, 1) for n, v in fk.items()},
        "write_size_kib_per_dispatch": {n: round(v, 1) for n, v in wk.items()},
        "dispatches": nf,
        "calibration": {"reference": "plain 1 GiB device copy (bench.py --calibrate-copy)",
                        "fetch_size_kib": round(cf, 1), "write_size_kib": round(cw, 1),
                        "fetch_factor": round(ff, 5), "write_factor": round(fw, 5)},
        "bytes_per_launch": int(round(fetch_b + write_b)),
        "fetch_bytes_per_launch": int(round(fetch_b)),
        "write_bytes_per_launch": int(round(write_b)),
        "algorithmic_bytes_per_launch": int(dec_b),
        "fetch_over_algorithmic": round(fetch_b / dec_b, 4),
        "counter_files": [os.path.relpath(p, ROOT) for p in paths],
    }
    key = traffic_key(w, grouped)
    with open(os.path.join(ROOT, "profiles", f"traffic_{key}.json"), "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    lines = [f"# HBM traffic of the timed decode launch ({key})", "",
             "rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE`, one counter per run, "
             "then the same two counters over `bench.py --calibrate-copy` (five 1 GiB "
             "device copies). Written by `python bench.py --workload "
             f"{w.index}{' --ungrouped' if (w.group_start is not None and not grouped) else ''}"
             f"{'' if w.block_size == 16 else f' --block-size {w.block_size}'} "
             "--traffic-summary <fetch csv> <write csv> <cal fetch csv> <cal write csv>`.", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | dispatches |",
             "|---|---|---|---|"]
    for n in sorted(fk):
        lines.append(f"| {n} | {fk[n]:,.1f} | {wk.get(n, float('nan')):,.1f} | {nf[n]} |")
    lines += ["", f"Calibration: the 1 GiB copy reads FETCH_SIZE {cf:,.1f} KiB and WRITE_SIZE "
              f"{cw:,.1f} KiB per dispatch, so the factors are {ff:.4f} (fetch) and {fw:.4f} "
              "(write).", "",
              f"Per launch: fetched {fetch_b / 1e9:.4f} GB, written {write_b / 1e6:.2f} MB; "
              f"algorithmic bytes {dec_b / 1e9:.4f} GB; fetch / algorithmic = "
              f"{fetch_b / dec_b:.4f}.", "", "Kernel source digest: "
              f"`{res['decode_source_digest']}`.", "", "Counter runs (repo root, MI355X):", ""]
    ung = " --ungrouped" if (w.group_start is not None and not grouped) else ""
    if w.block_size != 16:
        ung += f" --block-size {w.block_size}"
    run_args = f"--no-per-config --no-prefill --no-cpu-baseline --steps 10 --warmup 2 --workload {w.index}{ung}"
    for ctr, path, prog in (("FETCH_SIZE", paths[0], run_args),
                            ("WRITE_SIZE", paths[1], run_args),
                            ("FETCH_SIZE", paths[2], "--calibrate-copy"),
                            ("WRITE_SIZE", paths[3], "--calibrate-copy")):
        d = os.path.relpath(os.path.dirname(path), ROOT)
        o = os.path.basename(path).split("_counter_collection")[0]
        lines += ["```", f"rocprofv3 --pmc {ctr} --kernel-trace --output-format csv -d {d} -o {o} "
                  f"-- python -u bench.py {prog}", "```"]
    lines.append("")
    with open(os.path.join(ROOT, "profiles", f"traffic_{key}.md"), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(res, indent=1))


PCIE5_X16_GBS = 64.0   # host link of the MI355X platform: PCIe 5.0 x16, per direction


def swap_bench(args, w, dw, dev):
    """swap_blocks bandwidth: device -> pinned host and back, for every other
    sequence's blocks, timed with HIP events on the launch stream."""
    import torch

    import paged_kv_cache_159_amd as pkv
    from workloads import SwapSpace

    alloc = w.allocator
    seqs = list(range(0, w.num_seqs, 2))
    nhost = sum(len(alloc.block_table(s)) for s in seqs)
    sw = SwapSpace(alloc, nhost)
    out_pairs = np.concatenate([sw.swap_out(s) for s in seqs]).astype(np.int32)
    in_pairs = np.concatenate([sw.swap_in(s) for s in seqs]).astype(np.int32)
    shape = (nhost,) + tuple(dw.key_cache.shape[1:])
    hk = torch.empty(shape, dtype=dw.key_cache.dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=dw.key_cache.dtype, pin_memory=True)
    mo = torch.from_numpy(out_pairs).to(dev)
    mi = torch.from_numpy(in_pairs).to(dev)
    nbytes = 2 * len(out_pairs) * w.block_size * w.num_heads * w.head_dim * 2
    flat_dev = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    flat_host = torch.empty(nbytes // 2, dtype=torch.int16, pin_memory=True)

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e-3

    n = max(5, min(args.steps, 50))
    t_out = timed(lambda: pkv.swap_blocks(dw.key_cache, dw.value_cache, hk, hv, mo), n)
    t_in = timed(lambda: pkv.swap_blocks(hk, hv, dw.key_cache, dw.value_cache, mi), n)
    mo_h, mi_h = torch.from_numpy(out_pairs), torch.from_numpy(in_pairs)
    t_out_dma = timed(lambda: pkv.swap_blocks(dw.key_cache, dw.value_cache, hk, hv, mo_h,
                                              method="dma"), n)
    t_in_dma = timed(lambda: pkv.swap_blocks(hk, hv, dw.key_cache, dw.value_cache, mi_h,
                                             method="dma"), n)
    gbs = lambda t: nbytes / t / 1e9
    staged = {}
    for mib in (64, 256):
        stg = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
        t_i = timed(lambda: pkv.swap_blocks(hk, hv, dw.key_cache, dw.value_cache, mi_h,
                                            method="staged", staging=stg), n)
        t_o = timed(lambda: pkv.swap_blocks(dw.key_cache, dw.value_cache, hk, hv, mo_h,
                                            method="staged", staging=stg), n)
        staged[f"{mib}MiB"] = {"swap_in_gbs": round(gbs(t_i), 2), "swap_out_gbs": round(gbs(t_o), 2)}
        del stg
    runs_out = 1 + int(np.count_nonzero(np.any(np.diff(out_pairs, axis=0) != 1, axis=1)))
    runs_in = 1 + int(np.count_nonzero(np.any(np.diff(in_pairs, axis=0) != 1, axis=1)))
    t_d2h = timed(lambda: flat_host.copy_(flat_dev, non_blocking=True), n)
    t_h2d = timed(lambda: flat_dev.copy_(flat_host, non_blocking=True), n)
    res = {
        "metric": "swap_blocks host-link GB/s (swap-out, swap-in)",
        "value": round(gbs(t_out), 2),
        "unit": "GB/s",
        "swap_in_gbs": round(gbs(t_in), 2),
        "blocks_per_direction": int(len(out_pairs)),
        "bytes_per_direction": int(nbytes),
        "swap_out_ms": round(t_out * 1e3, 3),
        "swap_in_ms": round(t_in * 1e3, 3),
        "dma": {"swap_out_gbs": round(gbs(t_out_dma), 2), "swap_in_gbs": round(gbs(t_in_dma), 2),
                "copies_per_pool": {"out": runs_out, "in": runs_in}},
        "staged": staged,
        "contiguous_pinned_copy_gbs": {"d2h": round(gbs(t_d2h), 2), "h2d": round(gbs(t_h2d), 2)},
        "roofline": {"bound": "host link", "peak": PCIE5_X16_GBS, "unit": "GB/s",
                     "frac_out": round(gbs(t_out) / PCIE5_X16_GBS, 4),
                     "frac_in": round(gbs(t_in) / PCIE5_X16_GBS, 4)},
        "config": {"workload": f"{w.name}: every other sequence ({len(seqs)} of {w.num_seqs}), "
                               f"block_size {w.block_size}, {w.dtype}"},
        "data": "synthetic",
    }
    print(json.dumps(res), flush=True)


def unique_rows(tables, ctx, bs, num_blocks):
    """Distinct (physical block, row) slots a decode over these tables reads."""
    rows = np.zeros(num_blocks, dtype=np.int64)
    for s in range(tables.shape[0]):
        n = (int(ctx[s]) + bs - 1) // bs
        r = np.minimum(bs, int(ctx[s]) - bs * np.arange(n))
        np.maximum.at(rows, tables[s, :n].astype(np.int64), r)
    return int(rows.sum())


def beam_bench(args, dev):
    """Beam search over 32 steps: every step's inputs are built on the host and
    uploaded first; then each step (CoW copies, cache write, decode) is timed
    with HIP events. Three decode variants on identical inputs."""
    import torch

    import paged_kv_cache_159_amd as pkv
    from workloads import BeamSearch
    from workloads.device import bits_to_device

    steps = 32
    res = {"metric": "beam-search decode step, unique KV GB/s", "unit": "GB/s", "data": "synthetic"}
    for mode in ("prompt", "parent", "plain"):
        b = BeamSearch(prompts=16, beams=8, steps=steps, dtype="f16", block_size=args.block_size,
                       seed=7, groups="prompt" if mode == "plain" else mode)
        kc = bits_to_device(b.key_cache, b.dtype, dev)
        vc = bits_to_device(b.value_cache, b.dtype, dev)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        plan, ubytes, saving, shared = [], 0, [], []
        kvt = 2 * b.H * b.D * 2
        for _ in range(steps):
            st = b.step()
            plan.append(dict(pairs=up(st.copy_pairs), nk=bits_to_device(st.new_key, b.dtype, dev),
                             nv=bits_to_device(st.new_value, b.dtype, dev), slots=up(st.slot_mapping),
                             q=bits_to_device(st.query, b.dtype, dev), bt=up(st.block_tables),
                             ctx=up(st.context_lens), gs=up(st.group_start), sb=up(st.shared_blocks)))
            ubytes += unique_rows(st.block_tables, st.context_lens, b.bs, b.num_blocks) * kvt
            saving.append(1 - st.blocks_in_use / st.blocks_unshared)
            shared.append(float(np.mean(st.shared_blocks)))
        out = torch.empty_like(plan[0]["q"])
        gws = torch.empty(max(pkv.grouped_workspace_size(b.num_seqs, b.H, b.D, b.max_blocks, b.bs), 16),
                          dtype=torch.uint8, device=dev)
        ws = pkv.alloc_workspace(b.num_seqs, b.H, b.D, b.max_blocks, b.bs, device=dev)

        def run(record):
            evs = []
            for p in plan:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e2 = torch.cuda.Event(enable_timing=True)
                e0.record()
                if p["pairs"].shape[0]:
                    pkv.copy_blocks(kc, vc, p["pairs"])
                pkv.reshape_and_cache(p["nk"], p["nv"], kc, vc, p["slots"])
                e1.record()
                if mode == "plain":
                    pkv.paged_attention_decode(out, p["q"], kc, vc, p["bt"], p["ctx"], b.scale,
                                               workspace=ws)
                else:
                    pkv.paged_attention_decode_grouped(out, p["q"], kc, vc, p["bt"], p["ctx"],
                                                       p["gs"], p["sb"], b.scale, workspace=gws)
                e2.record()
                evs.append((e0, e1, e2))
            torch.cuda.synchronize()
            return evs

        run(False)
        evs = run(True)
        step_us = float(np.sum([a.elapsed_time(c) for a, _, c in evs])) * 1e3 / steps
        dec_us = float(np.sum([b_.elapsed_time(c) for _, b_, c in evs])) * 1e3 / steps
        res[mode] = {"step_us": round(step_us, 2), "decode_us": round(dec_us, 2),
                     "decode_unique_gbs": round(ubytes / steps / (dec_us * 1e-6) / 1e9, 1)}
        res["memory_saving_by_sharing"] = round(float(np.mean(saving)), 4)
        if mode != "plain":
            res[mode]["mean_shared_blocks_per_group"] = round(float(np.mean(shared)), 2)
        del kc, vc, plan
        torch.cuda.empty_cache()
    res["value"] = res["prompt"]["decode_unique_gbs"]
    res["config"] = {"workload": f"beam search: 16 prompts x 8 beams, prompts 256..1024 tokens, "
                                 f"32 steps, 32 heads x 128, f16, block_size {args.block_size}"}
    print(json.dumps(res), flush=True)


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # MI355X dense fp16 / bf16


def prefill_flops(w):
    """Algorithmic flops of the causal prefill: per head, each query at
    position p takes p + 1 keys, 2*D flops each for q.k and for p.v."""
    qs, ctx = w.query_start.astype(np.int64), w.context_lens.astype(np.int64)
    n = np.diff(qs)
    first = ctx - n
    keys = n * first + n * (n + 1) // 2
    return int(4 * w.head_dim * w.num_heads * keys.sum())


def prefill_records(dtype, steps, block_size, dev):
    """Time the two prefill workloads (HIP events, median of up to 30 calls
    after 0.3 s of warm-up); one record per workload."""
    import torch

    import paged_kv_cache_159_amd as pkv
    from workloads import make_prefill_case
    from workloads.device import upload

    rng = np.random.default_rng(2024)
    cases = {
        "whole_prompts": ([int(x) for x in rng.integers(1024, 4096, size=8, endpoint=True)],
                          [0] * 8),
        "chunks_512": ([512] * 16, [int(x) for x in rng.integers(1024, 3072, size=16, endpoint=True)]),
    }
    res = {}
    for name, (chunks, cached) in cases.items():
        w = make_prefill_case(chunks, cached, 32, 128, dtype, seed=len(name),
                              block_size=block_size, name=name)
        dw = upload(w, dev)
        pkv.reshape_and_cache(dw.new_key, dw.new_value, dw.key_cache, dw.value_cache, dw.slot_mapping)
        mq = max(chunks)
        f = lambda: pkv.paged_attention_prefill(dw.out, dw.query, dw.key_cache, dw.value_cache,
                                                dw.block_tables, dw.context_lens, dw.query_start,
                                                w.scale, max_query_len=mq)
        # Warm up for at least 0.3 s of back-to-back calls: building the
        # workload leaves the GPU idle for seconds, and the clock takes longer
        # than a few calls to come back up under this MFMA load (with 3 calls
        # of warm-up the timed calls ran ~14% slower than in steady state).
        t_end = time.perf_counter() + 0.3
        n = 0
        while n < 3 or time.perf_counter() < t_end:
            f()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        evs = []
        for _ in range(max(5, min(steps, 30))):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) * 1e3 for a, b in evs]
        us = float(np.median(times))
        fl = prefill_flops(w)
        tf = fl / (us * 1e-6) / 1e12
        res[name] = {"kernel_us": round(us, 1), "kernel_us_mean": round(float(np.mean(times)), 1),
                     "warmup_calls": n, "flops": fl, "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS[dtype], 4),
                     "tokens": int(sum(chunks)), "tokens_per_s": round(sum(chunks) / (us * 1e-6), 1),
                     "chunks": chunks, "cached": cached}
        del dw
        torch.cuda.empty_cache()
    return res


def prefill_bench(args, dev):
    res = {"metric": "paged prefill attention TFLOP/s (MFMA)", "unit": "TFLOP/s",
           "data": "synthetic", "dtype": args.dtype}
    res.update(prefill_records(args.dtype, args.steps, args.block_size, dev))
    res["value"] = res["whole_prompts"]["tflops"]
    res["roofline"] = {"bound": "mfma", "achieved": res["whole_prompts"]["tflops"],
                       "peak": MFMA_PEAK_TFLOPS[args.dtype], "unit": "TFLOP/s",
                       "frac": res["whole_prompts"]["frac_of_peak"],
                       "kernel": "prefill_kernel"}
    res["config"] = {"workload": f"prefill, 32 heads x 128, {args.dtype}, block_size {args.block_size}"}
    print(json.dumps(res), flush=True)


def load_traffic(key):
    """HBM traffic per decode launch from committed rocprofv3 counter runs,
    only if they were taken on the current decode kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_source_digest") != source_digest(key.endswith("_grouped")):
        return None
    return t.get("bytes_per_launch")


def hbm_context(nbytes=1 << 30, reps=10):
    """Measured HBM rates on this machine, as context for the 8 TB/s peak: a
    device-to-device copy of a 1 GiB buffer (bytes read + written per second)
    and a read-only pass over it (torch's fp32 sum). Medians of HIP events;
    nothing here is part of the timed decode."""
    import torch
    src = torch.randn(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    def med(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([x.elapsed_time(y) for x, y in ts])) * 1e-3
    t_copy = med(lambda: dst.copy_(src))
    t_read = med(lambda: src.sum())
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * nbytes / t_copy / 1e9, 1),
            "read_gbs": round(nbytes / t_read / 1e9, 1),
            "what": "1 GiB device copy (read + write bytes) and read-only sum, median of "
                    f"{reps} HIP-event timings; context for the 8 TB/s peak, not the denominator"}


def cpu_baseline(w, budget_s):
    """The float64 oracle (as it is) on whole sequences of the same workload,
    one thread, until about budget_s seconds of CPU work; scaled to K+V GB/s."""
    from threadpoolctl import threadpool_limits

    import oracle
    t0 = time.perf_counter()
    done_tokens = 0
    done_seqs = 0
    K, V = w.key_cache, w.value_cache
    if len(w.copy_pairs):
        K, V = oracle.copy_blocks(K, V, w.copy_pairs)
    K, V = oracle.reshape_and_cache(w.new_key, w.new_value, K, V, w.slot_mapping, w.block_size)
    t_prep = time.perf_counter() - t0
    t0 = time.perf_counter()
    passes = 0
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < budget_s:
            for s in range(w.num_seqs):
                pairs = [(s, h) for h in range(w.num_heads)]
                oracle.paged_attention_decode(w.query, K, V, w.block_tables, w.context_lens,
                                              w.scale, w.block_size, w.dtype, pairs=pairs)
                done_tokens += int(w.context_lens[s])
                done_seqs += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            passes += 1
    el = time.perf_counter() - t0
    gbs = done_tokens * w.kv_bytes_per_token / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 numpy oracle, one thread: {done_seqs} sequence decodes (all "
                      f"{w.num_heads} heads each; {passes} pass(es) over the {w.num_seqs} sequences, "
                      f"{done_tokens} tokens) in {el:.1f} s; host cache write/copy prep "
                      f"{t_prep:.1f} s not counted",
            "seqs_per_s": round(done_seqs / el, 4)}


# Workload and host-side cache state for the forked oracle workers (set by
# cpu_baseline_pool just before the fork; the children read it, never the GPU).
_CPU_STATE = None


def _cpu_pool_worker(wid):
    from threadpoolctl import threadpool_limits

    import oracle
    w, K, V, workers, budget_s = _CPU_STATE
    tokens = seqs = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < budget_s:
            for s in range(wid, w.num_seqs, workers):
                pairs = [(s, h) for h in range(w.num_heads)]
                oracle.paged_attention_decode(w.query, K, V, w.block_tables, w.context_lens,
                                              w.scale, w.block_size, w.dtype, pairs=pairs)
                tokens += int(w.context_lens[s])
                seqs += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
    return tokens, seqs


def cpu_baseline_pool(w, budget_s):
    """The same float64 oracle on all host cores (at most 16 worker processes,
    one thread each, sequences dealt round-robin), for about budget_s seconds.
    Must run before this process touches the GPU: the workers are forked and
    never hold a GPU handle."""
    import multiprocessing as mp

    import oracle
    global _CPU_STATE
    K, V = w.key_cache, w.value_cache
    if len(w.copy_pairs):
        K, V = oracle.copy_blocks(K, V, w.copy_pairs)
    K, V = oracle.reshape_and_cache(w.new_key, w.new_value, K, V, w.slot_mapping, w.block_size)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    _CPU_STATE = (w, K, V, workers, budget_s)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        parts = pool.map(_cpu_pool_worker, range(workers))
    el = time.perf_counter() - t0
    _CPU_STATE = None
    tokens = sum(p[0] for p in parts)
    seqs = sum(p[1] for p in parts)
    gbs = tokens * w.kv_bytes_per_token / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"float64 numpy oracle, {workers} processes x 1 thread (sequences dealt "
                      f"round-robin): {seqs} sequence decodes (all {w.num_heads} heads each, "
                      f"{tokens} tokens) in {el:.1f} s wall, pool start included",
            "seqs_per_s": round(seqs / el, 4)}


def make_replicas(dw, pkv, w, dev, min_total=4.0e9, max_r=16):
    """The pools and one output per replica: R copies of the K/V pools at
    different addresses (at least min_total bytes in all), so that rotating
    through them finds no K/V in the 256 MB last-level cache."""
    import torch
    pool_bytes = 2 * dw.key_cache.numel() * 2
    R = min(max_r, max(2, int(np.ceil(min_total / pool_bytes))))
    kcs = [dw.key_cache] + [dw.key_cache.clone() for _ in range(R - 1)]
    vcs = [dw.value_cache] + [dw.value_cache.clone() for _ in range(R - 1)]
    outs = [torch.empty_like(dw.query) for _ in range(R)]
    return R, kcs, vcs, outs


def _pct(x):
    return {k: round(float(np.percentile(x, q)), 2) for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}


def per_config_record(index, dev, runs=50, warmup=5, block_size=16):
    """One workload's decode step timed call by call with HIP events on the
    launch stream: copy_blocks | reshape_and_cache | decode kernel | merge,
    5 warm-up and 50 timed steps over rotated pool replicas. Reports the
    median (p10, p90) of each part, the decode's algorithmic bytes per second
    against the 8 TB/s peak (whole decode call, and its dominant kernel), and
    sequences per second. Workload 4 runs the grouped call (its kernel and
    merge are one call, timed together)."""
    import torch

    import paged_kv_cache_159_amd as pkv
    from workloads import make_config
    from workloads.device import upload

    w = make_config(index, block_size)
    dw = upload(w, dev)
    R, kcs, vcs, outs = make_replicas(dw, pkv, w, dev)
    grouped = w.group_start is not None
    if grouped:
        gs = torch.from_numpy(w.group_start).to(dev)
        sb = torch.from_numpy(w.shared_blocks).to(dev)
        ws = torch.empty(max(pkv.grouped_workspace_size(w.num_seqs, w.num_heads, w.head_dim,
                                                        w.max_blocks_per_seq, w.block_size), 16),
                         dtype=torch.uint8, device=dev)
    else:
        ws = pkv.alloc_workspace(w.num_seqs, w.num_heads, w.head_dim, w.max_blocks_per_seq,
                                 w.block_size, device=dev)
    has_copy = len(w.copy_pairs) > 0
    evs = []

    def one(i, record):
        r = i % R
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        rec = (lambda j: e[j].record()) if record else (lambda j: None)
        rec(0)
        if has_copy:
            pkv.copy_blocks(kcs[r], vcs[r], dw.copy_pairs)
        rec(1)
        pkv.reshape_and_cache(dw.new_key, dw.new_value, kcs[r], vcs[r], dw.slot_mapping)
        rec(2)
        if grouped:
            pkv.paged_attention_decode_grouped(outs[r], dw.query, kcs[r], vcs[r], dw.block_tables,
                                               dw.context_lens, gs, sb, w.scale, workspace=ws)
            rec(3)
        else:
            pkv.paged_attention_decode_partitions(outs[r], dw.query, kcs[r], vcs[r],
                                                  dw.block_tables, dw.context_lens, w.scale, ws)
            rec(3)
            pkv.paged_attention_decode_merge(outs[r], dw.context_lens, w.max_blocks_per_seq, ws,
                                             block_size=w.block_size)
        rec(4)
        if record:
            evs.append(e)

    for i in range(warmup):
        one(i, False)
    torch.cuda.synchronize()
    for i in range(runs):
        one(i, True)
    torch.cuda.synchronize()
    t = np.array([[a.elapsed_time(b) * 1e3 for a, b in zip(e[:-1], e[1:])] for e in evs])
    copy_us, write_us, kern_us, merge_us = t[:, 0], t[:, 1], t[:, 2], t[:, 3]
    call_us = kern_us + merge_us
    dec_b, write_b, copy_b, logical_b = algorithmic_bytes(w)
    kmed, cmed = float(np.median(kern_us)), float(np.median(call_us))
    traffic = load_traffic(traffic_key(w, grouped))
    rec = {
        "workload": f"{w.name}: {w.num_seqs} seqs x {w.num_heads} heads x {w.head_dim}, {w.dtype}, "
                    f"block_size {w.block_size}, sum(ctx)={w.total_context}, "
                    f"{len(w.slot_mapping)} new tokens, {len(w.copy_pairs)} CoW pairs",
        "decode_path": "grouped (shared-prefix MFMA units + tail partitions, then merge)" if grouped
                       else "plain (partition kernel, then merge)",
        "runs": runs, "warmup": warmup, "pool_replicas": R,
        "algorithmic_bytes": int(dec_b),
        "decode_call_us": _pct(call_us),
        "decode_kernel_us": _pct(kern_us) if not grouped else None,
        "decode_call_gbs": round(dec_b / (cmed * 1e-6) / 1e9, 1),
        "decode_call_frac": round(dec_b / (cmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_kernel_gbs": round(dec_b / (kmed * 1e-6) / 1e9, 1) if not grouped else None,
        "decode_kernel_frac": (round(dec_b / (kmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                               if not grouped else None),
        "seqs_per_s": round(w.num_seqs / (cmed * 1e-6), 1),
        "traffic_bytes": traffic,
        "traffic_over_algorithmic": round(traffic / dec_b, 4) if traffic else None,
        "cache_write_us": _pct(write_us),
        "cache_write_gbs": round(write_b / (float(np.median(write_us)) * 1e-6) / 1e9, 1),
    }
    if grouped:
        rec["logical_bytes"] = int(logical_b)
        rec["decode_call_logical_gbs"] = round(logical_b / (cmed * 1e-6) / 1e9, 1)
    if has_copy:
        rec["copy_blocks_us"] = _pct(copy_us)
        rec["copy_blocks_gbs"] = round(copy_b / (float(np.median(copy_us)) * 1e-6) / 1e9, 1)
    del kcs, vcs, outs, dw, ws
    torch.cuda.empty_cache()
    return rec


def stats_summary(csv_path, w, grouped):
    """profiles/kernels_<workload>.md from a rocprofv3 kernel_stats.csv of
    `bench.py --workload N --no-per-config --no-prefill --no-cpu-baseline`: the kernel
    table, and the decode kernels' algorithmic bytes over their average
    duration against the 8 TB/s peak."""
    import csv
    rows = []
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            name = r["Name"].split("(")[0].replace("void ", "")
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    dec_b = algorithmic_bytes(w)[0]
    names = TIMED_KERNELS["grouped" if grouped else "plain"]
    timed = [r for r in rows if any(k in r[0] for k in names)]
    us = sum(r[2] for r in timed)
    key = traffic_key(w, grouped)
    ung = "" if w.block_size == 16 else f" --block-size {w.block_size}"
    lines = [f"# rocprofv3 kernel stats: {key}", "",
             f"Workload: {w.name}, {w.num_seqs} sequences x {w.num_heads} heads x {w.head_dim}, "
             f"{w.dtype} KV, block size {w.block_size}, sum of contexts {w.total_context:,}, "
             f"{len(w.slot_mapping)} new tokens, {len(w.copy_pairs)} CoW pairs. One step = "
             f"{'copy_blocks + ' if len(w.copy_pairs) else ''}reshape_and_cache + "
             f"{'grouped decode (shared-prefix MFMA units and tail partitions) + merge' if grouped else 'decode partition launch + merge launch'}; "
             "pool replicas rotated.", "",
             "Command (repo root, MI355X):", "", "```",
             "rocprofv3 --kernel-trace --stats --output-format csv -d "
             f"{os.path.relpath(os.path.dirname(os.path.abspath(csv_path)), ROOT)} -o "
             f"{os.path.basename(csv_path).split('_kernel_stats')[0]} -- python -u bench.py "
             f"--workload {w.index}{ung} --no-per-config --no-prefill --no-cpu-baseline", "```", "",
             f"Decode kernel source digest (bench.py `source_digest`): `{source_digest(grouped)}`.", "",
             "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|"]
    for n, c, a, mn, mx, pc in rows:
        lines.append(f"| `{n}` | {c} | {a:.2f} | {mn:.2f} | {mx:.2f} | {pc:.1f}% |")
    lines += ["", "Kernels outside the step (`__amd_rocclr_copyBuffer`, `fillBuffer`, torch's "
              "`reduce_kernel` and random fills) are the uploads, the replica copies and the "
              "measured-HBM context of bench.py.", "",
              f"Algorithmic bytes of one decode launch: {dec_b:,} B. Timed kernels: "
              f"{', '.join(r[0] for r in timed)}; average {us:.2f} us in all: "
              f"{dec_b / (us * 1e-6) / 1e12:.3f} TB/s = {dec_b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f} "
              "of the 8 TB/s HBM peak.", ""]
    out = os.path.join(ROOT, "profiles", f"kernels_{key}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.beam or args.prefill:
        import torch
        torch.cuda.set_device(0)
        (beam_bench if args.beam else prefill_bench)(args, torch.device("cuda", 0))
        return
    if args.traffic_summary:
        sys.path.insert(0, ROOT)
        from workloads import make_config
        w = make_config(args.workload, args.block_size)
        traffic_summary(args.traffic_summary, w, w.group_start is not None and not args.ungrouped)
        return
    if args.stats_summary:
        sys.path.insert(0, ROOT)
        from workloads import make_config
        w = make_config(args.workload, args.block_size)
        stats_summary(args.stats_summary, w, w.group_start is not None and not args.ungrouped)
        return

    sys.path.insert(0, ROOT)
    from workloads import make_config

    t0 = time.time()
    w = make_config(args.workload, args.block_size)
    print(f"[bench] workload {w.index} {w.name}: S={w.num_seqs} H={w.num_heads} D={w.head_dim} "
          f"{w.dtype} NB={w.num_blocks} sum(ctx)={w.total_context} generated in {time.time() - t0:.1f} s",
          file=sys.stderr, flush=True)
    pool_baseline = None
    if not args.no_cpu_baseline:
        # before any GPU call: the oracle's worker processes are forked from here
        pool_baseline = cpu_baseline_pool(w, args.cpu_seconds)
        print(f"[bench] oracle on {pool_baseline['cores']} cores: {pool_baseline['value']} GB/s",
              file=sys.stderr, flush=True)

    import torch
    import paged_kv_cache_159_amd as pkv
    from workloads.device import upload

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    pkv.lib()
    dw = upload(w, dev)
    if args.swap:
        swap_bench(args, w, dw, dev)
        return
    pool_bytes = 2 * dw.key_cache.numel() * 2
    if args.replicas:
        R, kcs, vcs, outs = make_replicas(dw, pkv, w, dev, min_total=args.replicas * pool_bytes)
    else:
        R, kcs, vcs, outs = make_replicas(dw, pkv, w, dev)
    ws = pkv.alloc_workspace(w.num_seqs, w.num_heads, w.head_dim, w.max_blocks_per_seq,
                             w.block_size, device=dev)
    dec_b, write_b, copy_b, logical_b = algorithmic_bytes(w)
    step_bytes = dec_b + write_b + copy_b
    has_copy = len(w.copy_pairs) > 0
    print(f"[bench] {R} pool replicas of {pool_bytes / 1e9:.2f} GB; algorithmic bytes/step: "
          f"decode {dec_b} write {write_b} copy {copy_b}", file=sys.stderr, flush=True)

    ev = []
    grouped = w.group_start is not None and not args.ungrouped
    if grouped:
        gs = torch.from_numpy(w.group_start).to(dev)
        sb = torch.from_numpy(w.shared_blocks).to(dev)
        gws = torch.empty(max(pkv.grouped_workspace_size(w.num_seqs, w.num_heads, w.head_dim,
                                                         w.max_blocks_per_seq, w.block_size), 16),
                          dtype=torch.uint8, device=dev)

    def step(i, record):
        r = i % R
        kc, vc = kcs[r], vcs[r]
        if has_copy:
            pkv.copy_blocks(kc, vc, dw.copy_pairs)
        pkv.reshape_and_cache(dw.new_key, dw.new_value, kc, vc, dw.slot_mapping)
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        if grouped:
            # shared-prefix MFMA launch + tail partitions + merge, timed together
            pkv.paged_attention_decode_grouped(outs[r], dw.query, kc, vc, dw.block_tables,
                                               dw.context_lens, gs, sb, w.scale, workspace=gws)
            if record:
                e1.record()
                ev.append((e0, e1))
            return
        pkv.paged_attention_decode_partitions(outs[r], dw.query, kc, vc, dw.block_tables,
                                              dw.context_lens, w.scale, ws)
        if record:
            e1.record()
            ev.append((e0, e1))
        pkv.paged_attention_decode_merge(outs[r], dw.context_lens, w.max_blocks_per_seq, ws,
                                         block_size=w.block_size)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = wall / args.steps * 1e3
    dec_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    dec_avg_us = float(np.mean(dec_us))
    dec_med_us = float(np.median(dec_us))
    achieved = dec_b / (dec_med_us * 1e-6) / 1e9
    value = step_bytes / (ms * 1e-3) / 1e9
    print(f"[bench] {ms * 1e3:.1f} us/step; partition kernel median {dec_med_us:.1f} us, avg {dec_avg_us:.1f} us "
          f"(p10 {np.percentile(dec_us, 10):.1f}, p90 {np.percentile(dec_us, 90):.1f}) -> "
          f"{achieved:.0f} GB/s = {achieved / HBM_PEAK_GBS:.3f} of peak", file=sys.stderr, flush=True)

    traffic = load_traffic(traffic_key(w, grouped))
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, seeded shuffled block tables)",
        "config": {
            "workload": f"{w.name}: {w.num_seqs} seqs x {w.num_heads} heads x {w.head_dim}, {w.dtype} KV, "
                        f"block_size {w.block_size}, sum(ctx)={w.total_context}, "
                        f"{len(w.slot_mapping)} new tokens, {len(w.copy_pairs)} CoW pairs",
            "global_batch": w.num_seqs,
            "max_context": int(w.context_lens.max()),
            "parallelism": "single GPU",
        },
        "seqs_per_s": round(w.num_seqs / (ms * 1e-3), 1),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "decode_partition_us": round(dec_med_us, 2),
        "decode_partition_us_mean": round(dec_avg_us, 2),
        "decode_partition_us_pct": {k: round(float(np.percentile(dec_us, q)), 2)
                                    for k, q in (("p10", 10), ("p50", 50), ("p90", 90))},
        "decode_logical_kv_gbs": round(logical_b / (dec_med_us * 1e-6) / 1e9, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "grouped decode (shared-prefix MFMA + tail partitions + merge)" if grouped
                      else "decode_partition_kernel",
            "bytes_per_launch": dec_b,
            "duration": "median of the HIP-event durations of the timed region's launches",
        },
    }
    del kcs, vcs, outs, ws
    torch.cuda.empty_cache()
    if not args.no_per_config and args.block_size == 16:
        res["per_config"] = {}
        for idx in (2, 3, 4, 5):
            res["per_config"][str(idx)] = per_config_record(idx, dev)
            rc_ = res["per_config"][str(idx)]
            print(f"[bench] workload {idx}: decode call {rc_['decode_call_us']['p50']} us -> "
                  f"{rc_['decode_call_frac']:.3f} of peak, {rc_['seqs_per_s']:.0f} seqs/s",
                  file=sys.stderr, flush=True)
    if not args.no_prefill and args.block_size == 16:
        # f4 beside the decode records: fp16 prefill on MFMA (the --prefill run's workloads)
        pf = prefill_records("f16", 30, 16, dev)
        res["prefill_f16"] = {k: {f: v[f] for f in ("kernel_us", "tflops", "frac_of_peak", "tokens",
                                                    "tokens_per_s")}
                              for k, v in pf.items()}
        for k, v in res["prefill_f16"].items():
            print(f"[bench] prefill {k}: {v['kernel_us']} us -> {v['tflops']} TFLOP/s = "
                  f"{v['frac_of_peak']:.3f} of the MFMA peak", file=sys.stderr, flush=True)
    res["hbm_measured"] = hbm_context()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        res["cpu_baseline_all_cores"] = pool_baseline
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
