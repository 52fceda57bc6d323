"""Bench: one GPU's share of a Ulysses-4 attention layer at the Wan2.1 shape, on MI355X.

Workload (synthetic, seeded, N(0,1) bf16): global q/k/v [1, 27280, 40, 128]
cut into 4 rank shards [1, 6820, 40, 128].  One step = the whole hot path
for one simulated rank's 10 heads: pack (all head groups, one launch) ->
attention per head group (N = 27280, non-causal, fp32 LSE) -> unpack back
into the 4 output shards.  Steps cycle over the 4 simulated ranks so the
repack does not re-read one rank's bytes from cache.

`value` = attention TFLOP/s of the whole step (4*N^2*D*heads per step over
the step time, pack and unpack included).  The JSON line also carries the
attention launch's own rate (`roofline`: HIP events around each launch on the
launch stream; a launch is the attention kernel plus, under the automatic
range split, its merge kernel), the repack GB/s, the same steps under the two-stream group
pipeline (ulys_rank_pipeline; `--pipeline` times that one instead), a plain
device copy rate, and the CPU oracle timed on a bounded sample
(`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
ATTN_KERNEL = "attn_fwd_kernel<128, false, false>"   # D = 128, bf16 q/k, no key mask
MERGE_KERNEL = "range_merge_kernel<128>"             # the range split's merge, when the call uses one


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--groups", type=int, default=5, help="head groups per rank (5 = 2-head groups, run one at a time; 1 = one call over all 10 heads)")
    ap.add_argument("--pipeline", action="store_true",
                    help="time ulys_rank_pipeline (per-group repack on a second stream overlapping attention) "
                         "instead of the one-stream step (pack all groups, attend each, unpack all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=12288, help="query rows the oracle computes for cpu_baseline")
    ap.add_argument("--group-sweep", action="store_true",
                    help="time a rank's 10 heads (D=128) as G = 1, 2, 5, 10 attention calls for several sequence "
                         "lengths and print the automatic group count beside (calibrates ulys_auto_groups)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (HBM byte-counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="read the rocprofv3 runs under DIR (stats_g{1,5}, fetch_/write_ g1, g5 and copy), "
                         "write profiles/attn_fwd_traffic.json and print the summary tables (no GPU needed)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "ulysses_sequence_attention_amd", "csrc", f)
                  for f in ("attn.hip", "internal.h")]


def kernel_source_hash() -> str:
    """Hash of the attention kernel's sources and compile flags: counters taken
    on another version of the kernel are not reported as its traffic."""
    import hashlib
    from ulysses_sequence_attention_amd import build as ubuild
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(ubuild.FLAGS + ubuild.SOURCE_FLAGS.get("attn.hip", [])).encode())
    return h.hexdigest()


def measured_traffic(groups: int):
    """HBM bytes per attention launch from the stored rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, each scaled by the same counter's reading for a plain copy
    of known size; None when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = t.get("per_groups", {}).get(str(groups))
    if entry is None or t.get("source_sha256") != kernel_source_hash():
        return None
    return entry["hbm_bytes_per_launch"]


def fp8_attention(torch, ulys, L, shards, qs, os_, lse, flops_launch: float, steps: int) -> dict:
    """The same attention launches with e4m3 q/k: amax over the shards, the fp8 pack of rank 0's
    slots, then `steps` timed rounds of the G launches (HIP events).  Reported beside the bf16
    figure; the headline stays bf16."""
    amax = torch.zeros(2, dtype=torch.float32, device=qs.device)
    ulys.ulys_amax_bf16(shards["q"], amax[0:1])
    ulys.ulys_amax_bf16(shards["k"], amax[1:2])
    q8 = torch.empty(qs.shape, dtype=torch.uint8, device=qs.device)
    k8 = torch.empty_like(q8)
    v16 = torch.empty_like(qs)
    ulys.ulys_pack(L, 0, -1, shards["q"], shards["k"], shards["v"], q8, k8, v16,
                   qk_dtype=ulys.ULYS_FP8_E4M3, qk_amax=amax)
    G = qs.shape[0]
    run = lambda: [ulys.ulys_attend_group(q8[g], k8[g], v16[g], os_[g], lse[g], qk_dtype=ulys.ULYS_FP8_E4M3,
                                          qk_amax=amax) for g in range(G)]
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps / G
    return {"launch_ms": round(ms, 4), "tflops_bf16_equivalent": round(flops_launch / (ms * 1e-3) / 1e12, 2),
            "note": "e4m3 q/k (QK^T at the fp8 MFMA rate), bf16 V and P; FLOPs counted as for bf16"}


def merge_gbs(torch, ulys, o_slots, lse, steps: int) -> float:
    """ulys_lse_merge of the G head-group outputs taken as G partial results of one slot shape
    (a ring of G): algorithmic bytes (G partial o + lse read, one o + lse written) over the mean
    event time."""
    G = o_slots.shape[0]
    if G < 2:
        return float("nan")
    parts, lparts = [o_slots[g] for g in range(G)], [lse[g] for g in range(G)]
    out = torch.empty_like(o_slots[0])
    lout = torch.empty_like(lse[0])
    ulys.ulys_lse_merge(parts, lparts, out, lout)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        ulys.ulys_lse_merge(parts, lparts, out, lout)
    e1.record()
    torch.cuda.synchronize()
    nbytes = (G + 1) * (out.numel() * 2 + lout.numel() * 4)
    return nbytes / (e0.elapsed_time(e1) / steps * 1e-3) / 1e9


def device_copy_gbs(torch) -> float:
    """Practical HBM ceiling for a stream: a plain 1 GiB device-to-device copy
    (torch copy_), read + write bytes over the median of 5 timed copies."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del src, dst
    return 2 * n / (sorted(times)[2] * 1e-3) / 1e9


def group_sweep():
    """One JSON line per sequence length: attention time of 10 heads split into G calls (with the
    automatic key-range or range split, and with none), the split counts and the group count
    ulys_auto_groups picks for that shape (Wan-like layout, Ulysses degree 4)."""
    import torch
    from ulysses_sequence_attention_amd import ulys
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gen = torch.Generator(device="cpu").manual_seed(0)
    for rows in (2048, 4096, 8192, 16384, 27280):
        times = {0: {}, 1: {}}
        for splits in (0, 1):
            for gh in (10, 5, 2, 1):
                G = 10 // gh
                q = torch.randn((G, 1, rows, gh, 128), generator=gen).to(torch.bfloat16).cuda()
                k, v = q.roll(1, dims=2), q.roll(2, dims=2)
                o = torch.empty_like(q)
                lse = torch.empty((G, 1, gh, rows), device="cuda")
                run = lambda: [ulys.ulys_attend_group_ex(q[g], k[g], v[g], o[g], lse[g], key_splits=splits)
                               for g in range(G)]
                for _ in range(3):
                    run()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    run()
                e1.record()
                torch.cuda.synchronize()
                times[splits][G] = e0.elapsed_time(e1) / 10
        t = times[0]
        L = ulys.Layout(1, 4, rows // 4, 0, True, 40, 40, 128, 1)
        print(json.dumps({"rows": rows, "heads": 10, "cus": cus,
                          "key_splits": ulys.ulys_attend_splits(1, rows, rows, cus),
                          "range_split": ulys.ulys_attend_ranges(1, rows, rows, cus),
                          "ms_by_groups": {str(G): round(x, 4) for G, x in sorted(t.items())},
                          "relative_to_one_call": {str(G): round(x / t[1], 3) for G, x in sorted(t.items())},
                          "ms_by_groups_unsplit": {str(G): round(x, 4) for G, x in sorted(times[1].items())},
                          "auto_groups": ulys.ulys_auto_groups(L, cus)}), flush=True)


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, five times: reads 1 GiB and
    writes 1 GiB per launch.  Run under `rocprofv3 --pmc FETCH_SIZE` (then
    WRITE_SIZE) to get the counters' KiB per byte moved."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def summarize_profiles(d: str):
    """rocprofv3 runs -> profiles/attn_fwd_traffic.json + markdown tables on stdout.

    Expects under ``d``: stats_g1, stats_g5 (``--kernel-trace --stats``), fetch_g1, write_g1,
    fetch_g5, write_g5 (``--pmc FETCH_SIZE`` / ``WRITE_SIZE`` of the bench at G = 1, 5) and
    fetch_copy, write_copy (the same counters on ``--copy-calibration``), each with
    ``-o run --output-format csv``."""
    import csv
    import statistics

    def rows_of(sub, fname):
        path = os.path.join(d, sub, fname)
        with open(path) as fh:
            return list(csv.DictReader(fh))

    def counter(sub, name, kernel_substr):
        vals = {}
        for r in rows_of(sub, "run_counter_collection.csv"):
            if r["Counter_Name"] == name and kernel_substr in r["Kernel_Name"]:
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not vals:
            raise SystemExit(f"no {name} rows for {kernel_substr} in {sub}")
        return statistics.mean(vals.values()), len(vals)

    attn = "attn_fwd_kernel<128, false, false>"
    print("## Kernel statistics (rocprofv3 --kernel-trace --stats)\n")
    for G in (1, 5):
        print(f"### G = {G}\n\n| kernel | calls | total ms | avg us | min us | max us | % |\n|---|---|---|---|---|---|---|")
        for r in rows_of(f"stats_g{G}", "run_kernel_stats.csv"):
            name = r["Name"].replace("ulys::(anonymous namespace)::", "").replace("(ulys::AttnArgs)", "")
            print(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                  f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
        print()
    fcopy, ncopy = counter("fetch_copy", "FETCH_SIZE", "copyBuffer")
    wcopy, _ = counter("write_copy", "WRITE_SIZE", "copyBuffer")
    n = 1 << 30
    fscale, wscale = n / (fcopy * 1024), n / (wcopy * 1024)
    out = {"kernel": attn + " + range_merge_kernel<128> (when the launch takes a range split)",
           "workload": "Wan2.1 Ulysses-4 share: q/k/v slots [1,27280,10/G,128] bf16, non-causal, LSE",
           "source_sha256": kernel_source_hash(),
           "calibration": {"copy": f"__amd_rocclr_copyBuffer of 1 GiB (torch copy_), {ncopy} dispatches",
                           "fetch_kib_per_dispatch": round(fcopy, 3), "write_kib_per_dispatch": round(wcopy, 3),
                           "fetch_bytes_per_counted_byte": round(fscale, 5),
                           "write_bytes_per_counted_byte": round(wscale, 5)},
           "per_groups": {}}
    print("## HBM bytes per dispatch (FETCH_SIZE, WRITE_SIZE; scaled by the 1 GiB copy)\n")
    print(f"Calibration: FETCH_SIZE {fcopy:.1f} KiB and WRITE_SIZE {wcopy:.1f} KiB per 1 GiB copy "
          f"-> {fscale:.5f} and {wscale:.5f} bytes per counted byte.\n")
    print("| kernel | G | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | write bytes | algorithmic read / write | read / algorithmic |")
    print("|---|---|---|---|---|---|---|---|")
    rows = 27280
    for G in (1, 5):
        heads = 10 // G
        f, _ = counter(f"fetch_g{G}", "FETCH_SIZE", attn)
        w_, _ = counter(f"write_g{G}", "WRITE_SIZE", attn)
        try:   # the range split's merge belongs to the launch
            fm, _ = counter(f"fetch_g{G}", "FETCH_SIZE", "range_merge_kernel<128>")
            wm, _ = counter(f"write_g{G}", "WRITE_SIZE", "range_merge_kernel<128>")
        except SystemExit:
            fm = wm = 0.0
        print(f"| `range_merge_kernel<128>` | {G} | {fm:.1f} | {wm:.1f} | {fm * 1024 * fscale:.4g} | "
              f"{wm * 1024 * wscale:.4g} | | |")
        f, w_ = f + fm, w_ + wm
        rd, wr = f * 1024 * fscale, w_ * 1024 * wscale
        alg_r = 3 * rows * heads * 128 * 2
        alg_w = rows * heads * 128 * 2 + rows * heads * 4
        out["per_groups"][str(G)] = {"heads_per_launch": heads, "fetch_kib_per_dispatch": round(f, 2),
                                     "write_kib_per_dispatch": round(w_, 2), "hbm_read_bytes": int(rd),
                                     "hbm_write_bytes": int(wr), "hbm_bytes_per_launch": int(rd + wr),
                                     "algorithmic_read_bytes": alg_r, "algorithmic_write_bytes": alg_w,
                                     "read_over_algorithmic": round(rd / alg_r, 2)}
        print(f"| launch (`{attn}` + merge) | {G} | {f:.1f} | {w_:.1f} | {rd:.4g} | {wr:.4g} | "
              f"{alg_r:.4g} / {alg_w:.4g} | {rd / alg_r:.2f} |")
        for kname, alg in (("pack_kernel", None), ("unpack_kernel", None)):
            try:
                fk, nk = counter(f"fetch_g{G}", "FETCH_SIZE", kname)
                wk, _ = counter(f"write_g{G}", "WRITE_SIZE", kname)
            except SystemExit:
                continue
            print(f"| `{kname}` | {G} | {fk:.1f} | {wk:.1f} | {fk * 1024 * fscale:.4g} | {wk * 1024 * wscale:.4g} | | |")
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(f"\nwrote {TRAFFIC_FILE}")


def cpu_baseline(q, k, v, rows_sample: int):
    """The oracle as it stands (fp64 NumPy), on a bounded sample of the same workload:
    attention for `rows_sample` query rows of all 10 heads of rank 0 over all 27280 keys."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import layout as olay

    heads = list(range(10))
    qn = q[:, :, heads].double().numpy()
    kn = k[:, :, heads].double().numpy()
    vn = v[:, :, heads].double().numpy()
    n = qn.shape[1]
    rows = np.linspace(0, n - 1, rows_sample).astype(np.int64)
    t0 = time.perf_counter()
    oatt.attention(qn, kn, vn, oatt.default_scale(128), rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * rows_sample * n * 128 * len(heads)
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 NumPy attention, {rows_sample} of 27280 query rows x 10 heads x all 27280 keys "
                      f"(D=128), {dt:.1f} s"}


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.group_sweep:
        group_sweep()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from ulysses_sequence_attention_amd import inputs, ulys

    G = args.groups
    w = inputs.E2E_P4
    P, S_l, H, D = w.degree, w.s_local, w.hq, w.head_dim
    L = ulys.Layout(1, P, S_l, 0, True, H, H, D, G)
    rows = L.rows
    gh = L.gq
    q, k, v = inputs.global_qkv(w)          # CPU bf16 [1, 27280, 40, 128]
    dev = torch.device("cuda:0")
    shards = {n: [x[:, p * S_l:(p + 1) * S_l].contiguous().to(dev) for p in range(P)]
              for n, x in (("q", q), ("k", k), ("v", v))}
    slot_shape = (G, 1, rows, gh, D)
    qs = torch.empty(slot_shape, dtype=torch.bfloat16, device=dev)
    ks = torch.empty_like(qs)
    vs = torch.empty_like(qs)
    os_ = torch.empty_like(qs)
    lse = torch.empty((G, 1, gh, rows), dtype=torch.float32, device=dev)
    out = [torch.empty_like(s) for s in shards["q"]]
    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream()

    flops_step = 4.0 * rows * rows * D * (H // P)
    bytes_pack = 2 * 3 * rows * (H // P) * D * 2       # read + write, q/k/v bf16
    bytes_unpack = 2 * rows * (H // P) * D * 2

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(rank, pipelined, rec=None):
        if pipelined:
            # the pages' per-group pipeline: pack(g+2)/unpack(g) on the copy stream overlap attention(g)
            ulys.ulys_rank_pipeline(L, rank, shards["q"], shards["k"], shards["v"], qs, ks, vs, os_, out, lse=lse,
                                    stream=stream, copy_stream=copy_stream)
            return
        if rec is not None:
            rec["p0"].record(stream)
        ulys.ulys_pack(L, rank, -1, shards["q"], shards["k"], shards["v"], qs, ks, vs)
        if rec is not None:
            rec["p1"].record(stream)
        for g in range(G):
            ulys.ulys_attend_group(qs[g], ks[g], vs[g], os_[g], lse[g])
        if rec is not None:
            rec["a1"].record(stream)
        ulys.ulys_unpack(L, rank, -1, os_, out)
        if rec is not None:
            rec["u1"].record(stream)

    def timed(pipelined):
        """Warm-up, then exactly `steps` steps between two events; per-kernel events in sequential mode."""
        for i in range(args.warmup):
            step(i % P, pipelined)
        torch.cuda.synchronize()
        recs = None if pipelined else [{k_: ev() for k_ in ("p0", "p1", "a1", "u1")} for _ in range(args.steps)]
        t0, t1 = ev(), ev()
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            step(i % P, pipelined, None if recs is None else recs[i])
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps, recs

    pipelined = args.pipeline
    ms_step, recs = timed(pipelined)
    if pipelined:
        # per-kernel rates: the same steps again on one stream, events around each kernel group
        other_ms_step, recs = timed(False)
    else:
        # the two-stream schedule of the same steps, for comparison
        other_ms_step, _ = timed(True)
    pack_ms = sum(r["p0"].elapsed_time(r["p1"]) for r in recs) / args.steps
    attn_ms = sum(r["p1"].elapsed_time(r["a1"]) for r in recs) / args.steps
    unpack_ms = sum(r["a1"].elapsed_time(r["u1"]) for r in recs) / args.steps
    attn_launch_ms = attn_ms / G
    # an attention launch is the attention kernel plus, under the automatic range split, its merge
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ranges = ulys.ulys_attend_ranges(1, rows, rows, cus)
    launch_kernels = ATTN_KERNEL + (f" + {MERGE_KERNEL}" if ranges > 0 else "")
    attn_tflops = flops_step / (attn_ms * 1e-3) / 1e12
    value = flops_step / (ms_step * 1e-3) / 1e12
    repack_gbs = (bytes_pack + bytes_unpack) / ((pack_ms + unpack_ms) * 1e-3) / 1e9

    res = {
        "metric": "attention TFLOP/s + % MFMA peak at N=27280,H=10,D=128 bf16; repack GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1), seeded",
        "config": {"workload": f"Wan2.1 Ulysses-4 share: 4 shards [1,6820,40,128] -> pack 10 heads into {G} "
                               f"slot(s) [1,27280,{gh},128] -> attention N=27280 D=128 non-causal + LSE -> unpack",
                   "batch": 1, "seq_len": rows, "heads_per_gpu": H // P, "head_dim": D, "head_groups": G,
                   "ulysses_degree_simulated": P,
                   "schedule": "two-stream group pipeline" if pipelined else "one stream, sequential"},
        ("sequential_ms_per_step" if pipelined else "pipelined_ms_per_step"): round(other_ms_step, 4),
        "attention_tflops": round(attn_tflops, 2),
        "attention_frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "attention_ms": round(attn_ms, 4),
        "pack_ms": round(pack_ms, 4),
        "unpack_ms": round(unpack_ms, 4),
        "pack_gbs": round(bytes_pack / (pack_ms * 1e-3) / 1e9, 1),
        "unpack_gbs": round(bytes_unpack / (unpack_ms * 1e-3) / 1e9, 1),
        "repack_gbs": round(repack_gbs, 1),
        "repack_frac_hbm_peak": round(repack_gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "mfma", "achieved": round(flops_step / G / (attn_launch_ms * 1e-3) / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops_step / G / (attn_launch_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(G), "kernel": launch_kernels,
                     "launch_ms": round(attn_launch_ms, 4), "flops_per_launch": flops_step / G,
                     "range_split": ranges},
    }
    res["attention_fp8_qk"] = fp8_attention(torch, ulys, L, shards, qs, os_, lse, flops_step / G, args.steps)
    res["lse_merge_gbs"] = round(merge_gbs(torch, ulys, os_, lse, args.steps), 1)
    res["hbm_copy_gbs"] = round(device_copy_gbs(torch), 1)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(q, k, v, args.cpu_rows)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
