"""Bench: one GPU's share of a Ulysses-4 attention layer at the Wan2.1 shape, on MI355X.

Headline workload (synthetic, seeded, N(0,1) bf16): global q/k/v [1, 27280, 40, 128] cut into 4 rank
shards [1, 6820, 40, 128], resident in HBM.  One step = the whole hot path for one simulated rank's 10
heads: pack (all head groups, one launch) -> attention per head group (N = 27280, non-causal, fp32 LSE)
-> unpack into the 4 output shards.  Steps cycle over the 4 ranks and alternate between two slot sets
(558 MB, more than the 256 MB Infinity Cache), so no step re-reads what the previous one wrote.

Timing (the pages' protocol: warm-up 10, 50 timed iterations, median / P90 / min): HIP events on the
launch stream around every kernel group of every step; `ms_per_step` and `value` come from the events
bracketing all timed steps (their mean), the statistics from the per-step events.

`value` = attention TFLOP/s of the whole step (4*N^2*D*heads over the step time, pack and unpack
included).  `roofline` is the attention launch's (the attention kernel plus, under the automatic range
split, its merge): algorithmic FLOPs over the launch's mean event time, against the bf16 MFMA peak.
Further objects in the same line: the single 10-head call (G = 1), the joint text+image workload (valid-key
FLOPs), the GQA workload, the fp8 whole step (amax + e4m3 pack + attention + unpack), the repack rates,
the two-stream pipeline, an LSE merge, a plain device copy, and the CPU oracle on a bounded sample.
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
# e4m3 q/k: the QK^T half of the FLOPs at the fp8 rate, the PV half at the bf16 rate
PEAK_FP8_QK_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
ATTN_KERNEL = "attn_fwd_kernel<128, false, false, 2>"   # D = 128, bf16 q/k, no key mask (two row halves per wave)
MERGE_KERNEL = "range_merge_kernel<128>"             # the range split's merge, when the call uses one
METRIC = "attention TFLOP/s + % MFMA peak at N=27280,H=10,D=128 bf16; repack GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "ulysses_sequence_attention_amd", "csrc", f)
                  for f in ("attn.hip", "internal.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--groups", type=int, default=5,
                    help="head groups per rank in the headline step (5 = 2-head groups, run one at a time)")
    ap.add_argument("--only-headline", action="store_true",
                    help="time the headline step only (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=12288, help="query rows the oracle computes for cpu_baseline")
    ap.add_argument("--group-sweep", action="store_true",
                    help="time a rank's 10 heads (D=128) as G = 1, 2, 5, 10 attention calls for several sequence "
                         "lengths and print the automatic group count beside (calibrates ulys_auto_groups)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (checks the HBM byte counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="read the rocprofv3 runs under DIR, write profiles/attn_fwd_traffic.json and print the "
                         "summary tables (no GPU needed)")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------------- helpers

def stats(xs):
    s = sorted(xs)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    p90 = s[min(n - 1, int(round(0.9 * (n - 1))))]
    return {"median": round(med, 4), "p90": round(p90, 4), "min": round(s[0], 4), "mean": round(sum(s) / n, 4)}


def time_steps(torch, stream, fn, segments, warmup, steps):
    """Run fn(i, marks) `warmup` times, then `steps` times with HIP events on `stream`: marks(j) records the
    boundary before segment j (and marks(len) the end).  Returns (mean ms per step from the bracketing
    events, per-step ms list, {segment: per-step ms list})."""
    for i in range(warmup):
        fn(i, lambda j: None)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    recs = [[ev() for _ in range(len(segments) + 1)] for _ in range(steps)]
    t0, t1 = ev(), ev()
    t0.record(stream)
    for i in range(steps):
        fn(warmup + i, lambda j, r=recs[i]: r[j].record(stream))
    t1.record(stream)
    torch.cuda.synchronize()
    per_step = [r[0].elapsed_time(r[-1]) for r in recs]
    seg = {name: [r[j].elapsed_time(r[j + 1]) for r in recs] for j, name in enumerate(segments)}
    return t0.elapsed_time(t1) / steps, per_step, seg


def attention_roofline(flops_launch, launch_ms, peak, kernel, traffic=None, **extra):
    achieved = flops_launch / (launch_ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
         "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel, "launch_ms": round(launch_ms, 4),
         "flops_per_launch": flops_launch}
    r.update(extra)
    return r


def kernel_source_hash() -> str:
    """Hash of the attention kernel's code and compile flags: counters taken on another version of the
    kernel are not reported as its traffic.  Comments and whitespace are left out, so a change of comment
    text alone keeps the counters."""
    import hashlib
    import re
    from ulysses_sequence_attention_amd import build as ubuild
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)    # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    h.update(" ".join(ubuild.FLAGS + ubuild.SOURCE_FLAGS.get("attn.hip", [])).encode())
    return h.hexdigest()


def measured_traffic(groups: int):
    """HBM bytes per attention launch (kernel + merge) from the committed rocprofv3 DRAM request counters,
    or None when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = t.get("per_groups", {}).get(str(groups))
    if entry is None or t.get("source_sha256") != kernel_source_hash():
        return None
    return entry["hbm_bytes_per_launch"]


# ---------------------------------------------------------------------------------------------- workloads

class RankStep:
    """One simulated rank's path on a layout: [amax] -> pack (all groups) -> G attention calls -> unpack,
    with two rotating slot sets and one workspace, all allocated once."""

    def __init__(self, torch, ulys, L, shards, key_gaps=None, fp8=False, amax_each_step=False, key_mask=None):
        self.torch, self.ulys, self.L = torch, ulys, L
        self.shards, self.gaps, self.fp8, self.amax_each_step = shards, key_gaps, fp8, amax_each_step
        self.key_mask = key_mask
        dev = shards["q"][0].device
        G, B = L.groups, L.batch
        qk_dtype = torch.uint8 if fp8 else torch.bfloat16
        self.sets = []
        for _ in range(2):
            self.sets.append(dict(
                q=torch.empty((G, B, L.rows_q, L.gq, L.head_dim), dtype=qk_dtype, device=dev),
                k=torch.empty((G, B, L.rows, L.gkv, L.head_dim), dtype=qk_dtype, device=dev),
                v=torch.empty((G, B, L.rows, L.gkv, L.head_dim), dtype=torch.bfloat16, device=dev),
                o=torch.empty((G, B, L.rows_q, L.gq, L.head_dim), dtype=torch.bfloat16, device=dev),
                lse=torch.empty((G, B, L.gq, L.rows_q), dtype=torch.float32, device=dev)))
        self.out = [torch.empty_like(s) for s in shards["q"]]
        n = ulys.ulys_attend_workspace_bytes(B, L.rows_q, L.rows, L.gq, L.head_dim)
        self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.amax = torch.zeros(2, dtype=torch.float32, device=dev)
        if fp8:
            ulys.ulys_amax_bf16(shards["q"], self.amax[0:1])
            ulys.ulys_amax_bf16(shards["k"], self.amax[1:2])
        self.qk = ulys.ULYS_FP8_E4M3 if fp8 else ulys.ULYS_BF16

    def segments(self):
        return (["amax"] if self.amax_each_step else []) + ["pack", "attend", "unpack"]

    def __call__(self, i, mark):
        u, L, s = self.ulys, self.L, self.sets[i % 2]
        rank = i % L.degree
        j = 0
        if self.amax_each_step:
            mark(j); j += 1
            u.ulys_amax_bf16(self.shards["q"], self.amax[0:1])
            u.ulys_amax_bf16(self.shards["k"], self.amax[1:2])
        mark(j); j += 1
        u.ulys_pack(L, rank, -1, self.shards["q"], self.shards["k"], self.shards["v"], s["q"], s["k"], s["v"],
                    qk_dtype=self.qk, qk_amax=self.amax if self.fp8 else None)
        mark(j); j += 1
        for g in range(L.groups):
            if self.key_mask is None:
                u.ulys_attend_group(s["q"][g], s["k"][g], s["v"][g], s["o"][g], s["lse"][g], key_gaps=self.gaps,
                                    qk_dtype=self.qk, qk_amax=self.amax if self.fp8 else None, workspace=self.ws)
            else:
                u.ulys_attend_group_ex(s["q"][g], s["k"][g], s["v"][g], s["o"][g], s["lse"][g],
                                       key_gaps=self.gaps, key_mask=self.key_mask, qk_dtype=self.qk,
                                       qk_amax=self.amax if self.fp8 else None, workspace=self.ws)
        mark(j); j += 1
        u.ulys_unpack(L, rank, -1, s["o"], self.out)
        mark(j)

    def bytes_pack(self):
        L = self.L
        qk = 1 if self.fp8 else 2
        nq = L.batch * L.rows_q * L.hq // L.degree * L.head_dim
        nkv = L.batch * L.rows * L.hkv // L.degree * L.head_dim
        return (nq + 2 * nkv) * 2 + (nq + nkv) * qk + nkv * 2        # read bf16, write q/k (qk bytes) + v

    def bytes_unpack(self):
        L = self.L
        return 2 * L.batch * L.rows_q * L.hq // L.degree * L.head_dim * 2

    def bytes_amax(self):
        return sum(x.numel() * 2 for x in self.shards["q"]) + sum(x.numel() * 2 for x in self.shards["k"])


def shards_of(torch, inputs, w, dev):
    """Seeded global q/k/v cut into the P rank shards (the layout's own split), on the GPU."""
    q, k, v = inputs.global_qkv(w)
    P, S_l, R = w.degree, w.s_local, w.n_rep
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        if R > 0 and name == "q" and w.extra.get("kv_only_prefix"):   # the prefix is k/v only
            out[name] = [x[:, R + p * S_l:R + (p + 1) * S_l].contiguous().to(dev) for p in range(P)]
        elif R == 0:
            out[name] = [x[:, p * S_l:(p + 1) * S_l].contiguous().to(dev) for p in range(P)]
        else:                       # a replicated prefix: every shard carries it in front
            out[name] = [torch.cat([x[:, :R], x[:, R + p * S_l:R + (p + 1) * S_l]], dim=1).contiguous().to(dev)
                         for p in range(P)]
    return (q, k, v), out


def input_sha256(torch, tensors) -> str:
    """SHA-256 of the seeded inputs' bytes (q, then k, then v), so a run's data can be checked to be the same."""
    import hashlib
    h = hashlib.sha256()
    for x in tensors:
        h.update(x.contiguous().view(torch.int16).numpy().tobytes())
    return h.hexdigest()


def run_config(torch, ulys, args, stream, L, shards, flops_step, peak, kernel, gaps=None, fp8=False,
               amax_each_step=False, traffic=None, extra=None, key_mask=None):
    """Time RankStep over the config; returns the JSON object for it (attention roofline included)."""
    st = RankStep(torch, ulys, L, shards, gaps, fp8, amax_each_step, key_mask)
    ms, per_step, seg = time_steps(torch, stream, st, st.segments(), args.warmup, args.steps)
    launch_ms = sum(seg["attend"]) / len(seg["attend"]) / L.groups
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    r = {"ms_per_step": round(ms, 4), "step_ms": stats(per_step),
         "attention_ms": stats(seg["attend"]), "pack_ms": stats(seg["pack"]), "unpack_ms": stats(seg["unpack"]),
         "value_tflops": round(flops_step / (ms * 1e-3) / 1e12, 2),
         "attention_tflops": round(flops_step / (sum(seg["attend"]) / len(seg["attend"]) * 1e-3) / 1e12, 2),
         "roofline": attention_roofline(flops_step / L.groups, launch_ms, peak, kernel, traffic,
                                        range_split=ulys.ulys_attend_ranges(L.batch, L.rows_q, L.rows, cus),
                                        key_split=ulys.ulys_attend_splits(L.batch, L.rows_q, L.rows, cus))}
    mean = lambda xs: sum(xs) / len(xs)
    r["pack_gbs"] = round(st.bytes_pack() / (mean(seg["pack"]) * 1e-3) / 1e9, 1)
    r["unpack_gbs"] = round(st.bytes_unpack() / (mean(seg["unpack"]) * 1e-3) / 1e9, 1)
    if amax_each_step:
        r["amax_ms"] = stats(seg["amax"])
        r["amax_gbs"] = round(st.bytes_amax() / (mean(seg["amax"]) * 1e-3) / 1e9, 1)
    if extra:
        r.update(extra)
    return r, st


# ---------------------------------------------------------------------------------------------- side figures

def repack_back_to_back(torch, ulys, L, shards, reps: int) -> dict:
    """Kernel throughput of the repack without per-launch events: `reps` launches of each of pack (bf16 and
    e4m3 q/k), unpack and amax back to back between two events, ranks cycled and two slot sets rotated
    (nothing cache-resident).  GB/s of algorithmic bytes (read + write)."""
    dev = shards["q"][0].device
    G, P, D, rows = L.groups, L.degree, L.head_dim, L.rows
    heads = L.hq // P
    out = {}
    amax = torch.zeros(2, dtype=torch.float32, device=dev)
    ulys.ulys_amax_bf16(shards["q"], amax[0:1])
    ulys.ulys_amax_bf16(shards["k"], amax[1:2])

    def timed(fn, nbytes):
        for j in range(3):
            fn(j)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for j in range(reps):
            fn(j)
        e1.record()
        torch.cuda.synchronize()
        return round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    for fp8 in (False, True):
        qk = torch.uint8 if fp8 else torch.bfloat16
        sets = [[torch.empty((G, 1, rows, L.gq, D), dtype=qk, device=dev) for _ in range(2)] +
                [torch.empty((G, 1, rows, L.gkv, D), dtype=torch.bfloat16, device=dev)] for _ in range(2)]
        nbytes = rows * heads * D * (3 * 2 + 2 * (1 if fp8 else 2) + 2)
        out["fp8_pack_gbs" if fp8 else "pack_gbs"] = timed(
            lambda j: ulys.ulys_pack(L, j % P, -1, shards["q"], shards["k"], shards["v"], *sets[j % 2],
                                     qk_dtype=ulys.ULYS_FP8_E4M3 if fp8 else ulys.ULYS_BF16,
                                     qk_amax=amax if fp8 else None), nbytes)
        del sets
    oslots = [torch.empty((G, 1, rows, L.gq, D), dtype=torch.bfloat16, device=dev).normal_() for _ in range(2)]
    o_shards = [torch.empty_like(x) for x in shards["q"]]
    out["unpack_gbs"] = timed(lambda j: ulys.ulys_unpack(L, j % P, -1, oslots[j % 2], o_shards), 2 * rows * heads * D * 2)
    n_amax = sum(x.numel() * 2 for x in shards["q"])
    out["amax_gbs"] = timed(lambda j: ulys.ulys_amax_bf16(shards["q" if j % 2 == 0 else "k"], amax[j % 2:j % 2 + 1]),
                            n_amax)
    for k_ in ("pack_gbs", "fp8_pack_gbs", "unpack_gbs", "amax_gbs"):
        out[k_.replace("_gbs", "_frac_hbm_peak")] = round(out[k_] / PEAK_HBM_GBS, 4)
    out["launches_each"] = reps
    return out


def merge_gbs(torch, ulys, o_slots, lse, steps: int) -> float:
    """ulys_lse_merge of the G head-group outputs taken as G partial results of one slot shape (a ring of G):
    algorithmic bytes (G partial o + lse read, one o + lse written) over the mean event time."""
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
    """Practical HBM ceiling for a stream: a plain 1 GiB device-to-device copy (torch copy_), read + write
    bytes over the median of 5 timed copies."""
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


def pipelined_ms(torch, ulys, L, shards, warmup, steps):
    """ulys_rank_pipeline (packs and unpacks on a second stream beside the attention of each group): mean ms
    per rank step."""
    dev = shards["q"][0].device
    G = L.groups
    qs = torch.empty((G, L.batch, L.rows, L.gq, L.head_dim), dtype=torch.bfloat16, device=dev)
    ks, vs, os_ = torch.empty_like(qs), torch.empty_like(qs), torch.empty_like(qs)
    lse = torch.empty((G, L.batch, L.gq, L.rows), dtype=torch.float32, device=dev)
    out = [torch.empty_like(s) for s in shards["q"]]
    ws = torch.empty(max(ulys.ulys_attend_workspace_bytes(L.batch, L.rows, L.rows, L.gq, L.head_dim), 256),
                     dtype=torch.uint8, device=dev)
    events = [torch.cuda.Event() for _ in range(3)]
    xs = torch.cuda.Stream()
    run = lambda i: ulys.ulys_rank_pipeline(L, i % L.degree, shards["q"], shards["k"], shards["v"], qs, ks, vs, os_,
                                            out, lse=lse, events=events, workspace=ws, copy_stream=xs)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cpu_baseline(q, k, v, rows_sample: int):
    """The oracle as it stands (fp64 NumPy), on a bounded sample of the same workload: attention for
    `rows_sample` query rows of all 10 heads of rank 0 over all 27280 keys."""
    import numpy as np
    from oracle import attention as oatt

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


# ---------------------------------------------------------------------------------------------- other modes

def group_sweep():
    """One JSON line per sequence length: attention time of 10 heads split into G calls (with the automatic
    key-range or range split, and with none), the split counts and the group count ulys_auto_groups picks for
    that shape (Wan-like layout, Ulysses degree 4)."""
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
                ws = torch.empty(max(ulys.ulys_attend_workspace_bytes(1, rows, rows, gh, 128, splits), 256),
                                 dtype=torch.uint8, device="cuda")
                run = lambda: [ulys.ulys_attend_group_ex(q[g], k[g], v[g], o[g], lse[g], key_splits=splits,
                                                         workspace=ws) for g in range(G)]
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
    """A plain device-to-device copy of 1 GiB, five times: reads 1 GiB and writes 1 GiB per launch.  Under
    rocprofv3's DRAM request counters it checks their byte scale (32 bytes per counted request)."""
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

    Expects under ``d``: stats_g1, stats_g5 (``--kernel-trace --stats``); dram_g1, dram_g5, dram_copy
    (``--pmc TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_WRITE_DRAM_32B_sum``); mfma_g1, mfma_g5
    (``--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES SQ_WAVES SQ_INSTS_LDS
    SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU SQ_INSTS_SALU GRBM_GUI_ACTIVE``), each ``-o run --output-format csv``,
    of the headline bench at G = 1, 5 (and the copy calibration)."""
    import csv
    import statistics
    from collections import defaultdict

    def rows_of(sub, fname):
        with open(os.path.join(d, sub, fname)) as fh:
            return list(csv.DictReader(fh))

    def per_kernel(sub):
        """{kernel: {counter: mean per dispatch}} plus 'dur_ns' and 'n'."""
        acc = defaultdict(lambda: defaultdict(float))
        dur = {}
        for r in rows_of(sub, "run_counter_collection.csv"):
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            acc[key][r["Counter_Name"]] += float(r["Counter_Value"])
            dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        out = defaultdict(lambda: defaultdict(list))
        for (k, disp), cs in acc.items():
            for c, v in cs.items():
                out[k][c].append(v)
            out[k]["dur_ns"].append(dur[(k, disp)])
        return {k: {c: statistics.mean(v) for c, v in cs.items()} | {"n": len(cs["dur_ns"])} for k, cs in out.items()}

    def find(table, substr):
        for k, v in table.items():
            if substr in k:
                return v
        return None

    short = lambda n: n.replace("ulys::(anonymous namespace)::", "").replace("(ulys::AttnArgs)", "")
    print("## Kernel statistics (rocprofv3 --kernel-trace --stats)\n")
    for G in (1, 5):
        print(f"### G = {G}\n\n| kernel | calls | total ms | avg us | min us | max us | % |\n|---|---|---|---|---|---|---|")
        for r in rows_of(f"stats_g{G}", "run_kernel_stats.csv"):
            print(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                  f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
        print()
    RD, WR = "TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"
    copy = find(per_kernel("dram_copy"), "copyBuffer")
    n = 1 << 30
    print("## HBM bytes per dispatch (DRAM-bound request counters x 32 bytes)\n")
    print(f"Check on a plain 1 GiB device copy: {copy[RD] * 32 / n:.4f} GiB read, {copy[WR] * 32 / n:.4f} GiB "
          f"written per dispatch.\n")
    print("| kernel | G | read bytes | write bytes | algorithmic read / write | read / algorithmic | write / algorithmic |")
    print("|---|---|---|---|---|---|---|")
    rows = 27280
    out = {"kernel": ATTN_KERNEL + " + " + MERGE_KERNEL + " (when the launch takes a range split)",
           "workload": "Wan2.1 Ulysses-4 share: q/k/v slots [1,27280,10/G,128] bf16, non-causal, LSE",
           "source_sha256": kernel_source_hash(),
           "counters": f"{RD} and {WR} (32 bytes each); a 1 GiB copy reads {copy[RD] * 32:.0f} and writes "
                       f"{copy[WR] * 32:.0f} bytes by them",
           "per_groups": {}}
    for G in (1, 5):
        heads = 10 // G
        t = per_kernel(f"dram_g{G}")
        a = find(t, ATTN_KERNEL)
        m = find(t, MERGE_KERNEL) or {RD: 0.0, WR: 0.0}
        rd, wr = (a[RD] + m[RD]) * 32, (a[WR] + m[WR]) * 32
        alg_r = 3 * rows * heads * 128 * 2
        alg_w = rows * heads * 128 * 2 + rows * heads * 4
        out["per_groups"][str(G)] = {"heads_per_launch": heads, "hbm_read_bytes": int(rd), "hbm_write_bytes": int(wr),
                                     "hbm_bytes_per_launch": int(rd + wr), "algorithmic_read_bytes": alg_r,
                                     "algorithmic_write_bytes": alg_w, "read_over_algorithmic": round(rd / alg_r, 2)}
        print(f"| launch (`{ATTN_KERNEL}` + merge) | {G} | {rd:.4g} | {wr:.4g} | {alg_r:.4g} / {alg_w:.4g} | "
              f"{rd / alg_r:.2f} | {wr / alg_w:.2f} |")
        print(f"| `{MERGE_KERNEL}` alone | {G} | {m[RD] * 32:.4g} | {m[WR] * 32:.4g} | | | |")
        for kname, ar, aw in (("pack_kernel", 3 * rows * 10 * 128 * 2, 3 * rows * 10 * 128 * 2),
                              ("unpack_kernel", rows * 10 * 128 * 2, rows * 10 * 128 * 2)):
            k = find(t, kname)
            if k is not None:
                print(f"| `{kname}` (one rank, all groups) | {G} | {k[RD] * 32:.4g} | {k[WR] * 32:.4g} | "
                      f"{ar:.4g} / {aw:.4g} | {k[RD] * 32 / ar:.3f} | {k[WR] * 32 / aw:.3f} |")
    print("\n## MFMA utilisation of the attention kernel (SQ counters)\n")
    print("| G | kernel us | GRBM_GUI_ACTIVE / XCD | clock GHz | MFMA busy (of SIMD-cycles) | MFMA FLOPs / algorithmic | "
          "VALU per 32 rows x 32 keys | SALU per 32 x 32 | LDS per 32 x 32 | LDS bank conflicts |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for G in (1, 5):
        heads = 10 // G
        a = find(per_kernel(f"mfma_g{G}"), ATTN_KERNEL)
        xcd_cycles = a["GRBM_GUI_ACTIVE"] / 8
        ghz = xcd_cycles / a["dur_ns"]
        busy = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * 1024)
        flops = a["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        alg = 4.0 * rows * rows * 128 * heads
        blocks = heads * (rows / 32) * (rows / 32)      # (32 query rows, 32-key block) pairs
        mfma_insts = flops / (32 * 32 * 16 * 2)
        out["per_groups"][str(G)]["mfma"] = {"kernel_us": round(a["dur_ns"] / 1e3, 1), "clock_ghz": round(ghz, 3),
                                             "mfma_busy_frac": round(busy, 4),
                                             "mfma_flops_over_algorithmic": round(flops / alg, 4)}
        print(f"| {G} | {a['dur_ns'] / 1e3:.1f} | {xcd_cycles:.4g} | {ghz:.3f} | {busy:.3f} | {flops / alg:.4f} | "
              f"{(a['SQ_INSTS_VALU'] - mfma_insts) / blocks:.1f} | {a['SQ_INSTS_SALU'] / blocks:.1f} | "
              f"{a['SQ_INSTS_LDS'] / blocks:.1f} | {a['SQ_LDS_BANK_CONFLICT']:.4g} |")
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(f"\nwrote {TRAFFIC_FILE}")


# ---------------------------------------------------------------------------------------------- main

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
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is built and measured on one "
              f"GPU, with the all-to-all modelled as a local permutation; there is no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import dataclasses

    import torch
    from ulysses_sequence_attention_amd import inputs, ulys

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    G = args.groups
    w = inputs.E2E_P4
    (q, k, v), shards = shards_of(torch, inputs, w, dev)
    P, H, D = w.degree, w.hq, w.head_dim
    L = ulys.Layout(1, P, w.s_local, 0, True, H, H, D, G)
    rows = L.rows
    flops_step = 4.0 * rows * rows * D * (H // P)
    kernel = lambda layout: ATTN_KERNEL + (f" + {MERGE_KERNEL}" if ulys.ulys_attend_ranges(
        layout.batch, layout.rows_q, layout.rows, torch.cuda.get_device_properties(0).multi_processor_count) else "")

    head, st = run_config(torch, ulys, args, stream, L, shards, flops_step, PEAK_BF16_TFLOPS, kernel(L),
                          traffic=measured_traffic(G))
    res = {
        "metric": METRIC,
        "value": head["value_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1), seeded",
        "config": {"workload": f"Wan2.1 Ulysses-4 share: 4 shards [1,6820,40,128] -> pack 10 heads into {G} "
                               f"slot(s) [1,27280,{L.gq},128] -> attention N=27280 D=128 non-causal + LSE -> unpack",
                   "batch": 1, "seq_len": rows, "heads_per_gpu": H // P, "head_dim": D, "head_groups": G,
                   "ulysses_degree_simulated": P, "schedule": "one stream, sequential",
                   "slot_sets_rotated": 2, "input_sha256": input_sha256(torch, (q, k, v))},
        "roofline": head.pop("roofline"),
        "step_ms": head["step_ms"],
        "attention_tflops": head["attention_tflops"],
        "attention_frac_bf16_peak": round(head["attention_tflops"] / PEAK_BF16_TFLOPS, 4),
        "attention_ms": head["attention_ms"], "pack_ms": head["pack_ms"], "unpack_ms": head["unpack_ms"],
        "repack": {"pack_gbs": head["pack_gbs"], "unpack_gbs": head["unpack_gbs"],
                   "pack_frac_hbm_peak": round(head["pack_gbs"] / PEAK_HBM_GBS, 4),
                   "unpack_frac_hbm_peak": round(head["unpack_gbs"] / PEAK_HBM_GBS, 4),
                   "bytes": {"pack": st.bytes_pack(), "unpack": st.bytes_unpack()},
                   "note": "algorithmic bytes (read + write) over the mean time between the events around each kernel "
                           "inside the step (the event pair adds a few microseconds to kernels of 20-70 us); two "
                           "slot sets rotated (558 MB) and four ranks' shards cycled, so neither side is "
                           "cache-resident; repack_back_to_back times the kernels without per-launch events"},
    }
    res["repack"]["repack_gbs"] = round((st.bytes_pack() + st.bytes_unpack()) /
                                        ((res["pack_ms"]["mean"] + res["unpack_ms"]["mean"]) * 1e-3) / 1e9, 1)
    res["repack"]["repack_frac_hbm_peak"] = round(res["repack"]["repack_gbs"] / PEAK_HBM_GBS, 4)
    print(json.dumps({"progress": "headline", "ms_per_step": res["ms_per_step"], "roofline": res["roofline"]}),
          file=sys.stderr, flush=True)
    if not args.only_headline:
        del st
        configs = {}
        # the single 10-head call (G = 1)
        L1 = dataclasses.replace(L, groups=1)
        r, st1 = run_config(torch, ulys, args, stream, L1, shards, flops_step, PEAK_BF16_TFLOPS, kernel(L1),
                            traffic=measured_traffic(1))
        configs["wan_share_single_call"] = r
        res["lse_merge_gbs"] = round(merge_gbs(torch, ulys, _g5_view(torch, st1), _g5_lse(torch, st1), args.steps), 1)
        del st1
        print(json.dumps({"progress": "single call"}), file=sys.stderr, flush=True)
        # the fp8 whole step: amax + e4m3 pack + attention + unpack
        r, st8 = run_config(torch, ulys, args, stream, L, shards, flops_step, PEAK_FP8_QK_TFLOPS,
                            "attn_fwd_kernel<128, true, false, 1>" + (" + " + MERGE_KERNEL if res["roofline"]["range_split"]
                                                                   else ""),
                            fp8=True, amax_each_step=True,
                            extra={"note": "e4m3 q/k (QK^T at the fp8 rate), bf16 V and P; peak = the mixed bound "
                                           f"1 / (0.5 / {PEAK_FP8_TFLOPS:g} + 0.5 / {PEAK_BF16_TFLOPS:g})"})
        r["roofline"]["frac_of_bf16_peak"] = round(r["roofline"]["achieved"] / PEAK_BF16_TFLOPS, 4)
        configs["e2e_p4_fp8_step"] = r
        del st8, shards
        torch.cuda.empty_cache()
        print(json.dumps({"progress": "fp8 step"}), file=sys.stderr, flush=True)
        # the joint text+image workload (valid-key FLOPs) and the GQA workload, at P = 1 (pack = head slices)
        for name, wk in (("joint_varlen", inputs.JOINT_VARLEN), ("gqa", inputs.GQA)):
            _, sh = shards_of(torch, inputs, wk, dev)
            Lw = ulys.Layout(wk.batch, 1, wk.s_local, wk.n_rep, True, wk.hq, wk.hkv, wk.head_dim, wk.groups)
            gaps = None if wk.key_gap is None else [wk.key_gap] * wk.batch
            valid = Lw.rows - (0 if wk.key_gap is None else wk.key_gap[1] - wk.key_gap[0])
            fl = 4.0 * wk.batch * wk.hq * Lw.rows * valid * wk.head_dim
            r, stw = run_config(torch, ulys, args, stream, Lw, sh, fl, PEAK_BF16_TFLOPS, kernel(Lw), gaps=gaps,
                                extra={"flops_per_step": fl, "valid_keys": valid})
            configs[name] = r
            del stw, sh
            torch.cuda.empty_cache()
            print(json.dumps({"progress": name}), file=sys.stderr, flush=True)
        # cross-attention to a replicated text K/V prefix with its padding as a key mask (valid-key FLOPs)
        import numpy as np
        wk = inputs.KV_PREFIX_MASKED
        _, sh = shards_of(torch, inputs, wk, dev)
        Lw = ulys.Layout(wk.batch, wk.degree, wk.s_local, wk.n_rep, ulys.ULYS_REP_KV_PREFIX, wk.hq, wk.hkv,
                         wk.head_dim, wk.groups)
        valid_mask = np.ones((wk.batch, Lw.rows), dtype=bool)
        valid_mask[:, wk.extra["text_valid"]:wk.n_rep] = False
        words = inputs.key_mask_words(valid_mask).to(dev)
        valid = int(valid_mask.sum()) // wk.batch
        fl = 4.0 * wk.batch * (wk.hq // wk.degree) * Lw.rows_q * valid * wk.head_dim
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        r, stw = run_config(torch, ulys, args, stream, Lw, sh, fl, PEAK_BF16_TFLOPS,
                            "attn_fwd_kernel<128, false, true, 1>" + (f" + {MERGE_KERNEL}" if ulys.ulys_attend_ranges(
                                Lw.batch, Lw.rows_q, Lw.rows, cus) else ""),
                            key_mask=words,
                            extra={"flops_per_step": fl, "q_rows": Lw.rows_q, "kv_rows": Lw.rows, "valid_keys": valid,
                                   "note": "K/V-only text prefix (512 rows, 226 valid) replicated on the 4 ranks, "
                                           "padding as a key-mask bit array; q and o hold only the image rows"})
        configs["kv_prefix_masked"] = r
        del stw, sh
        torch.cuda.empty_cache()
        print(json.dumps({"progress": "kv_prefix_masked"}), file=sys.stderr, flush=True)
        res["configs"] = configs
        res["repack"]["fp8_pack_gbs"] = configs["e2e_p4_fp8_step"]["pack_gbs"]
        res["repack"]["amax_gbs"] = configs["e2e_p4_fp8_step"]["amax_gbs"]
        (q, k, v), shards = shards_of(torch, inputs, w, dev)
        res["pipelined_ms_per_step"] = round(pipelined_ms(torch, ulys, L, shards, args.warmup, args.steps), 4)
        res["repack_back_to_back"] = repack_back_to_back(torch, ulys, L, shards, args.steps)
        res["hbm_copy_gbs"] = round(device_copy_gbs(torch), 1)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(q, k, v, args.cpu_rows)
    print(json.dumps(res))


def _g5_view(torch, st1):
    """The single call's 10-head output slot viewed as five 2-head partial outputs (shape only)."""
    o = st1.sets[0]["o"][0]                       # [1, rows, 10, D]
    return o.view(1, o.shape[1], 5, 2, o.shape[3]).permute(2, 0, 1, 3, 4).contiguous()


def _g5_lse(torch, st1):
    lse = st1.sets[0]["lse"][0]                   # [1, 10, rows]
    return lse.view(1, 5, 2, lse.shape[2]).permute(1, 0, 2, 3).contiguous()


if __name__ == "__main__":
    main()
