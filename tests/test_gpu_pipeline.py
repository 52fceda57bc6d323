"""GPU: the two-stream head-group pipeline (ulys_rank_pipeline) against the same steps run one after
another on one stream, byte for byte (sglang PR #43521 "Motivation"/"Receive slots": the pipelined
exchange must give the sequential exchange's result bit for bit), with and without injected skew
between the streams; plus the tiny case against the oracle."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from gpu_common import bits, check_attention, f64, from_bits, layout_of, oatt, olay, shards_of
from ulysses_sequence_attention_amd import inputs

pytestmark = pytest.mark.gpu

# A GQA layout with a replicated suffix and a masked key range crossing a shard edge.
GQA_SUFFIX = dataclasses.replace(inputs.TINY, name="gqa_suffix", seed=11, batch=2, degree=2, s_local=300, n_rep=40,
                                 rep_first=False, hq=8, hkv=4, head_dim=128, groups=2, key_gap=(280, 330))


def _buffers(w, L, fp8):
    G = w.groups
    qk_dt = torch.uint8 if fp8 else torch.bfloat16
    qs = torch.full((G, w.batch, L.rows, L.gq, w.head_dim), 0x7f if fp8 else 0, dtype=qk_dt, device="cuda")
    ks = torch.full((G, w.batch, L.rows, L.gkv, w.head_dim), 0x7f if fp8 else 0, dtype=qk_dt, device="cuda")
    vs = torch.zeros((G, w.batch, L.rows, L.gkv, w.head_dim), dtype=torch.bfloat16, device="cuda")
    os_ = torch.zeros((G, w.batch, L.rows, L.gq, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((G, w.batch, L.gq, L.rows), dtype=torch.float32, device="cuda")
    return qs, ks, vs, os_, lse


def _run(gpu, w, dev, amax, pipelined, skew=None):
    """All ranks of workload w; returns (output shards, last rank's slots and lse) on the CPU."""
    L = layout_of(w)
    fp8 = w.fp8_qk
    qk = gpu.ULYS_FP8_E4M3 if fp8 else gpu.ULYS_BF16
    gaps = None if w.key_gap is None else [w.key_gap] * w.batch
    qs, ks, vs, os_, lse = _buffers(w, L, fp8)
    out = [torch.zeros_like(s) for s in dev["q"]]
    main = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    for rank in range(w.degree):
        if pipelined:
            if skew == "copy":                        # the copy stream is late: packs start after a spin
                with torch.cuda.stream(copy):
                    torch.cuda._sleep(20_000_000)
            elif skew == "main":                      # the compute stream is busy before the call
                torch.cuda._sleep(20_000_000)
            gpu.ulys_rank_pipeline(L, rank, dev["q"], dev["k"], dev["v"], qs, ks, vs, os_, out, lse=lse,
                                   key_gaps=gaps, qk_dtype=qk, qk_amax=amax, stream=main, copy_stream=copy)
        else:
            for g in range(w.groups):
                gpu.ulys_pack(L, rank, g, dev["q"], dev["k"], dev["v"], qs[g], ks[g], vs[g], qk, amax)
                gpu.ulys_attend_group(qs[g], ks[g], vs[g], os_[g], lse[g], key_gaps=gaps, qk_dtype=qk, qk_amax=amax)
                gpu.ulys_unpack(L, rank, g, os_[g], out)
    torch.cuda.synchronize()
    return ([bits(s) for s in out], qs.cpu().view(torch.uint8).numpy(), ks.cpu().view(torch.uint8).numpy(),
            bits(vs), bits(os_), lse.cpu().numpy().view(np.int32))


def _inputs(gpu, w):
    (q, k, v), sh = shards_of(w)
    dev = {n: [from_bits(s) for s in x] for n, x in sh.items()}
    amax = None
    if w.fp8_qk:
        amax = torch.empty(2, dtype=torch.float32, device="cuda")
        gpu.ulys_amax_bf16(dev["q"], amax[0:1])
        gpu.ulys_amax_bf16(dev["k"], amax[1:2])
    return (q, k, v), sh, dev, amax


def _same(a, b):
    out_a, *rest_a = a
    out_b, *rest_b = b
    for p, (x, y) in enumerate(zip(out_a, out_b)):
        assert np.array_equal(x, y), f"output shard {p} differs"
    for name, x, y in zip(("q slots", "k slots", "v slots", "o slots", "lse"), rest_a, rest_b):
        assert np.array_equal(x, y), f"{name} differ"


@pytest.mark.parametrize("w", [inputs.TINY, GQA_SUFFIX, inputs.E2E_P4], ids=lambda w: w.name)
def test_pipeline_equals_sequential(gpu, w):
    print(f"pipeline vs sequential: {w.name}", flush=True)
    _, _, dev, amax = _inputs(gpu, w)
    seq = _run(gpu, w, dev, amax, pipelined=False)
    pip = _run(gpu, w, dev, amax, pipelined=True)
    _same(seq, pip)


@pytest.mark.parametrize("skew", ["copy", "main"])
def test_pipeline_under_skew(gpu, skew):
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep not available")
    w = GQA_SUFFIX
    print(f"pipeline skew {skew}: {w.name}", flush=True)
    _, _, dev, amax = _inputs(gpu, w)
    seq = _run(gpu, w, dev, amax, pipelined=False)
    pip = _run(gpu, w, dev, amax, pipelined=True, skew=skew)
    _same(seq, pip)


def test_pipeline_one_stream(gpu):
    """copy_stream = stream: everything in order on one stream, same bytes."""
    w = inputs.TINY
    _, _, dev, amax = _inputs(gpu, w)
    seq = _run(gpu, w, dev, amax, pipelined=False)
    L = layout_of(w)
    qs, ks, vs, os_, lse = _buffers(w, L, False)
    out = [torch.zeros_like(s) for s in dev["q"]]
    for rank in range(w.degree):
        gpu.ulys_rank_pipeline(L, rank, dev["q"], dev["k"], dev["v"], qs, ks, vs, os_, out, lse=lse)
    torch.cuda.synchronize()
    for p, (x, y) in enumerate(zip(seq[0], [bits(s) for s in out])):
        assert np.array_equal(x, y), f"output shard {p} differs"


def test_pipeline_tiny_against_oracle(gpu):
    """Every output row of both shards of the tiny layout against the oracle's joint attention."""
    w = inputs.TINY
    (q, k, v), sh, dev, amax = _inputs(gpu, w)
    out, *_ = _run(gpu, w, dev, amax, pipelined=True)
    # global joint layout: prefix rows then the shards' own rows (prefix read from shard 0)
    joint = [olay.joint_for_rank(sh[n], 0, w.n_rep, w.rep_first) for n in ("q", "k", "v")]
    jq, jk, jv = (f64(from_bits(x, "cpu")) for x in joint)
    o_ref, lse_ref = oatt.attention(jq, jk, jv, oatt.default_scale(w.head_dim))
    got = np.concatenate([f64(from_bits(out[0], "cpu"))[:, :w.n_rep + w.s_local],
                          f64(from_bits(out[1], "cpu"))[:, w.n_rep:]], axis=1)
    err = np.abs(got - o_ref)
    assert err.max() <= 2e-2 and err.mean() <= 1e-3, (err.max(), err.mean())
    # the replicated prefix rows are written to every shard, identically
    assert np.array_equal(out[0][:, :w.n_rep], out[1][:, :w.n_rep])
