"""GPU: ulys_lse_merge (ring / hybrid merge of partial attention over key blocks, flashdreams cp.py
_impl_ring) against the fp64 oracle merge and against attention over all keys."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import bits, check_attention, f64, from_bits, sample_rows
from oracle import attention as oatt
from oracle import merge as omerge
from ulysses_sequence_attention_amd import inputs

pytestmark = pytest.mark.gpu


def _slot(b, rows, heads, d, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((b, rows, heads, d), generator=g, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("b,rows,heads,d", [(1, 300, 2, 64), (2, 517, 3, 128)])
def test_merge_of_two_key_halves_is_full_attention(gpu, b, rows, heads, d):
    """Attention over keys [0, h) and over [h, rows) (the other half masked with a key gap), merged,
    equals attention over all keys: against the oracle, and close to the one-call GPU result."""
    q, k, v = (_slot(b, rows, heads, d, s) for s in (1, 2, 3))
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    half = rows // 2 + 7
    parts = []
    for gap in ((half, rows), (0, half)):
        o = torch.empty_like(qg)
        lse = torch.empty((b, heads, rows), dtype=torch.float32, device="cuda")
        gpu.ulys_attend_group(qg, kg, vg, o, lse, key_gaps=[gap] * b)
        parts.append((o, lse))
    om = torch.empty_like(qg)
    lm = torch.empty((b, heads, rows), dtype=torch.float32, device="cuda")
    gpu.ulys_lse_merge([p[0] for p in parts], [p[1] for p in parts], om, lm)
    of = torch.empty_like(qg)
    lf = torch.empty_like(lm)
    gpu.ulys_attend_group(qg, kg, vg, of, lf)
    torch.cuda.synchronize()
    o_ref, lse_ref = oatt.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                    oatt.default_scale(d))
    check_attention(om, lm, o_ref, lse_ref, label="merged halves")
    assert np.abs(f64(om) - f64(of)).max() <= 2e-2
    assert np.abs(f64(lm) - f64(lf)).max() <= 1e-4


@pytest.mark.parametrize("n", [1, 3, 16])
def test_merge_against_oracle(gpu, n):
    """Random partials (one part -inf on some rows) against the oracle's pairwise merge, in fp64."""
    b, rows, heads, d = 2, 77, 3, 64
    rng = np.random.default_rng(n)
    o_parts = [_slot(b, rows, heads, d, 100 + i) for i in range(n)]
    lses = [rng.uniform(-6.0, 6.0, size=(b, heads, rows)).astype(np.float32) for _ in range(n)]
    if n > 1:
        lses[1][:, :, ::5] = -np.inf
    og = [x.cuda() for x in o_parts]
    lg = [torch.from_numpy(x).cuda() for x in lses]
    out = torch.empty_like(og[0])
    lout = torch.empty((b, heads, rows), dtype=torch.float32, device="cuda")
    gpu.ulys_lse_merge(og, lg, out, lout)
    torch.cuda.synchronize()
    o_ref, l_ref = omerge.merge_partials([x.double().numpy() for x in o_parts], lses)
    err = np.abs(f64(out) - o_ref)
    # bf16 output rounding (|o| < 4.5) plus fp32 weights
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    assert np.abs(f64(lout) - l_ref).max() <= 1e-5
    if n == 1:   # one part: the output is the part itself
        assert np.array_equal(bits(out), bits(o_parts[0]))


def test_merge_empty_rows_and_in_place(gpu):
    """Rows whose parts all have lse = -inf give o = 0 and lse = -inf; o_out may be a part."""
    b, rows, heads, d = 1, 40, 2, 128
    o_parts = [_slot(b, rows, heads, d, 200 + i).cuda() for i in range(2)]
    lses = [torch.randn((b, heads, rows), device="cuda") for _ in range(2)]
    for x in lses:
        x[:, :, 3] = -float("inf")
    ref = torch.empty_like(o_parts[0])
    lref = torch.empty_like(lses[0])
    gpu.ulys_lse_merge(o_parts, lses, ref, lref)
    torch.cuda.synchronize()
    assert torch.all(ref[:, 3] == 0) and torch.all(torch.isneginf(lref[:, :, 3]))
    inplace = o_parts[0].clone()
    gpu.ulys_lse_merge([inplace, o_parts[1]], lses, inplace)
    torch.cuda.synchronize()
    assert np.array_equal(bits(inplace), bits(ref))


def test_merge_wan_share_ring_of_two(gpu):
    """The Wan share (N = 27280, 2 heads, D = 128) split into two key halves and merged, sampled
    rows against the oracle over all keys."""
    w = inputs.WAN_SHARE_G5
    q, k, v = inputs.global_qkv(w)
    q, k, v = q[:, :, :2].contiguous(), k[:, :, :2].contiguous(), v[:, :, :2].contiguous()
    n = q.shape[1]
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    parts = []
    for gap in ((n // 2, n), (0, n // 2)):
        o = torch.empty_like(qg)
        lse = torch.empty((1, 2, n), dtype=torch.float32, device="cuda")
        gpu.ulys_attend_group(qg, kg, vg, o, lse, key_gaps=[gap])
        parts.append((o, lse))
    om = torch.empty_like(qg)
    lm = torch.empty((1, 2, n), dtype=torch.float32, device="cuda")
    gpu.ulys_lse_merge([p[0] for p in parts], [p[1] for p in parts], om, lm)
    torch.cuda.synchronize()
    rows = sample_rows(n, boundaries=(n // 2,), edge=4, extra=24)
    o_ref, lse_ref = oatt.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                    oatt.default_scale(128), rows=rows)
    check_attention(om, lm, o_ref, lse_ref, rows=rows, label="wan ring of two")
