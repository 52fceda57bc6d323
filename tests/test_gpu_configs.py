"""GPU parity at the workloads' own sizes: head-group calls equal the unsplit call byte for byte,
sampled rows of every head against the fp64 oracle, and the rank pipeline at the group count
ulys_auto_groups picks.

sglang PR #43521, "Motivation": the pipelined per-group result must be bit for bit that of the
sequential exchange; "Accuracy Tests": every case is compared byte for byte against attention over the
global layout with every head at once, including automatic groups accepted at a shape that fills the GPU
and declined at one that does not.  Slots are packed on the CPU by the oracle (or by the library's pack,
itself checked byte for byte against the oracle), so no expected value comes from the HIP path.
"""
import numpy as np
import pytest
import torch

from gpu_common import (bits, check_attention, f64, from_bits, inputs, layout_of, oatt, ofp8, olay, sample_rows,
                        shards_of)

pytestmark = pytest.mark.gpu


def _as_f64(a16):
    return torch.from_numpy(np.ascontiguousarray(a16)).view(torch.bfloat16).double().numpy()


def _attend(ulys, q, k, v, gaps=None, fp8=False, amax=None):
    b, rows, hq, d = q.shape
    o = torch.empty((b, rows, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, rows), dtype=torch.float32, device="cuda")
    ulys.ulys_attend_group(q, k, v, o, lse, key_gaps=gaps, qk_dtype=ulys.ULYS_FP8_E4M3 if fp8 else ulys.ULYS_BF16,
                           qk_amax=amax)
    torch.cuda.synchronize()
    return o, lse


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                       b.contiguous().view(torch.int32 if b.dtype == torch.float32 else torch.int16))


def test_joint_varlen_groups_equal_full_call(gpu):
    """Joint text+image workload at full size (512-row prefix with keys [226, 512) masked, 32760 image
    rows, 12 heads): the 12-head call under its automatic split equals its three 4-head group calls
    byte for byte (o and lse), and sampled rows of all 12 heads match the oracle."""
    w = inputs.JOINT_VARLEN
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    gaps = [w.key_gap]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"joint varlen: rows {w.rows}, range split {gpu.ulys_attend_ranges(1, w.rows, w.rows, cus)}, "
          f"key split {gpu.ulys_attend_splits(1, w.rows, w.rows, cus)}", flush=True)
    of, lf = _attend(gpu, from_bits(q), from_bits(k), from_bits(v), gaps=gaps)
    gh = w.hq // w.groups
    for g in range(w.groups):
        sl = slice(gh * g, gh * (g + 1))
        og, lg = _attend(gpu, from_bits(q[:, :, sl]), from_bits(k[:, :, sl]), from_bits(v[:, :, sl]), gaps=gaps)
        assert _same(og, of[:, :, sl]), f"group {g} o"
        assert _same(lg, lf[:, sl]), f"group {g} lse"
    rows = sample_rows(w.rows, boundaries=(226, 512, w.rows - 256), edge=4, extra=24)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(128), gaps, rows=rows)
    check_attention(of, lf, o_ref, l_ref, rows=rows, label="joint varlen, 12 heads")



def test_joint_varlen_masked_kv_adversarial(gpu):
    """Joint text+image workload at full size, one 4-head group: replacing the masked keys' K by +1e4 and
    V by -1e4 (keys [226, 512)) leaves o and lse byte for byte the same (masked keys take no part, under
    the automatic range split of this shape)."""
    w = inputs.JOINT_VARLEN
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    gh = w.hq // w.groups
    q, k, v = (np.ascontiguousarray(x[:, :, :gh]) for x in (q, k, v))
    gaps = [w.key_gap]
    o1, l1 = _attend(gpu, from_bits(q), from_bits(k), from_bits(v), gaps=gaps)
    k2, v2 = _as_f64(k).copy(), _as_f64(v).copy()
    k2[:, w.key_gap[0]:w.key_gap[1]] = 1e4
    v2[:, w.key_gap[0]:w.key_gap[1]] = -1e4
    o2, l2 = _attend(gpu, from_bits(q), torch.from_numpy(k2).to(torch.bfloat16).cuda(),
                     torch.from_numpy(v2).to(torch.bfloat16).cuda(), gaps=gaps)
    assert _same(o1, o2) and _same(l1, l2)

def test_gqa_groups_equal_full_call(gpu):
    """GQA workload at full size (batch 2, 16384 rows, 16 q heads over 4 kv heads, q x 2): the unsplit
    16-head call equals its four groups of 4 q heads over 1 kv head byte for byte; sampled rows of every
    head of both batches match the oracle."""
    w = inputs.GQA
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    of, lf = _attend(gpu, from_bits(q), from_bits(k), from_bits(v))
    for g in range(4):
        og, lg = _attend(gpu, from_bits(q[:, :, 4 * g:4 * g + 4]), from_bits(k[:, :, g:g + 1]),
                         from_bits(v[:, :, g:g + 1]))
        assert _same(og, of[:, :, 4 * g:4 * g + 4]), f"group {g} o"
        assert _same(lg, lf[:, 4 * g:4 * g + 4]), f"group {g} lse"
    rows = sample_rows(w.rows, boundaries=(8192,), edge=4, extra=16)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(128), rows=rows)
    check_attention(of, lf, o_ref, l_ref, rows=rows, label="gqa, 16 heads")


@pytest.fixture(scope="module")
def e2e():
    w = inputs.E2E_P4
    (qt, kt, vt), sh = shards_of(w)
    dev = {k_: [from_bits(s) for s in v_] for k_, v_ in sh.items()}
    return w, (qt, kt, vt), dev


def _e2e_rank_outputs(gpu, w, dev, groups, amax):
    """Every rank through amax-scaled fp8 pack -> attend per group -> unpack, with `groups` head groups.
    Returns (output shards, lse [rank][G, 1, Gq, rows])."""
    import dataclasses
    L = layout_of(dataclasses.replace(w, groups=groups))
    qs = torch.empty((groups, 1, L.rows, L.gq, 128), dtype=torch.uint8, device="cuda")
    ks = torch.empty_like(qs)
    vs = torch.empty((groups, 1, L.rows, L.gkv, 128), dtype=torch.bfloat16, device="cuda")
    os_ = torch.empty_like(vs)
    out = [torch.full_like(s, float("nan")) for s in dev["q"]]
    lses = []
    for rank in range(w.degree):
        lse = torch.empty((groups, 1, L.gq, L.rows), dtype=torch.float32, device="cuda")
        gpu.ulys_pack(L, rank, -1, dev["q"], dev["k"], dev["v"], qs, ks, vs, gpu.ULYS_FP8_E4M3, amax)
        for g in range(groups):
            gpu.ulys_attend_group(qs[g], ks[g], vs[g], os_[g], lse[g], qk_dtype=gpu.ULYS_FP8_E4M3, qk_amax=amax)
        gpu.ulys_unpack(L, rank, -1, os_, out)
        lses.append(lse)
    torch.cuda.synchronize()
    return out, lses


def test_e2e_p4_fp8_five_groups_equal_one_call(gpu, e2e):
    """End-to-end Ulysses-4 workload with e4m3 q/k: every rank's path at G = 5 (five 2-head slots) gives
    the same output shards and LSEs, byte for byte, as at G = 1 (one 10-head slot); sampled rows of the
    output and of the LSE match the oracle on the oracle's own quantisation."""
    w, (qt, kt, vt), dev = e2e
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    gpu.ulys_amax_bf16(dev["q"], amax[0:1])
    gpu.ulys_amax_bf16(dev["k"], amax[1:2])
    out5, lse5 = _e2e_rank_outputs(gpu, w, dev, 5, amax)
    out1, lse1 = _e2e_rank_outputs(gpu, w, dev, 1, amax)
    for p in range(w.degree):
        assert _same(out5[p], out1[p]), f"output shard {p}"
        # lse of G = 5 is [5, 1, 2, rows], of G = 1 [1, 1, 10, rows]: the same heads in the same order
        assert _same(lse5[p].reshape(10, -1), lse1[p].reshape(10, -1)), f"lse of rank {p}"
    aq = ofp8.amax([qt.float().numpy()])
    ak = ofp8.amax([kt.float().numpy()])
    assert amax[0].item() == aq and amax[1].item() == ak
    sq, iq = ofp8.scales_from_amax(aq)
    sk, ik = ofp8.scales_from_amax(ak)
    c = float(ofp8.score_scale(oatt.default_scale(128), sq, sk))
    rows = sample_rows(w.rows, boundaries=(6820, 13640, 20460), edge=3, extra=12)
    for rank in (0, 3):
        heads = [10 * rank + j for j in (0, 3, 9)]
        qd = ofp8.decode(ofp8.quantize(qt[:, :, heads].float().numpy(), iq))
        kd = ofp8.decode(ofp8.quantize(kt[:, :, heads].float().numpy(), ik))
        o_ref, l_ref = oatt.attention(qd, kd, vt[:, :, heads].double().numpy(), c, rows=rows)
        got_o = np.concatenate([f64(s) for s in out1], axis=1)[:, rows][:, :, heads]
        got_l = f64(lse1[rank].reshape(1, 10, -1))[:, [h - 10 * rank for h in heads]][:, :, rows]
        check_attention(got_o, got_l, o_ref, l_ref, label=f"e2e fp8 rank {rank}", fp8=True)


def test_tiny_reading_b_four_heads_per_rank(gpu):
    """The tiny workload's other reading of "4 q heads": 4 heads per rank (8 model heads over P = 2) in
    two groups of 2, with the 32-row replicated prefix: slots byte-exact against the oracle's pack, and
    the output shards within tolerance of the oracle on the whole joint layout, every row."""
    import dataclasses
    w = dataclasses.replace(inputs.TINY, name="tiny_b", hq=8, hkv=8)
    L = layout_of(w)
    (qt, kt, vt), sh = shards_of(w)
    dev = {k_: [from_bits(s) for s in v_] for k_, v_ in sh.items()}
    assert L.gq == 2 and L.rows == 256
    qs, ks, vs, os_ = (torch.empty((2, 1, 256, 2, 64), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    lse = torch.empty((2, 1, 2, 256), dtype=torch.float32, device="cuda")
    out = [torch.full_like(s, float("nan")) for s in dev["q"]]
    lses = {}
    for rank in range(2):
        gpu.ulys_pack(L, rank, -1, dev["q"], dev["k"], dev["v"], qs, ks, vs)
        for g in range(2):
            gpu.ulys_attend_group(qs[g], ks[g], vs[g], os_[g], lse[g], softmax_scale=1 / 8)
        gpu.ulys_unpack(L, rank, -1, os_, out)
        torch.cuda.synchronize()
        for g in range(2):
            for name, slot in (("q", qs), ("k", ks), ("v", vs)):
                ref = olay.pack(sh[name], rank, g, 2, w.n_rep, w.rep_first)
                assert np.array_equal(bits(slot[g]), ref), f"{name} slot rank {rank} group {g}"
        lses[rank] = f64(lse.permute(1, 0, 2, 3).reshape(1, 4, 256))
    o_ref, l_ref = oatt.attention(qt.double().numpy(), kt.double().numpy(), vt.double().numpy(), 1 / 8)
    got = olay.joint_for_rank([f64(s) for s in out], 0, w.n_rep, w.rep_first)
    got_lse = np.concatenate([lses[0], lses[1]], axis=1)
    check_attention(got, got_lse, o_ref, l_ref, label="tiny reading B")


# ---- the automatic group count on the GPU ----

def _pipeline_outputs(gpu, L, dev, key_gaps=None, copy_stream=True):
    qs = torch.empty((L.groups, L.batch, L.rows, L.gq, L.head_dim), dtype=torch.bfloat16, device="cuda")
    ks = torch.empty((L.groups, L.batch, L.rows, L.gkv, L.head_dim), dtype=torch.bfloat16, device="cuda")
    vs = torch.empty_like(ks)
    os_ = torch.empty_like(qs)
    lse = torch.empty((L.groups, L.batch, L.gq, L.rows), dtype=torch.float32, device="cuda")
    out = [torch.full_like(s, float("nan")) for s in dev["q"]]
    xs = torch.cuda.Stream() if copy_stream else None
    for rank in range(L.degree):
        gpu.ulys_rank_pipeline(L, rank, dev["q"], dev["k"], dev["v"], qs, ks, vs, os_, out, lse=lse,
                               key_gaps=key_gaps, copy_stream=xs)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case,expect", [("joint_varlen", 4), ("e2e_p4", 5), ("decline_8192", 1)])
def test_rank_pipeline_at_auto_groups(gpu, case, expect):
    """ulys_rank_pipeline run at the group count ulys_auto_groups picks on this device gives the output
    shards of the G = 1 pipeline byte for byte; sampled rows match the oracle.  The joint workload and the
    Ulysses-4 workload split (4 and 5 groups); a rank of 8192 joint rows declines (1 group), and its
    2-group pipeline still equals the single call."""
    import dataclasses
    if case == "joint_varlen":
        w = inputs.JOINT_VARLEN
    elif case == "e2e_p4":
        w = dataclasses.replace(inputs.E2E_P4, fp8_qk=False)
    else:
        w = inputs.small("decline", 81, degree=4, s_local=2048, hq=40, hkv=40, head_dim=128, groups=1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    G = gpu.ulys_auto_groups(layout_of(w), cus)
    print(f"{case}: rows {w.rows}, auto groups {G} on {cus} CUs", flush=True)
    if cus == 256:
        assert G == expect
    (qt, kt, vt), sh = shards_of(w)
    dev = {k_: [from_bits(s) for s in v_] for k_, v_ in sh.items()}
    gaps = None if w.key_gap is None else [w.key_gap] * w.batch
    ref = _pipeline_outputs(gpu, layout_of(dataclasses.replace(w, groups=1)), dev, gaps, copy_stream=False)
    Gt = G if G > 1 else 2
    got = _pipeline_outputs(gpu, layout_of(dataclasses.replace(w, groups=Gt)), dev, gaps)
    for p in range(w.degree):
        assert _same(got[p], ref[p]), f"shard {p} at G = {Gt}"
    heads = [0, w.hq // w.degree - 1, w.hq - 1]
    rows = sample_rows(w.rows, boundaries=(226, 512) if w.key_gap else (w.s_local,), edge=3, extra=12)
    o_ref, _ = oatt.attention(qt[:, :, heads].double().numpy(), kt[:, :, heads].double().numpy(),
                              vt[:, :, heads].double().numpy(), oatt.default_scale(128), gaps, rows=rows)
    joint = olay.joint_for_rank([f64(s) for s in got], 0, w.n_rep, w.rep_first)
    err = np.abs(joint[:, rows][:, :, heads] - o_ref)
    assert err.max() <= 2e-2 and err.mean() <= 1e-3, (err.max(), err.mean())
