"""GPU parity: ulys_attend_group against the fp64 oracle, plus bit-exactness rules.

Inputs are seeded (ulysses_sequence_attention_amd.inputs); slots are built on
the CPU by the oracle's pack and uploaded, so no oracle input comes from the
HIP path.  Tolerances (o max abs 2e-2, mean abs 1e-3; lse 1e-3 abs) sit in
gpu_common.
"""
import numpy as np
import pytest
import torch

from gpu_common import (bits, check_attention, f64, from_bits, inputs, oatt, ofp8, olay, sample_rows,
                        shards_of)

pytestmark = pytest.mark.gpu


def _slots(w, rank=0, group=0, groups=None):
    """Oracle-packed q/k/v slots (int16 bit views) for (rank, group)."""
    _, sh = shards_of(w)
    G = w.groups if groups is None else groups
    return [olay.pack(sh[n], rank, group, G, w.n_rep, w.rep_first) for n in ("q", "k", "v")]


def _attend(ulys, q, k, v, scale=0.0, gaps=None, lse=True, fp8=False, amax=None):
    b, rows, hq, d = q.shape
    o = torch.empty((b, rows, hq, d), dtype=torch.bfloat16, device="cuda")
    l = torch.empty((b, hq, rows), dtype=torch.float32, device="cuda") if lse else None
    ulys.ulys_attend_group(q, k, v, o, l, softmax_scale=scale, key_gaps=gaps,
                           qk_dtype=ulys.ULYS_FP8_E4M3 if fp8 else ulys.ULYS_BF16, qk_amax=amax)
    torch.cuda.synchronize()
    return o, l


def _as_f64(a16):
    return torch.from_numpy(a16).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("rank,group", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_tiny_config_all_rows(gpu, rank, group):
    w = inputs.TINY
    qs, ks, vs = _slots(w, rank, group)
    o, l = _attend(gpu, from_bits(qs), from_bits(ks), from_bits(vs), scale=1 / 8)
    o_ref, l_ref = oatt.attention(_as_f64(qs), _as_f64(ks), _as_f64(vs), 1 / 8)
    check_attention(o, l, o_ref, l_ref, label=f"tiny r{rank} g{group}")


@pytest.mark.parametrize("b,rows,hq,hkv,d,gaps", [
    (1, 1, 1, 1, 64, None),                      # one row, one key
    (1, 300, 2, 2, 128, None),                   # ragged: 2 q tiles, 5 key tiles
    (1, 1000, 3, 1, 64, None),                   # GQA 3:1, ragged
    (2, 777, 4, 2, 128, [(100, 300), (0, 64)]),  # per-batch gaps, one on a tile edge
    (1, 513, 2, 2, 128, [(1, 513)]),             # a single valid key
    (1, 600, 2, 2, 64, [(226, 600)]),            # tail padding
    (1, 700, 2, 2, 128, [(0, 699)]),             # only the last key valid
    (1, 640, 2, 2, 128, [(64, 576)]),            # gap aligned to whole tiles
    # a gap ending on a tile edge whose last tile is skipped, then a ragged last tile (whose keys past
    # the end must still be masked): D = 128 and 64, and one per batch
    (1, 1000, 2, 2, 128, [(100, 512)]),
    (2, 700, 2, 1, 64, [(65, 256), (300, 640)]),
])
def test_ragged_masked_gqa(gpu, b, rows, hq, hkv, d, gaps):
    w = inputs.small("case", 40 + rows, batch=b, s_local=rows, hq=hq, hkv=hkv, head_dim=d, q_mult=2.0)
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    o, l = _attend(gpu, from_bits(q), from_bits(k), from_bits(v), gaps=gaps)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), gaps)
    check_attention(o, l, o_ref, l_ref, label=f"b{b} n{rows} h{hq}/{hkv} d{d} gaps {gaps}")


@pytest.mark.parametrize("gap", [(5, 6), (31, 33), (32, 64), (63, 65), (100, 300), (0, 1), (449, 450),
                                 (200, 450), (1, 450)])
def test_gap_edges(gpu, gap):
    """Masked key ranges that start/end inside, on and across 32-key blocks and 64-key tiles."""
    w = inputs.small("gapedge", 70, s_local=450, hq=2, hkv=1, head_dim=128, q_mult=2.0)
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    o, l = _attend(gpu, from_bits(q), from_bits(k), from_bits(v), gaps=[gap])
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(128), [gap])
    check_attention(o, l, o_ref, l_ref, label=f"gap {gap}")


def test_masked_kv_contents_do_not_matter(gpu):
    """Masked keys get zero weight: replacing their K/V by +-1e4 leaves o and lse bit-identical."""
    w = inputs.small("adv", 50, s_local=900, hq=2, hkv=2, head_dim=128)
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    gaps = [(226, 512)]
    o1, l1 = _attend(gpu, from_bits(q), from_bits(k), from_bits(v), gaps=gaps)
    k2, v2 = _as_f64(k).copy(), _as_f64(v).copy()
    k2[:, 226:512] = 1e4
    v2[:, 226:512] = -1e4
    k2t = torch.from_numpy(k2).to(torch.bfloat16).cuda()
    v2t = torch.from_numpy(v2).to(torch.bfloat16).cuda()
    o2, l2 = _attend(gpu, from_bits(q), k2t, v2t, gaps=gaps)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_head_subset_is_bit_identical_to_full_call(gpu):
    """Attention of a head group equals, byte for byte, the same heads of the full call
    (the pipelined result must be bit for bit the sequential one)."""
    w = inputs.small("split", 51, s_local=1500, hq=10, hkv=10, head_dim=128, groups=5)
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    of, lf = _attend(gpu, from_bits(q), from_bits(k), from_bits(v))
    for g in range(5):
        sl = slice(2 * g, 2 * g + 2)
        og, lg = _attend(gpu, from_bits(q[:, :, sl]), from_bits(k[:, :, sl]), from_bits(v[:, :, sl]))
        assert torch.equal(og.view(torch.int16), of[:, :, sl].contiguous().view(torch.int16)), f"group {g}"
        assert torch.equal(lg, lf[:, sl].contiguous()), f"group {g} lse"


def test_gqa_split_bit_identical_and_repeat_kv(gpu):
    """GQA head groups (4 q heads over 1 kv head each) equal the unsplit call bit for bit;
    and GQA equals MHA with K/V repeated per q head."""
    w = inputs.small("gqa_split", 52, batch=2, s_local=700, hq=16, hkv=4, head_dim=128, q_mult=2.0)
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    of, lf = _attend(gpu, from_bits(q), from_bits(k), from_bits(v))
    for g in range(4):
        og, lg = _attend(gpu, from_bits(q[:, :, 4 * g:4 * g + 4]), from_bits(k[:, :, g:g + 1]),
                         from_bits(v[:, :, g:g + 1]))
        assert torch.equal(og.view(torch.int16), of[:, :, 4 * g:4 * g + 4].contiguous().view(torch.int16))
        assert torch.equal(lg, lf[:, 4 * g:4 * g + 4].contiguous())
    om, lm = _attend(gpu, from_bits(q), from_bits(np.repeat(k, 4, axis=2)), from_bits(np.repeat(v, 4, axis=2)))
    assert torch.equal(om.view(torch.int16), of.view(torch.int16)) and torch.equal(lm, lf)


def test_repeat_runs_are_deterministic(gpu):
    w = inputs.small("det", 53, s_local=2000, hq=4, hkv=4, head_dim=128)
    q, k, v = [from_bits(bits(x)) for x in inputs.global_qkv(w)]
    o1, l1 = _attend(gpu, q, k, v, gaps=[(10, 90)])
    for _ in range(3):
        o2, l2 = _attend(gpu, q, k, v, gaps=[(10, 90)])
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_lse_optional_and_output_unchanged(gpu):
    w = inputs.small("nolse", 54, s_local=333, hq=2, hkv=2, head_dim=64)
    q, k, v = [from_bits(bits(x)) for x in inputs.global_qkv(w)]
    o1, _ = _attend(gpu, q, k, v)
    o2, _ = _attend(gpu, q, k, v, lse=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ---- the workloads at full size, oracle on a deterministic row sample ----

def test_wan_share_full_size_sampled(gpu):
    w = inputs.WAN_SHARE
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    o, l = _attend(gpu, from_bits(q), from_bits(k), from_bits(v))
    rows = sample_rows(w.rows, boundaries=(256, 27136), extra=48)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(128), rows=rows)
    check_attention(o, l, o_ref, l_ref, rows=rows, label="wan share")


def test_wan_share_five_groups_bit_identical(gpu):
    w = inputs.WAN_SHARE
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    of, lf = _attend(gpu, from_bits(q), from_bits(k), from_bits(v))
    for g in range(5):
        sl = slice(2 * g, 2 * g + 2)
        og, lg = _attend(gpu, from_bits(q[:, :, sl]), from_bits(k[:, :, sl]), from_bits(v[:, :, sl]))
        assert torch.equal(og.view(torch.int16), of[:, :, sl].contiguous().view(torch.int16))
        assert torch.equal(lg, lf[:, sl].contiguous())


def test_joint_varlen_full_size_sampled(gpu):
    w = inputs.JOINT_VARLEN
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    gaps = [w.key_gap]
    rows = sample_rows(w.rows, boundaries=(226, 512), extra=48)
    for g in range(w.groups):
        sl = slice(4 * g, 4 * g + 4)
        o, l = _attend(gpu, from_bits(q[:, :, sl]), from_bits(k[:, :, sl]), from_bits(v[:, :, sl]), gaps=gaps)
        if g == 1:
            o_ref, l_ref = oatt.attention(_as_f64(q[:, :, sl]), _as_f64(k[:, :, sl]), _as_f64(v[:, :, sl]),
                                          oatt.default_scale(128), gaps, rows=rows)
            check_attention(o, l, o_ref, l_ref, rows=rows, label="joint varlen")


def test_gqa_full_size_sampled(gpu):
    w = inputs.GQA
    q, k, v = [bits(x) for x in inputs.global_qkv(w)]
    o, l = _attend(gpu, from_bits(q[:, :, 4:8]), from_bits(k[:, :, 1:2]), from_bits(v[:, :, 1:2]))
    rows = sample_rows(w.rows, extra=32)
    o_ref, l_ref = oatt.attention(_as_f64(q[:, :, 4:8]), _as_f64(k[:, :, 1:2]), _as_f64(v[:, :, 1:2]),
                                  oatt.default_scale(128), rows=rows)
    check_attention(o, l, o_ref, l_ref, rows=rows, label="gqa")


# ---- fp8 q/k ----

@pytest.mark.parametrize("d,rows,gaps", [(128, 700, None), (64, 450, [(100, 200)]), (128, 1030, [(0, 1000)])])
def test_fp8_attention_vs_oracle_on_decoded_codes(gpu, d, rows, gaps):
    """e4m3 q/k codes (oracle-quantised), bf16 v: the kernel must match fp64 attention on
    the decoded codes with c = (softmax_scale * q_scale) * k_scale."""
    w = inputs.small("fp8", 60 + d, s_local=rows, hq=2, hkv=2, head_dim=d)
    qt, kt, vt = inputs.global_qkv(w)
    aq = ofp8.amax([qt.float().numpy()])
    ak = ofp8.amax([kt.float().numpy()])
    sq, iq = ofp8.scales_from_amax(aq)
    sk, ik = ofp8.scales_from_amax(ak)
    qc = ofp8.quantize(qt.float().numpy(), iq)
    kc = ofp8.quantize(kt.float().numpy(), ik)
    amax = torch.tensor([aq, ak], dtype=torch.float32, device="cuda")
    o, l = _attend(gpu, torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), vt.cuda(), gaps=gaps,
                   fp8=True, amax=amax)
    c = ofp8.score_scale(oatt.default_scale(d), sq, sk)
    o_ref, l_ref = oatt.attention(ofp8.decode(qc), ofp8.decode(kc), vt.double().numpy(), float(c), gaps)
    check_attention(o, l, o_ref, l_ref, label=f"fp8 d{d}", fp8=True)


def test_e2e_p4_fp8_pipeline(gpu):
    """The Wan Ulysses-4 path for one simulated rank and for all four: amax -> pack 5 groups
    (e4m3 q/k, bf16 v) -> attend each group -> unpack; sampled rows of every output shard
    against the oracle on the whole joint layout with the oracle's own quantisation."""
    w = inputs.E2E_P4
    from gpu_common import layout_of
    L = layout_of(w)
    (qt, kt, vt), sh = shards_of(w)
    dev = {k_: [from_bits(s) for s in v_] for k_, v_ in sh.items()}
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    gpu.ulys_amax_bf16(dev["q"], amax[0:1])
    gpu.ulys_amax_bf16(dev["k"], amax[1:2])
    qs = torch.empty((w.groups, 1, L.rows, L.gq, 128), dtype=torch.uint8, device="cuda")
    ks = torch.empty_like(qs)
    vs = torch.empty((w.groups, 1, L.rows, L.gkv, 128), dtype=torch.bfloat16, device="cuda")
    os_ = torch.empty_like(vs)
    out = [torch.zeros_like(s) for s in dev["q"]]
    for rank in range(w.degree):
        gpu.ulys_pack(L, rank, -1, dev["q"], dev["k"], dev["v"], qs, ks, vs, gpu.ULYS_FP8_E4M3, amax)
        for g in range(w.groups):
            gpu.ulys_attend_group(qs[g], ks[g], vs[g], os_[g], None, qk_dtype=gpu.ULYS_FP8_E4M3, qk_amax=amax)
        gpu.ulys_unpack(L, rank, -1, os_, out)
    torch.cuda.synchronize()
    aq = ofp8.amax([qt.float().numpy()])
    ak = ofp8.amax([kt.float().numpy()])
    assert amax[0].item() == aq and amax[1].item() == ak
    sq, iq = ofp8.scales_from_amax(aq)
    sk, ik = ofp8.scales_from_amax(ak)
    heads = [0, 9, 10, 21, 39]
    qd = ofp8.decode(ofp8.quantize(qt[:, :, heads].float().numpy(), iq))
    kd = ofp8.decode(ofp8.quantize(kt[:, :, heads].float().numpy(), ik))
    c = float(ofp8.score_scale(oatt.default_scale(128), sq, sk))
    rows = sample_rows(w.rows, boundaries=(6820, 13640, 20460), edge=3, extra=12)
    o_ref, _ = oatt.attention(qd, kd, vt[:, :, heads].double().numpy(), c, rows=rows)
    got = np.concatenate([f64(s) for s in out], axis=1)[:, rows][:, :, heads]
    err = np.abs(got - o_ref)
    assert err.max() <= 2e-2 and err.mean() <= 1e-3, (err.max(), err.mean())
