"""GPU parity of the range split: R workgroups per (b, head), each taking an equal run of the
(query tile, key tile) sequence; the pieces of a tile cut by run ends are merged by a second
kernel, in run order.

Against the fp64 oracle (which never splits): run counts from 3 to 128 over ragged shapes, gaps,
key masks, runs that are empty or hold one key tile, fp8 q/k, and the 27280-row Wan shape on
sampled rows.  Byte rules: head subsets and masks equal to gaps give the same bytes at the same run
count; repeated calls (before and after a call of another shape, which reuses the workspace) and
calls on another stream give the same bytes; the automatic choice is the reported one.  Inputs are seeded (ulysses_sequence_attention_amd.inputs).
"""
import numpy as np
import pytest
import torch

from gpu_common import bits, check_attention, from_bits, inputs, oatt, ofp8, sample_rows

pytestmark = pytest.mark.gpu


def _qkv(seed, b, nq, nk, hq, hkv, d):
    q = bits(inputs.random_bf16((b, nq, hq, d), seed))
    k = bits(inputs.random_bf16((b, nk, hkv, d), seed + 1))
    v = bits(inputs.random_bf16((b, nk, hkv, d), seed + 2))
    return q, k, v


def _run(ulys, q, k, v, ranges, gaps=None, mask=None, fp8=False, amax=None, stream=None):
    b, nq, hq, d = q.shape
    o = torch.full((b, nq, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((b, hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    words = None if mask is None else inputs.key_mask_words(mask).cuda()
    ulys.ulys_attend_group_ex(q, k, v, o, l, key_gaps=gaps, key_mask=words, key_splits=-ranges,
                              qk_dtype=ulys.ULYS_FP8_E4M3 if fp8 else ulys.ULYS_BF16, qk_amax=amax, stream=stream)
    torch.cuda.synchronize()
    return o, l


def _as_f64(a16):
    return torch.from_numpy(a16).view(torch.bfloat16).double().numpy()


def _same(x, y):
    o1, l1 = x
    o2, l2 = y
    return torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


RANGE_CASES = [  # b, nq, nk, hq, hkv, d, ranges, gaps
    (1, 700, 1500, 2, 1, 128, 5, None),            # 3 query tiles x 24 key tiles in 5 runs
    (2, 300, 2100, 2, 2, 64, 3, [(100, 700), (0, 0)]),
    (1, 513, 4000, 2, 2, 128, 64, [(1000, 2500)]),  # up to 22 pieces per tile
    (1, 1000, 1000, 4, 4, 128, 7, None),
    (1, 1, 4100, 1, 1, 128, 32, None),              # one query row, 65 key tiles in 32 runs
    (3, 100, 1000, 2, 2, 64, 20, None),             # 16 units in 20 runs: 4 runs empty
    (1, 2, 33, 2, 2, 128, 32, None),                # one unit: 31 empty runs, one whole tile
    (1, 1030, 3333, 2, 2, 128, 9, [(3300, 3333)]),  # ragged last query tile and key tile
    (1, 500, 1000, 2, 2, 128, 6, [(100, 512)]),     # a skipped tile-aligned gap end, then a ragged last tile
]


@pytest.mark.parametrize("case", RANGE_CASES)
def test_ranges_vs_oracle(gpu, case):
    b, nq, nk, hq, hkv, d, ranges, gaps = case
    q, k, v = _qkv(1100 + nq, b, nq, nk, hq, hkv, d)
    o, l = _run(gpu, from_bits(q), from_bits(k), from_bits(v), ranges, gaps=gaps)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), gaps)
    check_attention(o, l, o_ref, l_ref, label=f"ranges {ranges}")


@pytest.mark.parametrize("ranges", [2, 5, 13])
def test_ranges_with_key_masks(gpu, ranges):
    """Random masks plus long masked runs: the runs are taken over the listed tiles."""
    b, nq, nk, hq, hkv, d = 2, 600, 5000, 2, 2, 128
    q, k, v = _qkv(1150, b, nq, nk, hq, hkv, d)
    mask = inputs.random_key_mask(b, nk, seed=1151, p_valid=0.4)
    mask[0, 300:3000] = False
    mask[1, :4000] = False
    o, l = _run(gpu, from_bits(q), from_bits(k), from_bits(v), ranges, mask=mask)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), key_mask=mask)
    check_attention(o, l, o_ref, l_ref, label=f"mask ranges {ranges}")


def test_ranges_fully_masked_batch(gpu):
    """A batch whose mask leaves no key: each tile is one empty unit, written as o = 0, lse = -inf."""
    b, nq, nk, hq, d = 2, 600, 2000, 2, 128
    q, k, v = _qkv(1160, b, nq, nk, hq, hq, d)
    mask = np.ones((b, nk), dtype=bool)
    mask[1] = False
    o, l = _run(gpu, from_bits(q), from_bits(k), from_bits(v), 5, mask=mask)
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(l[1]))
    o_ref, l_ref = oatt.attention(_as_f64(q[:1]), _as_f64(k[:1]), _as_f64(v[:1]), oatt.default_scale(d))
    check_attention(o[:1], l[:1], o_ref, l_ref, label="batch 0")


def test_ranges_mask_of_gap_head_subset_and_repeats(gpu):
    """At one run count: a mask marking exactly the keys outside the gap gives the gap's bytes, a
    head subset gives the full call's bytes for those heads, and repeated calls give the same bytes
    (before and after a call of another shape)."""
    b, nq, nk, hq, hkv, d, ranges = 1, 900, 3000, 6, 3, 128, 7
    q, k, v = _qkv(1170, b, nq, nk, hq, hkv, d)
    qd, kd, vd = from_bits(q), from_bits(k), from_bits(v)
    gaps = [(700, 1900)]
    full = _run(gpu, qd, kd, vd, ranges, gaps=gaps)
    mask = np.ones((b, nk), dtype=bool)
    mask[0, 700:1900] = False
    assert _same(_run(gpu, qd, kd, vd, ranges, mask=mask), full)
    og, lg = _run(gpu, from_bits(q[:, :, 2:4]), from_bits(k[:, :, 1:2]), from_bits(v[:, :, 1:2]), ranges, gaps=gaps)
    assert torch.equal(og.view(torch.int16), full[0][:, :, 2:4].contiguous().view(torch.int16))
    assert torch.equal(lg, full[1][:, 2:4].contiguous())
    assert _same(_run(gpu, qd, kd, vd, ranges, gaps=gaps), full)
    q2, k2, v2 = _qkv(1175, 2, 300, 700, 2, 2, 64)
    _run(gpu, from_bits(q2), from_bits(k2), from_bits(v2), 3)
    assert _same(_run(gpu, qd, kd, vd, ranges, gaps=gaps), full)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), gaps)
    check_attention(full[0], full[1], o_ref, l_ref, label="ranges 7, gap")


def test_ranges_on_another_stream(gpu):
    side = torch.cuda.Stream()
    for i, (b, nq, nk, hq, d, r) in enumerate([(1, 600, 2000, 2, 128, 3), (1, 2000, 9000, 4, 128, 11)]):
        q, k, v = _qkv(1180 + i, b, nq, nk, hq, hq, d)
        qd, kd, vd = from_bits(q), from_bits(k), from_bits(v)
        first = _run(gpu, qd, kd, vd, r)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            other = _run(gpu, qd, kd, vd, r, stream=side)
        assert _same(first, other), f"shape {i}"


def test_fp8_with_ranges(gpu):
    d, rows = 128, 1200
    w = inputs.small("fp8ranges", 62, s_local=rows, hq=2, hkv=2, head_dim=d)
    qt, kt, vt = inputs.global_qkv(w)
    aq = ofp8.amax([qt.float().numpy()])
    ak = ofp8.amax([kt.float().numpy()])
    sq, iq = ofp8.scales_from_amax(aq)
    sk, ik = ofp8.scales_from_amax(ak)
    qc = ofp8.quantize(qt.float().numpy(), iq)
    kc = ofp8.quantize(kt.float().numpy(), ik)
    amax = torch.tensor([aq, ak], dtype=torch.float32, device="cuda")
    o, l = _run(gpu, torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), vt.cuda(), 6, gaps=[(10, 300)],
                fp8=True, amax=amax)
    c = ofp8.score_scale(oatt.default_scale(d), sq, sk)
    o_ref, l_ref = oatt.attention(ofp8.decode(qc), ofp8.decode(kc), vt.double().numpy(), float(c), [(10, 300)])
    check_attention(o, l, o_ref, l_ref, label="fp8 ranges 6", fp8=True)


def test_ranges_wan_shape_sampled_rows(gpu):
    """The 27280-row, 2-head launch in 128 runs (0.84 query tile each, so nearly every tile is cut):
    sampled rows against the oracle, and head 1 alone gives the 2-head call's bytes."""
    b, n, hq, d, ranges = 1, 27280, 2, 128, 128
    q, k, v = _qkv(1190, b, n, n, hq, hq, d)
    qd, kd, vd = from_bits(q), from_bits(k), from_bits(v)
    o, l = _run(gpu, qd, kd, vd, ranges)
    rows = sample_rows(n, boundaries=(256, 215 * 128, n - 100), extra=24)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), rows=rows)
    check_attention(o, l, o_ref, l_ref, rows=rows, label="Wan shape, 128 runs")
    o1, l1 = _run(gpu, qd[:, :, 1:2].contiguous(), kd[:, :, 1:2].contiguous(), vd[:, :, 1:2].contiguous(), ranges)
    assert torch.equal(o1.view(torch.int16), o[:, :, 1:2].contiguous().view(torch.int16))
    assert torch.equal(l1, l[:, 1:2].contiguous())


def test_automatic_ranges_is_the_reported_one(gpu):
    """key_splits = 0 at the Wan shape gives the bytes of -R, R as ulys_attend_ranges reports for the device."""
    b, n, hq, d = 1, 27280, 2, 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert gpu.ulys_attend_splits(b, n, n, cus) == 1
    r = gpu.ulys_attend_ranges(b, n, n, cus)
    q, k, v = _qkv(1195, b, n, n, hq, hq, d)
    qd, kd, vd = from_bits(q), from_bits(k), from_bits(v)
    o = torch.empty((b, n, hq, d), dtype=torch.bfloat16, device="cuda")
    l = torch.empty((b, hq, n), dtype=torch.float32, device="cuda")
    gpu.ulys_attend_group_ex(qd, kd, vd, o, l, key_splits=0)
    torch.cuda.synchronize()
    assert r > 0
    assert _same((o, l), _run(gpu, qd, kd, vd, r))


def test_ranges_heads_in_several_launches(gpu):
    """4096 runs over 128 query tiles need 1.03 GB of partials per head, so the 2 GiB workspace
    takes one head per launch: 3 launches, each head as in a one-head call."""
    b, n, hq, d, ranges = 1, 32768, 3, 128, 4096
    q, k, v = _qkv(1200, b, n, n, hq, 1, d)
    qd, kd, vd = from_bits(q), from_bits(k), from_bits(v)
    o, l = _run(gpu, qd, kd, vd, ranges)
    rows = sample_rows(n, boundaries=(256, n - 200), extra=16)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), rows=rows)
    check_attention(o, l, o_ref, l_ref, rows=rows, label="3 launches")
    o1, l1 = _run(gpu, qd[:, :, 2:3].contiguous(), kd, vd, ranges)
    assert torch.equal(o1.view(torch.int16), o[:, :, 2:3].contiguous().view(torch.int16))
    assert torch.equal(l1, l[:, 2:3].contiguous())


def test_ranges_gqa_mask_fp8_d64(gpu):
    """GQA 4:1, head_dim 64, e4m3 q/k and a key mask with per-batch tile counts, in 11 runs."""
    b, nq, nk, hq, hkv, d, ranges = 3, 700, 2600, 4, 1, 64, 11
    q = inputs.random_bf16((b, nq, hq, d), 1210).float().numpy()
    k = inputs.random_bf16((b, nk, hkv, d), 1211).float().numpy()
    v = inputs.random_bf16((b, nk, hkv, d), 1212)
    mask = inputs.random_key_mask(b, nk, seed=1213, p_valid=0.5)
    mask[1, 700:2400] = False
    mask[2, :64] = False
    aq, ak = ofp8.amax([q]), ofp8.amax([k])
    sq, iq = ofp8.scales_from_amax(aq)
    sk, ik = ofp8.scales_from_amax(ak)
    qc, kc = ofp8.quantize(q, iq), ofp8.quantize(k, ik)
    amax = torch.tensor([aq, ak], dtype=torch.float32, device="cuda")
    o, l = _run(gpu, torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), v.cuda(), ranges, mask=mask,
                fp8=True, amax=amax)
    c = ofp8.score_scale(oatt.default_scale(d), sq, sk)
    o_ref, l_ref = oatt.attention(ofp8.decode(qc), ofp8.decode(kc), v.double().numpy(), float(c), key_mask=mask)
    check_attention(o, l, o_ref, l_ref, label="GQA fp8 mask ranges 11", fp8=True)
