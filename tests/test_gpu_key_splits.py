"""GPU parity of the key-range split: each (b, head, query tile) computed as several
workgroups over contiguous runs of its key tiles, merged by log-sum-exp weights.

Against the fp64 oracle (which never splits): forced run counts from 2 to 16 over
ragged shapes, gaps, key masks, empty runs, fp8 q/k, and a call large enough to run
its heads in several launches.  Byte rules: head subsets and masks equal to gaps give
the same bytes at the same run count; the automatic count is the one the library
reports; calls on another stream give the same bytes.  Inputs are seeded
(ulysses_sequence_attention_amd.inputs).
"""
import numpy as np
import pytest
import torch

from gpu_common import bits, check_attention, f64, from_bits, inputs, oatt, ofp8, sample_rows

pytestmark = pytest.mark.gpu


def _qkv(seed, b, nq, nk, hq, hkv, d, q_mult=1.0):
    q = bits(inputs.random_bf16((b, nq, hq, d), seed, q_mult))
    k = bits(inputs.random_bf16((b, nk, hkv, d), seed + 1))
    v = bits(inputs.random_bf16((b, nk, hkv, d), seed + 2))
    return q, k, v


def _run(ulys, q, k, v, splits, gaps=None, mask=None, fp8=False, amax=None, stream=None):
    b, nq, hq, d = q.shape
    o = torch.full((b, nq, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((b, hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    words = None if mask is None else inputs.key_mask_words(mask).cuda()
    ulys.ulys_attend_group_ex(q, k, v, o, l, key_gaps=gaps, key_mask=words, key_splits=splits,
                              qk_dtype=ulys.ULYS_FP8_E4M3 if fp8 else ulys.ULYS_BF16, qk_amax=amax, stream=stream)
    torch.cuda.synchronize()
    return o, l


def _as_f64(a16):
    return torch.from_numpy(a16).view(torch.bfloat16).double().numpy()


SPLIT_CASES = [  # b, nq, nk, hq, hkv, d, splits, gaps
    (1, 700, 1500, 4, 2, 128, 2, None),
    (2, 300, 2100, 2, 1, 64, 3, [(100, 700), (0, 0)]),
    (1, 513, 4000, 2, 2, 128, 7, [(1000, 2500)]),
    (1, 200, 200, 2, 2, 128, 16, None),          # 4 key tiles: 12 runs are empty
    (3, 100, 1000, 4, 4, 64, 16, None),          # 16 tiles: one per run
    (1, 1030, 3333, 2, 2, 128, 5, [(3300, 3333)]),
    (1, 1, 4100, 1, 1, 128, 4, None),            # one query row
    (2, 33, 65, 2, 2, 64, 2, None),              # two tiles, the second holding one key
    (1, 500, 1000, 2, 2, 128, 3, [(100, 512)]),  # a skipped tile-aligned gap end, then a ragged last tile
]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_forced_splits_vs_oracle(gpu, case):
    b, nq, nk, hq, hkv, d, splits, gaps = case
    q, k, v = _qkv(900 + nq, b, nq, nk, hq, hkv, d)
    o, l = _run(gpu, from_bits(q), from_bits(k), from_bits(v), splits, gaps=gaps)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), gaps)
    check_attention(o, l, o_ref, l_ref, label=f"splits {splits}")


@pytest.mark.parametrize("splits", [1, 4, 9])
def test_splits_with_key_masks(gpu, splits):
    """Random masks plus long masked runs (whole tiles skipped, the runs taken over the listed tiles)."""
    b, nq, nk, hq, hkv, d = 2, 400, 5000, 2, 2, 128
    q, k, v = _qkv(950, b, nq, nk, hq, hkv, d)
    mask = inputs.random_key_mask(b, nk, seed=951, p_valid=0.4)
    mask[0, 300:3000] = False
    mask[1, :4000] = False
    o, l = _run(gpu, from_bits(q), from_bits(k), from_bits(v), splits, mask=mask)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), key_mask=mask)
    check_attention(o, l, o_ref, l_ref, label=f"mask splits {splits}")


def test_splits_fully_masked_batch(gpu):
    b, nq, nk, hq, d = 2, 300, 2000, 2, 128
    q, k, v = _qkv(960, b, nq, nk, hq, hq, d)
    mask = np.ones((b, nk), dtype=bool)
    mask[1] = False
    o, l = _run(gpu, from_bits(q), from_bits(k), from_bits(v), 4, mask=mask)
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(l[1]))
    o_ref, l_ref = oatt.attention(_as_f64(q[:1]), _as_f64(k[:1]), _as_f64(v[:1]), oatt.default_scale(d))
    check_attention(o[:1], l[:1], o_ref, l_ref, label="batch 0")


def test_splits_mask_of_gap_and_head_subset_bytes(gpu):
    """At one run count: a mask marking exactly the keys outside the gap gives the gap's bytes,
    and a head subset gives the full call's bytes for those heads."""
    b, nq, nk, hq, hkv, d, splits = 1, 600, 3000, 6, 3, 128, 6
    q, k, v = _qkv(970, b, nq, nk, hq, hkv, d)
    gaps = [(700, 1900)]
    of, lf = _run(gpu, from_bits(q), from_bits(k), from_bits(v), splits, gaps=gaps)
    mask = np.ones((b, nk), dtype=bool)
    mask[0, 700:1900] = False
    om, lm = _run(gpu, from_bits(q), from_bits(k), from_bits(v), splits, mask=mask)
    assert torch.equal(om.view(torch.int16), of.view(torch.int16)) and torch.equal(lm, lf)
    og, lg = _run(gpu, from_bits(q[:, :, 2:4]), from_bits(k[:, :, 1:2]), from_bits(v[:, :, 1:2]), splits, gaps=gaps)
    assert torch.equal(og.view(torch.int16), of[:, :, 2:4].contiguous().view(torch.int16))
    assert torch.equal(lg, lf[:, 2:4].contiguous())


def test_automatic_count_is_the_reported_one(gpu):
    """key_splits = 0 gives the bytes of the count ulys_attend_splits reports for the device."""
    b, nq, nk, hq, d = 1, 1500, 6000, 2, 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    c = gpu.ulys_attend_splits(b, nq, nk, cus)
    assert c > 1                                   # 6 query tiles per head cannot fill the device
    q, k, v = _qkv(980, b, nq, nk, hq, hq, d)
    oa, la = _run(gpu, from_bits(q), from_bits(k), from_bits(v), 0)
    oc, lc = _run(gpu, from_bits(q), from_bits(k), from_bits(v), c)
    assert torch.equal(oa.view(torch.int16), oc.view(torch.int16)) and torch.equal(la, lc)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d))
    check_attention(oa, la, o_ref, l_ref, label=f"auto {c}")


def test_splits_on_another_stream_and_workspace_growth(gpu):
    """Calls of growing and shrinking size on two streams: each stream has its own workspace,
    results equal the default stream's bytes."""
    shapes = [(1, 300, 2000, 2, 128), (1, 2000, 9000, 4, 128), (1, 300, 2000, 2, 128)]
    side = torch.cuda.Stream()
    for i, (b, nq, nk, hq, d) in enumerate(shapes):
        q, k, v = _qkv(990 + i, b, nq, nk, hq, hq, d)
        o1, l1 = _run(gpu, from_bits(q), from_bits(k), from_bits(v), 5)
        qd, kd, vd = from_bits(q), from_bits(k), from_bits(v)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            o2, l2 = _run(gpu, qd, kd, vd, 5, stream=side)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), f"shape {i}"


def test_fp8_with_splits(gpu):
    d, rows = 128, 1200
    w = inputs.small("fp8split", 61, s_local=rows, hq=2, hkv=2, head_dim=d)
    qt, kt, vt = inputs.global_qkv(w)
    aq = ofp8.amax([qt.float().numpy()])
    ak = ofp8.amax([kt.float().numpy()])
    sq, iq = ofp8.scales_from_amax(aq)
    sk, ik = ofp8.scales_from_amax(ak)
    qc = ofp8.quantize(qt.float().numpy(), iq)
    kc = ofp8.quantize(kt.float().numpy(), ik)
    amax = torch.tensor([aq, ak], dtype=torch.float32, device="cuda")
    o, l = _run(gpu, torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), vt.cuda(), 3, gaps=[(10, 300)],
                fp8=True, amax=amax)
    c = ofp8.score_scale(oatt.default_scale(d), sq, sk)
    o_ref, l_ref = oatt.attention(ofp8.decode(qc), ofp8.decode(kc), vt.double().numpy(), float(c), [(10, 300)])
    check_attention(o, l, o_ref, l_ref, label="fp8 splits 3", fp8=True)


def test_splits_heads_in_several_launches(gpu):
    """16 runs over 140000 query rows need 1.15 GB of partials per head, so the 2 GiB workspace
    takes one head per launch: 3 launches, each head as in a one-head call."""
    b, n, hq, d, splits = 1, 140000, 3, 128, 16
    q, k, v = _qkv(1000, b, n, n, hq, 1, d)
    qd, kd, vd = from_bits(q), from_bits(k), from_bits(v)
    o, l = _run(gpu, qd, kd, vd, splits)
    rows = sample_rows(n, boundaries=(256, n - 200), extra=24)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), rows=rows)
    check_attention(o, l, o_ref, l_ref, rows=rows, label="3 launches")
    o1, l1 = _run(gpu, qd[:, :, 1:2].contiguous(), kd, vd, splits)
    assert torch.equal(o1.view(torch.int16), o[:, :, 1:2].contiguous().view(torch.int16))
    assert torch.equal(l1, l[:, 1:2].contiguous())
