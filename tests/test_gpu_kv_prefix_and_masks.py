"""GPU parity for the replicated K/V-only prefix layout (more keys than queries) and for
arbitrary key masks, against the fp64 oracle; plus the byte rules that tie them to the
plain calls (a mask equal to a gap gives the gap's bytes, head subsets give the full
call's bytes, the pipeline gives the sequential path's bytes).

Masks are seeded (ulysses_sequence_attention_amd.inputs.random_key_mask) and encoded
as the library's bit words on the host; slots are packed by the oracle on the CPU.
"""
import numpy as np
import pytest
import torch

from gpu_common import bits, check_attention, f64, from_bits, inputs, oatt, olay, sample_rows

pytestmark = pytest.mark.gpu


def _as_f64(a16):
    return torch.from_numpy(a16).view(torch.bfloat16).double().numpy()


def _attend_ex(ulys, q, k, v, gaps=None, mask=None, scale=0.0):
    b, nq, hq, d = q.shape
    o = torch.full((b, nq, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((b, hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    words = None if mask is None else inputs.key_mask_words(mask).cuda()
    ulys.ulys_attend_group_ex(q, k, v, o, l, softmax_scale=scale, key_gaps=gaps, key_mask=words)
    torch.cuda.synchronize()
    return o, l


def _kv_prefix_shards(seed, batch, degree, s_local, n_rep, hq, hkv, d):
    """q shards [B, S_l, Hq, D]; k/v shards [B, R + S_l, Hkv, D] sharing one replicated prefix."""
    q = [bits(inputs.random_bf16((batch, s_local, hq, d), seed + p)) for p in range(degree)]
    rep_k = bits(inputs.random_bf16((batch, n_rep, hkv, d), seed + 100))
    rep_v = bits(inputs.random_bf16((batch, n_rep, hkv, d), seed + 101))
    k = [np.concatenate([rep_k, bits(inputs.random_bf16((batch, s_local, hkv, d), seed + 200 + p))], axis=1)
         for p in range(degree)]
    v = [np.concatenate([rep_v, bits(inputs.random_bf16((batch, s_local, hkv, d), seed + 300 + p))], axis=1)
         for p in range(degree)]
    return q, k, v


KV_CASES = [  # batch, P, S_l, R, hq, hkv, D, G
    (1, 2, 200, 77, 4, 4, 128, 2),
    (2, 4, 96, 130, 8, 4, 64, 1),
    (1, 4, 1706, 512, 8, 8, 128, 2),
]


@pytest.mark.parametrize("case", KV_CASES)
def test_kv_prefix_pack_unpack_byte_exact(gpu, case):
    b, P, s_l, R, hq, hkv, d, G = case
    q, k, v = _kv_prefix_shards(11, b, P, s_l, R, hq, hkv, d)
    L = gpu.Layout(b, P, s_l, R, gpu.ULYS_REP_KV_PREFIX, hq, hkv, d, G)
    dq = [from_bits(x) for x in q]
    dk = [from_bits(x) for x in k]
    dv = [from_bits(x) for x in v]
    gq, gkv = hq // P // G, hkv // P // G
    for rank in range(P):
        qs = torch.empty((G, b, L.rows_q, gq, d), dtype=torch.bfloat16, device="cuda")
        ks = torch.empty((G, b, L.rows, gkv, d), dtype=torch.bfloat16, device="cuda")
        vs = torch.empty_like(ks)
        gpu.ulys_pack(L, rank, -1, dq, dk, dv, qs, ks, vs)
        torch.cuda.synchronize()
        for g in range(G):
            rq, rk, rv = olay.pack_kv_prefix(q, k, v, rank, g, G, R)
            assert np.array_equal(bits(qs[g]), rq), f"q slot r{rank} g{g}"
            assert np.array_equal(bits(ks[g]), rk), f"k slot r{rank} g{g}"
            assert np.array_equal(bits(vs[g]), rv), f"v slot r{rank} g{g}"
    # unpack: a seeded output slot per (rank, group) scattered back into [B, S_l, Hq, D] shards
    out = [torch.zeros((b, s_l, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    ref = [np.zeros((b, s_l, hq, d), dtype=np.int16) for _ in range(P)]
    for rank in range(P):
        for g in range(G):
            o_slot = bits(inputs.random_bf16((b, L.rows_q, gq, d), 900 + 10 * rank + g))
            gpu.ulys_unpack(L, rank, g, from_bits(o_slot), out)
            olay.unpack_kv_prefix(o_slot, ref, rank, g, G)
    torch.cuda.synchronize()
    for p in range(P):
        assert np.array_equal(bits(out[p]), ref[p]), f"o shard {p}"


@pytest.mark.parametrize("case,gap", [(KV_CASES[0], None), (KV_CASES[0], (30, 77)), (KV_CASES[1], (0, 100)),
                                      (KV_CASES[2], (226, 512))])
def test_kv_prefix_attention(gpu, case, gap):
    """Cross-attention of the P*S_l gathered q rows over the R + P*S_l keys (text keys partly masked)."""
    b, P, s_l, R, hq, hkv, d, G = case
    q, k, v = _kv_prefix_shards(21, b, P, s_l, R, hq, hkv, d)
    rq, rk, rv = olay.pack_kv_prefix(q, k, v, 1, 0, G, R)
    gaps = None if gap is None else [gap] * b
    o, l = _attend_ex(gpu, from_bits(rq), from_bits(rk), from_bits(rv), gaps=gaps)
    o_ref, l_ref = oatt.attention(_as_f64(rq), _as_f64(rk), _as_f64(rv), oatt.default_scale(d), gaps)
    check_attention(o, l, o_ref, l_ref, label=f"kv prefix {case} gap {gap}")


def test_kv_prefix_pipeline_matches_sequential(gpu):
    b, P, s_l, R, hq, hkv, d, G = 1, 2, 300, 64, 8, 4, 128, 2
    q, k, v = _kv_prefix_shards(31, b, P, s_l, R, hq, hkv, d)
    L = gpu.Layout(b, P, s_l, R, gpu.ULYS_REP_KV_PREFIX, hq, hkv, d, G)
    dq, dk, dv = [from_bits(x) for x in q], [from_bits(x) for x in k], [from_bits(x) for x in v]
    gq, gkv = hq // P // G, hkv // P // G
    rank = 1
    gaps = [(20, 64)]

    def slots():
        return (torch.empty((G, b, L.rows_q, gq, d), dtype=torch.bfloat16, device="cuda"),
                torch.empty((G, b, L.rows, gkv, d), dtype=torch.bfloat16, device="cuda"),
                torch.empty((G, b, L.rows, gkv, d), dtype=torch.bfloat16, device="cuda"),
                torch.empty((G, b, L.rows_q, gq, d), dtype=torch.bfloat16, device="cuda"))

    qs, ks, vs, os_ = slots()
    out_seq = [torch.zeros((b, s_l, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    lse_seq = torch.empty((G, b, gq, L.rows_q), dtype=torch.float32, device="cuda")
    for g in range(G):
        gpu.ulys_pack(L, rank, g, dq, dk, dv, qs[g], ks[g], vs[g])
        gpu.ulys_attend_group_ex(qs[g], ks[g], vs[g], os_[g], lse_seq[g], key_gaps=gaps)
        gpu.ulys_unpack(L, rank, g, os_[g], out_seq)
    qs2, ks2, vs2, os2 = slots()
    out_pipe = [torch.zeros_like(x) for x in out_seq]
    lse_pipe = torch.empty_like(lse_seq)
    side = torch.cuda.Stream()
    gpu.ulys_rank_pipeline(L, rank, dq, dk, dv, qs2, ks2, vs2, os2, out_pipe, lse_pipe, key_gaps=gaps,
                           copy_stream=side)
    torch.cuda.synchronize()
    for p in range(P):
        assert np.array_equal(bits(out_pipe[p]), bits(out_seq[p]))
    assert np.array_equal(lse_pipe.cpu().numpy().view(np.int32), lse_seq.cpu().numpy().view(np.int32))
    # and the result is the oracle's
    for g in range(G):
        rq, rk, rv = olay.pack_kv_prefix(q, k, v, rank, g, G, R)
        o_ref, l_ref = oatt.attention(_as_f64(rq), _as_f64(rk), _as_f64(rv), oatt.default_scale(d), gaps)
        check_attention(os2[g], lse_pipe[g], o_ref, l_ref, label=f"pipeline g{g}")


MASK_CASES = [  # batch, nq, nk, hq, hkv, d, p_valid
    (1, 300, 300, 2, 2, 128, 0.9),
    (2, 257, 700, 4, 2, 64, 0.5),
    (1, 500, 1000, 3, 1, 128, 0.1),
    (2, 129, 33, 2, 2, 128, 0.7),
]


@pytest.mark.parametrize("case", MASK_CASES)
def test_random_key_masks(gpu, case):
    b, nq, nk, hq, hkv, d, p = case
    q = bits(inputs.random_bf16((b, nq, hq, d), 41, 2.0))
    k = bits(inputs.random_bf16((b, nk, hkv, d), 42))
    v = bits(inputs.random_bf16((b, nk, hkv, d), 43))
    m = inputs.random_key_mask(b, nk, 44, p)
    m[:, 7] = True
    o, l = _attend_ex(gpu, from_bits(q), from_bits(k), from_bits(v), mask=m)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), key_mask=m)
    check_attention(o, l, o_ref, l_ref, label=f"mask {case}")


@pytest.mark.parametrize("pattern", ["tiles", "alternate", "tail", "head", "one_key", "gap_and_mask",
                                     "gap_in_full_mask"])
def test_masks_that_skip_tiles(gpu, pattern):
    """Masks that leave whole 64-key tiles empty (the tile list skips them) or single keys."""
    b, nq, nk, h, d = 1, 200, 1100, 2, 128
    q = bits(inputs.random_bf16((b, nq, h, d), 51, 2.0))
    k = bits(inputs.random_bf16((b, nk, h, d), 52))
    v = bits(inputs.random_bf16((b, nk, h, d), 53))
    m = np.ones((b, nk), dtype=bool)
    gaps = None
    if pattern == "tiles":
        m[:, 64:256] = False
        m[:, 500:640] = False
    elif pattern == "alternate":
        for t in range(0, nk, 128):
            m[:, t:t + 64] = False
    elif pattern == "tail":
        m[:, 130:] = False
    elif pattern == "head":
        m[:, :1000] = False
    elif pattern == "one_key":
        m[:] = False
        m[:, 777] = True
    elif pattern == "gap_and_mask":
        m = inputs.random_key_mask(b, nk, 54, 0.6)
        gaps = [(300, 700)]
    elif pattern == "gap_in_full_mask":   # mask words all ones where the gap cuts tiles 4 and 10
        m[:, 900:960] = False
        gaps = [(300, 700)]
    o, l = _attend_ex(gpu, from_bits(q), from_bits(k), from_bits(v), gaps=gaps, mask=m)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), gaps, key_mask=m)
    check_attention(o, l, o_ref, l_ref, label=f"mask pattern {pattern}")


def test_mask_of_gap_gives_the_gap_bytes(gpu):
    """A mask marking exactly the keys outside the gaps reproduces the gap call bit for bit,
    and ulys_attend_group equals ulys_attend_group_ex without a mask."""
    b, n, h, d = 2, 900, 2, 128
    q = bits(inputs.random_bf16((b, n, h, d), 61))
    k = bits(inputs.random_bf16((b, n, h, d), 62))
    v = bits(inputs.random_bf16((b, n, h, d), 63))
    gaps = [(100, 450), (0, 64)]
    m = np.ones((b, n), dtype=bool)
    for i, (g0, g1) in enumerate(gaps):
        m[i, g0:g1] = False
    o1 = torch.empty((b, n, h, d), dtype=torch.bfloat16, device="cuda")
    l1 = torch.empty((b, h, n), dtype=torch.float32, device="cuda")
    gpu.ulys_attend_group(from_bits(q), from_bits(k), from_bits(v), o1, l1, key_gaps=gaps)
    o2, l2 = _attend_ex(gpu, from_bits(q), from_bits(k), from_bits(v), gaps=gaps)
    o3, l3 = _attend_ex(gpu, from_bits(q), from_bits(k), from_bits(v), mask=m)
    for o, l in ((o2, l2), (o3, l3)):
        assert np.array_equal(bits(o), bits(o1))
        assert np.array_equal(l.cpu().numpy().view(np.int32), l1.cpu().numpy().view(np.int32))


def test_mask_head_subset_is_bit_identical(gpu):
    b, n, hq, hkv, d = 1, 640, 8, 4, 128
    q = bits(inputs.random_bf16((b, n, hq, d), 71))
    k = bits(inputs.random_bf16((b, n, hkv, d), 72))
    v = bits(inputs.random_bf16((b, n, hkv, d), 73))
    m = inputs.random_key_mask(b, n, 74, 0.4)
    m[:, 0] = True
    o, l = _attend_ex(gpu, from_bits(q), from_bits(k), from_bits(v), mask=m)
    for g in range(2):   # 2 groups of 4 q heads over 2 kv heads
        qs = np.ascontiguousarray(q[:, :, 4 * g:4 * g + 4])
        ks = np.ascontiguousarray(k[:, :, 2 * g:2 * g + 2])
        vs = np.ascontiguousarray(v[:, :, 2 * g:2 * g + 2])
        og, lg = _attend_ex(gpu, from_bits(qs), from_bits(ks), from_bits(vs), mask=m)
        assert np.array_equal(bits(og), bits(o[:, :, 4 * g:4 * g + 4]))
        assert np.array_equal(lg.cpu().numpy().view(np.int32), l[:, 4 * g:4 * g + 4].cpu().numpy().view(np.int32))


def test_fully_masked_batch_gives_zero_and_neg_inf(gpu):
    b, nq, nk, h, d = 2, 100, 300, 2, 64
    q = bits(inputs.random_bf16((b, nq, h, d), 81))
    k = bits(inputs.random_bf16((b, nk, h, d), 82))
    v = bits(inputs.random_bf16((b, nk, h, d), 83))
    m = inputs.random_key_mask(b, nk, 84, 0.5)
    m[1] = False
    o, l = _attend_ex(gpu, from_bits(q), from_bits(k), from_bits(v), mask=m)
    assert np.all(f64(o[1]) == 0.0)
    assert np.all(np.isneginf(f64(l[1])))
    o_ref, l_ref = oatt.attention(_as_f64(q[:1]), _as_f64(k[:1]), _as_f64(v[:1]), oatt.default_scale(d),
                                  key_mask=m[:1])
    check_attention(o[:1], l[:1], o_ref, l_ref, label="batch 0 beside a fully masked batch")


def test_mask_fp8_qk(gpu):
    """A key mask with e4m3 q/k (codes and scales from the oracle)."""
    from oracle import fp8 as ofp8
    b, n, h, d = 1, 520, 2, 128
    qf = inputs.random_bf16((b, n, h, d), 91, 2.0)
    kf = inputs.random_bf16((b, n, h, d), 92)
    v = bits(inputs.random_bf16((b, n, h, d), 93))
    aq, ak = ofp8.amax([qf.float().numpy()]), ofp8.amax([kf.float().numpy()])
    sq, iq = ofp8.scales_from_amax(aq)
    sk, ik = ofp8.scales_from_amax(ak)
    qc = ofp8.quantize(qf.float().numpy(), iq)
    kc = ofp8.quantize(kf.float().numpy(), ik)
    m = inputs.random_key_mask(b, n, 94, 0.3)
    m[:, 3] = True
    amax = torch.tensor([float(aq), float(ak)], dtype=torch.float32, device="cuda")
    o = torch.empty((b, n, h, d), dtype=torch.bfloat16, device="cuda")
    l = torch.empty((b, h, n), dtype=torch.float32, device="cuda")
    gpu.ulys_attend_group_ex(torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), from_bits(v), o, l,
                             key_mask=inputs.key_mask_words(m).cuda(), qk_dtype=gpu.ULYS_FP8_E4M3, qk_amax=amax)
    torch.cuda.synchronize()
    c = float(ofp8.score_scale(oatt.default_scale(d), sq, sk))
    o_ref, l_ref = oatt.attention(ofp8.decode(qc), ofp8.decode(kc), _as_f64(v), c, key_mask=m)
    check_attention(o, l, o_ref, l_ref, label="fp8 + mask", fp8=True)


def test_mask_at_the_key_limit(gpu):
    """262144 keys (the 4096-tile list limit) with a sparse mask; sampled query rows."""
    b, nq, nk, h, d = 1, 256, 262144, 1, 128
    q = bits(inputs.random_bf16((b, nq, h, d), 101, 2.0))
    k = bits(inputs.random_bf16((b, nk, h, d), 102))
    v = bits(inputs.random_bf16((b, nk, h, d), 103))
    m = inputs.random_key_mask(b, nk, 104, 0.02)
    m[:, -1] = True
    o, l = _attend_ex(gpu, from_bits(q), from_bits(k), from_bits(v), mask=m)
    rows = sample_rows(nq, every=16, extra=16)
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), rows=rows, key_mask=m)
    check_attention(o, l, o_ref, l_ref, rows=rows, label="262144 keys")


@pytest.mark.parametrize("splits", [0, 3, -6])
def test_mask_bits_past_the_last_key_are_ignored(gpu, splits):
    """The header's rule: bits of the last mask word for keys j >= kv_rows are ignored.  The words here have
    every such bit set (the last word all ones), with a ragged key count and a gap whose end is a tile edge
    (so its last tile is skipped); the result must be the oracle's over the real keys only, without a split,
    under a key-range split and under a range split."""
    b, nq, nk, hq, hkv, d = 1, 300, 1000, 2, 2, 128
    q = bits(inputs.random_bf16((b, nq, hq, d), 91))
    k = bits(inputs.random_bf16((b, nk, hkv, d), 92))
    v = bits(inputs.random_bf16((b, nk, hkv, d), 93))
    m = inputs.random_key_mask(b, nk, 94, 0.8)
    m[:, 960:] = True                                   # the last 64-key tile: every real key valid
    words = inputs.key_mask_words(m)
    words[:, -1] = -1                                   # ... and the 24 bits past the 1000th key set too
    gaps = [(100, 512)]
    o = torch.full((b, nq, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((b, hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    gpu.ulys_attend_group_ex(from_bits(q), from_bits(k), from_bits(v), o, l, key_gaps=gaps, key_mask=words.cuda(),
                             key_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oatt.attention(_as_f64(q), _as_f64(k), _as_f64(v), oatt.default_scale(d), gaps, key_mask=m)
    check_attention(o, l, o_ref, l_ref, label=f"mask bits past the end, splits {splits}")


def test_kv_prefix_masked_wan_share_full_size(gpu):
    """The bench's K/V-only-prefix workload at full size: four ranks' q shards hold only their 6820 image
    rows; the k/v shards carry 512 replicated text rows in front, of which the first 226 are valid by a
    key-mask bit array.  For rank 1, group 2 (2 of its 10 heads): the library's pack equals the oracle's
    K/V-prefix pack byte for byte; attention with the mask equals the same call with the padding given as
    a key gap byte for byte (o and lse); sampled rows match the oracle with the mask."""
    w = inputs.KV_PREFIX_MASKED
    q, k, v = inputs.global_qkv(w)
    P, S_l, R, G = w.degree, w.s_local, w.n_rep, w.groups
    qs = [bits(q[:, R + p * S_l:R + (p + 1) * S_l]) for p in range(P)]
    ks = [np.concatenate([bits(k[:, :R]), bits(k[:, R + p * S_l:R + (p + 1) * S_l])], axis=1) for p in range(P)]
    vs = [np.concatenate([bits(v[:, :R]), bits(v[:, R + p * S_l:R + (p + 1) * S_l])], axis=1) for p in range(P)]
    L = gpu.Layout(w.batch, P, S_l, R, gpu.ULYS_REP_KV_PREFIX, w.hq, w.hkv, w.head_dim, G)
    rank, g = 1, 2
    print(f"kv prefix masked: q rows {L.rows_q}, kv rows {L.rows}, rank {rank} group {g}", flush=True)
    dq = torch.empty((w.batch, L.rows_q, L.gq, w.head_dim), dtype=torch.bfloat16, device="cuda")
    dk = torch.empty((w.batch, L.rows, L.gkv, w.head_dim), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    gpu.ulys_pack(L, rank, g, [from_bits(x) for x in qs], [from_bits(x) for x in ks], [from_bits(x) for x in vs],
                  dq, dk, dv)
    torch.cuda.synchronize()
    rq, rk, rv = olay.pack_kv_prefix(qs, ks, vs, rank, g, G, R)
    assert np.array_equal(bits(dq), rq) and np.array_equal(bits(dk), rk) and np.array_equal(bits(dv), rv)
    mask = np.ones((w.batch, L.rows), dtype=bool)
    mask[:, w.extra["text_valid"]:R] = False
    om, lm = _attend_ex(gpu, dq, dk, dv, mask=mask)
    og, lg = _attend_ex(gpu, dq, dk, dv, gaps=[(w.extra["text_valid"], R)] * w.batch)
    assert np.array_equal(bits(om), bits(og)), "o: mask path differs from gap path"
    assert np.array_equal(lm.cpu().numpy().view(np.int32), lg.cpu().numpy().view(np.int32)), "lse differs"
    rows = sample_rows(L.rows_q, boundaries=(S_l, 2 * S_l, 3 * S_l), edge=4, extra=24)
    o_ref, l_ref = oatt.attention(_as_f64(rq), _as_f64(rk), _as_f64(rv), oatt.default_scale(w.head_dim),
                                  rows=rows, key_mask=mask)
    check_attention(om, lm, o_ref, l_ref, rows=rows, label="kv prefix masked, Wan share")
