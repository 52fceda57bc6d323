"""Pins for oracle.attention (CPU only).

* brute force: pure-Python loops with exactly rounded sums (oracle.brute);
* a library routine: torch CPU float64 scaled_dot_product_attention with a
  boolean key mask and K/V ``repeat_interleave`` for GQA (what sglang's
  ``LocalAttention.forward`` does), and scipy's logsumexp for the LSE;
* closed forms: q = 0, a single valid key, identical keys, constant V;
* invariants: key permutation, masked K/V contents, the ring LSE merge of
  two key halves (flashdreams ``cp.py`` ``_impl_ring``), GQA = MHA over
  repeated K/V, the suffix layout = the prefix layout rotated
  (sglang ``_forward_with_replicated_suffix``).
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention as oa
from oracle import brute


def _rand(shape, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * mult).to(torch.bfloat16).double().numpy()


def _sdpa_ref(q, k, v, scale, gaps):
    """torch float64 SDPA: [B,N,H,D] -> transpose to [B,H,N,D], bool mask, repeat_interleave."""
    qt = torch.from_numpy(q).transpose(1, 2)
    kt = torch.from_numpy(k).transpose(1, 2)
    vt = torch.from_numpy(v).transpose(1, 2)
    rep = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(rep, dim=1)
    vt = vt.repeat_interleave(rep, dim=1)
    nk = kt.shape[2]
    mask = torch.ones(q.shape[0], 1, 1, nk, dtype=torch.bool)
    for b, (g0, g1) in enumerate(gaps or []):
        mask[b, :, :, g0:g1] = False
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out.transpose(1, 2).numpy()


@pytest.mark.parametrize("b,n,hq,hkv,d,gaps", [
    (1, 12, 2, 2, 8, None),
    (2, 9, 4, 2, 4, [(2, 5), (0, 3)]),
    (1, 10, 3, 1, 6, [(7, 10)]),
])
def test_matches_bruteforce(b, n, hq, hkv, d, gaps):
    q, k, v = _rand((b, n, hq, d), 1), _rand((b, n, hkv, d), 2), _rand((b, n, hkv, d), 3)
    scale = 0.37
    o, lse = oa.attention(q, k, v, scale, gaps, block=4)
    ob, lseb = brute.attention(q.tolist(), k.tolist(), v.tolist(), float(np.float32(scale)), gaps)
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lseb))) < 1e-12


@pytest.mark.parametrize("b,n,hq,hkv,d,gaps", [
    (1, 64, 4, 4, 16, None),
    (2, 80, 8, 2, 32, [(10, 30), (60, 80)]),
    (1, 50, 4, 1, 8, [(0, 49)]),
])
def test_matches_torch_sdpa_f64(b, n, hq, hkv, d, gaps):
    q, k, v = _rand((b, n, hq, d), 4, 2.0), _rand((b, n, hkv, d), 5), _rand((b, n, hkv, d), 6)
    scale = float(np.float32(d ** -0.5))
    o, _ = oa.attention(q, k, v, scale, gaps)
    assert np.max(np.abs(o - _sdpa_ref(q, k, v, scale, gaps))) < 1e-12


def test_lse_is_logsumexp_of_scores():
    b, n, h, d = 2, 33, 2, 8
    q, k, v = _rand((b, n, h, d), 7), _rand((b, n, h, d), 8), _rand((b, n, h, d), 9)
    gaps = [(5, 9), (30, 33)]
    scale = 0.25
    _, lse = oa.attention(q, k, v, scale, gaps)
    for bb in range(b):
        keep = np.ones(n, bool)
        keep[gaps[bb][0]:gaps[bb][1]] = False
        for hh in range(h):
            s = scale * np.einsum("id,jd->ij", q[bb, :, hh], k[bb, keep, hh])
            assert np.allclose(lse[bb, hh], logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_closed_forms():
    b, n, h, d = 1, 20, 2, 8
    k, v = _rand((b, n, h, d), 10), _rand((b, n, h, d), 11)
    gap = [(3, 8)]
    valid = np.r_[0:3, 8:20]
    # q = 0: uniform weights over the valid keys, lse = ln |J|
    o, lse = oa.attention(np.zeros((b, n, h, d)), k, v, 0.5, gap)
    assert np.allclose(o[0, 5], v[0, valid].mean(axis=0), atol=1e-14)
    assert np.allclose(lse, np.log(len(valid)), atol=1e-14)
    # one valid key: o = v_j, lse = s_j
    q = _rand((b, n, h, d), 12)
    o, lse = oa.attention(q, k, v, 0.5, [(1, n)])
    assert np.allclose(o, np.broadcast_to(v[:, :1], o.shape), atol=1e-14)
    assert np.allclose(lse[0, 1], 0.5 * q[0, :, 1] @ k[0, 0, 1], atol=1e-12)
    # identical keys: o = mean of v
    kk = np.broadcast_to(k[:, :1], k.shape).copy()
    o, _ = oa.attention(q, kk, v, 0.5)
    assert np.allclose(o[0, 3], v[0].mean(axis=0), atol=1e-12)
    # constant V: o = V
    vc = np.broadcast_to(v[:, :1], v.shape).copy()
    o, _ = oa.attention(q, k, vc, 0.5, gap)
    assert np.allclose(o, np.broadcast_to(v[:, :1], o.shape), atol=1e-12)


def test_invariants():
    b, n, hq, hkv, d = 1, 40, 4, 2, 8
    q, k, v = _rand((b, n, hq, d), 13, 2.0), _rand((b, n, hkv, d), 14), _rand((b, n, hkv, d), 15)
    gap = [(11, 17)]
    o, lse = oa.attention(q, k, v, 0.3, gap)
    # changing masked K/V changes nothing
    k2, v2 = k.copy(), v.copy()
    k2[:, 11:17] = 1e4
    v2[:, 11:17] = -1e4
    o2, lse2 = oa.attention(q, k2, v2, 0.3, gap)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # permuting keys (K, V and the mask together): the masked rows are moved to the end
    perm = np.r_[0:11, 17:40, 11:17][np.random.default_rng(0).permutation(34).tolist() + list(range(34, 40))]
    o3, lse3 = oa.attention(q, k[:, perm], v[:, perm], 0.3, [(34, 40)])
    assert np.allclose(o3, o, atol=1e-13) and np.allclose(lse3, lse, atol=1e-13)
    # GQA = MHA with each kv head repeated Hq/Hkv times (repeat_interleave)
    o4, lse4 = oa.attention(q, np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2), 0.3, gap)
    assert np.allclose(o4, o, atol=1e-14) and np.allclose(lse4, lse, atol=1e-14)


def test_ring_lse_merge_equals_full():
    """flashdreams cp.py, ring path: taking in the second block's (out, lse) with the logistic
    weight of the LSE difference, and the LSE as the log of the two summed exponentials,
    reproduces attention over all keys."""
    b, n, h, d = 1, 30, 2, 8
    q, k, v = _rand((b, n, h, d), 16), _rand((b, 2 * n, h, d), 17), _rand((b, 2 * n, h, d), 18)
    o, lse = oa.attention(q, k, v, 0.4)
    o1, l1 = oa.attention(q, k[:, :n], v[:, :n], 0.4)
    o2, l2 = oa.attention(q, k[:, n:], v[:, n:], 0.4)
    l1t, l2t = l1.transpose(0, 2, 1)[..., None], l2.transpose(0, 2, 1)[..., None]
    sig = 1.0 / (1.0 + np.exp(-(l2t - l1t)))
    om = o1 - sig * (o1 - o2)
    lm = l1 - np.log(1.0 / (1.0 + np.exp(-(l1 - l2))))
    assert np.allclose(om, o, atol=1e-13) and np.allclose(lm, lse, atol=1e-13)


def test_suffix_layout_is_rotated_prefix():
    """Non-causal attention is permutation equivariant: attention over
    [shards | rep] equals attention over [rep | shards] with rows rotated back."""
    n_rep, n = 5, 24
    q, k, v = _rand((1, n, 2, 8), 19), _rand((1, n, 2, 8), 20), _rand((1, n, 2, 8), 21)
    o, lse = oa.attention(q, k, v, 0.3)
    rot = np.r_[n - n_rep:n, 0:n - n_rep]
    orot, lrot = oa.attention(q[:, rot], k[:, rot], v[:, rot], 0.3)
    back = np.argsort(rot)
    assert np.allclose(orot[:, back], o, atol=1e-13) and np.allclose(lrot[:, :, back], lse, atol=1e-13)


def test_row_sample_is_exact():
    q, k, v = _rand((1, 50, 2, 8), 22), _rand((1, 50, 2, 8), 23), _rand((1, 50, 2, 8), 24)
    o, lse = oa.attention(q, k, v, 0.3)
    rows = np.array([0, 7, 13, 49])
    os_, ls_ = oa.attention(q, k, v, 0.3, rows=rows)
    assert np.array_equal(os_, o[:, rows]) and np.array_equal(ls_, lse[:, :, rows])


def test_errors():
    q = np.zeros((1, 4, 1, 2))
    with pytest.raises(ValueError):
        oa.attention(q, q, q, 1.0, [(0, 4)])      # no valid key
    with pytest.raises(ValueError):
        oa.attention(q, q, q, 1.0, [(3, 5)])      # gap out of range
    with pytest.raises(ValueError):
        oa.attention(np.zeros((1, 4, 3, 2)), q.repeat(2, axis=2), q.repeat(2, axis=2), 1.0)


def _sdpa_mask_ref(q, k, v, scale, key_mask):
    """torch float64 SDPA with an arbitrary [B, Nk] boolean key mask (broadcast over heads and rows)."""
    qt = torch.from_numpy(q).transpose(1, 2)
    kt = torch.from_numpy(k).transpose(1, 2)
    vt = torch.from_numpy(v).transpose(1, 2)
    rep = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(rep, dim=1)
    vt = vt.repeat_interleave(rep, dim=1)
    mask = torch.from_numpy(key_mask)[:, None, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out.transpose(1, 2).numpy()


def _rand_mask(b, nk, seed, p=0.5):
    m = np.random.default_rng(seed).random((b, nk)) < p
    m[:, 0] = True            # every batch keeps a valid key
    return m


@pytest.mark.parametrize("b,nq,nk,hq,hkv,d", [(1, 7, 12, 2, 2, 8), (2, 9, 5, 4, 2, 4), (2, 6, 11, 3, 1, 6)])
def test_mask_matches_bruteforce(b, nq, nk, hq, hkv, d):
    """Arbitrary key masks and Nq != Nk against exactly rounded loops."""
    q, k, v = _rand((b, nq, hq, d), 11), _rand((b, nk, hkv, d), 12), _rand((b, nk, hkv, d), 13)
    m = _rand_mask(b, nk, 5)
    o, lse = oa.attention(q, k, v, 0.41, key_mask=m, block=3)
    ob, lseb = brute.attention(q.tolist(), k.tolist(), v.tolist(), float(np.float32(0.41)), key_mask=m.tolist())
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lseb))) < 1e-12


@pytest.mark.parametrize("b,nq,nk,hq,hkv,d,p", [(1, 40, 90, 4, 4, 16, 0.3), (2, 64, 64, 8, 2, 32, 0.8),
                                               (1, 33, 130, 2, 1, 8, 0.05)])
def test_mask_matches_sdpa(b, nq, nk, hq, hkv, d, p):
    q, k, v = _rand((b, nq, hq, d), 21), _rand((b, nk, hkv, d), 22), _rand((b, nk, hkv, d), 23)
    m = _rand_mask(b, nk, 7, p)
    scale = oa.default_scale(d)
    o, _ = oa.attention(q, k, v, scale, key_mask=m)
    assert np.max(np.abs(o - _sdpa_mask_ref(q, k, v, scale, m))) < 1e-12


def test_mask_of_gap_equals_gap_and_combines():
    """A mask marking the keys outside a gap is the gap; gap and mask together keep their intersection."""
    b, n, h, d = 2, 50, 2, 8
    q, k, v = _rand((b, n, h, d), 31), _rand((b, n, h, d), 32), _rand((b, n, h, d), 33)
    gaps = [(10, 30), (0, 17)]
    m = np.ones((b, n), dtype=bool)
    for i, (g0, g1) in enumerate(gaps):
        m[i, g0:g1] = False
    o1, l1 = oa.attention(q, k, v, 0.3, gaps)
    o2, l2 = oa.attention(q, k, v, 0.3, key_mask=m)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    m2 = _rand_mask(b, n, 9)
    o3, _ = oa.attention(q, k, v, 0.3, gaps, key_mask=m2)
    o4, _ = oa.attention(q, k, v, 0.3, key_mask=m & m2)
    assert np.array_equal(o3, o4)


def test_masked_kv_contents_do_not_matter():
    b, nq, nk, h, d = 1, 20, 45, 2, 8
    q, k, v = _rand((b, nq, h, d), 41), _rand((b, nk, h, d), 42), _rand((b, nk, h, d), 43)
    m = _rand_mask(b, nk, 11)
    o1, l1 = oa.attention(q, k, v, 0.5, key_mask=m)
    k2, v2 = k.copy(), v.copy()
    k2[:, ~m[0]] = 1e4
    v2[:, ~m[0]] = -1e4
    o2, l2 = oa.attention(q, k2, v2, 0.5, key_mask=m)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_all_masked_batch_gives_zero_and_neg_inf():
    b, n, h, d = 2, 10, 2, 4
    q, k, v = _rand((b, n, h, d), 51), _rand((b, n, h, d), 52), _rand((b, n, h, d), 53)
    m = np.ones((b, n), dtype=bool)
    m[1] = False
    o, lse = oa.attention(q, k, v, 0.5, key_mask=m)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    ob, lseb = brute.attention(q.tolist(), k.tolist(), v.tolist(), 0.5, key_mask=m.tolist())
    assert np.all(np.array(ob)[1] == 0) and np.all(np.isneginf(np.array(lseb)[1]))
    assert np.all(np.isfinite(lse[0]))


@pytest.mark.parametrize("d", [64, 128, 96, 8])
def test_default_scale_is_head_dim_inverse_sqrt(d):
    """sglang layer.py, UlyssesAttention / USPAttention: the softmax scale defaults to head_size**-0.5.
    The oracle passes it to the kernel as a float32; torch's SDPA uses the same default
    (1/sqrt(E) for scale=None), so attention with default_scale matches SDPA's own default to the
    float32 rounding of the scale (exactly when d is a power of 4)."""
    c = oa.default_scale(d)
    assert c == float(np.float32(d ** -0.5))
    assert abs(c - 1.0 / np.sqrt(d)) <= 2.0 ** -24 / np.sqrt(d)
    q, k, v = _rand((1, 20, 2, d), 30), _rand((1, 20, 2, d), 31), _rand((1, 20, 2, d), 32)
    o, _ = oa.attention(q, k, v, c)
    qt, kt, vt = (torch.from_numpy(x).transpose(1, 2) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).transpose(1, 2).numpy()
    tol = 1e-12 if d in (64, 16, 4) else 1e-6
    assert np.allclose(o, ref, rtol=0, atol=tol)
    # a planted mistake (1/d instead of 1/sqrt(d)) is visibly different
    o_bad, _ = oa.attention(q, k, v, 1.0 / d)
    assert not np.allclose(o_bad, ref, rtol=0, atol=1e-3)
