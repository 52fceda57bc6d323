"""Pins for oracle.layout (CPU only).

``oracle.layout.pack`` is written as "build the rank's joint sequence, slice
the group's heads".  These tests re-derive the same slots a different way,
from the exchange steps two pages print, with the all-to-all simulated as an
explicit exchange of chunks between simulated ranks:

* flashdreams ``cp.py`` ``_impl_ulysses`` (bhsd layout): reshape to
  ``[B, W, H_l, S_l, D]``, permute ``(1, 3, 0, 2, 4)``, all_to_all_single
  over dim 0, flatten(0, 1), permute ``(1, 2, 0, 3)``; and the inverse chain
  for the output;
* sglang ``layer.py`` ``_forward_with_replicated_prefix`` (bshd layout):
  split replicated/sharded rows, all-to-all the sharded rows (scatter heads,
  gather sequence), slice the replicated rows to the rank's heads (q and k/v
  separately for GQA), concatenate; ``_forward_with_replicated_suffix``
  rotates the suffix to the front and back.
"""
import numpy as np
import pytest
import torch

from oracle import layout


def _alltoall_single(chunks_per_rank):
    """all_to_all_single over dim 0: rank r's output chunk j = rank j's input chunk r."""
    w = len(chunks_per_rank)
    return [torch.cat([chunks_per_rank[j][r:r + 1] for j in range(w)], dim=0) for r in range(w)]


def _flashdreams_ulysses_in(shards_bhsd):
    """Per rank: [B, H, S_l, D] -> [B, H_l, W*S_l, D] following _impl_ulysses."""
    w = len(shards_bhsd)
    b, h, s_l, d = shards_bhsd[0].shape
    hl = h // w
    sent = [x.reshape(b, w, hl, s_l, d).permute(1, 3, 0, 2, 4).contiguous() for x in shards_bhsd]
    recv = _alltoall_single(sent)
    return [x.flatten(0, 1).permute(1, 2, 0, 3).contiguous() for x in recv]


def _flashdreams_ulysses_out(outs_bhsd, s_l):
    """Per rank: [B, H_l, W*S_l, D] -> [B, H, S_l, D], the inverse chain of _impl_ulysses."""
    w = len(outs_bhsd)
    b, hl, _, d = outs_bhsd[0].shape
    sent = [x.reshape(b, hl, w, s_l, d).permute(2, 1, 0, 3, 4).contiguous() for x in outs_bhsd]
    recv = _alltoall_single(sent)
    # [W, H_l, B, S_l, D] -> flatten(0,1) -> [H, B, S_l, D] -> permute(1,0,2,3) -> [B, H, S_l, D]
    return [x.flatten(0, 1).permute(1, 0, 2, 3).contiguous() for x in recv]


def _sglang_a2a_in(shards_bshd, rank):
    """sequence_model_parallel_all_to_all_4D(scatter_dim=2, gather_dim=1), rank's result."""
    w = len(shards_bshd)
    hl = shards_bshd[0].shape[2] // w
    return torch.cat([s[:, :, rank * hl:(rank + 1) * hl] for s in shards_bshd], dim=1)


def _sglang_prefix_joint(shards, rank, n_rep):
    """_forward_with_replicated_prefix steps 1-4 for one tensor, rank's attention input."""
    rep = shards[rank][:, :n_rep]
    gathered = _sglang_a2a_in([s[:, n_rep:] for s in shards], rank)
    hl = gathered.shape[2]
    return torch.cat([rep[:, :, rank * hl:(rank + 1) * hl], gathered], dim=1)


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("w,b,s_l,h,d,groups", [(2, 1, 5, 4, 8, 2), (4, 2, 3, 8, 4, 1), (4, 1, 7, 8, 2, 2),
                                                (3, 2, 4, 6, 2, 2)])
def test_pack_matches_flashdreams_chain(w, b, s_l, h, d, groups):
    shards = [_rand((b, s_l, h, d), 100 + p) for p in range(w)]
    joint = _flashdreams_ulysses_in([s.permute(0, 2, 1, 3).contiguous() for s in shards])
    np_shards = [s.float().numpy() for s in shards]
    gh = h // w // groups
    for r in range(w):
        for g in range(groups):
            slot = layout.pack(np_shards, r, g, groups, n_rep=0, rep_first=True)
            ref = joint[r][:, g * gh:(g + 1) * gh].permute(0, 2, 1, 3).float().numpy()
            assert slot.shape == (b, w * s_l, gh, d)
            assert np.array_equal(slot, ref)


@pytest.mark.parametrize("w,b,s_l,h,d,groups", [(2, 1, 5, 4, 8, 2), (4, 2, 3, 8, 4, 2)])
def test_unpack_matches_flashdreams_output_chain(w, b, s_l, h, d, groups):
    hl = h // w
    gh = hl // groups
    outs_bhsd = [_rand((b, hl, w * s_l, d), 200 + r) for r in range(w)]
    ref = _flashdreams_ulysses_out(outs_bhsd, s_l)           # per rank [B, H, S_l, D]
    got = [np.zeros((b, s_l, h, d), dtype=np.float32) for _ in range(w)]
    for r in range(w):
        slot_all = outs_bhsd[r].permute(0, 2, 1, 3).float().numpy()   # [B, rows, H_l, D]
        for g in range(groups):
            layout.unpack(np.ascontiguousarray(slot_all[:, :, g * gh:(g + 1) * gh]), got, r, g, groups,
                          n_rep=0, rep_first=True)
    for p in range(w):
        assert np.array_equal(got[p], ref[p].permute(0, 2, 1, 3).float().numpy())


@pytest.mark.parametrize("w,b,s_l,n_rep,hq,hkv,d,groups", [(2, 1, 6, 3, 4, 4, 4, 2), (4, 2, 3, 5, 8, 4, 2, 1),
                                                           (2, 2, 4, 2, 8, 4, 2, 2)])
def test_pack_prefix_matches_sglang_steps(w, b, s_l, n_rep, hq, hkv, d, groups):
    gx = [_rand((b, n_rep + w * s_l, h, d), 300 + i) for i, h in enumerate((hq, hkv, hkv))]
    for x in gx:
        h = x.shape[2]
        shards_t = layout.split_global(x.float().numpy(), w, n_rep, True)
        shards = [torch.from_numpy(s) for s in shards_t]
        gh = h // w // groups
        for r in range(w):
            ref = _sglang_prefix_joint(shards, r, n_rep)
            for g in range(groups):
                slot = layout.pack(shards_t, r, g, groups, n_rep, True)
                assert np.array_equal(slot, ref[:, :, g * gh:(g + 1) * gh].numpy())


@pytest.mark.parametrize("w,s_l,n_rep,h,groups", [(2, 5, 3, 4, 2), (4, 2, 6, 8, 1)])
def test_pack_suffix_is_rotated_prefix(w, s_l, n_rep, h, groups):
    """_forward_with_replicated_suffix: rotate rep rows to the front, run the prefix
    path, rotate back.  Our suffix slot keeps the caller's order, so it must equal
    the prefix derivation with the rep rows moved from the front to the back."""
    d = 2
    x = _rand((1, n_rep + w * s_l, h, d), 7)
    xs = x.float().numpy()
    shards = layout.split_global(xs, w, n_rep, rep_first=False)
    gh = h // w // groups
    for r in range(w):
        rotated = [torch.from_numpy(np.concatenate([s[:, s_l:], s[:, :s_l]], axis=1)) for s in shards]
        pre = _sglang_prefix_joint(rotated, r, n_rep)
        ref = torch.cat([pre[:, n_rep:], pre[:, :n_rep]], dim=1)
        for g in range(groups):
            slot = layout.pack(shards, r, g, groups, n_rep, rep_first=False)
            assert np.array_equal(slot, ref[:, :, g * gh:(g + 1) * gh].numpy())


@pytest.mark.parametrize("rep_first", [True, False])
def test_split_global_then_unpack_roundtrip(rep_first):
    """unpack(pack(x)) over every (rank, group) rebuilds every shard exactly,
    and the shards re-assemble the joint layout."""
    w, s_l, n_rep, h, d, groups = 4, 3, 2, 8, 2, 2
    x = _rand((2, n_rep + w * s_l, h, d), 11).float().numpy()
    shards = layout.split_global(x, w, n_rep, rep_first)
    assert np.array_equal(layout.joint_for_rank(shards, 1, n_rep, rep_first), x)
    out = [np.full_like(s, np.nan) for s in shards]
    for r in range(w):
        for g in range(groups):
            layout.unpack(layout.pack(shards, r, g, groups, n_rep, rep_first), out, r, g, groups, n_rep,
                          rep_first)
    for s, o in zip(shards, out):
        assert np.array_equal(s, o)


def test_unique_ids_source_formula():
    """Every slot element carries a unique id naming its source (shard, b, row, head, d);
    check the row map the pages describe: replicated rows first from the rank's own
    copy, then sharded rows source-rank-major."""
    w, b, s_l, n_rep, h, d, groups = 3, 2, 4, 2, 6, 3, 1
    shards = []
    for p in range(w):
        ids = np.zeros((b, n_rep + s_l, h, d), dtype=np.int64)
        for bb in range(b):
            for t in range(n_rep + s_l):
                for hh in range(h):
                    for dd in range(d):
                        ids[bb, t, hh, dd] = ((((p * 10 + bb) * 100 + t) * 100 + hh) * 10) + dd
        shards.append(ids)
    gh = h // w // groups
    for r in range(w):
        for g in range(groups):
            slot = layout.pack(shards, r, g, groups, n_rep, True)
            for t in range(n_rep + w * s_l):
                src_p, src_t = (r, t) if t < n_rep else ((t - n_rep) // s_l, n_rep + (t - n_rep) % s_l)
                for j in range(gh):
                    hh = r * (h // w) + g * gh + j
                    assert slot[1, t, j, 2] == ((((src_p * 10 + 1) * 100 + src_t) * 100 + hh) * 10) + 2


def test_divisibility_errors():
    with pytest.raises(ValueError):
        layout.group_heads(10, 4, 1)
    with pytest.raises(ValueError):
        layout.group_heads(8, 4, 3)


def _sglang_kv_prefix_inputs(q_shards, k_shards, v_shards, rank, n_rep):
    """_forward_with_replicated_kv_prefix_split for rank: all-to-all q and the k/v shard
    rows, slice the replicated k/v prefix to the rank's k/v heads, join it in front."""
    q = _sglang_a2a_in(q_shards, rank)
    k_sh = _sglang_a2a_in([s[:, n_rep:] for s in k_shards], rank)
    v_sh = _sglang_a2a_in([s[:, n_rep:] for s in v_shards], rank)
    h_kv_local = k_sh.shape[2]
    h0 = rank * h_kv_local
    k_rep = k_shards[rank][:, :n_rep, h0:h0 + h_kv_local]
    v_rep = v_shards[rank][:, :n_rep, h0:h0 + h_kv_local]
    return q, torch.cat([k_rep, k_sh], dim=1), torch.cat([v_rep, v_sh], dim=1)


@pytest.mark.parametrize("w,b,s_l,n_rep,hq,hkv,d", [(2, 1, 5, 3, 4, 4, 8), (4, 2, 3, 6, 8, 4, 4), (4, 1, 2, 1, 4, 4, 2)])
def test_pack_kv_prefix_matches_sglang_steps(w, b, s_l, n_rep, hq, hkv, d):
    """K/V-only prefix: q has no replicated rows; k/v = [rep sliced to the rank's heads | gathered rows]."""
    q_shards = [_rand((b, s_l, hq, d), 10 + p) for p in range(w)]
    k_shards = [_rand((b, n_rep + s_l, hkv, d), 20 + p) for p in range(w)]
    v_shards = [_rand((b, n_rep + s_l, hkv, d), 30 + p) for p in range(w)]
    # every rank holds the same replicated k/v prefix
    for lst in (k_shards, v_shards):
        for p in range(1, w):
            lst[p][:, :n_rep] = lst[0][:, :n_rep]
    for r in range(w):
        q_ref, k_ref, v_ref = _sglang_kv_prefix_inputs(q_shards, k_shards, v_shards, r, n_rep)
        qs, ks, vs = layout.pack_kv_prefix([x.float().numpy() for x in q_shards], [x.float().numpy() for x in k_shards],
                                           [x.float().numpy() for x in v_shards], r, 0, 1, n_rep)
        assert np.array_equal(qs, q_ref.float().numpy())
        assert np.array_equal(ks, k_ref.float().numpy())
        assert np.array_equal(vs, v_ref.float().numpy())


def test_unpack_kv_prefix_restores_q_shards():
    """Round trip: unpacking a copy of every rank's q slot (every group) gives the q shards back."""
    w, b, s_l, h, d, groups = 4, 2, 3, 8, 4, 2
    q_shards = [_rand((b, s_l, h, d), 40 + p).float().numpy() for p in range(w)]
    out = [np.zeros_like(x) for x in q_shards]
    for r in range(w):
        for g in range(groups):
            qs = layout.pack(q_shards, r, g, groups, 0, True)
            layout.unpack_kv_prefix(qs.copy(), out, r, g, groups)
    for p in range(w):
        assert np.array_equal(out[p], q_shards[p])
