"""Pins for oracle.layout (CPU only).

``oracle.layout.pack`` is written as "build the rank's joint sequence, slice
the group's heads" (array concatenation).  These tests rebuild every slot
element by element from the index map the pages state in words, with no
concatenation or reshaping:

* flashdreams ``core/attention/cp.py``, ``ContextParallelAttention`` (the
  Ulysses path): before the exchange rank p holds sequence rows
  ``[p*S_l, (p+1)*S_l)`` of every head; after it rank r holds heads
  ``[r*H/P, (r+1)*H/P)`` of the whole sequence, the rows ordered by source
  rank, then by local row.  The output exchange is the inverse map.
* sglang ``layer.py``, ``USPAttention`` with a replicated prefix: the
  replicated rows never enter the exchange; rank r takes its own copy,
  restricted to its heads (q heads for q, k/v heads for k and v), and puts
  it in front of the gathered rows.  A replicated suffix is handled by
  moving the replicated rows to the front and back again, which the tests
  check as an equivalence.  With a K/V-only prefix, q carries no replicated
  rows and k/v carry them in front.
* sglang PR #43521, "Receive slots": group g of rank r holds the contiguous
  head block ``[h0, h0 + Gh)``, ``h0 = r*H/P + g*Gh``.
"""
import numpy as np
import pytest

from oracle import layout


def _source_of(t, rank, p_deg, s_l, n_rep, rep_first):
    """(source rank, row within that rank's shard) of joint row t of ``rank``."""
    if rep_first:
        if t < n_rep:
            return rank, t
        u = t - n_rep
        return u // s_l, n_rep + u % s_l
    if t < p_deg * s_l:
        return t // s_l, t % s_l
    return rank, s_l + (t - p_deg * s_l)


def _slot_by_index_map(shards, rank, group, groups, n_rep, rep_first):
    """slot[b, t, j, d] = shard[src(t)][b, row(t), h0 + j, d], one (t, j) at a time."""
    p_deg = len(shards)
    bsz, shard_rows, h, d = shards[0].shape
    s_l = shard_rows - n_rep
    gh = h // p_deg // groups
    h0 = rank * (h // p_deg) + group * gh
    rows = n_rep + p_deg * s_l
    out = np.empty((bsz, rows, gh, d), dtype=shards[0].dtype)
    for t in range(rows):
        src, row = _source_of(t, rank, p_deg, s_l, n_rep, rep_first)
        for j in range(gh):
            for b in range(bsz):
                for dd in range(d):
                    out[b, t, j, dd] = shards[src][b, row, h0 + j, dd]
    return out


def _shards_by_output_map(slots, p_deg, s_l, h, groups):
    """Output exchange with no replicated rows: out_p[b, s, h0 + j, d] = slot(r, g)[b, p*S_l + s, j, d]
    for every rank r and group g (slots[r][g])."""
    bsz, _, gh, d = slots[0][0].shape
    out = [np.full((bsz, s_l, h, d), np.nan) for _ in range(p_deg)]
    for r in range(p_deg):
        for g in range(groups):
            h0 = r * (h // p_deg) + g * gh
            for p in range(p_deg):
                for s in range(s_l):
                    for j in range(gh):
                        out[p][:, s, h0 + j, :] = slots[r][g][:, p * s_l + s, j, :]
    return out


def _rand(shape, seed):
    """bf16-representable float32 values (the slots are exact copies either way)."""
    g = np.random.default_rng(seed)
    x = g.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


@pytest.mark.parametrize("w,b,s_l,h,d,groups", [(2, 1, 5, 4, 8, 2), (4, 2, 3, 8, 4, 1), (4, 1, 7, 8, 2, 2),
                                                (3, 2, 4, 6, 2, 2)])
def test_pack_matches_exchange_index_map(w, b, s_l, h, d, groups):
    """No replicated rows: slot (r, g) row t = source rank t // S_l, local row t % S_l, heads h0.."""
    shards = [_rand((b, s_l, h, d), 100 + p) for p in range(w)]
    gh = h // w // groups
    for r in range(w):
        for g in range(groups):
            slot = layout.pack(shards, r, g, groups, n_rep=0, rep_first=True)
            assert slot.shape == (b, w * s_l, gh, d)
            assert np.array_equal(slot, _slot_by_index_map(shards, r, g, groups, 0, True))


@pytest.mark.parametrize("w,b,s_l,h,d,groups", [(2, 1, 5, 4, 8, 2), (4, 2, 3, 8, 4, 2)])
def test_unpack_matches_output_index_map(w, b, s_l, h, d, groups):
    """The output exchange: joint row p*S_l + s of rank r's slot goes to shard p, row s, rank r's heads."""
    gh = h // w // groups
    slots = [[_rand((b, w * s_l, gh, d), 200 + 10 * r + g) for g in range(groups)] for r in range(w)]
    ref = _shards_by_output_map(slots, w, s_l, h, groups)
    got = [np.zeros((b, s_l, h, d), dtype=np.float32) for _ in range(w)]
    for r in range(w):
        for g in range(groups):
            layout.unpack(slots[r][g], got, r, g, groups, n_rep=0, rep_first=True)
    for p in range(w):
        assert np.array_equal(got[p], ref[p])


@pytest.mark.parametrize("w,b,s_l,n_rep,hq,hkv,d,groups", [(2, 1, 6, 3, 4, 4, 4, 2), (4, 2, 3, 5, 8, 4, 2, 1),
                                                           (2, 2, 4, 2, 8, 4, 2, 2)])
def test_pack_prefix_matches_index_map(w, b, s_l, n_rep, hq, hkv, d, groups):
    """Replicated prefix, q and k/v with their own head counts (GQA): rows t < R from the rank's
    own copy, the rest source-rank-major."""
    for i, h in enumerate((hq, hkv, hkv)):
        x = _rand((b, n_rep + w * s_l, h, d), 300 + i)
        shards = layout.split_global(x, w, n_rep, True)
        for r in range(w):
            for g in range(groups):
                slot = layout.pack(shards, r, g, groups, n_rep, True)
                assert np.array_equal(slot, _slot_by_index_map(shards, r, g, groups, n_rep, True))


@pytest.mark.parametrize("w,s_l,n_rep,h,groups", [(2, 5, 3, 4, 2), (4, 2, 6, 8, 1)])
def test_pack_suffix_is_rotated_prefix(w, s_l, n_rep, h, groups):
    """The suffix path of sglang's USPAttention moves the replicated rows to the front, runs the
    prefix path and moves them back.  Our suffix slot keeps the caller's order, so it must equal
    the prefix index map on rotated shards with the replicated rows then moved to the back."""
    d = 2
    x = _rand((1, n_rep + w * s_l, h, d), 7)
    shards = layout.split_global(x, w, n_rep, rep_first=False)
    for r in range(w):
        rotated = [np.concatenate([s[:, s_l:], s[:, :s_l]], axis=1) for s in shards]
        for g in range(groups):
            pre = _slot_by_index_map(rotated, r, g, groups, n_rep, True)
            ref = np.concatenate([pre[:, n_rep:], pre[:, :n_rep]], axis=1)
            slot = layout.pack(shards, r, g, groups, n_rep, rep_first=False)
            assert np.array_equal(slot, ref)
            assert np.array_equal(slot, _slot_by_index_map(shards, r, g, groups, n_rep, False))


@pytest.mark.parametrize("rep_first", [True, False])
def test_split_global_then_unpack_roundtrip(rep_first):
    """unpack(pack(x)) over every (rank, group) rebuilds every shard exactly,
    and the shards re-assemble the joint layout."""
    w, s_l, n_rep, h, d, groups = 4, 3, 2, 8, 2, 2
    x = _rand((2, n_rep + w * s_l, h, d), 11)
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


def _kv_prefix_by_index_map(q_shards, k_shards, v_shards, rank, n_rep):
    """K/V-only prefix (sglang layer.py, _forward_with_replicated_kv_prefix): q rows are the
    gathered shard rows alone; k/v rows are the rank's own replicated rows at its k/v heads,
    then the gathered shard rows -- one group holding all of the rank's heads."""
    return (_slot_by_index_map(q_shards, rank, 0, 1, 0, True),
            _slot_by_index_map(k_shards, rank, 0, 1, n_rep, True),
            _slot_by_index_map(v_shards, rank, 0, 1, n_rep, True))


@pytest.mark.parametrize("w,b,s_l,n_rep,hq,hkv,d", [(2, 1, 5, 3, 4, 4, 8), (4, 2, 3, 6, 8, 4, 4), (4, 1, 2, 1, 4, 4, 2)])
def test_pack_kv_prefix_matches_index_map(w, b, s_l, n_rep, hq, hkv, d):
    """K/V-only prefix: q has no replicated rows; k/v = [rep sliced to the rank's heads | gathered rows]."""
    q_shards = [_rand((b, s_l, hq, d), 10 + p) for p in range(w)]
    k_shards = [_rand((b, n_rep + s_l, hkv, d), 20 + p) for p in range(w)]
    v_shards = [_rand((b, n_rep + s_l, hkv, d), 30 + p) for p in range(w)]
    # every rank holds the same replicated k/v prefix
    for lst in (k_shards, v_shards):
        for p in range(1, w):
            lst[p][:, :n_rep] = lst[0][:, :n_rep]
    for r in range(w):
        q_ref, k_ref, v_ref = _kv_prefix_by_index_map(q_shards, k_shards, v_shards, r, n_rep)
        qs, ks, vs = layout.pack_kv_prefix(q_shards, k_shards, v_shards, r, 0, 1, n_rep)
        assert np.array_equal(qs, q_ref)
        assert np.array_equal(ks, k_ref)
        assert np.array_equal(vs, v_ref)


def test_unpack_kv_prefix_restores_q_shards():
    """Round trip: unpacking a copy of every rank's q slot (every group) gives the q shards back."""
    w, b, s_l, h, d, groups = 4, 2, 3, 8, 4, 2
    q_shards = [_rand((b, s_l, h, d), 40 + p) for p in range(w)]
    out = [np.zeros_like(x) for x in q_shards]
    for r in range(w):
        for g in range(groups):
            qs = layout.pack(q_shards, r, g, groups, 0, True)
            layout.unpack_kv_prefix(qs.copy(), out, r, g, groups)
    for p in range(w):
        assert np.array_equal(out[p], q_shards[p])
