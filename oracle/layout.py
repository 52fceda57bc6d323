"""Oracle: the Ulysses layout permutation (pack / unpack) -- test infrastructure.

What Ulysses does to the layout (one rank's view, all-to-all modelled as a
local permutation):

* Every rank p holds a shard ``[B, n_rep + s_local, H, D]``: its own
  ``s_local`` sequence rows plus, when present, ``n_rep`` replicated text rows
  that every rank holds identically.  The replicated rows sit in front
  (prefix) or behind (suffix) the sharded rows.
  (sglang ``layer.py``, ``USPAttention.forward`` docstring on
  num_replicated_prefix / num_replicated_suffix.)
* After the exchange rank r owns heads ``[r*H/P, (r+1)*H/P)`` over the whole
  joint sequence; the sharded rows arrive source-rank-major.
  (flashdreams ``cp.py``, ``ContextParallelAttention._impl_ulysses``: the
  reshape to ``[B, W, H_l, S_l, D]``, all-to-all, and flatten of the world
  dimension into the sequence.)
* Replicated rows stay out of the exchange: each rank slices its own copy to
  its head range and joins it to the gathered shard rows, in front for a
  prefix, behind for a suffix.
  (sglang ``layer.py``, ``_forward_with_replicated_prefix`` steps 1-4 and
  ``_forward_with_replicated_suffix``; sglang PR #43521, "Layouts".)
* The receive slot of head group g is one contiguous ``[B, rows, Gh, D]``
  tensor holding that group's heads in exactly the order attention reads.
  (sglang PR #43521, "Receive slots".)
* The output goes back by the inverse permutation; replicated rows' output
  for this rank's heads reaches every rank (the all-gather over heads).
  (sglang ``layer.py``, ``_forward_with_replicated_prefix`` step 5.)

Reading adopted where the pages are silent: the G groups of a rank are
contiguous blocks of ``H/(P*G)`` heads in head order, for q and for k/v
separately (GQA).  The suffix slot keeps the caller's row order
``[shard_0 | ... | shard_{P-1} | rep]`` (no rotation).

The definition used here is the plainest one: build the joint layout the
rank attends over, then slice the group's heads.  All arrays are NumPy; the
permutation is exact for any dtype.
"""
from __future__ import annotations

import numpy as np


def rows_of(degree: int, s_local: int, n_rep: int) -> int:
    """Joint sequence length seen by attention: replicated + all shard rows."""
    return n_rep + degree * s_local


def group_heads(h: int, degree: int, groups: int) -> int:
    """Heads per group for a tensor with ``h`` heads (H / (P*G))."""
    if h % degree or (h // degree) % groups:
        raise ValueError(f"heads {h} not divisible by degree {degree} x groups {groups}")
    return h // degree // groups


def head_offset(h: int, degree: int, groups: int, rank: int, group: int) -> int:
    """First head of (rank, group): r*H/P + g*H/(P*G)."""
    return rank * (h // degree) + group * group_heads(h, degree, groups)


def split_global(x: np.ndarray, degree: int, n_rep: int, rep_first: bool) -> list[np.ndarray]:
    """Cut a joint ``[B, rows, H, D]`` tensor into the P shards the ranks hold.

    Joint order: prefix ``[rep | shard_0 | ... | shard_{P-1}]``, suffix
    ``[shard_0 | ... | shard_{P-1} | rep]``.  Each shard carries a copy of
    the replicated rows on the same side.
    """
    b, rows, h, d = x.shape
    s_local, rem = divmod(rows - n_rep, degree)
    if rem:
        raise ValueError("rows - n_rep must divide by the degree")
    if rep_first:
        rep = x[:, :n_rep]
        body = x[:, n_rep:]
    else:
        rep = x[:, rows - n_rep:]
        body = x[:, : rows - n_rep]
    shards = []
    for p in range(degree):
        own = body[:, p * s_local:(p + 1) * s_local]
        shards.append(np.ascontiguousarray(
            np.concatenate([rep, own], axis=1) if rep_first else np.concatenate([own, rep], axis=1)))
    return shards


def joint_for_rank(shards: list[np.ndarray], rank: int, n_rep: int, rep_first: bool) -> np.ndarray:
    """The joint ``[B, rows, H, D]`` sequence rank ``rank`` attends over (all heads).

    Sharded rows of every source rank in rank order; replicated rows from
    ``rank``'s own copy.
    """
    own = shards[rank]
    if rep_first:
        rep = own[:, :n_rep]
        body = [s[:, n_rep:] for s in shards]
        return np.concatenate([rep] + body, axis=1)
    s_local = own.shape[1] - n_rep
    rep = own[:, s_local:]
    body = [s[:, :s_local] for s in shards]
    return np.concatenate(body + [rep], axis=1)


def pack(shards: list[np.ndarray], rank: int, group: int, groups: int,
         n_rep: int, rep_first: bool) -> np.ndarray:
    """Receive slot ``[B, rows, Gh, D]`` of (rank, group) for one tensor.

    slot[b, t, j, :] = joint_for_rank(...)[b, t, h0 + j, :],
    h0 = rank*H/P + group*H/(P*G).
    """
    degree = len(shards)
    h = shards[0].shape[2]
    gh = group_heads(h, degree, groups)
    h0 = head_offset(h, degree, groups, rank, group)
    joint = joint_for_rank(shards, rank, n_rep, rep_first)
    return np.ascontiguousarray(joint[:, :, h0:h0 + gh, :])


def unpack(o_slot: np.ndarray, out_shards: list[np.ndarray], rank: int, group: int,
           groups: int, n_rep: int, rep_first: bool) -> None:
    """Scatter an output slot ``[B, rows, Gq, D]`` back into the P output shards.

    Inverse of ``pack`` on the shard rows: the rows of source rank p go back
    to ``out_shards[p]`` at heads ``h0 .. h0+Gq``.  Replicated rows' output
    goes to every shard (the all-gather over heads).  Modifies ``out_shards``
    in place.
    """
    degree = len(out_shards)
    h = out_shards[0].shape[2]
    gh = group_heads(h, degree, groups)
    h0 = head_offset(h, degree, groups, rank, group)
    s_local = out_shards[0].shape[1] - n_rep
    if rep_first:
        rep = o_slot[:, :n_rep]
        body = o_slot[:, n_rep:]
    else:
        rep = o_slot[:, degree * s_local:]
        body = o_slot[:, : degree * s_local]
    for p in range(degree):
        own = body[:, p * s_local:(p + 1) * s_local]
        if rep_first:
            out_shards[p][:, :n_rep, h0:h0 + gh] = rep
            out_shards[p][:, n_rep:, h0:h0 + gh] = own
        else:
            out_shards[p][:, :s_local, h0:h0 + gh] = own
            out_shards[p][:, s_local:, h0:h0 + gh] = rep


def pack_kv_prefix(q_shards: list[np.ndarray], k_shards: list[np.ndarray], v_shards: list[np.ndarray],
                   rank: int, group: int, groups: int, n_rep: int):
    """Receive slots of (rank, group) with a replicated K/V-only prefix.

    sglang ``layer.py`` ``_forward_with_replicated_kv_prefix``: q is
    sequence-sharded with no replicated part; k/v are ``[rep | shard]`` on
    every rank.  Steps: all-to-all q and the k/v shard rows (seq -> head
    shard), slice the replicated k/v prefix to the rank's heads, join it in
    front of the gathered k/v rows.  That is the plain joint layout with no
    replicated rows for q and the prefix layout for k/v, so the slots are
    ``pack`` with ``n_rep = 0`` for q and ``n_rep`` in front for k and v.
    Returns ``(q_slot [B, P*S_l, Gq, D], k_slot, v_slot [B, R + P*S_l, Gkv, D])``.
    """
    return (pack(q_shards, rank, group, groups, 0, True),
            pack(k_shards, rank, group, groups, n_rep, True),
            pack(v_shards, rank, group, groups, n_rep, True))


def unpack_kv_prefix(o_slot: np.ndarray, out_shards: list[np.ndarray], rank: int, group: int,
                     groups: int) -> None:
    """Inverse of the q permutation of ``pack_kv_prefix`` for the output: the
    output carries no replicated rows (``_usp_output_all_to_all`` of the
    attention output alone), so it is ``unpack`` with ``n_rep = 0``."""
    unpack(o_slot, out_shards, rank, group, groups, 0, True)
