"""Oracle: dense non-causal softmax attention with log-sum-exp, fp64 -- test infrastructure.

Definition (per batch b, query head h, query row i), on exactly the values
the kernel reads (bf16 widened, or decoded e4m3 codes):

* J = keys outside the masked key gap ``[gap_start, gap_end)`` of batch b
  (a key mask gives masked keys zero weight: sglang ``layer.py``,
  ``LocalAttention.forward`` turns a boolean key mask into an additive
  ``(mask - 1) * finfo.max`` bias broadcast over queries; the pad span
  ``[pad_start, pad_end)`` of ``USPAttention.forward``'s masked branch);
* kv head ``h' = h // (Hq / Hkv)`` (GQA: ``LocalAttention.forward`` repeats
  each K/V head ``Hq/Hkv`` times with ``repeat_interleave``);
* ``s_ij = c * sum_d q[i,h,d] k[j,h',d]``, c the float32 score scale
  (default ``head_dim ** -0.5``: sglang ``UlyssesAttention.__init__``);
* ``m_i = max_J s_ij``, ``l_i = sum_J exp(s_ij - m_i)``,
  ``o_i = sum_J exp(s_ij - m_i) v[j,h'] / l_i``,
  ``lse_i = m_i + ln l_i`` (natural log: flashdreams ``cp.py`` merges ring
  partial outputs with ``sigmoid``/``logsigmoid`` of LSE differences, which
  only holds for a natural-log LSE).

An arbitrary boolean key mask ``[B, Nk]`` may be given as well (sglang
``layer.py`` ``build_varlen_mask_meta``: a ``[B, S]`` key mask; masked keys
take part in no row's softmax); the valid keys are then those outside the gap
that the mask keeps.  Query rows inside the gap or at masked positions are
computed like every other row (SDPA semantics: the mask is on keys only).
The number of queries ``Nq`` may differ from the number of keys ``Nk``
(attention over a replicated K/V-only prefix plus the sharded keys: sglang
``layer.py`` ``_forward_with_replicated_kv_prefix``).

A batch with no valid key: with a gap alone this is an error, not a result;
when a key mask leaves no valid key the row's output is 0 and its LSE
``-inf`` (reading adopted: an empty softmax contributes nothing, as a
partial with LSE ``-inf`` carries zero weight in the ring merge).

Implementation: ``numpy`` fp64, one (b, h) at a time, query rows in blocks
so the score block stays small; two passes over each score row (max, then
exp-sum), no online rescaling.
"""
from __future__ import annotations

import numpy as np


def default_scale(head_dim: int) -> float:
    return float(np.float32(head_dim ** -0.5))


def valid_key_mask(n_keys: int, gap: tuple[int, int] | None, mask=None) -> np.ndarray:
    """Valid keys of one batch: outside ``gap`` and, when ``mask`` is given, where it is True."""
    keep = np.ones(n_keys, dtype=bool)
    if gap is not None:
        g0, g1 = int(gap[0]), int(gap[1])
        if not (0 <= g0 <= g1 <= n_keys):
            raise ValueError(f"key gap {gap} outside [0, {n_keys}]")
        keep[g0:g1] = False
        if not keep.any():
            raise ValueError("no valid key")
    if mask is not None:
        keep &= np.asarray(mask, dtype=bool)
    return keep


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              key_gaps: list[tuple[int, int]] | None = None,
              rows: np.ndarray | None = None, block: int = 512, key_mask: np.ndarray | None = None):
    """Exact attention.

    q: ``[B, Nq, Hq, D]``, k/v: ``[B, Nk, Hkv, D]`` (any float dtype; widened
    to fp64).  ``key_gaps``: per batch ``(start, end)`` masked key range, or
    None.  ``key_mask``: boolean ``[B, Nk]`` (True = valid key), or None.
    ``rows``: optional sorted array of query rows to compute (query
    rows are independent, so a sample is exact); default all.

    Returns ``(o, lse)``: o ``[B, len(rows), Hq, D]`` fp64 and lse
    ``[B, Hq, len(rows)]`` fp64.
    """
    bsz, nq, hq, d = q.shape
    _, nk, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    rep = hq // hkv
    c = float(np.float32(scale))
    sel = np.arange(nq) if rows is None else np.asarray(rows)
    o = np.zeros((bsz, len(sel), hq, d), dtype=np.float64)
    lse = np.zeros((bsz, hq, len(sel)), dtype=np.float64)
    for b in range(bsz):
        keep = valid_key_mask(nk, None if key_gaps is None else key_gaps[b],
                              None if key_mask is None else key_mask[b])
        if not keep.any():
            lse[b] = -np.inf
            continue
        for h in range(hq):
            hk = h // rep
            kb = np.asarray(k[b, :, hk, :], dtype=np.float64)[keep]
            vb = np.asarray(v[b, :, hk, :], dtype=np.float64)[keep]
            for i0 in range(0, len(sel), block):
                qi = np.asarray(q[b, sel[i0:i0 + block], h, :], dtype=np.float64)
                s = c * (qi @ kb.T)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                o[b, i0:i0 + block, h, :] = (p @ vb) / l
                lse[b, h, i0:i0 + block] = (m + np.log(l))[:, 0]
    return o, lse
