"""Oracle: merging partial attention results over key blocks by their LSE -- test infrastructure.

What is merged (flashdreams ``core/attention/cp.py``, ``ContextParallelAttention``,
ring path): every ring step attends the local queries to one block of keys and
yields an output and its log-sum-exp.  The running result takes in each new
block in turn: the new block's share of the weight is the logistic function of
its LSE minus the running LSE, the running output moves towards the block's
output by that share, and the running LSE becomes the log of the sum of the two
exponentials (written with the log-logistic function, which stays finite for
large LSE gaps).  The page can do this in float32; here every step runs in
float64 on the exact values the kernel reads (bf16 outputs widened, float32
LSEs widened), blocks in the order given.

A block whose LSE is -inf (no valid key in it) has weight 0.  The merged
result is attention over the union of the blocks' keys; that, not this
formula, is what the tests pin it to.
"""
from __future__ import annotations

import numpy as np


def _sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore", invalid="ignore"):
        return np.where(x >= 0, 1.0 / (1.0 + np.exp(-x)), np.exp(x) / (1.0 + np.exp(x)))


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    # log(1 / (1 + exp(-x))) = -log1p(exp(-x)), written stably for both signs
    with np.errstate(over="ignore"):
        return np.where(x >= 0, -np.log1p(np.exp(-x)), x - np.log1p(np.exp(x)))


def merge_partials(outs: list[np.ndarray], lses: list[np.ndarray]):
    """Merge ``n`` partial results in order.

    outs: each ``[B, rows, H, D]``; lses: each ``[B, H, rows]``.
    Returns ``(out [B, rows, H, D] fp64, lse [B, H, rows] fp64)``.
    """
    if len(outs) != len(lses) or not outs:
        raise ValueError("need one lse per output and at least one block")
    prev_out = np.asarray(outs[0], dtype=np.float64)
    prev_lse = np.asarray(lses[0], dtype=np.float64)
    for o, l in zip(outs[1:], lses[1:]):
        o = np.asarray(o, dtype=np.float64)
        l = np.asarray(l, dtype=np.float64)
        with np.errstate(invalid="ignore"):
            d = l - prev_lse                       # [B, H, rows]
        # a block (or the running result) with no valid key has weight 0
        w = np.where(np.isneginf(l), 0.0, np.where(np.isneginf(prev_lse), 1.0, _sigmoid(np.nan_to_num(d))))
        wt = w.transpose(0, 2, 1)[..., None]       # [B, rows, H, 1]
        prev_out = prev_out - wt * (prev_out - o)
        with np.errstate(invalid="ignore"):
            new_lse = prev_lse - _logsigmoid(np.nan_to_num(prev_lse - l))
        prev_lse = np.where(np.isneginf(l), prev_lse, np.where(np.isneginf(prev_lse), l, new_lse))
    return prev_out, prev_lse
