"""Pins of oracle.merge (CPU): merging the (out, lse) of attention over disjoint key blocks
reproduces attention over all keys (flashdreams cp.py _impl_ring), for any number of blocks,
any order and empty blocks; one block is the identity."""
import numpy as np
import pytest

from oracle import attention as oa
from oracle import merge as om


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("cuts", [[0, 40], [0, 17, 40], [0, 5, 6, 23, 40], [0, 1, 2, 3, 39, 40]])
def test_merge_of_key_blocks_is_full_attention(cuts):
    b, nq, nk, h, d = 2, 13, 40, 3, 8
    q, k, v = _rand((b, nq, h, d), 1), _rand((b, nk, h, d), 2), _rand((b, nk, h, d), 3)
    o, lse = oa.attention(q, k, v, 0.5)
    parts = [oa.attention(q, k[:, a:z], v[:, a:z], 0.5) for a, z in zip(cuts[:-1], cuts[1:])]
    mo, ml = om.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert np.allclose(mo, o, atol=1e-13) and np.allclose(ml, lse, atol=1e-13)
    # the order of the blocks does not matter
    rev = parts[::-1]
    mo2, ml2 = om.merge_partials([p[0] for p in rev], [p[1] for p in rev])
    assert np.allclose(mo2, o, atol=1e-13) and np.allclose(ml2, lse, atol=1e-13)


def test_single_block_is_identity():
    o, l = _rand((1, 5, 2, 4), 4), _rand((1, 2, 5), 5)
    mo, ml = om.merge_partials([o], [l])
    assert np.array_equal(mo, o) and np.array_equal(ml, l)


def test_block_without_keys_has_no_weight():
    """A fully masked block (lse = -inf, output arbitrary) leaves the others' merge unchanged,
    in any position, including first."""
    b, nq, nk, h, d = 1, 6, 20, 2, 4
    q, k, v = _rand((b, nq, h, d), 6), _rand((b, nk, h, d), 7), _rand((b, nk, h, d), 8)
    o, lse = oa.attention(q, k, v, 0.7)
    p1 = oa.attention(q, k[:, :9], v[:, :9], 0.7)
    p2 = oa.attention(q, k[:, 9:], v[:, 9:], 0.7)
    empty = (_rand((b, nq, h, d), 9) * 100.0, np.full((b, h, nq), -np.inf))
    for order in ([empty, p1, p2], [p1, empty, p2], [p1, p2, empty]):
        mo, ml = om.merge_partials([p[0] for p in order], [p[1] for p in order])
        assert np.allclose(mo, o, atol=1e-13) and np.allclose(ml, lse, atol=1e-13)


def test_extreme_lse_gaps_stay_finite():
    """Weights of blocks whose LSEs differ by hundreds: no overflow, the larger block wins."""
    o1, o2 = np.ones((1, 2, 1, 3)), np.full((1, 2, 1, 3), 2.0)
    l1, l2 = np.array([[[0.0, 800.0]]]), np.array([[[800.0, 0.0]]])
    mo, ml = om.merge_partials([o1, o2], [l1, l2])
    assert np.all(np.isfinite(mo)) and np.all(np.isfinite(ml))
    assert np.allclose(mo[0, 0, 0], 2.0) and np.allclose(mo[0, 1, 0], 1.0)
    assert np.allclose(ml, 800.0)
