"""The masked attention kernel's clean-run rule, modelled on the CPU (attn.hip: the tile list's 'full' and
'next listed' bits, clean_run, run_clean, step).

A piece walks positions [p0, p0 + n) of the list of key tiles that hold a valid key.  Step i computes the
second block of position i and the first block of position i + 1 and loads position i + 2 (the general step
clamps that load, and loads the ragged last tile with rows past the end clamped).  At ring stage 0 a clean
run of 3r steps may start: it computes positions i .. i + 3r without masking and loads positions
i + 2 .. i + 3r + 1 by advancing one pointer a tile per step, with plain row offsets.  The rule: a run covers
positions whose tile is full (every key valid) and whose next tile is listed and is not the ragged last tile.
This model checks, over seeded random masks and piece bounds, that a run then (1) loads consecutive tiles
only, (2) never loads the ragged last tile, and (3) computes only full tiles without a mask -- and that the
rule without the last-tile condition breaks (2).
"""
import numpy as np

KBN = 64


def _tile_list(valid_keys, rows, exclude_last_tile=True):
    ntiles = (rows + KBN - 1) // KBN
    tail = ntiles - 1 if rows % KBN else -1
    tvalid = lambda t: t < ntiles and bool(valid_keys[t * KBN:min(rows, (t + 1) * KBN)].any())
    tfull = lambda t: t < ntiles and (t + 1) * KBN <= rows and bool(valid_keys[t * KBN:(t + 1) * KBN].all())
    out = []
    for t in range(ntiles):
        if tvalid(t):
            link = tvalid(t + 1) and (t + 1 != tail or not exclude_last_tile)
            out.append((t, tfull(t), link))
    return out, tail


def _violations(valid_keys, rows, rng, exclude_last_tile=True, pieces=12):
    lst, tail = _tile_list(valid_keys, rows, exclude_last_tile)
    nseq, found = len(lst), []
    for _ in range(pieces if nseq else 0):
        p0 = int(rng.integers(0, nseq))
        n = int(rng.integers(1, nseq - p0 + 1))

        def clean_run(i):
            room = n - 2 - i
            if room <= 0:
                return 0
            k = 0
            while p0 + i + k < nseq and lst[p0 + i + k][1] and lst[p0 + i + k][2] and k <= room:
                k += 1
            return max(0, min(room, k - 1))

        i, stage = 0, 0
        while True:
            if stage == 0:
                r = clean_run(i) // 3
                if r > 0:
                    first = lst[p0 + i + 2][0]
                    for j in range(3 * r):
                        pos = p0 + i + 2 + j
                        if pos >= nseq or lst[pos][0] != first + j:
                            found.append("non-consecutive load")
                        if first + j == tail:
                            found.append("ragged last tile loaded by a clean run")
                    for pos in range(p0 + i, p0 + i + 3 * r + 1):
                        if not lst[pos][1]:
                            found.append("partial tile computed without a mask")
                    i += 3 * r
            if i + 1 >= n:
                break
            stage = (stage + 1) % 3
            i += 1
    return found


def _masks(rng, count):
    for case in range(count):
        rows = int(rng.integers(1, 3000))
        m = np.ones(rows, dtype=bool)
        kind = case % 4
        if kind == 0:
            m[int(rng.integers(0, rows)):] = rng.random() < 0.5
        elif kind == 1:
            a = int(rng.integers(0, rows))
            m[a:int(rng.integers(a, rows + 1))] = False
        elif kind == 2:
            m = rng.random(rows) < 0.97
        if not m.any():
            m[0] = True
        yield m, rows


def test_clean_runs_keep_their_invariants():
    rng = np.random.default_rng(1)
    bad = [(rows, v) for m, rows in _masks(rng, 1500) for v in _violations(m, rows, rng)]
    assert bad == [], bad[:5]


def test_rule_without_the_last_tile_condition_loads_it():
    rng = np.random.default_rng(1)
    kinds = {v for m, rows in _masks(rng, 1500) for v in _violations(m, rows, rng, exclude_last_tile=False)}
    assert "ragged last tile loaded by a clean run" in kinds
