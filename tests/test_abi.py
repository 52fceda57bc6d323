"""The C ABI on the CPU: the library loads, exports every entry point include/ulys.h
declares, and every invalid call is refused with its status before any HIP call
(so these run without a GPU; no valid compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulys.h")


@pytest.fixture(scope="module")
def U():
    lib = os.path.join(ROOT, "ulysses_sequence_attention_amd", "libulys.so")
    if not os.path.exists(lib):
        from ulysses_sequence_attention_amd import build
        build.build()
    from ulysses_sequence_attention_amd import ulys
    return ulys


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:long\s+long|\w+)\*?\s+\*?(ulys_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_path():
    names = _declared()
    for n in ("ulys_pack", "ulys_attend_group", "ulys_attend_group_ex", "ulys_attend_splits", "ulys_unpack",
              "ulys_rank_pipeline", "ulys_attend_workspace_bytes",
              "ulys_lse_merge", "ulys_auto_groups", "ulys_amax_bf16", "ulys_strerror", "ulys_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(U):
    lib = ctypes.CDLL(U.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(U.EXPORTED)


FAKE = 0x10000          # an aligned, never-dereferenced address (calls below fail validation first)
MIS = 0x10008           # 8-byte aligned only


def _arr(n, val=FAKE):
    a = (ctypes.c_void_p * n)()
    for i in range(n):
        a[i] = val
    return a


def _pack(U, L, rank=0, group=0, q=None, k=None, v=None, slots=(FAKE, FAKE, FAKE), dtype=0, amax=FAKE):
    c = U.Layout(**L).c_struct() if isinstance(L, dict) else L
    P = c.degree if c.degree > 0 else 1
    q = _arr(P) if q is None else q
    k = _arr(P) if k is None else k
    v = _arr(P) if v is None else v
    return U.call_raw("ulys_pack", ctypes.byref(c), rank, group, q, k, v, *slots, dtype, amax, None)


GOOD = dict(batch=1, degree=4, s_local=10, n_rep=0, rep_first=True, hq=40, hkv=40, head_dim=128, groups=5)


@pytest.mark.parametrize("change,status", [
    (dict(degree=0), -1), (dict(batch=0), -1), (dict(s_local=0), -1), (dict(groups=0), -1),
    (dict(n_rep=-1), -1), (dict(hq=42), -1), (dict(hkv=20, hq=40, groups=5), 0),
    (dict(hkv=12, hq=40), -1), (dict(groups=3), -1), (dict(head_dim=96), -2), (dict(degree=65, hq=65 * 2, hkv=130, groups=1), -1),
])
def test_pack_layout_rules(U, change, status):
    L = dict(GOOD, **change)
    st = _pack(U, L, group=-2 if status == 0 else 0)   # a valid layout still fails on group -2
    assert st == (-1 if status == 0 else status), U.last_error()
    assert U.last_error()


def test_pack_rules(U):
    assert _pack(U, GOOD, rank=4) == -1
    assert _pack(U, GOOD, rank=-1) == -1
    assert _pack(U, GOOD, group=5) == -1
    assert _pack(U, GOOD, dtype=7) == -1
    assert _pack(U, GOOD, dtype=1, amax=None) == -1                    # fp8 needs amax
    assert _pack(U, GOOD, q=_arr(4, MIS)) == -1                        # misaligned shard
    bad = _arr(4)
    bad[3] = None
    assert _pack(U, GOOD, k=bad) == -1                                  # NULL shard
    assert _pack(U, GOOD, slots=(FAKE, None, FAKE)) == -1
    assert _pack(U, GOOD, slots=(FAKE, FAKE, MIS)) == -1
    c = U.Layout(**GOOD).c_struct()
    c.rep_first = 3                                                     # modes are 0, 1, 2
    assert _pack(U, c) == -1
    assert U.call_raw("ulys_pack", None, 0, 0, _arr(4), _arr(4), _arr(4), FAKE, FAKE, FAKE, 0, None, None) == -1
    assert "layout" in U.last_error()


def _attend(U, batch=1, rows=100, hq=2, hkv=2, d=128, q=FAKE, o=FAKE, dtype=0, scale=0.0, amax=None, gaps=None, lse=None):
    g = None
    if gaps is not None:
        g = (ctypes.c_int32 * len(gaps))(*gaps)
    return U.call_raw("ulys_attend_group", batch, rows, hq, hkv, d, q, FAKE, FAKE, dtype, ctypes.c_float(scale),
                      amax, g, o, lse, None, 0, None)


def test_attend_rules(U):
    assert _attend(U, rows=0) == -1
    assert _attend(U, batch=0) == -1
    assert _attend(U, hq=3, hkv=2) == -1
    assert _attend(U, d=80) == -2
    assert _attend(U, q=MIS) == -1
    assert _attend(U, o=None) == -1
    assert _attend(U, lse=FAKE + 2) == -1
    assert _attend(U, dtype=1) == -1                                   # fp8 without amax
    assert _attend(U, scale=float("nan")) == -1
    assert _attend(U, scale=float("inf")) == -1
    assert _attend(U, gaps=[5, 3]) == -1                               # end < start
    assert _attend(U, gaps=[-1, 3]) == -1
    assert _attend(U, gaps=[90, 101]) == -1                            # past rows
    assert _attend(U, gaps=[0, 100]) == -1                             # no valid key
    assert "no valid key" in U.last_error()
    assert _attend(U, batch=2, gaps=[0, 10, 0, 100]) == -1
    assert _attend(U, batch=300, gaps=[0, 1] * 300) == -1             # too many gap batches


def _attend_ex(U, batch=1, nq=100, nk=140, hq=2, hkv=2, d=128, dtype=0, gaps=None, mask=None, splits=0, ws=None,
               ws_bytes=0):
    g = None
    if gaps is not None:
        g = (ctypes.c_int32 * len(gaps))(*gaps)
    return U.call_raw("ulys_attend_group_ex", batch, nq, nk, hq, hkv, d, FAKE, FAKE, FAKE, dtype, ctypes.c_float(0.0),
                      None, g, mask, splits, FAKE, None, ws, ctypes.c_size_t(ws_bytes), None)


def test_attend_ex_rules(U):
    assert _attend_ex(U, nq=0) == -1
    assert _attend_ex(U, nk=0) == -1
    assert _attend_ex(U, hq=3, hkv=2) == -1
    assert _attend_ex(U, d=96) == -2
    assert _attend_ex(U, gaps=[120, 141]) == -1                        # gaps are on keys: past nk = 140
    assert _attend_ex(U, gaps=[0, 140]) == -1                          # no valid key
    assert _attend_ex(U, mask=FAKE + 2) == -1                          # mask words 4-byte aligned
    assert _attend_ex(U, nk=262144 + 64, mask=FAKE) == -2              # key-mask tile list limit
    assert "key mask" in U.last_error()
    assert _attend_ex(U, splits=-4097) == -1                           # key_splits in [-4096, 16]
    assert _attend_ex(U, splits=17) == -1
    assert "key_splits" in U.last_error()
    assert _attend_ex(U, splits=-33) == -1                             # ranges: at most 32 per query tile
    assert "per query tile" in U.last_error()
    assert _attend_ex(U, nq=257, splits=-65) == -1                     # (2 query tiles: 64 ranges)


def _ws_bytes(U, batch, nq, nk, heads, d, splits, cus=256):
    return U.call_raw("ulys_attend_workspace_bytes", batch, nq, nk, heads, d, splits, cus)


def test_workspace_bytes_arithmetic(U):
    """Workspace of a split call: fp32 partial o (D floats) and lse (one float) per query row and run
    (key-range split C: every row of every run; range split R: two 256-row tile pieces per run), per
    head, plus 256 bytes for the per-batch tile counts."""
    lib = ctypes.CDLL(U.LIB_PATH)
    lib.ulys_attend_workspace_bytes.restype = ctypes.c_longlong
    f = lambda *a: lib.ulys_attend_workspace_bytes(*a)
    assert f(1, 100, 140, 2, 128, 1, 256) == 0                         # no split, no workspace
    assert f(2, 1000, 3000, 3, 64, 4, 256) == 256 + 3 * 4 * 2 * 1000 * (64 + 1) * 4
    assert f(1, 27280, 27280, 2, 128, -128, 256) == 256 + 2 * 128 * 2 * 256 * (128 + 1) * 4
    assert f(1, 27280, 27280, 10, 128, -128, 256) == 256 + 10 * 128 * 2 * 256 * (128 + 1) * 4
    # the automatic choice at the Wan share on 256 CUs is the range split into 128 runs
    assert f(1, 27280, 27280, 2, 128, 0, 256) == f(1, 27280, 27280, 2, 128, -128, 256)
    assert f(1, 1, 1, 1, 128, 0, 0) == -1
    assert f(1, 1, 1, 1, 96, 0, 1) == -2
    assert f(1, 1, 1, 1, 128, 17, 1) == -1


def test_workspace_rules(U):
    """A split call needs a workspace of at least one head's partials, 256-byte aligned (explicit splits,
    so the rule is checked before any HIP call)."""
    lib = ctypes.CDLL(U.LIB_PATH)
    lib.ulys_attend_workspace_bytes.restype = ctypes.c_longlong
    one = lib.ulys_attend_workspace_bytes(1, 100, 140, 1, 128, 2, 256)
    assert one > 0
    assert _attend_ex(U, splits=2) == -1                               # no workspace
    assert "workspace" in U.last_error()
    assert _attend_ex(U, splits=2, ws=FAKE, ws_bytes=one - 1) == -1    # below one head's partials
    assert "ulys_attend_workspace_bytes" in U.last_error()
    assert _attend_ex(U, splits=2, ws=FAKE + 16, ws_bytes=one) == -1   # not 256-byte aligned
    assert "aligned" in U.last_error()
    assert _attend_ex(U, splits=-2, ws=FAKE, ws_bytes=100) == -1       # a range split too


def test_attend_splits_rule(U):
    """The automatic key-range split: host arithmetic only."""
    # the Wan share, 107 query tiles per head on 256 CUs: no key-range split (measured: 2 or 7 runs are 4%
    # slower for a 2-head call); the range split is taken instead
    assert U.ulys_attend_splits(1, 27280, 27280, 256) == 1
    # a short sequence, 6 query tiles per head: 4 runs of 23 key tiles (measured at 2 heads: 3 runs 2.4x,
    # 5 runs 3.4x; fewer runs suit more heads)
    assert U.ulys_attend_splits(1, 1500, 6000, 256) == 4
    # few keys: 16 key tiles in 4 runs of 4 (measured at 1024-1500 rows: 4 runs 1.4-1.6x at 2 heads,
    # 1.1-1.4x at 8); one key tile: no split
    assert U.ulys_attend_splits(1, 256, 1000, 256) == 4
    assert U.ulys_attend_splits(1, 1000, 2047, 256) == 4
    assert U.ulys_attend_splits(1, 256, 64, 256) == 1
    # many query tiles already fill the CUs (4096 tiles)
    assert U.ulys_attend_splits(16, 65536, 65536, 256) == 1
    for args in [(1, 27280, 27280, 256), (2, 5000, 90000, 256), (1, 300, 300000, 80), (4, 8192, 8192, 304)]:
        c = U.ulys_attend_splits(*args)
        assert 1 <= c <= 16
        assert c == 1 or (args[2] + 63) // 64 >= 4 * c
    assert U.call_raw("ulys_attend_splits", 0, 1, 1, 1) == -1
    assert U.call_raw("ulys_attend_splits", 1, 1, 1, 0) == -1


def test_attend_ranges_rule(U):
    """The automatic range split (taken only where the key-range split is 1): host arithmetic only."""
    # the Wan share: 107 query tiles per head -> 128 runs (0.84 tile each): a 2-head call is one full
    # round of 256 workgroups, a 10-head call five (measured: +1 to +7% and +7% over no split)
    assert U.ulys_attend_ranges(1, 27280, 27280, 256) == 128
    assert U.ulys_attend_ranges(1, 1500, 6000, 256) == 0                 # the key-range split (5) applies
    assert U.ulys_attend_ranges(1, 65536, 65536, 256) == 0               # 256 tiles per head fill the CUs
    assert U.ulys_attend_ranges(1, 32760, 32760, 256) == 0               # 128 tiles: 2 heads fill the CUs
    # 130 query tiles (the joint prefix + image shape): 256 runs of half a tile (measured at 2 and 4 heads:
    # 1.58x and 1.26x over no split, against 1.32x and 1.17x for 3 key-range runs)
    assert U.ulys_attend_ranges(1, 32760 + 512, 32760 + 512, 256) == 256
    assert U.ulys_attend_splits(1, 32760 + 512, 32760 + 512, 256) == 1
    assert U.ulys_attend_ranges(1, 256, 1000, 256) == 0                  # one query tile: no candidate
    for args in [(1, 27280, 27280, 256), (1, 24000, 24000, 256), (2, 20000, 30000, 304), (1, 9000, 70000, 80),
                 (3, 27280, 27280, 256)]:
        r = U.ulys_attend_ranges(*args)
        qt = (args[1] + 255) // 256
        cus = args[3]
        assert r == 0 or (r % (cus // 8) == 0 and qt < r <= 4 * qt and r <= 4096)
        assert r == 0 or U.ulys_attend_splits(*args) == 1
    assert U.call_raw("ulys_attend_ranges", 0, 1, 1, 1) == -1
    assert U.call_raw("ulys_attend_ranges", 1, 1, 1, 0) == -1


def test_unpack_and_amax_rules(U):
    c = U.Layout(**GOOD).c_struct()
    assert U.call_raw("ulys_unpack", ctypes.byref(c), 0, 0, None, _arr(4), None) == -1
    assert U.call_raw("ulys_unpack", ctypes.byref(c), 0, 0, FAKE, None, None) == -1
    assert U.call_raw("ulys_unpack", ctypes.byref(c), 9, 0, FAKE, _arr(4), None) == -1
    c.hq = 41
    assert U.call_raw("ulys_unpack", ctypes.byref(c), 0, 0, FAKE, _arr(4), None) == -1
    assert U.call_raw("ulys_amax_bf16", _arr(1), 0, 8, FAKE, None) == -1
    assert U.call_raw("ulys_amax_bf16", _arr(1), 1, 12, FAKE, None) == -1
    assert U.call_raw("ulys_amax_bf16", _arr(1), 1, 8, None, None) == -1
    assert U.call_raw("ulys_amax_bf16", _arr(1, MIS), 1, 8, FAKE, None) == -1


def _pipeline(U, L, rank=0, slots=(FAKE,) * 4, lse=None, out=None, dtype=0, amax=FAKE, scale=0.0, gaps=None,
              events="fake"):
    events = _arr(3) if events == "fake" else events
    c = U.Layout(**L).c_struct()
    P = c.degree
    out = _arr(P) if out is None else out
    g = None if gaps is None else (ctypes.c_int32 * len(gaps))(*gaps)
    return U.call_raw("ulys_rank_pipeline", ctypes.byref(c), rank, _arr(P), _arr(P), _arr(P), *slots, lse, out,
                      dtype, amax, ctypes.c_float(scale), g, events, None, ctypes.c_size_t(0), None, None)


def test_pipeline_rules(U):
    """Every rule of pack, attend and unpack is checked before anything is enqueued."""
    assert _pipeline(U, dict(GOOD, hq=42)) == -1                       # layout
    assert _pipeline(U, GOOD, rank=4) == -1
    assert _pipeline(U, GOOD, slots=(FAKE, None, FAKE, FAKE)) == -1    # k slots
    assert _pipeline(U, GOOD, slots=(FAKE, FAKE, FAKE, MIS)) == -1     # o slots misaligned
    assert _pipeline(U, GOOD, out=_arr(4, MIS)) == -1                  # output shards
    assert _pipeline(U, GOOD, lse=FAKE + 2) == -1
    assert _pipeline(U, GOOD, dtype=1, amax=None) == -1                # fp8 without amax
    assert _pipeline(U, GOOD, scale=float("nan")) == -1
    assert _pipeline(U, GOOD, gaps=[0, 40]) == -1                      # no valid key (40 joint rows)
    assert "no valid key" in U.last_error()
    assert _pipeline(U, dict(GOOD, head_dim=96)) == -2
    assert _pipeline(U, dict(GOOD, hq=4 * 65, hkv=4 * 65, groups=65)) == -2   # more than 64 groups
    assert _pipeline(U, GOOD, events=None) == -1                       # the caller's three events
    assert _pipeline(U, GOOD, events=_arr(3, 0)) == -1
    assert "events" in U.last_error()


def _merge(U, n=2, o=None, lse=None, b=1, rows=10, heads=2, d=64, out=FAKE, lse_out=None):
    o = _arr(n) if o is None else o
    lse = _arr(n) if lse is None else lse
    return U.call_raw("ulys_lse_merge", n, o, lse, b, rows, heads, d, out, lse_out, None)


def test_merge_rules(U):
    assert _merge(U, n=0) == -1
    assert _merge(U, n=17, o=_arr(17), lse=_arr(17)) == -1
    assert _merge(U, rows=0) == -1
    assert _merge(U, d=12) == -1
    assert _merge(U, d=2048) == -1
    assert _merge(U, o=_arr(2, MIS)) == -1
    assert _merge(U, lse=_arr(2, FAKE + 2)) == -1
    assert _merge(U, out=None) == -1
    assert _merge(U, lse_out=FAKE) == -1                     # lse_out is one of the lse parts
    assert "lse_out" in U.last_error()


def _groups(U, **kw):
    L = dict(batch=1, degree=4, s_local=6820, n_rep=0, rep_first=True, hq=40, hkv=40, head_dim=128, groups=1)
    L.update(kw)
    return U.ulys_auto_groups(U.Layout(**L), kw.pop("cus", 256) if "cus" in kw else 256)


def test_auto_groups_follow_the_rounds_rule(U):
    """Wan2.1 at Ulysses 4 (27280 rows, 10 heads per rank, no key-range split): one call takes
    ceil(1070/256) = 5 rounds of workgroups, five 2-head calls 5 x 1 -> 5 groups.  With the key-range
    split (2 runs below 27280 rows) the workgroups double.  Measured on MI355X (group-split sweep):
    16384 rows: one call 5 rounds, five calls 5 x 1 (1.358 vs 1.350 ms) -> 5; 8192 rows: one call
    3 rounds, two calls 2 x 2 (0.491 vs 0.430 ms) -> 1; 4096 rows: 2 rounds either way -> 2."""
    assert _groups(U) == 5
    assert _groups(U, s_local=16384 // 4) == 5
    assert _groups(U, s_local=8192 // 4) == 1
    assert _groups(U, s_local=4096 // 4) == 2
    assert _groups(U, s_local=2048 // 4) == 1                          # 8 x 10 x 2 = 160 workgroups: one call
    assert _groups(U, groups=3) == 5                                   # the layout's own count is ignored
    # 12 heads per rank, 32760 rows (no key split): W = 12 x 128 = 1536 -> 6 rounds; 7 and 5 do not
    # divide 12, 4 groups take 4 x 2 = 8 rounds, 3 groups 3 x 2 = 6
    assert _groups(U, hq=48, hkv=48, s_local=8190) == 3
    # GQA 40/8 at P 4: only 2 divides the 2 k/v heads per rank; 2 x 3 rounds > 5, and at 8192 rows
    # (2 key runs) 2 x 2 > 3
    assert _groups(U, hq=40, hkv=8) == 1
    assert _groups(U, hq=40, hkv=8, s_local=8192 // 4) == 1
    assert U.call_raw("ulys_auto_groups", None, 256) == -1
    c = U.Layout(**dict(GOOD)).c_struct()
    assert U.call_raw("ulys_auto_groups", ctypes.byref(c), 0) == -1
    c.hq = 42
    assert U.call_raw("ulys_auto_groups", ctypes.byref(c), 256) == -1


def test_strerror(U):
    lib = ctypes.CDLL(U.LIB_PATH)
    lib.ulys_strerror.restype = ctypes.c_char_p
    assert lib.ulys_strerror(0) == b"ok"
    assert lib.ulys_strerror(-1) == b"invalid argument"
    assert lib.ulys_strerror(-2) == b"unsupported configuration"
    assert lib.ulys_strerror(-3) == b"HIP runtime error"
    assert lib.ulys_strerror(5) == b"unknown status"


def test_binding_refuses_cpu_tensors(U):
    import torch
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        U.ulys_attend_group(x, x, x, x)


def test_key_mask_word_encoding():
    """inputs.key_mask_words follows the header's encoding: key j of batch b valid iff bit j % 32 of
    word [b][j // 32] is set (checked bit by bit)."""
    import numpy as np
    from ulysses_sequence_attention_amd import inputs
    m = inputs.random_key_mask(3, 100, 5, 0.5)
    w = inputs.key_mask_words(m).numpy().view(np.uint32)
    assert w.shape == (3, 4)
    for b in range(3):
        for j in range(128):
            bit = (int(w[b, j // 32]) >> (j % 32)) & 1
            assert bit == (int(m[b, j]) if j < 100 else 0)


def test_split_choice_invariants(U):
    """Over seeded random shapes and CU counts: the automatic key-range runs C and range runs R are
    never both taken, C has at least 4 key tiles per run, and R is a multiple of cus/8 in (T, 4T]."""
    import random
    rng = random.Random(7)
    for _ in range(400):
        batch = rng.choice([1, 1, 2, 3, 8])
        q_rows = rng.randint(1, 120000)
        kv_rows = rng.choice([q_rows, rng.randint(1, 200000)])
        cus = rng.choice([80, 256, 304])
        c = U.ulys_attend_splits(batch, q_rows, kv_rows, cus)
        r = U.ulys_attend_ranges(batch, q_rows, kv_rows, cus)
        qt, nt = (q_rows + 255) // 256, (kv_rows + 63) // 64
        assert 1 <= c <= 16 and r >= 0
        assert c == 1 or r == 0
        assert c == 1 or nt >= 4 * c
        assert r == 0 or (r % (cus // 8) == 0 and qt < r <= min(4 * qt, 32 * qt, 4096))
