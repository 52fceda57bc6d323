"""Python binding of libulys (argument marshalling only).

Each function has the name of the C entry point it wraps and does nothing
but check tensor dtypes/devices/sizes, collect raw device pointers and the
current HIP stream, call the library, and turn a negative status into an
exception (ValueError for ULYS_EINVAL, NotImplementedError for
ULYS_EUNSUPPORTED, RuntimeError for ULYS_EHIP).  Every step of the path runs
in the library's HIP kernels; there is no other implementation here.
Importing this module fails loudly if libulys.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libulys.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m ulysses_sequence_attention_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

ULYS_OK, ULYS_EINVAL, ULYS_EUNSUPPORTED, ULYS_EHIP = 0, -1, -2, -3
ULYS_BF16, ULYS_FP8_E4M3 = 0, 1

_vp = ctypes.c_void_p
_i = ctypes.c_int


class ulys_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "degree", "s_local", "n_rep", "rep_first", "hq", "hkv", "head_dim", "groups")]


_lib.ulys_pack.argtypes = [ctypes.POINTER(ulys_layout), _i, _i, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                           ctypes.POINTER(_vp), _vp, _vp, _vp, _i, _vp, _vp]
_lib.ulys_pack.restype = _i
_lib.ulys_amax_bf16.argtypes = [ctypes.POINTER(_vp), _i, ctypes.c_size_t, _vp, _vp]
_lib.ulys_amax_bf16.restype = _i
_sz = ctypes.c_size_t
_lib.ulys_attend_group.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _i, ctypes.c_float, _vp,
                                   ctypes.POINTER(ctypes.c_int32), _vp, _vp, _vp, _sz, _vp]
_lib.ulys_attend_group.restype = _i
_lib.ulys_attend_group_ex.argtypes = [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, ctypes.c_float, _vp,
                                      ctypes.POINTER(ctypes.c_int32), _vp, _i, _vp, _vp, _vp, _sz, _vp]
_lib.ulys_attend_group_noalloc.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _i, ctypes.c_float, _vp,
                                           ctypes.POINTER(ctypes.c_int32), _vp, _vp, _vp]
_lib.ulys_attend_group_noalloc.restype = _i
_lib.ulys_attend_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
_lib.ulys_attend_workspace_bytes.restype = ctypes.c_longlong
_lib.ulys_attend_group_ex.restype = _i
_lib.ulys_attend_splits.argtypes = [_i, _i, _i, _i]
_lib.ulys_attend_splits.restype = _i
_lib.ulys_attend_ranges.argtypes = [_i, _i, _i, _i]
_lib.ulys_attend_ranges.restype = _i
_lib.ulys_unpack.argtypes = [ctypes.POINTER(ulys_layout), _i, _i, _vp, ctypes.POINTER(_vp), _vp]
_lib.ulys_unpack.restype = _i
_lib.ulys_rank_pipeline.argtypes = [ctypes.POINTER(ulys_layout), _i, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                    ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_vp), _i, _vp,
                                    ctypes.c_float, _vp, ctypes.POINTER(_vp), _vp, _sz, _vp, _vp]
_lib.ulys_rank_pipeline.restype = _i
_lib.ulys_lse_merge.argtypes = [_i, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _i, _i, _i, _vp, _vp, _vp]
_lib.ulys_lse_merge.restype = _i
_lib.ulys_auto_groups.argtypes = [ctypes.POINTER(ulys_layout), _i]
_lib.ulys_auto_groups.restype = _i
_lib.ulys_strerror.argtypes = [_i]
_lib.ulys_strerror.restype = ctypes.c_char_p
_lib.ulys_last_error.argtypes = []
_lib.ulys_last_error.restype = ctypes.c_char_p

EXPORTED = ("ulys_pack", "ulys_amax_bf16", "ulys_attend_group", "ulys_attend_group_ex", "ulys_attend_splits",
            "ulys_attend_ranges", "ulys_attend_workspace_bytes", "ulys_attend_group_noalloc",
            "ulys_unpack", "ulys_rank_pipeline", "ulys_lse_merge", "ulys_auto_groups", "ulys_strerror",
            "ulys_last_error")

ULYS_REP_SUFFIX, ULYS_REP_PREFIX, ULYS_REP_KV_PREFIX = 0, 1, 2


@dataclass(frozen=True)
class Layout:
    """Python mirror of ``ulys_layout``; ``rep_first`` is a ``ULYS_REP_*`` mode (True/False = prefix/suffix)."""
    batch: int
    degree: int
    s_local: int
    n_rep: int
    rep_first: int
    hq: int
    hkv: int
    head_dim: int
    groups: int

    @property
    def rows(self) -> int:
        """Joint rows of the k/v slots (and of q/o unless the replicated rows are K/V-only)."""
        return self.n_rep + self.degree * self.s_local

    @property
    def shard_rows(self) -> int:
        """Rows of a k/v shard."""
        return self.n_rep + self.s_local

    @property
    def rows_q(self) -> int:
        """Joint rows of the q and o slots."""
        return self.rows - (self.n_rep if int(self.rep_first) == ULYS_REP_KV_PREFIX else 0)

    @property
    def shard_rows_q(self) -> int:
        """Rows of a q or o shard."""
        return self.shard_rows - (self.n_rep if int(self.rep_first) == ULYS_REP_KV_PREFIX else 0)

    @property
    def gq(self) -> int:
        return self.hq // self.degree // self.groups

    @property
    def gkv(self) -> int:
        return self.hkv // self.degree // self.groups

    def c_struct(self) -> ulys_layout:
        return ulys_layout(self.batch, self.degree, self.s_local, self.n_rep, int(self.rep_first), self.hq, self.hkv,
                           self.head_dim, self.groups)


def _check(status: int) -> None:
    if status == ULYS_OK:
        return
    msg = f"{_lib.ulys_strerror(status).decode()}: {_lib.ulys_last_error().decode()}"
    if status == ULYS_EINVAL:
        raise ValueError(msg)
    if status == ULYS_EUNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes, numel: int | None = None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _ptrs(ts, name, dtypes, numel):
    arr = (_vp * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _dev(t, f"{name}[{i}]", dtypes, numel)
    return arr


def _cus(device) -> int:
    return torch.cuda.get_device_properties(device).multi_processor_count


def ulys_attend_workspace_bytes(batch: int, q_rows: int, kv_rows: int, heads: int, head_dim: int,
                                key_splits: int = 0, compute_units: int | None = None) -> int:
    """Workspace bytes an attention call of this shape needs for all ``heads`` in one launch (0: no split).

    ``compute_units`` defaults to the current device's count (the automatic split depends on it)."""
    cus = _cus(torch.cuda.current_device()) if compute_units is None else int(compute_units)
    n = _lib.ulys_attend_workspace_bytes(int(batch), int(q_rows), int(kv_rows), int(heads), int(head_dim),
                                         int(key_splits), cus)
    _check(int(min(n, 0)))
    return int(n)


def _workspace(workspace, device, batch, q_rows, kv_rows, heads, head_dim, key_splits, stream):
    """(pointer, bytes) of the caller's workspace, or of a new torch buffer sized for the call (kept alive by
    torch's allocator until the work on ``stream`` that uses it is done)."""
    if workspace is None:
        n = ulys_attend_workspace_bytes(batch, q_rows, kv_rows, heads, head_dim, key_splits, _cus(device))
        if n == 0:
            return None, 0, None
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
        workspace.record_stream(torch.cuda.current_stream(device) if stream is None else stream)
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


_BF16 = (torch.bfloat16,)
_QK8 = (torch.uint8, torch.float8_e4m3fn)


def ulys_pack(layout: Layout, rank: int, group: int, q_shards, k_shards, v_shards, q_slot, k_slot, v_slot,
              qk_dtype: int = ULYS_BF16, qk_amax: torch.Tensor | None = None, stream=None) -> None:
    """Fill the receive slots of (rank, group); group = -1 packs all groups."""
    L = layout
    if len(q_shards) != L.degree or len(k_shards) != L.degree or len(v_shards) != L.degree:
        raise ValueError("need one shard per rank for q, k and v")
    ng = L.groups if group < 0 else 1
    nq = L.batch * L.shard_rows_q * L.hq * L.head_dim
    nkv = L.batch * L.shard_rows * L.hkv * L.head_dim
    qa = _ptrs(q_shards, "q_shards", _BF16, nq)
    ka = _ptrs(k_shards, "k_shards", _BF16, nkv)
    va = _ptrs(v_shards, "v_shards", _BF16, nkv)
    qk_t = _QK8 if qk_dtype == ULYS_FP8_E4M3 else _BF16
    qs = _dev(q_slot, "q_slot", qk_t, ng * L.batch * L.rows_q * L.gq * L.head_dim)
    ks = _dev(k_slot, "k_slot", qk_t, ng * L.batch * L.rows * L.gkv * L.head_dim)
    vs = _dev(v_slot, "v_slot", _BF16, ng * L.batch * L.rows * L.gkv * L.head_dim)
    am = None
    if qk_amax is not None:
        am = _dev(qk_amax, "qk_amax", (torch.float32,), 2)
    c = L.c_struct()
    _check(_lib.ulys_pack(ctypes.byref(c), rank, group, qa, ka, va, qs, ks, vs, qk_dtype, am, _stream(stream)))


def ulys_amax_bf16(tensors, out: torch.Tensor, stream=None) -> None:
    """out[0] = max |x| over all ``tensors`` (bf16, same element count)."""
    n = tensors[0].numel()
    arr = _ptrs(tensors, "tensors", _BF16, n)
    o = _dev(out, "out", (torch.float32,))
    _check(_lib.ulys_amax_bf16(arr, len(tensors), n, o, _stream(stream)))


def ulys_attend_group(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                      lse: torch.Tensor | None = None, softmax_scale: float = 0.0,
                      key_gaps=None, qk_dtype: int = ULYS_BF16, qk_amax: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> None:
    """Attention on one slot: q ``[B, rows, hq, D]``, k/v ``[B, rows, hkv, D]`` -> o (and lse ``[B, hq, rows]``).

    ``key_gaps``: per-batch ``(start, end)`` masked key ranges, or None.  ``workspace``: a GPU byte buffer of at
    least the size :func:`ulys_attend_workspace_bytes` gives for one head (None: a torch buffer of the full size
    is allocated for the call).
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.dim() != 4:
        raise ValueError("q, k, v, o must be 4-D [B, rows, heads, D]")
    b, rows, hq, d = q.shape
    hkv = k.shape[2]
    if tuple(k.shape) != (b, rows, hkv, d) or tuple(v.shape) != (b, rows, hkv, d) or tuple(o.shape) != (b, rows, hq, d):
        raise ValueError("shape mismatch between q, k, v and o")
    qk_t = _QK8 if qk_dtype == ULYS_FP8_E4M3 else _BF16
    qp = _dev(q, "q", qk_t)
    kp = _dev(k, "k", qk_t)
    vp = _dev(v, "v", _BF16)
    op = _dev(o, "o", _BF16)
    lp = None if lse is None else _dev(lse, "lse", (torch.float32,), b * hq * rows)
    am = None if qk_amax is None else _dev(qk_amax, "qk_amax", (torch.float32,), 2)
    gaps = None
    if key_gaps is not None:
        if len(key_gaps) != b:
            raise ValueError("key_gaps needs one (start, end) per batch")
        gaps = (ctypes.c_int32 * (2 * b))(*[int(x) for g in key_gaps for x in g])
    wp, wn, _keep = _workspace(workspace, q.device, b, rows, rows, hq, d, 0, stream)
    _check(_lib.ulys_attend_group(b, rows, hq, hkv, d, qp, kp, vp, qk_dtype, float(softmax_scale), am, gaps, op, lp,
                                  wp, wn, _stream(stream)))


def ulys_attend_group_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                              lse: torch.Tensor | None = None, softmax_scale: float = 0.0, key_gaps=None,
                              qk_dtype: int = ULYS_BF16, qk_amax: torch.Tensor | None = None, stream=None) -> None:
    """:func:`ulys_attend_group` without a workspace: the library's static per-GPU scratch holds the split
    partials (no allocation anywhere in the call).  Calls that overlap on one GPU race on that scratch."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.dim() != 4:
        raise ValueError("q, k, v, o must be 4-D [B, rows, heads, D]")
    b, rows, hq, d = q.shape
    hkv = k.shape[2]
    if tuple(k.shape) != (b, rows, hkv, d) or tuple(v.shape) != (b, rows, hkv, d) or tuple(o.shape) != (b, rows, hq, d):
        raise ValueError("shape mismatch between q, k, v and o")
    qk_t = _QK8 if qk_dtype == ULYS_FP8_E4M3 else _BF16
    qp = _dev(q, "q", qk_t)
    kp = _dev(k, "k", qk_t)
    vp = _dev(v, "v", _BF16)
    op = _dev(o, "o", _BF16)
    lp = None if lse is None else _dev(lse, "lse", (torch.float32,), b * hq * rows)
    am = None if qk_amax is None else _dev(qk_amax, "qk_amax", (torch.float32,), 2)
    gaps = None
    if key_gaps is not None:
        if len(key_gaps) != b:
            raise ValueError("key_gaps needs one (start, end) per batch")
        gaps = (ctypes.c_int32 * (2 * b))(*[int(x) for g in key_gaps for x in g])
    _check(_lib.ulys_attend_group_noalloc(b, rows, hq, hkv, d, qp, kp, vp, qk_dtype, float(softmax_scale), am, gaps,
                                          op, lp, _stream(stream)))


def ulys_attend_group_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                         lse: torch.Tensor | None = None, softmax_scale: float = 0.0, key_gaps=None,
                         key_mask: torch.Tensor | None = None, qk_dtype: int = ULYS_BF16,
                         qk_amax: torch.Tensor | None = None, key_splits: int = 0,
                         workspace: torch.Tensor | None = None, stream=None) -> None:
    """Attention with q ``[B, Nq, hq, D]`` and k/v ``[B, Nk, hkv, D]`` (Nq may differ from Nk) -> o ``[B, Nq, hq, D]``
    (and lse ``[B, hq, Nq]``).

    ``key_mask``: device int32/uint32 words ``[B, ceil(Nk/32)]``, bit ``j % 32`` of word ``j // 32`` set for a
    valid key ``j``, or None (all keys valid).  ``key_gaps`` as for :func:`ulys_attend_group`.
    ``key_splits``: 0 = automatic (:func:`ulys_attend_splits`, else :func:`ulys_attend_ranges`), 1 = none,
    2..16 = that many key-range runs per query tile, ``-R`` = a range split into R runs per (b, head).
    ``workspace`` as for :func:`ulys_attend_group` (sized with the same ``key_splits``).
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.dim() != 4:
        raise ValueError("q, k, v, o must be 4-D [B, rows, heads, D]")
    b, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (b, nk, hkv, d) or tuple(v.shape) != (b, nk, hkv, d) or tuple(o.shape) != (b, nq, hq, d):
        raise ValueError("shape mismatch between q, k, v and o")
    qk_t = _QK8 if qk_dtype == ULYS_FP8_E4M3 else _BF16
    qp = _dev(q, "q", qk_t)
    kp = _dev(k, "k", qk_t)
    vp = _dev(v, "v", _BF16)
    op = _dev(o, "o", _BF16)
    lp = None if lse is None else _dev(lse, "lse", (torch.float32,), b * hq * nq)
    am = None if qk_amax is None else _dev(qk_amax, "qk_amax", (torch.float32,), 2)
    mp = None
    if key_mask is not None:
        mp = _dev(key_mask, "key_mask", (torch.int32, torch.uint32), b * ((nk + 31) // 32))
    gaps = None
    if key_gaps is not None:
        if len(key_gaps) != b:
            raise ValueError("key_gaps needs one (start, end) per batch")
        gaps = (ctypes.c_int32 * (2 * b))(*[int(x) for g in key_gaps for x in g])
    wp, wn, _keep = _workspace(workspace, q.device, b, nq, nk, hq, d, key_splits, stream)
    _check(_lib.ulys_attend_group_ex(b, nq, nk, hq, hkv, d, qp, kp, vp, qk_dtype, float(softmax_scale), am, gaps, mp,
                                     int(key_splits), op, lp, wp, wn, _stream(stream)))


def ulys_unpack(layout: Layout, rank: int, group: int, o_slot: torch.Tensor, o_shards, stream=None) -> None:
    """Scatter the output slot(s) of (rank, group) into the P output shards."""
    L = layout
    if len(o_shards) != L.degree:
        raise ValueError("need one output shard per rank")
    ng = L.groups if group < 0 else 1
    sp = _dev(o_slot, "o_slot", _BF16, ng * L.batch * L.rows_q * L.gq * L.head_dim)
    oa = _ptrs(o_shards, "o_shards", _BF16, L.batch * L.shard_rows_q * L.hq * L.head_dim)
    c = L.c_struct()
    _check(_lib.ulys_unpack(ctypes.byref(c), rank, group, sp, oa, _stream(stream)))


def ulys_rank_pipeline(layout: Layout, rank: int, q_shards, k_shards, v_shards, q_slots, k_slots, v_slots,
                       o_slots, o_shards, lse: torch.Tensor | None = None, softmax_scale: float = 0.0,
                       key_gaps=None, qk_dtype: int = ULYS_BF16, qk_amax: torch.Tensor | None = None,
                       events=None, workspace: torch.Tensor | None = None, stream=None, copy_stream=None) -> None:
    """Pack, attend and unpack every head group of ``rank``; repack on ``copy_stream`` overlaps attention.

    Slots hold all G groups (``[G, B, rows, Gh, D]``; q/o with ``rows_q`` rows), lse ``[G, B, Gq, rows_q]`` or None.
    ``copy_stream`` None means the same stream as ``stream`` (sequential).  ``events``: three
    ``torch.cuda.Event`` objects the library records and waits on (reusable across calls; None: three new
    ones).  ``workspace`` as for :func:`ulys_attend_group`, for one group's attention.
    """
    L = layout
    if len(q_shards) != L.degree or len(k_shards) != L.degree or len(v_shards) != L.degree:
        raise ValueError("need one shard per rank for q, k and v")
    if len(o_shards) != L.degree:
        raise ValueError("need one output shard per rank")
    G = L.groups
    nq = L.batch * L.shard_rows_q * L.hq * L.head_dim
    nkv = L.batch * L.shard_rows * L.hkv * L.head_dim
    qa = _ptrs(q_shards, "q_shards", _BF16, nq)
    ka = _ptrs(k_shards, "k_shards", _BF16, nkv)
    va = _ptrs(v_shards, "v_shards", _BF16, nkv)
    qk_t = _QK8 if qk_dtype == ULYS_FP8_E4M3 else _BF16
    qs = _dev(q_slots, "q_slots", qk_t, G * L.batch * L.rows_q * L.gq * L.head_dim)
    ks = _dev(k_slots, "k_slots", qk_t, G * L.batch * L.rows * L.gkv * L.head_dim)
    vs = _dev(v_slots, "v_slots", _BF16, G * L.batch * L.rows * L.gkv * L.head_dim)
    os_ = _dev(o_slots, "o_slots", _BF16, G * L.batch * L.rows_q * L.gq * L.head_dim)
    oa = _ptrs(o_shards, "o_shards", _BF16, nq)
    lp = None if lse is None else _dev(lse, "lse", (torch.float32,), G * L.batch * L.gq * L.rows_q)
    am = None if qk_amax is None else _dev(qk_amax, "qk_amax", (torch.float32,), 2)
    gaps = None
    if key_gaps is not None:
        if len(key_gaps) != L.batch:
            raise ValueError("key_gaps needs one (start, end) per batch")
        gaps = (ctypes.c_int32 * (2 * L.batch))(*[int(x) for g in key_gaps for x in g])
    s = _stream(stream)
    x = s if copy_stream is None else _stream(copy_stream)
    if events is None:
        events = [torch.cuda.Event() for _ in range(3)]
    if len(events) != 3:
        raise ValueError("need three events")
    ev = (_vp * 3)()
    for i, e in enumerate(events):
        if e.cuda_event == 0:            # torch creates the HIP event on its first record
            e.record(torch.cuda.current_stream() if stream is None else stream)
        ev[i] = e.cuda_event
    wp, wn, _keep = _workspace(workspace, q_slots.device, L.batch, L.rows_q, L.rows, L.gq, L.head_dim, 0, stream)
    c = L.c_struct()
    _check(_lib.ulys_rank_pipeline(ctypes.byref(c), rank, qa, ka, va, qs, ks, vs, os_, lp, oa, qk_dtype, am,
                                   float(softmax_scale), gaps, ev, wp, wn, s, x))


def ulys_lse_merge(o_parts, lse_parts, o_out: torch.Tensor, lse_out: torch.Tensor | None = None,
                   stream=None) -> None:
    """Merge partial attention results over disjoint key blocks: o ``[B, rows, heads, D]`` bf16,
    lse ``[B, heads, rows]`` fp32 per part -> o_out (and lse_out)."""
    if len(o_parts) != len(lse_parts) or not o_parts:
        raise ValueError("need one lse per partial output and at least one part")
    b, rows, heads, d = o_out.shape
    n = b * rows * heads * d
    oa = _ptrs(o_parts, "o_parts", _BF16, n)
    la = _ptrs(lse_parts, "lse_parts", (torch.float32,), b * heads * rows)
    op = _dev(o_out, "o_out", _BF16, n)
    lp = None if lse_out is None else _dev(lse_out, "lse_out", (torch.float32,), b * heads * rows)
    _check(_lib.ulys_lse_merge(len(o_parts), oa, la, b, rows, heads, d, op, lp, _stream(stream)))


def ulys_attend_splits(batch: int, q_rows: int, kv_rows: int, compute_units: int = 256) -> int:
    """The automatic key-range split (run count) of an attention call of this shape on ``compute_units`` CUs."""
    st = _lib.ulys_attend_splits(int(batch), int(q_rows), int(kv_rows), int(compute_units))
    _check(min(st, 0))
    return st


def ulys_attend_ranges(batch: int, q_rows: int, kv_rows: int, compute_units: int = 256) -> int:
    """The automatic range split (runs per (b, head), 0 = none) of an attention call of this shape."""
    st = _lib.ulys_attend_ranges(int(batch), int(q_rows), int(kv_rows), int(compute_units))
    _check(min(st, 0))
    return st


def ulys_auto_groups(layout: Layout, compute_units: int = 256) -> int:
    """Head-group count for ulys_rank_pipeline (1 = keep one call); ``layout.groups`` is ignored."""
    c = layout.c_struct()
    st = _lib.ulys_auto_groups(ctypes.byref(c), int(compute_units))
    _check(min(st, 0))
    return st


def call_raw(name: str, *args) -> int:
    """Call an entry point with raw ctypes arguments and return its status (for ABI tests)."""
    return getattr(_lib, name)(*args)


def last_error() -> str:
    return _lib.ulys_last_error().decode()
