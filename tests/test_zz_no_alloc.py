"""ulys_attend_group_noalloc (static per-GPU scratch, no allocation) against ulys_attend_group with a
caller workspace: byte-identical o and lse, over calls in a row on the same scratch, the second with a
smaller input, then a call whose heads need more than the scratch (several launches), and the rejection of
a call whose single head needs more than it."""
import numpy as np
import pytest
import torch

from gpu_common import bits, check_attention, from_bits, inputs, oatt, sample_rows

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20


def _inputs(name, seed, rows, heads):
    w = inputs.small(name, seed, s_local=rows, hq=heads, hkv=heads, head_dim=128)
    return [from_bits(bits(x)) for x in inputs.global_qkv(w)]


def _pair(gpu, q, k, v):
    b, rows, hq, d = q.shape
    o1 = torch.full((b, rows, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((b, hq, rows), float("nan"), dtype=torch.float32, device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    gpu.ulys_attend_group_noalloc(q, k, v, o1, l1)
    ws = torch.empty(max(gpu.ulys_attend_workspace_bytes(b, rows, rows, hq, d), 256), dtype=torch.uint8,
                     device="cuda")
    gpu.ulys_attend_group(q, k, v, o2, l2, workspace=ws)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def _same(a, b):
    return torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


def test_noalloc_equals_workspace_call(gpu):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # 1) the Wan share's 2-head group: the range split's partials fill 68 MB of the scratch
    q, k, v = _inputs("noalloc_a", 91, 27280, 2)
    need = gpu.ulys_attend_workspace_bytes(1, 27280, 27280, 2, 128, 0, cus)
    print(f"call 1: 27280 rows x 2 heads, workspace {need} bytes", flush=True)
    o1, l1, o2, l2 = _pair(gpu, q, k, v)
    assert _same(o1, o2) and _same(l1, l2)
    # 2) a smaller call right after it on the same scratch (key-range split of 4096 rows)
    q, k, v = _inputs("noalloc_b", 92, 4096, 2)
    need2 = gpu.ulys_attend_workspace_bytes(1, 4096, 4096, 2, 128, 0, cus)
    print(f"call 2: 4096 rows x 2 heads, workspace {need2} bytes", flush=True)
    assert 0 < need2 < need
    o1, l1, o2, l2 = _pair(gpu, q, k, v)
    assert _same(o1, o2) and _same(l1, l2)
    rows = sample_rows(4096, extra=24)
    to = lambda t: t.cpu().double().numpy()
    o_ref, l_ref = oatt.attention(to(q), to(k), to(v), oatt.default_scale(128), rows=rows)
    check_attention(o1, l1, o_ref, l_ref, rows=rows, label="noalloc 4096 rows")
    # 3) heads needing more than the scratch: the call runs them in several launches, same bytes
    q, k, v = _inputs("noalloc_c", 93, 27280, 10)
    need3 = gpu.ulys_attend_workspace_bytes(1, 27280, 27280, 10, 128, 0, cus)
    print(f"call 3: 27280 rows x 10 heads, workspace {need3} bytes (scratch {SCRATCH})", flush=True)
    o1, l1, o2, l2 = _pair(gpu, q, k, v)
    assert _same(o1, o2) and _same(l1, l2)
    assert not torch.isnan(l1).any()


def test_noalloc_rejects_a_head_above_the_scratch(gpu):
    """One head of 136000 rows takes a range split whose partials need more than 128 MiB: refused with
    nothing enqueued (the output keeps its sentinel)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = 136000
    need = gpu.ulys_attend_workspace_bytes(1, rows, rows, 1, 128, 0, cus)
    if need <= SCRATCH:
        pytest.skip(f"on {cus} CUs this shape needs only {need} bytes")
    q = torch.zeros((1, rows, 1, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(ValueError, match="static"):
        gpu.ulys_attend_group_noalloc(q, q, q, o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
