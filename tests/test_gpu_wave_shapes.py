"""The attention kernel's two wave shapes give the same bytes (GPU).

bf16 q/k at head_dim 128 without a key mask run 64 query rows per wave (one wave per SIMD, inline-asm MFMAs); the
same call with a key mask runs 32 rows per wave (two per SIMD, builtin MFMAs).  A mask that marks exactly the keys
outside the gaps selects the second shape without changing what is computed, so the two calls must agree bit for
bit.  Seeded sweep over batch, lengths (ragged and tile-aligned, Nq < Nk as with a K/V-only prefix), GQA, gaps (none,
tile-aligned ends, inside one tile, at the start) and the split choices (automatic, none, key-range runs, range
runs).
"""
import numpy as np
import pytest
import torch

from gpu_common import bits, from_bits, inputs

pytestmark = pytest.mark.gpu

# (batch, nq, nk, hq, hkv, gaps per batch or None, key_splits)
CASES = [
    (1, 256, 256, 1, 1, None, 0),
    (1, 300, 300, 2, 2, None, 0),
    (2, 1000, 1000, 2, 1, [(100, 512), (0, 64)], 0),
    (1, 1024, 1024, 4, 4, [(128, 640)], 1),
    (1, 1500, 1500, 2, 2, [(700, 705)], 2),
    (2, 2048, 2048, 2, 2, None, 3),
    (1, 2000, 2100, 4, 2, [(0, 100)], 0),
    (1, 777, 1536, 2, 2, [(512, 1024)], -3),
    (2, 1300, 1300, 1, 1, [(64, 128), (1200, 1300)], -7),
    (1, 3000, 3000, 8, 2, [(226, 512)], 0),
    (1, 513, 513, 2, 2, None, -5),
    (1, 4096, 4096, 2, 2, None, 0),
    (1, 27280, 27280, 2, 2, None, 0),            # the Wan share's 2-head launch (range split, 128 runs)
    (1, 33272, 33272, 2, 2, [(226, 512)], 0),    # the joint text+image workload's gap
]


def _call(gpu, q, k, v, gaps, mask, splits):
    b, nq, hq, d = q.shape
    o = torch.full((b, nq, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((b, hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    words = None if mask is None else inputs.key_mask_words(mask).cuda()
    gpu.ulys_attend_group_ex(q, k, v, o, l, key_gaps=gaps, key_mask=words, key_splits=splits)
    torch.cuda.synchronize()
    return bits(o), l.cpu().numpy().view(np.int32)


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}-q{c[1]}-k{c[2]}-h{c[3]}/{c[4]}-s{c[6]}" for c in CASES])
def test_wave_shapes_bit_identical(gpu, case):
    b, nq, nk, hq, hkv, gaps, splits = case
    seed = 9000 + 17 * CASES.index(case)
    print(f"wave shapes: b={b} nq={nq} nk={nk} hq={hq} hkv={hkv} gaps={gaps} splits={splits}", flush=True)
    q = from_bits(bits(inputs.random_bf16((b, nq, hq, 128), seed)))
    k = from_bits(bits(inputs.random_bf16((b, nk, hkv, 128), seed + 1)))
    v = from_bits(bits(inputs.random_bf16((b, nk, hkv, 128), seed + 2)))
    mask = np.ones((b, nk), dtype=bool)
    if gaps is not None:
        for i, (g0, g1) in enumerate(gaps):
            mask[i, g0:g1] = False
    o64, l64 = _call(gpu, q, k, v, gaps, None, splits)       # 64 rows per wave
    o32, l32 = _call(gpu, q, k, v, None, mask, splits)       # 32 rows per wave (key mask)
    assert not torch.isnan(from_bits(o64, device="cpu").float()).any(), "unwritten output rows"
    assert np.array_equal(o64, o32), "outputs differ between the wave shapes"
    assert np.array_equal(l64, l32), "LSE differs between the wave shapes"
