"""Seeded random sweep of pack (bf16 and e4m3 q/k) and unpack against the oracle's layout map, byte-exact.

Layouts drawn from a fixed seed: batch, Ulysses degree, sharded rows, a replicated prefix or suffix (or
none), GQA head counts, head dim and the group count; every rank, all groups in one launch and one group
alone.  Unpack writes into shards filled with a sentinel, so a row or head it should not touch shows."""
import numpy as np
import pytest
import torch

from gpu_common import bits, from_bits, inputs, layout_of, ofp8, olay, shards_of

pytestmark = pytest.mark.gpu

N_CASES = 40


def _workload(i):
    rng = np.random.default_rng(9000 + i)
    degree = int(rng.choice([1, 2, 3, 4, 8]))
    groups = int(rng.choice([1, 2, 3]))
    hkv_rank = groups * int(rng.choice([1, 2]))
    hq_rank = hkv_rank * int(rng.choice([1, 2, 4]))
    return inputs.small(f"rand{i}", 4000 + i, batch=int(rng.choice([1, 2])), degree=degree,
                        s_local=int(rng.choice([1, 3, 17, 64, 100])), n_rep=int(rng.choice([0, 0, 1, 9, 64])),
                        rep_first=bool(rng.random() < 0.6), hq=hq_rank * degree, hkv=hkv_rank * degree,
                        head_dim=int(rng.choice([64, 128])), groups=groups), bool(rng.random() < 0.3)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layout_pack_unpack(gpu, i):
    w, fp8 = _workload(i)
    L = layout_of(w)
    _, sh = shards_of(w)
    dev = {k: [from_bits(s) for s in v] for k, v in sh.items()}
    amax = inv = None
    if fp8:
        amax = torch.empty(2, dtype=torch.float32, device="cuda")
        gpu.ulys_amax_bf16(dev["q"], amax[0:1])
        gpu.ulys_amax_bf16(dev["k"], amax[1:2])
        torch.cuda.synchronize()
        inv = {n: ofp8.scales_from_amax(ofp8.amax([torch.from_numpy(s).view(torch.bfloat16).float().numpy()
                                                    for s in sh[n]]))[1] for n in ("q", "k")}
    qk_dt = torch.uint8 if fp8 else torch.bfloat16
    for rank in range(w.degree):
        for group in (-1, w.groups - 1):
            ng = w.groups if group < 0 else 1
            qs = torch.empty((ng, w.batch, L.rows, L.gq, w.head_dim), dtype=qk_dt, device="cuda")
            ks = torch.empty((ng, w.batch, L.rows, L.gkv, w.head_dim), dtype=qk_dt, device="cuda")
            vs = torch.empty((ng, w.batch, L.rows, L.gkv, w.head_dim), dtype=torch.bfloat16, device="cuda")
            gpu.ulys_pack(L, rank, group, dev["q"], dev["k"], dev["v"], qs, ks, vs,
                          gpu.ULYS_FP8_E4M3 if fp8 else gpu.ULYS_BF16, amax)
            torch.cuda.synchronize()
            for j in range(ng):
                g = j if group < 0 else group
                for name, slot in (("q", qs), ("k", ks), ("v", vs)):
                    ref = olay.pack(sh[name], rank, g, w.groups, w.n_rep, w.rep_first)
                    if fp8 and name != "v":
                        ref = ofp8.quantize(torch.from_numpy(ref).view(torch.bfloat16).float().numpy(), inv[name])
                        got = slot[j].cpu().numpy()
                    else:
                        got = bits(slot[j])
                    assert np.array_equal(got, ref), f"{w} rank {rank} group {g} {name} fp8={fp8}"
        # unpack of a random output slot (all groups) into sentinel-filled shards
        sentinel = np.full((w.batch, L.shard_rows, w.hq, w.head_dim), 0x7FC1, dtype=np.int16)
        slot = bits(inputs.random_bf16((w.groups, w.batch, L.rows, L.gq, w.head_dim), seed=5000 + 37 * i + rank))
        ref = [sentinel.copy() for _ in range(w.degree)]
        for g in range(w.groups):
            olay.unpack(slot[g], ref, rank, g, w.groups, w.n_rep, w.rep_first)
        out = [from_bits(sentinel) for _ in range(w.degree)]
        gpu.ulys_unpack(L, rank, -1, from_bits(slot), out)
        torch.cuda.synchronize()
        for p in range(w.degree):
            assert np.array_equal(bits(out[p]), ref[p]), f"{w} rank {rank} unpack shard {p}"
