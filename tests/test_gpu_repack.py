"""GPU parity: pack / unpack / amax through the C ABI, byte-exact against the oracle."""
import numpy as np
import pytest
import torch

from gpu_common import bits, from_bits, layout_of, ofp8, olay, inputs, shards_of

pytestmark = pytest.mark.gpu

CASES = [
    inputs.TINY,                                                                   # prefix, P=2, G=2
    inputs.small("suffix", 31, degree=4, s_local=37, n_rep=9, rep_first=False, hq=8, hkv=8, groups=2),
    inputs.small("gqa_prefix", 32, batch=2, degree=2, s_local=50, n_rep=13, hq=8, hkv=4, head_dim=128, groups=2),
    inputs.small("ragged_p3", 33, degree=3, s_local=1, n_rep=0, hq=6, hkv=3, head_dim=64, groups=1),
    inputs.small("p8_many_groups", 34, degree=8, s_local=5, n_rep=3, hq=32, hkv=16, head_dim=128, groups=2),
]


def _pack_gpu(ulys, w, sh, rank, group, fp8=False, amax=None):
    L = layout_of(w)
    ng = w.groups if group < 0 else 1
    dev = {k: [from_bits(s) for s in v] for k, v in sh.items()}
    qk_dt = torch.uint8 if fp8 else torch.bfloat16
    q_slot = torch.empty((ng, w.batch, L.rows, L.gq, w.head_dim), dtype=qk_dt, device="cuda")
    k_slot = torch.empty((ng, w.batch, L.rows, L.gkv, w.head_dim), dtype=qk_dt, device="cuda")
    v_slot = torch.empty((ng, w.batch, L.rows, L.gkv, w.head_dim), dtype=torch.bfloat16, device="cuda")
    ulys.ulys_pack(L, rank, group, dev["q"], dev["k"], dev["v"], q_slot, k_slot, v_slot,
                   ulys.ULYS_FP8_E4M3 if fp8 else ulys.ULYS_BF16, amax)
    torch.cuda.synchronize()
    return q_slot, k_slot, v_slot


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_pack_bf16_byte_exact(gpu, w):
    _, sh = shards_of(w)
    for rank in range(w.degree):
        qs, ks, vs = _pack_gpu(gpu, w, sh, rank, -1)
        for g in range(w.groups):
            for name, slot in (("q", qs), ("k", ks), ("v", vs)):
                ref = olay.pack(sh[name], rank, g, w.groups, w.n_rep, w.rep_first)
                assert np.array_equal(bits(slot[g]), ref), f"{w.name} rank {rank} group {g} {name}"
        # single-group launches give the same bytes as the all-groups launch
        g = w.groups - 1
        q1, k1, v1 = _pack_gpu(gpu, w, sh, rank, g)
        assert torch.equal(q1[0].view(torch.int16), qs[g].view(torch.int16))
        assert torch.equal(v1[0].view(torch.int16), vs[g].view(torch.int16))


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_unpack_byte_exact(gpu, w):
    L = layout_of(w)
    sentinel = np.full((w.batch, L.shard_rows, w.hq, w.head_dim), 0x7FC1, dtype=np.int16)
    for rank in range(w.degree):
        slot = bits(inputs.random_bf16((w.groups, w.batch, L.rows, L.gq, w.head_dim), seed=900 + rank))
        ref = [sentinel.copy() for _ in range(w.degree)]
        for g in range(w.groups):
            olay.unpack(slot[g], ref, rank, g, w.groups, w.n_rep, w.rep_first)
        out = [from_bits(sentinel) for _ in range(w.degree)]
        gpu.ulys_unpack(L, rank, -1, from_bits(slot), out)
        torch.cuda.synchronize()
        for p in range(w.degree):
            assert np.array_equal(bits(out[p]), ref[p]), f"{w.name} rank {rank} shard {p}"


def test_full_rank_roundtrip_e2e_shape(gpu):
    """Wan P=4 shards [1, 6820, 40, 128]: pack every rank and group, unpack the q slots
    back: every shard is rebuilt exactly (the exchange is a permutation)."""
    w = inputs.E2E_P4
    L = layout_of(w)
    _, sh = shards_of(w)
    dev = {k: [from_bits(s) for s in v] for k, v in sh.items()}
    out = [torch.empty_like(s) for s in dev["q"]]
    q_slot = torch.empty((w.groups, 1, L.rows, L.gq, w.head_dim), dtype=torch.bfloat16, device="cuda")
    k_slot = torch.empty_like(q_slot)
    v_slot = torch.empty_like(q_slot)
    for rank in range(w.degree):
        gpu.ulys_pack(L, rank, -1, dev["q"], dev["k"], dev["v"], q_slot, k_slot, v_slot)
        if rank == 2:
            torch.cuda.synchronize()
            for g in (0, 4):
                assert np.array_equal(bits(q_slot[g]), olay.pack(sh["q"], rank, g, w.groups, 0, True))
                assert np.array_equal(bits(v_slot[g]), olay.pack(sh["v"], rank, g, w.groups, 0, True))
        gpu.ulys_unpack(L, rank, -1, q_slot, out)
    torch.cuda.synchronize()
    for p in range(w.degree):
        assert torch.equal(out[p].view(torch.int16), dev["q"][p].view(torch.int16))


@pytest.mark.parametrize("w", [CASES[0], CASES[2], CASES[4]], ids=lambda w: w.name)
def test_amax_and_fp8_pack_byte_exact(gpu, w):
    _, sh = shards_of(w)
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    qd = [from_bits(s) for s in sh["q"]]
    kd = [from_bits(s) for s in sh["k"]]
    gpu.ulys_amax_bf16(qd, amax[0:1])
    gpu.ulys_amax_bf16(kd, amax[1:2])
    torch.cuda.synchronize()
    ref_aq = ofp8.amax([torch.from_numpy(s).view(torch.bfloat16).float().numpy() for s in sh["q"]])
    ref_ak = ofp8.amax([torch.from_numpy(s).view(torch.bfloat16).float().numpy() for s in sh["k"]])
    assert amax[0].item() == ref_aq and amax[1].item() == ref_ak
    _, inv_q = ofp8.scales_from_amax(ref_aq)
    _, inv_k = ofp8.scales_from_amax(ref_ak)
    for rank in range(w.degree):
        qs, ks, vs = _pack_gpu(gpu, w, sh, rank, -1, fp8=True, amax=amax)
        for g in range(w.groups):
            for name, slot, inv in (("q", qs, inv_q), ("k", ks, inv_k)):
                ref_bf16 = olay.pack(sh[name], rank, g, w.groups, w.n_rep, w.rep_first)
                ref = ofp8.quantize(torch.from_numpy(ref_bf16).view(torch.bfloat16).float().numpy(), inv)
                got = slot[g].cpu().numpy()
                assert np.array_equal(got, ref), f"{w.name} rank {rank} group {g} {name}: " \
                    f"{int((got != ref).sum())} codes differ"
            assert np.array_equal(bits(vs[g]), olay.pack(sh["v"], rank, g, w.groups, w.n_rep, w.rep_first))


def test_fp8_cast_exhaustive_bf16(gpu):
    """Every finite bf16 pattern through the pack kernel's e4m3fn cast, several scales,
    against the oracle's codec (the cast decides integer codes, so byte-exact)."""
    pat = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    x = pat[torch.isfinite(pat.float())]
    n = (x.numel() // 64) * 64
    x = x[:n].reshape(1, n // 64, 1, 64).contiguous()          # one "shard", D = 64, one head
    w = inputs.small("codec", 0, degree=1, s_local=n // 64, hq=1, hkv=1, head_dim=64)
    L = layout_of(w)
    xd = x.cuda()
    for amax_val in (448.0, 3.75, 0.0, 1e-30, 65280.0, 7.0e37):
        amax = torch.tensor([amax_val, amax_val], dtype=torch.float32, device="cuda")
        qs = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        ks = torch.empty_like(qs)
        vs = torch.empty_like(xd)
        gpu.ulys_pack(L, 0, 0, [xd], [xd], [xd], qs, ks, vs, gpu.ULYS_FP8_E4M3, amax)
        torch.cuda.synchronize()
        _, inv = ofp8.scales_from_amax(np.float32(amax_val))
        ref = ofp8.quantize(x.float().numpy(), inv)
        got = qs.cpu().numpy()
        assert np.array_equal(got, ref), f"amax {amax_val}: {int((got != ref).sum())} codes differ"
