"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle.

This module only draws random numbers and names the workload shapes; it
holds none of the method's arithmetic (no permutation, no attention, no
quantisation).  Draws: ``torch.Generator('cpu').manual_seed(seed)``, float32
``randn`` for q, then k, then v, each cast to bfloat16 (round to nearest
even).  Shapes follow the workloads the pages measure (Wan2.1 at Ulysses 4:
40 heads of 128 over 27280 rows, 6820 rows per rank; a 512-row text prefix
with 226 valid tokens joined to 32760 image rows; GQA 16/4 heads).  The
activations of the trained models are not available, so N(0, 1) stands in.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes and the seed, nothing else."""
    name: str
    seed: int
    batch: int
    degree: int          # simulated Ulysses degree P (1 = the slot is the whole call)
    s_local: int         # sharded rows per rank
    n_rep: int           # replicated text rows (0 = none)
    rep_first: bool      # True: replicated prefix, False: suffix
    hq: int              # model q heads (all ranks)
    hkv: int             # model k/v heads (all ranks)
    head_dim: int
    groups: int          # head groups per rank
    key_gap: tuple[int, int] | None = None   # masked key range [start, end) of the joint sequence
    q_mult: float = 1.0                      # q drawn as q_mult * N(0,1) (peaky softmax)
    fp8_qk: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.n_rep + self.degree * self.s_local


# The five workloads (sizes only).
TINY = Workload("tiny", 1, batch=1, degree=2, s_local=112, n_rep=32, rep_first=True,
                hq=4, hkv=4, head_dim=64, groups=2)
WAN_SHARE = Workload("wan_share", 2, batch=1, degree=1, s_local=27280, n_rep=0, rep_first=True,
                     hq=10, hkv=10, head_dim=128, groups=1)
WAN_SHARE_G5 = Workload("wan_share_g5", 2, batch=1, degree=1, s_local=27280, n_rep=0, rep_first=True,
                        hq=10, hkv=10, head_dim=128, groups=5)
JOINT_VARLEN = Workload("joint_varlen", 3, batch=1, degree=1, s_local=32760, n_rep=512, rep_first=True,
                        hq=12, hkv=12, head_dim=128, groups=3, key_gap=(226, 512))
GQA = Workload("gqa", 4, batch=2, degree=1, s_local=16384, n_rep=0, rep_first=True,
               hq=16, hkv=4, head_dim=128, groups=4, q_mult=2.0)
E2E_P4 = Workload("e2e_p4", 5, batch=1, degree=4, s_local=6820, n_rep=0, rep_first=True,
                  hq=40, hkv=40, head_dim=128, groups=5, fp8_qk=True)
# Cross-attention to a replicated text K/V prefix at the Wan share: each rank's q holds only its image rows,
# its k/v shards carry the 512 text rows (the first 226 valid, the padding given as a key mask) in front.
KV_PREFIX_MASKED = Workload("kv_prefix_masked", 6, batch=1, degree=4, s_local=6820, n_rep=512, rep_first=True,
                            hq=40, hkv=40, head_dim=128, groups=5,
                            extra={"kv_only_prefix": True, "text_valid": 226})

ALL = {w.name: w for w in (TINY, WAN_SHARE, WAN_SHARE_G5, JOINT_VARLEN, GQA, E2E_P4, KV_PREFIX_MASKED)}


def randn_bf16(gen: torch.Generator, shape, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult
    return x.to(torch.bfloat16)


def global_qkv(w: Workload, seed: int | None = None):
    """Joint (global-layout) q, k, v as CPU bfloat16 tensors ``[B, rows, H, D]``."""
    gen = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    q = randn_bf16(gen, (w.batch, w.rows, w.hq, w.head_dim), w.q_mult)
    k = randn_bf16(gen, (w.batch, w.rows, w.hkv, w.head_dim))
    v = randn_bf16(gen, (w.batch, w.rows, w.hkv, w.head_dim))
    return q, k, v


def small(name: str, seed: int, **kw) -> Workload:
    """A small ad-hoc workload for parity cases (same recipe, other sizes)."""
    base = dict(batch=1, degree=1, s_local=64, n_rep=0, rep_first=True, hq=2, hkv=2,
                head_dim=64, groups=1)
    base.update(kw)
    return Workload(name, seed, **base)


def random_bf16(shape, seed: int, mult: float = 1.0) -> torch.Tensor:
    """Any other seeded bf16 tensor (e.g. a synthetic output slot for unpack tests)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    return randn_bf16(gen, shape, mult)


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Raw 16-bit patterns of a bf16 tensor (for byte-exact comparisons)."""
    return x.contiguous().view(torch.int16)


def random_key_mask(batch: int, n_keys: int, seed: int, p_valid: float = 0.5) -> "np.ndarray":
    """Seeded boolean key mask ``[batch, n_keys]`` (True = valid), each key kept with probability p_valid."""
    import numpy as np
    gen = torch.Generator("cpu").manual_seed(seed)
    return (torch.rand(batch, n_keys, generator=gen) < p_valid).numpy().astype(np.bool_)


def key_mask_words(mask) -> torch.Tensor:
    """Encode a boolean ``[B, N]`` key mask as the library's bit words: int32 ``[B, ceil(N/32)]``,
    bit ``j % 32`` of word ``j // 32`` set for a valid key ``j`` (an encoding of the input, no arithmetic
    of the method)."""
    import numpy as np
    m = np.asarray(mask, dtype=bool)
    b, n = m.shape
    words = (n + 31) // 32
    padded = np.zeros((b, words * 32), dtype=bool)
    padded[:, :n] = m
    w = np.packbits(padded.reshape(b, words, 4, 8), axis=-1, bitorder="little").reshape(b, words, 4)
    return torch.from_numpy(w.astype(np.uint8).copy()).view(torch.int32).reshape(b, words)
