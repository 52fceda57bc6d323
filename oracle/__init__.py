"""CPU oracle for the Ulysses attention hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy/fp64 definitions of what the GPU path
computes: the Ulysses layout permutation (pack / unpack), the OCP e4m3fn cast
used for fp8 q/k, and dense non-causal softmax attention with log-sum-exp.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import, call or execute anything in this package.  The product path
(``ulysses_sequence_attention_amd``) never imports it and shares no code with
it; the only module both sides use is the seeded input generator
``ulysses_sequence_attention_amd.inputs``, which holds none of the method's
arithmetic.

Modules
  layout     -- shard/global layout, pack(r, g), unpack(r, g)
  fp8        -- e4m3fn encode/decode and the per-tensor amax scale
  attention  -- fp64 softmax attention + LSE, key gap, GQA
  brute      -- pure-Python loops for tiny inputs (a pin for ``attention``)

Every function here is pinned by ``tests/test_oracle_*.py`` against
something other than itself (brute force, library routines, closed forms,
invariants, an independent derivation of the permutation from a second page).
"""
