"""Ulysses sequence-parallel attention, one GPU's hot path, native on MI355X (gfx950).

The C-ABI library ``libulys.so`` (HIP kernels, see ``include/ulys.h``) does
the work; ``ulysses_sequence_attention_amd.ulys`` is its thin ctypes binding
and ``ulysses_sequence_attention_amd.inputs`` holds the seeded synthetic
input generators.  Import ``ulys`` explicitly: it raises ImportError when
the library has not been built (there is no fallback path).
"""
