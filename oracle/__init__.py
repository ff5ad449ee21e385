"""CPU oracle for the batched K-token verify pass — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct reference implementations of what the HIP
library computes: explicit dequantisation followed by a float64 matmul, float64
multi-row attention, and the exact-integer Leviathan–Chen acceptance procedure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The product path (the
``speculative_decoding_verify_vq_amd`` package and its C-ABI library) never
imports, links or calls it, and this package imports nothing from the product
path. The two share no code.

Sources (pages, cited by title and section):
  * "The fastest way to run local LLMs on a Mac" (mtplx.com docs), sections
    "Decode is a memory-bandwidth problem", "Why native MTP doubles decode",
    "Why exact acceptance matters".
  * "Speculative decoding and MTP on Apple silicon" (llms-explorer.com), section
    "Facts" (the claims on the quantized-matmul re-read, the multi-row
    attention kernel, Leviathan–Chen rejection sampling and identical
    truncation of draft and target distributions).

Parity status of every function is stated in its module docstring. Every
function here is pinned by the ``-m "not gpu"`` tests (brute force, closed
forms, invariants, special cases, exact rational enumeration and a chi-square
distribution test); none is "parity unpinned".
"""
from . import qmm, attn, accept, stack  # noqa: F401
