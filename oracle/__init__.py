"""Oracle for the Kimi K3 Gated MLA layer and the Kimi K3.1 Gated DSA decode step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import or call anything in this package. The HIP library and its Python
binding never import it, and it imports nothing from them: the two share no code, header,
table or helper. The only module both sides use is ``workloads`` (seeded inputs, no arithmetic
of the method).

Everything here is plain float64 NumPy written from the pages' description of the layer, in
the pages' order and notation, with no blocking, fusion or reordering. Inputs arrive as bf16
values widened to float64. The one place the oracle rounds is where the pages fix a storage
format: the KV cache and the index-key cache are held in bfloat16.

Parity pins (tests/test_oracle_*.py) tie every function here to facts fixed by the pages and
the mathematics: page-printed cache sizes, float64 brute force on tiny inputs, the absorbed ==
expanded identity, causality, prefill == prefill-then-decode, closed forms of the norms, the
gate at W_g = 0, the ReLU identity of the index score, and sort-based top-k. End-to-end
numeric values of the layer are otherwise unpinned: the pages print no worked example.
"""
from .mla import *  # noqa: F401,F403
from .mla import __all__  # noqa: F401
