"""CPU oracle for the Unweight-style compressed-MLP matmul.  TEST INFRASTRUCTURE.

A plain, slow, obviously correct numpy/Python statement of what the hot path
computes: the lossless exponent codec (field split, top-16 palette, verbatim
64-element groups, canonical Huffman, per-tile stream) and the fp64 matmul it
feeds.  It shares no code with the HIP path and imports nothing from it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
never routes through it.

Source: Cloudflare, "Unweight: how we compressed an LLM 22% without
sacrificing quality" (DocsDigest translation), sections "How to compress model
weights effectively", "Four ways to use compressed weights" and "How the
reconstructive matmul works".  Every function here is pinned by a
``-m "not gpu"`` test against something other than itself; none is
"parity unpinned".
"""
from . import codec, numerics  # noqa: F401
