"""Plain fp64 CPU oracle for the VeriCache draft/verify/accept hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The HIP library and its Python binding never import it, and it imports nothing
from them: the two sides share only the seeded input generators in ``synth``.

Every function cites the passage of the source pages it follows.  The pages are
"VeriCache: Turning Lossy KV Cache into Lossless LLM Inference" (gist.science,
English and Korean versions; cited as [VC <section>]) and "CacheGen: KV Cache
Compression and Streaming ..." (context only).  Where the pages are silent the
function states the reading it takes.

Parity status: every function is pinned by ``tests/test_oracle.py`` to closed
forms, invariants or brute force; none is "parity unpinned".
"""
from .vc_oracle import *  # noqa: F401,F403
