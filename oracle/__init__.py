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

Parity status: every function has a pin of its own in ``tests/test_oracle.py``
(closed forms, invariants, brute force or hand-worked values; ``dequant_v``
and ``logits`` by hand-worked examples), each shown to fail on planted
mistakes; none is "parity unpinned".  The oracle holds only the method's
canonical data forms, none of the kernels' internal layouts.
"""
from .vc_oracle import *  # noqa: F401,F403
