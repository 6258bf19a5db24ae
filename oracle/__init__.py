"""Slow, plain fp64 CPU oracle for the paged-KV attention path.

THIS IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP library (``paged_kv_cache_176_amd``), and neither imports the other; the only
thing both sides consume is the seeded input generators in ``workloads``.

Contents
  * ``e4m3fn``   -- OCP E4M3FN decode (closed form) and the saturating RNE
                    quantiser used by the fp8 cache write.
  * ``paged_ref`` -- cache write (any cache strides: NHD, HND, padded pitches),
                    paged gather, exact softmax attention with GQA, causal
                    offsets and optional sink logits, split-KV partials under a
                    fixed count or a context-bucket split policy, and the
                    log-sum-exp merge.

Every function is pinned by ``-m "not gpu"`` tests (closed forms, invariants,
library special cases such as torch's fp8 cast and fp64 SDPA, brute force on tiny
inputs); no oracle function is "parity unpinned".
"""
from . import e4m3fn, paged_ref  # noqa: F401
