"""CPU oracle for the TurboQuant KV-cache hot path — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 restatement of what the quantise/store
and decode-attention path computes, written from the pages' description of
the method.  It exists to check the HIP path; nothing in the product
(``kv_cache_vector_03_amd``) imports it, and it imports nothing from the
product.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.

Sources (cited by page title and section throughout):

* "From paper to practice: the TurboQuant integration roadmap of vLLM,
  SGLang and TRT-LLM" (miraclefarms notes, 2026-04-21) — called *Roadmap*.
* "TurboQuant: extreme KV-cache compression for LLM inference" (pomoai hub
  page on the 0xSero/turboquant project) — called *Hub*.
* The iThome article on TurboQuant KV-cache quantisation (article 10406003)
  — called *iThome*.
* "TurboQuant KV cache 3-bit" (yage.ai share page, 2026-03-25) — called
  *Yage*.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (closed forms, textbook values, brute force, statistics).  The
whole-pipeline attention *quality* against unquantised attention has no
number on the pages for synthetic data: that comparison is reported, never
asserted ("parity unpinned" in that narrow sense only).
"""

from . import bits, codebook, rotation, keys, values, paged, attention  # noqa: F401
