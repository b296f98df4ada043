"""Reference oracle for the hybrid sliding-window attention forward (TEST INFRASTRUCTURE).

This package is a plain, slow, fp64 CPU implementation of what the GPU library
computes.  It exists only to check that library: nothing in the product path may
import it.  The only permitted callers are the tests under ``tests/``, the
``smoke()`` check in ``__graft_entry__.py`` and the ``cpu_baseline`` leg of
``bench.py``.  It shares no code, constants or helpers with the HIP kernels or
their Python binding, and it never touches a GPU.

Sources (titles of the web pages the method is described on):

* "MiMo-V2-Flash Technical Report" digest (mlpod.com), section 2.2 "Hybrid SWA":
  2.2.1 gives the window of 128 tokens and the 5:1 SWA:GA interleave; 2.2.2
  "Learnable Attention Sink Bias" puts a learnable term in the softmax
  denominator so a query can send attention mass to a virtual sink.  Section 2.3
  describes MTP drafts verified in parallel by the main model.
* "MiMo-V2 全解" blog (kokolerk.github.io), section 2.2: the sink adds a learnable
  term to the softmax denominator (borrowed from gpt-oss).
* ICML 2026 keynote write-up (hzrcw.cc), section 02: 128-token window, GQA,
  learnable sink bias; Q&A: RoPE positions keep increasing as the window slides.

Modules:
  swa_oracle  -- vectorised (numpy, fp64) definition, used for every parity check.
  brute       -- pure-Python per-query loops with math.fsum, for tiny inputs; used
                 only to pin swa_oracle.
"""
