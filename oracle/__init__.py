"""Float64 CPU oracle for TurboQuant-style KV-cache quantize-append and
compressed-domain decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the GPU library computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library under ``kv_cache_vector_append_amd/`` never does, and
the two share no code (only the seeded input generators in ``workloads/``).

Sources, cited by page title and section throughout:

* [Design Study]  "TurboQuant Family Design Study for CPU and Browser WASM KV
  Caches" (iarpg.com report).
* [Reconstruction]  "Mathematical Reconstruction, Lineage, and Accuracy Limits
  of TurboQuant and TurboVec" (iarpg.com report).  Its formulas are missing
  from the extracted text; every place where this oracle had to choose a
  reading is marked READING.
* [README]  "TurboQuant: KV Cache Compression for LLM Inference"
  (electron-rare/turboquant README).

Pinning status (what each function is checked against) is listed in
``tests/test_oracle_*.py``.  Parity unpinned: none of the functions below is
without a pin; the one reading that no page fixes numerically (the
structured two-round QJL sketch) is pinned by its unbiasedness bound.
"""

from . import rng, codebook, rotation, layout, tq  # noqa: F401
