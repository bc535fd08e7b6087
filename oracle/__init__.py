"""CPU oracle for the DistFlashAttn hot path — TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct float64 reference that the GPU
path is checked against.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product
path (``long_context_exact_amd``) never imports, calls or links anything
here, and nothing here imports the product path.

Source: "DISTFLASHATTN: Distributed Memory-efficient Attention for
Long-context LLMs Training" (arXiv 2310.03294), as summarised section by
section on its paperlayer.ai abstract page.  Citations below name the
paper's section / figure / appendix as that page tags them.

Modules
-------
attention  exact causal softmax attention (forward, LSE merge, backward),
           optionally restricted to a local sliding window, with or without
           global tokens
schedule   the chunk-pair schedules (unbalanced, load-balanced, sliding-window
           and sliding-window with replicated global tokens) and the causal
           tile map of one chunk pair

Every function here is pinned by ``tests/test_oracle_*.py`` against facts the
oracle does not compute itself (brute force, closed forms, invariants,
finite differences, a library special case).  No function is "parity
unpinned".
"""

from .attention import (  # noqa: F401
    attention_fwd,
    lse_merge,
    attention_bwd,
    attention_delta,
)
from .schedule import (  # noqa: F401
    balanced_schedule,
    unbalanced_schedule,
    window_schedule,
    global_window_schedule,
    causal_tile_map,
)
