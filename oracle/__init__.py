"""fp64 CPU oracle of the H2O chunked sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product (the HIP
library and its Python binding) never imports or calls it, and it shares no
code with the product: it is a plain, slow restatement of the method written
from the pages of "Learning how to Forget: Fine-tuning for Long-Context Sparse
Attention" (montaan paper page, sections "Improvements to Heavy-Hitter Oracle
(H2O)" and "Kernel Support Needs").

Pins (tests/test_oracle.py) tie it to things other than itself: exact causal
attention from ``torch.nn.functional.scaled_dot_product_attention`` when no
eviction happens, closed forms under uniform attention, a hand-derived worked
example (tests/golden/), brute-force subset enumeration and a dense-masked
replay on tiny caches, and conservation / invariance properties.
"""
from .h2o_oracle import (  # noqa: F401
    H2OState,
    attend_buffer,
    attend_chunk,
    attend_chunk_backward,
    buffer_step,
    evict_and_insert,
    h2o_step,
    lastrec_step,
    select_victims,
    select_victims_lastrec,
    selection_scores,
    update_scores,
)
