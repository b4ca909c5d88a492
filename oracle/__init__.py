"""CPU oracle for the MoBA prefill forward pass, its backward, packed sequences, the
short key convolution and the full-attention decode that follows a prefill (float64,
NumPy).

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``, and by
nothing else.  The product path (the HIP library ``libmoba.so`` and its Python
binding) never imports, calls or links it, and fails loudly when its own extension is
missing instead of falling back to this code.

It shares no code with the HIP path: no kernels, headers, helpers, tables or pre/post
processing.  The only module both sides use is ``workloads`` (seeded random inputs).

Two independent implementations live here:

* ``moba_oracle``  the plain definition, row by row: centroids, gate scores, top-k
  with the current block forced, one softmax over the union of the attended keys.
* ``bruteforce``   the attention-mask formulation (the pages' "moba_naive" idea): a
  full T x nb gate matrix and a T x T boolean mask, for tiny inputs only.

Every function is pinned by ``tests/test_oracle.py`` against facts fixed by the pages
or by mathematics (dense-attention equivalence against torch's SDPA, closed forms,
exact-tie rules, hand-derived routings, brute force).  No function here is
"parity unpinned".
"""
from .moba_oracle import (  # noqa: F401
    num_blocks, centroids, gate_scores_rows, select_rows, select_blocks,
    attended_keys, attend_row, attend_rows, attend_parts_row, merge_parts,
    moba_forward, moba_rows, attended_pairs, attend_row_grad, moba_backward,
    moba_forward_varlen, key_short_conv, moba_backward_varlen, decode_attention,
)
from .bruteforce import moba_bruteforce, moba_bruteforce_packed  # noqa: F401
