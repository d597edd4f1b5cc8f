"""CPU oracle for striped ring attention: TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
path is checked against. Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (``striped_ring_attention_amd``) never imports,
calls or falls back to it, and this package imports nothing from there.

Everything here is numpy in float64 on the inputs exactly as stored (bf16 or
fp32 values widened to fp64). Sources, cited by page and section:

* "Striped Attention: Faster Ring Attention for Causal Transformers", summary
  page at research.elamur.ai ("Summary" paragraphs 1-2, "Key points"):
  ring attention over N devices with K/V blocks circulating, contiguous
  chunks vs. the striped layout in which each device holds every N-th token,
  exactness through permutation equivariance.
* The same paper's abstract (pith.science/paper/2311.09431): ring attention
  is an exact attention algorithm; striped devices hold tokens spread
  uniformly through the sequence.
* Notes page at phantomic12.github.io (paragraphs 1-2): causal load imbalance
  of contiguous shards, uniform stripes.

Modules:
  stripes    -- stripe/contiguous position maps and brute-force tile census.
  attention  -- dense causal attention, per-round ring partials, the
                log-sum-exp merge, the full ring and the backward pass.
  rotary     -- rotary position embedding of model inputs at their original
                positions, and its composition with the stripe gather.

Parity status of each function is stated in its docstring; every function
here is pinned by ``tests/test_oracle.py`` and ``tests/test_oracle_rope.py``
(brute force, closed forms, invariants, a library special case) -- none is
"parity unpinned".
"""

from .stripes import (  # noqa: F401
    CONTIGUOUS,
    STRIPED,
    positions,
    stripe_index,
    unstripe_index,
    to_device_layout,
    from_device_layout,
    round_source,
    live_mask,
    live_tiles,
    live_pairs,
)
from .attention import (  # noqa: F401
    dense_causal_attention,
    attention_rows,
    ring_partial,
    lse_merge,
    ring_attention,
    dense_causal_backward,
    backward_key_rows,
    backward_query_rows,
)
from .rotary import (  # noqa: F401
    inv_freq,
    rope,
    rope_device_layout,
)
