"""Plain CPU oracle for CLEAR circular-window attention (forward pass).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The library in ``dit_circular_local_amd``
never imports it, and this package imports nothing from the library: the two
share no code.

What it computes comes from the pages about CLEAR (arXiv 2412.16112):

* the attention mask M of the pith.science review of the paper ("Core claim"):
  a pair (i, j) is admitted when either token is a text token or the two image
  tokens lie within Euclidean radius r on the token grid;
* plain softmax attention with 1/sqrt(c) logit scaling (the same review,
  "Assumptions & free parameters": Eq. 1; "What carries the argument": Eq. 7);
* text queries attend to every key (the review's referee summary: text-token
  attention is kept global).

Everything is evaluated in float64 on the exact input values.

Modules
-------
attention  -- masked softmax attention by definition (full layer, or chosen rows)
tilemap    -- tile lists (runs of keys per query tile, chunk flags) by brute force
counts     -- lattice-point and admitted-pair counts by enumeration

Parity status: every function here has at least one pin in
``tests/test_oracle_pins.py`` / ``tests/test_oracle_tilemap.py``.
"""

from .attention import (  # noqa: F401
    clear_mask,
    attention_rows,
    attention_head,
    attention,
    in_window_pairs,
)
from .tilemap import tile_map_bruteforce  # noqa: F401
from .counts import lattice_count, pair_count, pair_count_bruteforce  # noqa: F401
