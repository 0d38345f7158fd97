"""Plain CPU oracle for CLEAR circular-window attention (forward pass).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The library in ``dit_circular_local_amd``
never imports it, and this package imports nothing from the library: the two
share no code.

What it computes comes from the pages about CLEAR (arXiv 2412.16112):

* the attention mask of the pith.science review of the paper ("Core claim"),
  written here 0-based as M_ij = [i < n_text] or [j < n_text] or
  [dy_ij^2 + dx_ij^2 <= r2], with (dy, dx) the grid offset of two image tokens;
* plain softmax attention with 1/sqrt(c) logit scaling (the same review,
  "Assumptions & free parameters": Eq. 1; "What carries the argument": Eq. 7);
* text queries attend to every key (the review's referee summary: text-token
  attention is kept global);
* two variants the same pages discuss: the square window the circle is
  inscribed in ("What carries the argument": the circle costs about pi/4 of it),
  and the patch-averaged text rows of Eq. 7 used for multi-GPU patch-parallel
  inference;
* the gradients of that attention (dQ, dK, dV), the step that follows it in the
  paper's attention-only distillation fine-tuning, by the chain rule.

Everything is evaluated in float64 on the exact input values.

Modules
-------
attention  -- masked softmax attention by definition (full layer, or chosen rows)
backward   -- its gradients by the chain rule (full layer, chosen query rows or keys)
tilemap    -- tile lists (key tiles per query tile, sub-tile flags) by brute force
counts     -- lattice-point and admitted-pair counts by enumeration

Parity status: every exported function has at least one pin against values
the pages or plain mathematics fix (closed forms, library routines, brute
force, finite differences), in ``tests/test_oracle_pins.py`` (attention,
counts and the admitted-pair counter ``in_window_pairs``),
``tests/test_oracle_tilemap.py``, ``tests/test_oracle_square.py``,
``tests/test_oracle_strips.py`` or ``tests/test_oracle_backward.py``.
"""

from .attention import (  # noqa: F401
    WINDOWS,
    clear_mask,
    strip_rows,
    text_rows_patch_average,
    attention_rows,
    attention_head,
    attention,
    in_window_pairs,
)
from .backward import attention_backward, attention_backward_head, key_grads  # noqa: F401
from .tilemap import tile_map_bruteforce  # noqa: F401
from .counts import lattice_count, pair_count, pair_count_bruteforce  # noqa: F401
