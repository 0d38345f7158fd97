"""The window-box reference used for grids too large for the host: on grids the
oracle handles whole, it must give the oracle's rows of the full problem."""

import numpy as np
import pytest
import torch

from oracle import attention_rows
from window_box import box_reference


@pytest.mark.parametrize("window", ["circle", "square"])
@pytest.mark.parametrize("n_text,gh,gw,r2", [(3, 23, 17, 9), (0, 12, 30, 20), (5, 9, 9, 200), (2, 31, 7, 0)])
def test_box_rows_equal_full_problem_rows(n_text, gh, gw, r2, window):
    g = torch.Generator().manual_seed(gh * 100 + gw)
    n = n_text + gh * gw
    q, k, v = (torch.randn(n, 16, generator=g, dtype=torch.float64) for _ in range(3))
    cells = [(0, 0), (gh - 1, gw - 1), (0, gw - 1), (gh - 1, 0), (gh // 2, gw // 2), (1, gw - 2), (gh - 2, 1)]
    rows, ref = box_reference(q, k, v, n_text, gh, gw, r2, cells, window=window)
    full, _ = attention_rows(q.numpy(), k.numpy(), v.numpy(), n_text, gh, gw, r2, rows, window=window)
    np.testing.assert_allclose(ref, full, rtol=0, atol=1e-12)
