"""bench.py's in-window pair count (its FLOP numerator) against the oracle's counts."""

import pytest

import bench
from oracle import pair_count, pair_count_bruteforce


@pytest.mark.parametrize("n_text,gh,gw,r2", [(512, 512, 512, 64), (512, 512, 512, 1024), (512, 64, 64, 256),
                                             (512, 128, 128, 1024), (7, 9, 13, 5), (0, 5, 5, 100), (3, 4, 6, -1)])
def test_admitted_pairs_match_oracle(n_text, gh, gw, r2):
    assert bench.admitted_pairs(n_text, gh, gw, r2) == pair_count(n_text, gh, gw, r2)["total"]


def test_admitted_pairs_small_bruteforce():
    for args in [(2, 7, 5, 8), (0, 6, 6, 2), (4, 3, 11, 13)]:
        assert bench.admitted_pairs(*args) == pair_count_bruteforce(*args)


def test_flux_8192_flop_counts():
    # 4 * d * pairs * heads: 3.928 / 13.097 TFLOP per layer at r = 8 / 32
    f8 = 4 * 128 * bench.admitted_pairs(512, 512, 512, 64) * 24
    f32 = 4 * 128 * bench.admitted_pairs(512, 512, 512, 1024) * 24
    assert round(f8 / 1e12, 3) == 3.928
    assert round(f32 / 1e12, 3) == 13.097


@pytest.mark.parametrize("n_text,gh,gw,r2", [(512, 512, 512, 1024), (512, 64, 64, 256), (7, 9, 13, 5),
                                             (0, 5, 5, 100), (3, 4, 6, -1)])
def test_square_admitted_pairs_match_oracle(n_text, gh, gw, r2):
    assert bench.admitted_pairs(n_text, gh, gw, r2, "square") == \
        pair_count(n_text, gh, gw, r2, "square")["total"]
    if (n_text + gh * gw) <= 200:
        assert bench.admitted_pairs(n_text, gh, gw, r2, "square") == \
            pair_count_bruteforce(n_text, gh, gw, r2, "square")


@pytest.mark.parametrize("window", ["circle", "square"])
@pytest.mark.parametrize("n_text,gh,gw,r2", [(512, 64, 64, 256), (7, 9, 13, 5), (0, 19, 13, 9), (40, 4, 4, 0)])
def test_computed_work_covers_every_admitted_pair(n_text, gh, gw, r2, window):
    """The kernels' chunk count (tile waste included) never falls below the
    admitted pairs: every admitted pair lies in a chunk its wavefront computes."""
    import dit_circular_local_amd as ca

    assert bench.computed_pairs(ca, n_text, gh, gw, r2, window) >= bench.admitted_pairs(n_text, gh, gw, r2, window)
