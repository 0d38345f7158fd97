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


def test_cpu_baseline_workers_run_one_blas_thread_each(monkeypatch):
    # hosts may export BLAS / OpenMP thread counts equal to the core count; the
    # pool's workers must still run one thread each, and the parent's
    # environment must come back unchanged
    from dit_circular_local_amd.inputs import WORKLOADS

    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        monkeypatch.setenv(k, "16")
    r = bench.cpu_baseline(WORKLOADS["tiny"], 4, 0.5)
    assert r["blas_threads_per_worker"] == 1
    assert r["value"] > 0 and r["worker_processes"] >= 1 and r["kind"] == "oracle"
    assert " 0 block rows" not in r["sample"]
    import os
    assert all(os.environ[k] == "16" for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"))


def test_cpu_oracle_runs_report_whole_heads_and_samples():
    # a whole head where the budget allows it, a proportional sample where it
    # does not (every worker still runs at least one unit); pairs as counted by
    # the oracle's pair counter for exactly the rows that ran
    from dit_circular_local_amd.inputs import WORKLOADS

    tiny, part = bench.cpu_oracle_runs([("tiny", 4, 5.0), ("flux1k", 8, 1e-3)])
    assert tiny["whole_heads"] and tiny["value"] > 0
    n_workers = tiny["worker_processes"]
    w = WORKLOADS["tiny"]
    assert f"{bench.admitted_pairs(w.n_text, w.grid_h, w.grid_w, 16) * n_workers} admitted pairs" in tiny["sample"]
    assert not part["whole_heads"] and part["value"] > 0 and "proportional share" in part["sample"]


def test_oracle_units_cover_a_head_once_in_proportion():
    from dit_circular_local_amd.inputs import WORKLOADS

    w = WORKLOADS["flux1k"]
    for index in (0, 3):
        u = bench._oracle_units(w, index, 8)
        rows = [r for k, p in u if k == "text" for r in p]
        blocks = [b for k, p in u if k == "blocks" for b in p]
        assert sorted(rows) == list(range(w.n_text))
        assert sorted(blocks) == [(y, x) for y in range(w.grid_h // 8) for x in range(w.grid_w // 8)]
        # any prefix holds about the same share of text groups and block rows
        half = u[:len(u) // 2]
        nt = sum(k == "text" for k, _ in half) / sum(k == "text" for k, _ in u)
        nb = sum(k == "blocks" for k, _ in half) / sum(k == "blocks" for k, _ in u)
        assert abs(nt - nb) < 0.15


def test_committed_profiles_match_the_kernel_sources():
    # the forward figures bench.py reports beside its own timing come from
    # profiles taken on the current kernel sources and device flags; a kernel
    # change without new profiles fails here instead of dropping them silently
    for r in (32, 8):
        e = bench.load_profile("flux8k", r)
        assert e is not None, f"profiles/traffic.json has no entry for the current sources at r={r}"
        assert e["hbm_bytes_per_launch"] > 0 and 0 < e["mfma_busy"] < 1 and e["kernel_ms"] > 0


def test_profile_of_other_sources_is_not_used(tmp_path, monkeypatch):
    import json

    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(
        {"flux8k_r32": {"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 1.0}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_profile("flux8k", 32) is None
    assert bench.load_profile("flux8k", 8) is None
