"""The rocprofv3 harness's reduction (dit_circular_local_amd.profiling) on
hand-made CSV files shaped like the profiler's, without a GPU: kernel-name
parsing, per-dispatch counter sums, the derived matrix-core share, shader
clock and calibrated byte counts."""

import csv
import json
import os

from dit_circular_local_amd import profiling as P

KNAME = ("void clear::(anonymous namespace)::clear_attn_fwd_kernel<clear::(anonymous namespace)::Bf16G>"
         "(clear::(anonymous namespace)::Params)")


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _counter_rows(disp, kname, values):
    # the profiler reports some counters per XCD/SE instance: several rows per counter
    rows = []
    for c, v in values.items():
        parts = v if isinstance(v, list) else [v]
        rows += [[disp, disp, "Agent 1", 1, 1, 1, 1, 1, kname, 256, 0, 0, 0, 0, 0, c, float(x), 0, 1]
                 for x in parts]
    return rows


CHEAD = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
         "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
         "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def test_kernel_name_drops_only_the_argument_list():
    assert P._short(KNAME) == ("void clear::(anonymous namespace)::clear_attn_fwd_kernel"
                               "<clear::(anonymous namespace)::Bf16G>")
    assert P._short("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_summary_figures(tmp_path):
    root = str(tmp_path)
    # trace: the first dispatch (tile-map build) is skipped; the others last 10 and 12 ms
    th = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
          "Correlation_Id", "Start_Timestamp", "End_Timestamp"]
    _write(os.path.join(root, "trace", "trace_kernel_trace.csv"), th,
           [["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, i, 1, KNAME, i, 0, dur]
            for i, dur in enumerate([30e6, 10e6, 12e6])])
    # SIMD cycles per dispatch = GRBM_GUI_ACTIVE / 8 * 1024; GUI = 8 * 2e7 -> 2.048e10 SIMD cycles
    sq = {"GRBM_GUI_ACTIVE": 8 * 2.0e7, "SQ_VALU_MFMA_BUSY_CYCLES": [0.5e10, 0.524e10],
          "SQ_ACTIVE_INST_VALU": 1.024e9, "SQ_VALU_MFMA_COEXEC_CYCLES": 2.048e9, "SQ_INSTS_MFMA": 1.6e8,
          "SQ_INSTS_VALU": 8.0e8}
    _write(os.path.join(root, "sq", "sq_counter_collection.csv"), CHEAD,
           sum((_counter_rows(d, KNAME, sq) for d in (1, 2, 3)), []))
    _write(os.path.join(root, "fetch", "fetch_counter_collection.csv"), CHEAD,
           sum((_counter_rows(d, KNAME, {"FETCH_SIZE": 1000.0}) for d in (1, 2, 3)), []))
    _write(os.path.join(root, "write", "write_counter_collection.csv"), CHEAD,
           sum((_counter_rows(d, KNAME, {"WRITE_SIZE": 300.0}) for d in (1, 2, 3)), []))
    # calibration: a 1 MiB copy reads FETCH 512 KiB and WRITE 1024 KiB
    _write(os.path.join(root, "copy_fetch", "copy_fetch_counter_collection.csv"), CHEAD,
           _counter_rows(1, "__amd_rocclr_copyBuffer", {"FETCH_SIZE": 512.0}))
    _write(os.path.join(root, "copy_write", "copy_write_counter_collection.csv"), CHEAD,
           _counter_rows(1, "__amd_rocclr_copyBuffer", {"WRITE_SIZE": 1024.0}))
    with open(os.path.join(root, "copy_fetch.cmd"), "w") as f:
        f.write("rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --copy-probe-mib 1\n")
    res = P.summarize(root, "clear_attn_fwd_kernel", flop=2.2e13, alg_bytes=1.0e6, skip_first=1)
    d = res["derived"]
    assert abs(res["trace"]["mean_ms"] - 11.0) < 1e-9
    assert abs(d["mfma_busy"] - 1.024e10 / 2.048e10) < 1e-12          # instance rows summed per dispatch
    assert abs(d["valu_active"] - 4 * 1.024e9 / 2.048e10) < 1e-12
    assert abs(d["shader_clock_ghz"] - 2.0e7 / 11e-3 / 1e9) < 1e-9
    assert abs(d["fetch_scale"] - 2.0) < 1e-12 and abs(d["write_scale"] - 1.0) < 1e-12
    assert d["bytes"] == (1000.0 * 2.0 + 300.0) * 1024
    assert abs(d["achieved_tflops"] - 2.2e13 / 11e-3 / 1e12) < 1e-9
    assert abs(d["per_16_mfma"]["SQ_INSTS_VALU"] - 80.0) < 1e-12
    md = P.markdown(res, "t")
    assert "mfma_busy" in md and "FETCH_SIZE" in md
    rec = os.path.join(root, "rec.json")
    P.record(rec, "flux8k_r32", res, "x.md")
    e = json.load(open(rec))["flux8k_r32"]
    assert e["hbm_bytes_per_launch"] == d["bytes"] and e["kernel_ms"] == res["trace"]["mean_ms"]


def test_pass_commands_put_the_program_after_the_separator():
    c = P.rocprof_command("sq", "/x/sq", ["python3", "bench.py", "--steps", "2"])
    assert c[:2] == ["rocprofv3", "--output-format"] and c[c.index("--") + 1:] == ["python3", "bench.py", "--steps", "2"]
    assert "--pmc" in c and "--kernel-trace" not in c and "-s" not in c
    t = P.rocprof_command("trace", "/x/t", ["python3", "bench.py"])
    assert "--kernel-trace" in t and "--pmc" not in t
    # each counter pass stays within the per-block limits of one profiler run
    for name, cs in P.PASSES.items():
        sq = [c for c in cs if c.startswith("SQ_")]
        grbm = [c for c in cs if c.startswith("GRBM_")]
        assert len(sq) <= 8 and len(grbm) <= 2, name


def test_one_summary_for_several_kernels_of_a_run(tmp_path):
    root = str(tmp_path)
    ka = "void clear::(anonymous namespace)::clear_attn_bwd_dkdv_kernel<X>(P)"
    kb = "void clear::(anonymous namespace)::clear_attn_bwd_dq_kernel<X>(P)"
    th = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
          "Correlation_Id", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for i in range(3):
        rows.append(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, 2 * i, 1, ka, 2 * i, 0, 30e6])
        rows.append(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, 2 * i + 1, 2, kb, 2 * i + 1, 0, 20e6])
    _write(os.path.join(root, "trace", "trace_kernel_trace.csv"), th, rows)
    recs = [P.summarize(root, k, flop=None, alg_bytes=None) for k in ("bwd_dkdv", "bwd_dq")]
    assert abs(recs[0]["trace"]["mean_ms"] - 30.0) < 1e-9 and abs(recs[1]["trace"]["mean_ms"] - 20.0) < 1e-9
    md = P.markdown(recs, "t", "note")
    assert md.count("## ") == 2 and "All kernels of the run" in md and "note" in md
    assert md.index("## bwd_dkdv") < md.index("## bwd_dq")
