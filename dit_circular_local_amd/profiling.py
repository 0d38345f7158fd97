"""rocprofv3 harness: kernel times, matrix-core utilisation and memory traffic
of the CLEAR attention kernels against the MI355X (gfx950) peaks.

This module never touches the GPU itself.  ``collect`` starts ``rocprofv3`` as
a child process around a command (normally ``python3 bench.py ...``), one pass
per counter set, because the profiler does not split counters over passes;
``summarize`` reduces the CSV files the passes wrote to per-kernel figures and
writes a Markdown summary plus a JSON record.  Run ``collect`` on the machine with the GPU
and ``summarize`` anywhere.

    python -m dit_circular_local_amd.profiling collect --out prof/fwd8k -- \\
        python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline ...
    python -m dit_circular_local_amd.profiling summarize prof/fwd8k \\
        --kernel clear_attn_fwd_kernel --flop 1.3097e13 --bytes 6.455e9 --md profiles/x.md

Passes (each its own profiler run):

* ``trace``   -- ``--kernel-trace --stats``: every dispatch's duration;
* ``sq``      -- SQ counters: MFMA busy cycles, VALU / MFMA co-execution,
                 instruction mix, wave cycles, GRBM_GUI_ACTIVE (shader clock);
* ``fetch`` / ``write`` -- FETCH_SIZE, then WRITE_SIZE (L2-to-fabric KiB per
                 dispatch);
* ``copy_fetch`` / ``copy_write`` -- the same two counters for a plain device
                 copy of known size (``bench.py --copy-probe-mib``), which
                 calibrates them into bytes.

Derived figures (per dispatch of the named kernel, averaged over its
dispatches):

* SIMD cycles = GRBM_GUI_ACTIVE / XCDs x SIMDs (GRBM_GUI_ACTIVE sums the
  active cycles of the 8 XCDs' graphics blocks);
* MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD cycles (the counter already
  weights each MFMA by its cycles);
* VALU active = 4 x SQ_ACTIVE_INST_VALU / SIMD cycles (quad-cycle units);
* co-execution = SQ_VALU_MFMA_COEXEC_CYCLES / SIMD cycles;
* running shader clock = GRBM_GUI_ACTIVE / XCDs / kernel duration;
* bytes = FETCH_SIZE x f_fetch + WRITE_SIZE x f_write (KiB x 1024), with the
  factors that make the copy's readings equal its size; GB/s = bytes / the
  kernel's mean duration from the trace pass.
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shlex
import subprocess
import sys
from collections import defaultdict
from typing import Dict, List, Optional

# MI355X (gfx950): 256 compute units in 8 XCDs, 4 SIMDs per CU, 2.4 GHz peak
# engine clock; dense bf16 matrix-core peak 256 x 2.4e9 x 4096 flop/clk; HBM3E
# 8 TB/s.
N_CU = 256
N_XCD = 8
SIMD_PER_CU = 4
PEAK_CLOCK_HZ = 2.4e9
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0

# Each set fits the per-block hardware limits of one pass (at most 8 SQ, 4 TCC
# and 2 GRBM counters; FETCH_SIZE takes 3 TCC counters, WRITE_SIZE 2).
PASSES = {
    "sq": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
           "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE"],
    "sq2": ["SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAIT_INST_ANY", "SQ_INSTS_VMEM_RD",
            "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_BRANCH", "SQ_INSTS_SMEM"],
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
}


def rocprof_command(kind: str, out_dir: str, cmd: List[str]) -> List[str]:
    """The rocprofv3 command line of one pass (the program goes after --)."""
    base = ["rocprofv3", "--output-format", "csv", "-d", out_dir, "-o", kind]
    if kind == "trace":
        return base + ["--kernel-trace", "--stats", "--"] + cmd
    counters = PASSES[kind.replace("copy_", "")]
    return base + ["--pmc", *counters, "--"] + cmd


def collect(out: str, cmd: List[str], passes: List[str], copy_cmd: Optional[List[str]],
            timeout_s: int) -> int:
    """Run each pass as a child process (from /tmp, where the profiler keeps its
    scratch files; ``out`` is made absolute first).  Stops at the first failing
    pass."""
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ)
    env.setdefault("TMPDIR", "/tmp")
    todo = [(p, cmd) for p in passes]
    if copy_cmd:
        todo += [("copy_fetch", copy_cmd), ("copy_write", copy_cmd)]
    for kind, c in todo:
        full = ["timeout", "-s", "KILL", str(timeout_s)] + rocprof_command(kind, os.path.join(out, kind), c)
        print("pass", kind, ":", " ".join(shlex.quote(x) for x in full), flush=True)
        with open(os.path.join(out, f"{kind}.cmd"), "w") as f:
            f.write(" ".join(shlex.quote(x) for x in rocprof_command(kind, os.path.join(out, kind), c)) + "\n")
        r = subprocess.run(full, env=env, cwd="/tmp")
        # the profiler itself may end with SIGSEGV after a complete run (cooperative
        # launches); the pass is kept when its CSV files are there
        if r.returncode != 0 and not _csvs(os.path.join(out, kind)):
            print(f"pass {kind} failed with exit code {r.returncode}", flush=True)
            return r.returncode
        print(f"pass {kind} done (exit {r.returncode})", flush=True)
    return 0


def _csvs(d: str) -> List[str]:
    return sorted(glob.glob(os.path.join(d, "**", "*.csv"), recursive=True))


def _rows(d: str, suffix: str):
    for p in _csvs(d):
        if p.endswith(suffix):
            with open(p, newline="") as f:
                yield from csv.DictReader(f)


def _short(name: str) -> str:
    """Kernel name without its final (argument list) group; demangled names
    hold other parentheses, e.g. "(anonymous namespace)"."""
    name = name.strip()
    if not name.endswith(")"):
        return name
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        depth += {")": 1, "(": -1}.get(name[i], 0)
        if depth == 0:
            return name[:i].strip()
    return name


def kernel_durations(d: str) -> Dict[str, List[float]]:
    """Dispatch durations (ns) per kernel from a kernel-trace pass, in order."""
    out: Dict[str, List[float]] = defaultdict(list)
    for r in _rows(d, "kernel_trace.csv"):
        out[_short(r["Kernel_Name"])].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return out


def counters(d: str) -> Dict[str, Dict[str, List[float]]]:
    """Counter values per kernel and counter, one entry per dispatch."""
    per: Dict[tuple, Dict[str, float]] = defaultdict(dict)
    names: Dict[tuple, str] = {}
    for r in _rows(d, "counter_collection.csv"):
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), _short(r["Kernel_Name"]))
        names[key] = key[1]
        per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out: Dict[str, Dict[str, List[float]]] = defaultdict(lambda: defaultdict(list))
    for key in sorted(per, key=lambda k: int(k[0]) if str(k[0]).isdigit() else 0):
        for c, v in per[key].items():
            out[names[key]][c].append(v)
    return out


def _match(d: Dict[str, object], kernel: str) -> List[str]:
    return [k for k in d if kernel in k]


def _mean(x: List[float]) -> float:
    return sum(x) / len(x) if x else float("nan")


def summarize(root: str, kernel: str, flop: Optional[float], alg_bytes: Optional[float],
              skip_first: int = 1) -> dict:
    """Per-kernel figures from the passes under ``root`` (see the module doc).
    ``skip_first`` dispatches of the kernel (tile-map build, warm-up) are left
    out of the averages."""
    res: dict = {"kernel": kernel, "root": root}
    tr = kernel_durations(os.path.join(root, "trace"))
    ks = _match(tr, kernel)
    if ks:
        ns = [x for k in ks for x in tr[k]]
        timed = ns[skip_first:] or ns
        res["trace"] = {"dispatches": len(ns), "mean_ms": _mean(timed) / 1e6, "min_ms": min(timed) / 1e6,
                        "max_ms": max(timed) / 1e6, "names": ks}
        res["kernels"] = {k: {"dispatches": len(v), "mean_ms": _mean(v) / 1e6} for k, v in tr.items()}
    ms = res.get("trace", {}).get("mean_ms")
    cnt: Dict[str, float] = {}
    for p in ("sq", "sq2", "fetch", "write"):
        c = counters(os.path.join(root, p))
        for k in _match(c, kernel):
            for name, vals in c[k].items():
                cnt[name] = _mean(vals[skip_first:] or vals)
    res["counters"] = cnt
    der: dict = {}
    if "GRBM_GUI_ACTIVE" in cnt:
        simd_cycles = cnt["GRBM_GUI_ACTIVE"] / N_XCD * N_CU * SIMD_PER_CU
        der["simd_cycles"] = simd_cycles
        if "SQ_VALU_MFMA_BUSY_CYCLES" in cnt:
            der["mfma_busy"] = cnt["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles
        if "SQ_ACTIVE_INST_VALU" in cnt:
            der["valu_active"] = 4.0 * cnt["SQ_ACTIVE_INST_VALU"] / simd_cycles
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in cnt:
            der["valu_mfma_coexec"] = cnt["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles
        if ms:
            der["shader_clock_ghz"] = cnt["GRBM_GUI_ACTIVE"] / N_XCD / (ms * 1e-3) / 1e9
    if "SQ_INSTS_MFMA" in cnt and cnt["SQ_INSTS_MFMA"] > 0:
        chunks = cnt["SQ_INSTS_MFMA"] / 16.0
        der["per_16_mfma"] = {c: cnt[c] / chunks for c in cnt if c.startswith("SQ_INSTS_")}
    cal = {}
    for p, counter in (("copy_fetch", "FETCH_SIZE"), ("copy_write", "WRITE_SIZE")):
        c = counters(os.path.join(root, p))
        vals = [v for k in c for v in c[k].get(counter, []) if "copy" in k.lower()]
        if vals:
            cal[counter] = _mean(vals)
    res["copy_readings_kib"] = cal
    if "FETCH_SIZE" in cnt and "WRITE_SIZE" in cnt and cal.get("FETCH_SIZE") and cal.get("WRITE_SIZE"):
        copy_kib = res.get("copy_kib")
        if copy_kib is None:
            copy_kib = _copy_kib(root)
        if copy_kib:
            ff = copy_kib / cal["FETCH_SIZE"]
            fw = copy_kib / cal["WRITE_SIZE"]
            rd = cnt["FETCH_SIZE"] * ff * 1024
            wr = cnt["WRITE_SIZE"] * fw * 1024
            der["fetch_scale"], der["write_scale"] = ff, fw
            der["read_bytes"], der["write_bytes"], der["bytes"] = rd, wr, rd + wr
            if ms:
                der["fabric_gbs"] = (rd + wr) / (ms * 1e-3) / 1e9
                der["fabric_frac_of_hbm_peak"] = der["fabric_gbs"] / PEAK_HBM_GBS
            if alg_bytes:
                der["bytes_over_algorithmic"] = (rd + wr) / alg_bytes
    if ms and flop:
        der["achieved_tflops"] = flop / (ms * 1e-3) / 1e12
        der["frac_of_bf16_peak"] = der["achieved_tflops"] / PEAK_BF16_TFLOPS
    if ms and alg_bytes:
        der["algorithmic_gbs"] = alg_bytes / (ms * 1e-3) / 1e9
    res["derived"] = der
    return res


def _copy_kib(root: str) -> Optional[float]:
    """Size of the calibration copy, from the recorded command (--copy-probe-mib N)."""
    p = os.path.join(root, "copy_fetch.cmd")
    if not os.path.exists(p):
        return None
    parts = open(p).read().split()
    if "--copy-probe-mib" in parts:
        return float(parts[parts.index("--copy-probe-mib") + 1]) * 1024.0
    return None


def _repo_relative(cmd: str) -> str:
    """A recorded command with the checkout's absolute path written as $REPO."""
    import re

    return re.sub(r"/\S*?/repo(?=/)", "$REPO", cmd)


def markdown(res, title: str, note: Optional[str] = None, summary_cmd: Optional[str] = None) -> str:
    """A short Markdown summary of ``summarize``'s record, or of several
    records of one run (one section per kernel); ``summary_cmd`` is the
    command that wrote it."""
    recs = [res] if isinstance(res, dict) else list(res)
    lines = [f"# {title}", ""]
    if note:
        lines += [note, ""]
    if summary_cmd:
        lines += [f"Summary written by `{_repo_relative(summary_cmd)}` from the CSV files of the passes below.", ""]
    lines += ["Commands (each pass its own profiler run, from /tmp; `$REPO` is the repository root):", ""]
    for p in ("trace", "sq", "sq2", "fetch", "write", "copy_fetch", "copy_write"):
        cmdf = os.path.join(recs[0]["root"], f"{p}.cmd")
        if os.path.exists(cmdf):
            lines.append(f"- `{p}`: `{_repo_relative(open(cmdf).read().strip())}`")
    lines.append("")
    if recs[0].get("kernels"):
        lines += ["All kernels of the run:", "", "| kernel | dispatches | mean ms |", "|---|---|---|"]
        for k, v in sorted(recs[0]["kernels"].items(), key=lambda kv: -kv[1]["mean_ms"] * kv[1]["dispatches"]):
            lines.append(f"| `{k[:90]}` | {v['dispatches']} | {v['mean_ms']:.4f} |")
        lines.append("")
    for rec in recs:
        if len(recs) > 1:
            lines += [f"## {rec['kernel']}", ""]
        t = rec.get("trace")
        if t:
            lines += ["| kernel | dispatches | mean ms (timed) | min ms | max ms |", "|---|---|---|---|---|",
                      f"| {rec['kernel']} | {t['dispatches']} | {t['mean_ms']:.4f} | {t['min_ms']:.4f} | "
                      f"{t['max_ms']:.4f} |", ""]
        if rec["counters"]:
            lines += ["| counter | per dispatch |", "|---|---|"]
            lines += [f"| {k} | {v:.4g} |" for k, v in sorted(rec["counters"].items())]
            lines.append("")
        d = rec["derived"]
        if d:
            lines += ["| derived | value |", "|---|---|"]
            for k, v in d.items():
                if isinstance(v, dict):
                    for kk, vv in v.items():
                        lines.append(f"| {k}.{kk} | {vv:.4g} |")
                else:
                    lines.append(f"| {k} | {v:.4g} |")
            lines.append("")
    return "\n".join(lines)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect", help="run rocprofv3 passes around a command (on the machine with the GPU)")
    c.add_argument("--out", required=True)
    c.add_argument("--passes", default="trace,sq,sq2,fetch,write")
    c.add_argument("--copy-mib", type=int, default=1024,
                   help="calibration copy size for FETCH_SIZE/WRITE_SIZE (0: none)")
    c.add_argument("--timeout", type=int, default=240, help="seconds per pass")
    c.add_argument("command", nargs=argparse.REMAINDER)
    s = sub.add_parser("summarize", help="reduce collected CSVs (anywhere)")
    s.add_argument("root")
    s.add_argument("--kernel", action="append", default=None,
                   help="kernel name (substring); repeat for several kernels of one run "
                        "(default clear_attn_fwd_kernel)")
    s.add_argument("--flop", type=float, action="append", default=None,
                   help="algorithmic flops per dispatch (one per --kernel)")
    s.add_argument("--bytes", type=float, action="append", default=None,
                   help="algorithmic bytes per dispatch (one per --kernel)")
    s.add_argument("--skip-first", type=int, default=1)
    s.add_argument("--md", default=None)
    s.add_argument("--json", default=None)
    s.add_argument("--title", default="rocprofv3 summary")
    s.add_argument("--note", default=None, help="text placed under the title")
    s.add_argument("--record", default=None, help="JSON file to add this run's figures to (profiles/traffic.json)")
    s.add_argument("--key", default=None, help="entry name in --record, e.g. flux8k_r32")
    s.add_argument("--source", default=None, help="name of the Markdown summary the entry refers to")
    a = ap.parse_args(argv)
    if a.cmd == "collect":
        cmd = a.command[1:] if a.command and a.command[0] == "--" else a.command
        if not cmd:
            ap.error("give the command to profile after --")
        copy_cmd = None
        if a.copy_mib > 0:
            bench = [x for x in cmd if x.endswith("bench.py")]
            if bench:
                copy_cmd = [cmd[0], bench[0], "--copy-probe-mib", str(a.copy_mib)]
        passes = [p for p in a.passes.split(",") if p]
        return collect(a.out, cmd, passes, copy_cmd, a.timeout)
    kernels = a.kernel or ["clear_attn_fwd_kernel"]
    flops = a.flop or [None] * len(kernels)
    nbytes = a.bytes or [None] * len(kernels)
    if len(flops) != len(kernels) or len(nbytes) != len(kernels):
        ap.error("give --flop and --bytes once per --kernel (or not at all)")
    recs = [summarize(a.root, k, f, b, a.skip_first) for k, f, b in zip(kernels, flops, nbytes)]
    if a.record and len(recs) != 1:
        ap.error("--record takes one kernel")
    res = recs[0] if len(recs) == 1 else recs
    # the command line, with the title and note texts elided
    shown, skip = [], False
    for x in (argv if argv is not None else sys.argv[1:]):
        if skip:
            shown.append("...")
            skip = False
            continue
        shown.append(x)
        skip = x in ("--title", "--note")
    md = markdown(res, a.title, a.note, "python -m dit_circular_local_amd.profiling " + shlex.join(shown))
    if a.md:
        with open(a.md, "w") as f:
            f.write(md + "\n")
    else:
        print(md)
    if a.json:
        with open(a.json, "w") as f:
            json.dump(res, f, indent=1)
    if a.record:
        record(a.record, a.key, res, a.source)
    return 0


def record(path: str, key: str, res: dict, source: Optional[str]) -> None:
    """Add the figures bench.py reads (keyed by the forward kernel's source
    hash) to a JSON file, as entry `key`."""
    from dit_circular_local_amd.build import kernel_source_hash

    d = res["derived"]
    entry = {
        "kernel_source_hash": kernel_source_hash(),
        "kernel": res["kernel"],
        "kernel_ms": res.get("trace", {}).get("mean_ms"),
        "hbm_bytes_per_launch": d.get("bytes"),
        "read_bytes": d.get("read_bytes"),
        "write_bytes": d.get("write_bytes"),
        "fetch_scale": d.get("fetch_scale"),
        "write_scale": d.get("write_scale"),
        "mfma_busy": d.get("mfma_busy"),
        "valu_active": d.get("valu_active"),
        "valu_mfma_coexec": d.get("valu_mfma_coexec"),
        "shader_clock_ghz": d.get("shader_clock_ghz"),
        "source": source,
    }
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[key] = entry
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    sys.exit(main())
