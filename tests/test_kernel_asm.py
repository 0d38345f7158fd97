"""Structural checks on the gfx950 assembly of the attention kernels, compiled
here with the build's own flags.

The chunk walk's two LDS stages are filled by direct-to-LDS copies, which are
vector-memory loads: the compiler orders them at most against the same
wavefront's own LDS reads (and the d = 128 bf16 forward issues them in
assembly, out of the compiler's sight).  Other wavefronts may read a stage
only after every wavefront's copies into it have landed, so every barrier of
the walk must come after a wait for all of the wavefront's vector-memory
operations (vmcnt(0)) in the same basic block.  Without that wait the kernels'
results depended on the instruction schedule (a wavefront could pass the
barrier with its last copy in flight).  The assembly copies of the d = 128
bf16 forward come in groups of four per staged chunk (two copy blocks of K,
two of V)."""

import os
import re
import subprocess

import pytest

from dit_circular_local_amd import build as B

KERNELS = {"attn_fwd.hip": r"clear_attn_fwd_kernel", "attn_bwd.hip": r"clear_attn_bwd_(dkdv|dq)_kernel"}

# copies per wavefront and chunk of the d = 128 bf16 forward (K and V, two
# copy blocks each), issued in assembly
BF16_FWD_COPIES = {"Bf16G": 4}


def _allowed_vmcnt(name):
    for tag, n in BF16_FWD_COPIES.items():
        if "clear_attn_fwd_kernel" in name and tag in name:
            return {0}, n
    return {0}, None


def _device_asm(src, tmp_path):
    out = os.path.join(tmp_path, os.path.basename(src) + ".s")
    cmd = [B.HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S", *B.DEVICE_FLAGS,
           "-I", B.INCLUDE, "-I", B.CSRC, os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().split("\n")


def _functions(lines, name_re):
    """(name, body lines) of every kernel whose mangled name matches name_re."""
    out, cur, body = [], None, []
    for l in lines:
        m = re.match(r"^(_Z\S+):", l)
        if m:
            cur, body = (m.group(1) if re.search(name_re, m.group(1)) else None), []
            continue
        if cur and l.startswith(".Lfunc_end"):
            out.append((cur, body))
            cur = None
        elif cur:
            body.append(l)
    return out


@pytest.mark.parametrize("src", sorted(KERNELS))
def test_every_walk_barrier_waits_for_the_wavefronts_copies(src, tmp_path):
    funcs = _functions(_device_asm(src, str(tmp_path)), KERNELS[src])
    assert funcs, f"no attention kernel found in {src}"
    barriers = 0
    for name, body in funcs:
        allowed, group = _allowed_vmcnt(name)
        code = [l.split(";")[0].strip() for l in body]
        for i, ins in enumerate(code):
            if not ins.startswith("s_barrier"):
                continue
            barriers += 1
            got = None
            for prev in reversed(code[:i]):
                if not prev:
                    continue
                if prev.endswith(":"):  # block boundary: the wait must sit in the barrier's own block
                    break
                if prev.startswith(("buffer_", "global_")):
                    break
                if prev.startswith("s_waitcnt"):
                    m = re.search(r"vmcnt\((\d+)\)", prev)
                    got = int(m.group(1)) if m else None
                    break
            assert got in allowed, f"{name}: barrier #{barriers} waits vmcnt({got}), allowed {sorted(allowed)}"
        if group is not None:
            # the assembly copies come in groups of exactly `group` per staged chunk
            copies = [i for i, ins in enumerate(code) if ins.startswith("buffer_load_dwordx4") and ins.endswith("lds")]
            assert copies and len(copies) % group == 0, f"{name}: {len(copies)} copies"
    assert barriers > 0
