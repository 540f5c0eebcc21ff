"""Build the gfx950 HIP library ``libattn.so`` in-tree with hipcc.

Usage: ``python -m exact_attention_64_amd.build`` (or ``build()`` from Python).
Always recompiles; the result lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libattn.so")
# The HBM read probe (include/attn_probe.h) the benchmark measures the read
# ceiling with; a library of its own, outside the attention boundary.
PROBE_LIB = os.path.join(HERE, "libattn_probe.so")
PROBE_SRC = "attn_probe.hip"

# (source, object name, extra flags).  The prefill kernels are compiled once per
# (input type, causal, paged cache) triple so that the eight sets build in parallel.
SOURCES = [("attn_api.cpp", "attn_api", []),
           *[("attn_fwd.hip", f"attn_fwd_t{t}_c{c}_p{g}",
              [f"-DATTN_FWD_DTYPE={t}", f"-DATTN_FWD_CAUSAL={c}", f"-DATTN_FWD_PAGED={g}"])
             for t in (0, 1) for c in (0, 1) for g in (0, 1)],
           ("attn_decode.hip", "attn_decode", []),
           ("attn_combine.hip", "attn_combine", []),
           ("attn_small.hip", "attn_small", []),
           ("attn_bwd.hip", "attn_bwd", [])]

# Packed fp32 VALU instructions are switched off for every HIP translation unit.
# MFMA accumulators are kept in VGPRs: the vector ALU works on the score tiles
# the matrix core produces, and AGPR-held scores would cost a copy per element
# (left to itself, the compiler also moved the backward's dK/dV accumulators
# between AGPRs and VGPRs on every step).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
VGPR_ACC_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link ``libattn.so`` (and the read probe
    ``libattn_probe.so``). Returns the path of ``libattn.so``."""
    cc = hipcc()
    objs = []
    procs = []
    for src, name, extra in [*SOURCES, (PROBE_SRC, "attn_probe", [])]:
        obj = os.path.join(HERE, "_build", name + ".o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [cc, *HIP_FLAGS, *VGPR_ACC_FLAGS, *extra, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-x")
            cmd.insert(2, "hip")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        keep = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if pr.returncode != 0:
            failed.append((src, "\n".join(keep)))
        elif verbose and keep:
            print("\n".join(keep))
    if failed:
        msg = "\n\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    probe_obj = objs.pop()
    for out, parts in ((LIB, objs), (PROBE_LIB, [probe_obj])):
        tmp = out + ".tmp"
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *parts, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
