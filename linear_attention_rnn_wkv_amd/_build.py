"""Build librwkv_wkv.so (the C-ABI library) and libstream_probe.so (the
bench's bandwidth reference) for gfx950 with hipcc.

Usage: python -m linear_attention_rnn_wkv_amd._build [--verbose]
The library is written next to this file; objects go to <repo>/_build/.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "librwkv_wkv.so")
SOURCES = ["rwkv_wkv_abi.hip", "rwkv4_scan.hip", "rwkv4_step.hip", "wkv_step.hip",
           "wkv_chunk.hip", "wkv_chunk_bwd.hip", "decay_lora.hip"]
# plain streaming kernels: the HBM bandwidth the bench measures against
PROBE_LIBRARY = os.path.join(PKG, "libstream_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]
# The RWKV-4 chain counts arrivals with one lane's returning atomic whose
# result is only needed at the end of the workgroup; the atomic optimizer
# would broadcast it at once and so wait for the round trip right there.
SOURCE_FLAGS = {"rwkv4_scan.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # no packed fp32 math (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        # the host pass does not know the packed-fp32 feature: drop that note
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(" ".join(cmd))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))


def _compile_link(sources, output, verbose):
    os.makedirs(OBJDIR, exist_ok=True)
    objs, cmds = [], []
    for src in sources:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    _run(cmds, verbose)
    tmp = output + ".tmp"
    _run([[HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]], verbose)
    os.replace(tmp, output)
    return output


def build(verbose: bool = False) -> str:
    """Compile every HIP source, link librwkv_wkv.so (the operators) and
    libstream_probe.so (the bench's bandwidth reference); returns the
    operator library's path."""
    _compile_link(SOURCES, LIBRARY, verbose)
    _compile_link(PROBE_SOURCES, PROBE_LIBRARY, verbose)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
