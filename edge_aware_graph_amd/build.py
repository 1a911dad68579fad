"""Build the gfx950 HIP library in-tree: edge_aware_graph_amd/libedge_attn.so."""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libedge_attn.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("ea_kernels.hip", "ea_block.hip", "ea_generic.hip", "ea_probe.hip", "ea_api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are disabled: only scalar fp32 VALU and MFMA are used.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def scratch_users(remarks: str):
    """Kernels whose resource-usage remarks report scratch (private) memory."""
    users, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            users.append((name, int(m.group(1))))
    return users


def missing_stubs(lib_path: str):
    """Kernel launch stubs the library references but does not define (the
    host pass can drop a kernel's stub without an error when a device builtin
    in its body does not type-check for the host); such a library fails to
    load with an undefined symbol."""
    res = subprocess.run(["nm", "-u", lib_path], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("nm failed on %s: %s" % (lib_path, res.stderr))
    return [line.split()[-1] for line in res.stdout.splitlines() if "__device_stub__" in line]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP source into the shared library (always rebuilds).

    Every kernel must run without scratch memory: register spills are a
    performance cliff here, and spill code has been seen to reload a
    spilled fragment incompletely. The build fails if any kernel spills.
    """
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage"] + list(extra) + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB)
    spills = scratch_users(res.stderr)
    if spills:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch memory: %s" % ", ".join("%s (%d B/lane)" % s for s in spills))
    stubs = missing_stubs(tmp)
    if stubs:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the library: %s" % ", ".join(stubs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
