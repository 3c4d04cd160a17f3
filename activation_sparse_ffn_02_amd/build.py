"""Build libasf.so (HIP, gfx950) in-tree with hipcc: each source compiled to an
object in parallel, then linked.  The same kernel objects with the host API
compiled under ASF_DEBUG give libasf_debug.so, which checks the caller's
device content (list ids, counts, the neuron table) before use."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libasf.so")
LIB_DEBUG = os.path.join(HERE, "libasf_debug.so")
SOURCES = ["asf_api.hip", "asf_kernels.hip", "asf_batched.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _link(objs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking %s" % os.path.basename(out))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(HERE, "..", "include")]
    tmpdir = tempfile.mkdtemp(prefix="asf_build_")
    try:
        jobs = [(src, src.replace(".hip", ".o"), []) for src in SOURCES]
        jobs.append(("asf_api.hip", "asf_api_debug.o", ["-DASF_DEBUG"]))
        procs = []
        for src, obj, extra in jobs:
            cmd = [HIPCC] + FLAGS + extra + inc + ["-c", os.path.join(CSRC, src), "-o",
                                                   os.path.join(tmpdir, obj)]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                          text=True))
        failed = False
        for p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(out)
                failed = True
        if failed:
            raise RuntimeError("hipcc failed compiling libasf.so")
        objs = {obj: os.path.join(tmpdir, obj) for _, obj, _ in jobs}
        kernels = [objs["asf_kernels.o"], objs["asf_batched.o"]]
        _link([objs["asf_api.o"]] + kernels, LIB, verbose)
        _link([objs["asf_api_debug.o"]] + kernels, LIB_DEBUG, verbose)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
