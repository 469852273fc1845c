"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

Every .hip source under csrc/ is compiled to an object in parallel, then
linked into gated_deltanet_layer_causal_amd/libgdn.so.  Packed-fp32 VALU
instructions are disabled for all device code.

The build fails if any kernel uses scratch memory (register spills or
stack): the sequential chunk kernels count their outstanding memory
operations by hand (s_waitcnt vmcnt(N)), and a spill would add memory
operations that the count does not know about.  The compiler's per-kernel
resource report is kept in _build/resources.txt.

A digest of the sources (csrc/ and include/) is written beside the library
(libgdn.so.sources); capi.load() refuses a library whose digest does not
match the sources in the tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
DIGEST = LIB + ".sources"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-variable",
    "-Wno-unused-but-set-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
    # MFMA results and accumulators in ordinary VGPRs: the sequential passes
    # keep their state in accumulators and scale it every chunk, which with
    # AGPRs costs a read and a write per element around each multiply
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def source_digest() -> str:
    """sha256 over every file of csrc/ and include/ (names and contents)."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for f in sorted(os.listdir(d)):
            p = os.path.join(d, f)
            if os.path.isfile(p) and f.endswith((".hip", ".h")):
                h.update(f.encode())
                with open(p, "rb") as fh:
                    h.update(fh.read())
    return h.hexdigest()


_FN = re.compile(r"remark: Function Name: (\S+)")
_KV = re.compile(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\d+)")


def resource_report(stderr: str):
    """[(kernel, {field: value})] from hipcc's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in stderr.splitlines():
        m = _FN.search(line)
        if m:
            cur = (m.group(1), {})
            out.append(cur)
            continue
        m = _KV.search(line)
        if m and cur is not None:
            cur[1][m.group(1).strip()] = int(m.group(2))
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, resource_report(r.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libgdn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    lines, spills = [], []
    for src, (_, rep) in zip(srcs, results):
        for name, kv in rep:
            lines.append(f"{os.path.basename(src)} {name} " +
                         " ".join(f"{k.replace(' ', '_')}={v}" for k, v in kv.items()))
            if kv.get("ScratchSize [bytes/lane]", 0) > 0:
                spills.append(f"{name} ({os.path.basename(src)}): "
                              f"{kv['ScratchSize [bytes/lane]']} bytes/lane of scratch")
    with open(os.path.join(BUILD, "resources.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if spills:
        raise RuntimeError("kernels use scratch memory (spills), which the hand-counted memory "
                           "waits of the chunk kernels do not allow:\n  " + "\n  ".join(spills))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(DIGEST, "w") as fh:
        fh.write(source_digest() + "\n")
    if verbose:
        print(f"built {LIB} ({len(lines)} kernels, no scratch)")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
