"""Build libkvq.so (HIP for gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object and linked into one
shared library next to this file.  The quantize translation unit is built
without floating-point contraction so that its fp32 arithmetic is exactly the
operations the header's quantizer contract lists.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no packed-fp32 VALU instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]
PER_FILE = {
    "quantize.hip": ["-ffp-contract=off"],
}
# Comparison builds (made only on request, never by build()): extra flags per
# source and the library name.  "keys-dot2" runs the decode kernel's
# quantized-key loop on v_dot2 instead of matrix cores for one query head per
# kv head; the binding loads it when KVQ_LIBRARY names it.
VARIANTS = {
    "keys-dot2": ({"decode.hip": ["-DKVQ_KEY_LOOP_DOT2"]}, "libkvq_keys_dot2.so"),
}
SOURCES = ["api.hip", "quantize.hip", "reorder.hip", "decode.hip", "search.hip", "pq.hip", "vq.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build(verbose: bool = False, jobs: int = 4, variant: str | None = None) -> str:
    """Compile every kernel source for gfx950 and link libkvq.so (or a
    comparison library of VARIANTS); returns its path."""
    cc = hipcc()
    extra, lib = ({}, LIB) if variant is None else (VARIANTS[variant][0], os.path.join(HERE, VARIANTS[variant][1]))
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *COMMON, *PER_FILE.get(src, []), *extra.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            while len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
            if p.returncode != 0:
                failed.append((src, "\n".join(lines)))
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n\n".join(f"[{s}]\n{t}" for s, t in failed))
        tmp_lib = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
        os.replace(tmp_lib, lib)
    return lib


if __name__ == "__main__":
    v = sys.argv[sys.argv.index("--variant") + 1] if "--variant" in sys.argv else None
    print(build(verbose="-v" in sys.argv, variant=v))
