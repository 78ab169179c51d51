"""Build libqkv.so (HIP for gfx950) in-tree with hipcc.

    python -m tiered_quantization_eviction_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqkv.so")
ARCH = os.environ.get("QKV_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 instructions stay disabled (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False) -> str:
    objs = []
    with tempfile.TemporaryDirectory(prefix="qkv_build_") as tmp:
        procs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [hipcc(), *FLAGS, *lang, "-c", src, "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = False
        for cmd, p in procs:
            out, _ = p.communicate()
            noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0 or (verbose and noise):
                sys.stderr.write(" ".join(cmd) + "\n" + "\n".join(noise) + "\n")
            failed |= p.returncode != 0
        if failed:
            raise RuntimeError("hipcc failed")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout)
            raise RuntimeError("link failed")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
