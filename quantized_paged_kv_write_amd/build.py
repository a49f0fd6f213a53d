"""Build libkvq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m quantized_paged_kv_write_amd.build

Compiles every csrc/*.hip to an object under _build/ and links the shared
library next to this file.  Flags: no fast-math, denormals preserved, fp32
contraction off in the write kernels (their quotient sequence is written out
with explicit FMAs and must not be re-associated), packed FP32 disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
ARCH = "gfx950"

SOURCES = {
    "kvq_api.hip": [],
    "kvq_write.hip": ["-ffp-contract=off"],
    "kvq_decode.hip": [],
    "kvq_decode_kint8.hip": [],
    "kvq_decode_kfp8.hip": [],
    "kvq_decode_kkivi.hip": [],
    "kvq_decode_ke5m2.hip": [],
    "kvq_decode_kint4.hip": [],
    "kvq_decode_kint4_rot.hip": [],
    "kvq_decode_kint8_rot.hip": [],
    "kvq_decode_kfp8_rot.hip": [],
    "kvq_decode_ke5m2_rot.hip": [],
    "kvq_offload.hip": [],
    "kvq_prefill.hip": [],
    "kvq_prefill_kint8.hip": [],
    "kvq_prefill_kfp8.hip": [],
    "kvq_prefill_kkivi.hip": [],
    "kvq_prefill_ke5m2.hip": [],
    "kvq_prefill_kint4.hip": [],
}

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq.so)")


PROBE_SRC = "kvq_probe.hip"  # benchmark reference points, its own library
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    probe_obj = os.path.join(BUILD, PROBE_SRC.replace(".hip", ".o"))
    procs.append((PROBE_SRC, subprocess.Popen([cc, *COMMON, "-c", os.path.join(CSRC, PROBE_SRC), "-o", probe_obj],
                                              stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", probe_obj, "-o", tmp], check=True)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
