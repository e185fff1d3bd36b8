"""Build libdspark.so (all HIP sources, gfx950) into the package directory.

Usage: python -m draft_sampling_verify_markov_amd.build [--jobs N]
"""

import argparse
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdspark.so")
ARCH = os.environ.get("DSPARK_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source extra flags.  The one-launch draft and the resident-W2 residual
# pass keep their W2 fragments in the AGPRs, so their MFMAs write their
# results to VGPRs.
EXTRA_FLAGS = {
    "draft_fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "verify.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def build(jobs=None, verbose=False):
    """Compile every csrc/*.hip and link libdspark.so.  Returns the library path."""
    cc = hipcc()
    srcs = sources()
    tmp = tempfile.mkdtemp(prefix="dspark_build_")
    try:
        objs, procs = [], []
        for s in srcs:
            o = os.path.join(tmp, os.path.basename(s) + ".o")
            objs.append(o)
            cmd = [cc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            if jobs and len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[-1][1].wait()
        for s, p in procs:
            out = p.communicate()[0].decode(errors="replace")
            lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
            if p.returncode != 0:
                raise RuntimeError(f"hipcc failed on {s}:\n" + "\n".join(lines))
            if verbose and lines:
                print("\n".join(lines))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
    sys.exit(0)
