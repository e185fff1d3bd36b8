"""The library's host code under AddressSanitizer, on the CPU.

Every csrc/*.hip source is compiled again with the host side instrumented
(the device code is built as usual and never runs here), linked against the
shared sanitizer runtime, and the C-ABI argument, workspace-size and status
checks of test_abi_cpu.py run against that library in a child process with
the runtime preloaded.  Any invalid host memory access in those paths aborts
the child with a sanitizer report."""

import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from draft_sampling_verify_markov_amd import build as B  # noqa: E402


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(600)
def test_abi_checks_under_address_sanitizer():
    rt = _runtime()
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if rt is None or not os.path.exists(cc):
        pytest.skip("hipcc or the sanitizer runtime is not installed")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1"]
    tmp = tempfile.mkdtemp(prefix="dspark_asan_")
    try:
        objs, procs = [], []
        for s in B.sources():
            o = os.path.join(tmp, os.path.basename(s) + ".o")
            objs.append(o)
            cmd = [cc, *flags, *B.EXTRA_FLAGS.get(os.path.basename(s), []), *host_asan, "-c", s, "-o", o]
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        for s, p in procs:
            out = p.communicate()[0].decode(errors="replace")
            assert p.returncode == 0, f"{s}:\n{out}"
        lib = os.path.join(tmp, "libdspark_asan.so")
        link = [cc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                "-shared-libasan", *objs, "-o", lib]
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        assert r.returncode == 0, r.stdout.decode(errors="replace")

        env = dict(os.environ, DSPARK_LIB=lib, LD_PRELOAD=rt,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
        r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                            "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                           cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
        out = r.stdout.decode(errors="replace")
        assert "AddressSanitizer" not in out, out[-4000:]
        assert r.returncode == 0, out[-4000:]
        assert " passed" in out, out[-2000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
