"""The C ABI's host code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (host only, no GPU).

tests/sanitize/abi_sanitize.cpp drives every validation path of include/dcn.h
(descriptors, NULL / misaligned pointers, short workspaces: all refused before
any launch) and runs each oracle function on small inputs.  The library's
sources are compiled with the sanitizers on the
host side; any leak, out-of-bounds access or undefined behaviour aborts the
program.  The device code is compiled as usual (the host objects refer to
it) but never runs: nothing here launches a kernel.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "modulated_deformable_convolution_dcn_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm compilers")
def test_abi_and_oracle_under_asan_ubsan(tmp_path):
    build = str(tmp_path)
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I",
              CSRC, "-I", os.path.join(ROOT, "oracle")]
    srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp"))]
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(build, os.path.basename(src) + ".o")
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-fno-gpu-rdc", "-Xclang",
               "-target-feature", "-Xclang", "-packed-fp32-ops"] + common + SAN + \
            ["-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    for plain in (os.path.join(ROOT, "oracle", "dcn_oracle.cpp"),
                  os.path.join(ROOT, "tests", "sanitize", "abi_sanitize.cpp")):
        obj = os.path.join(build, os.path.basename(plain) + ".o")
        cmd = [CLANG, "-x", "c++", "-ffp-contract=off"] + common + \
            ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c", plain, "-o", obj]
        procs.append((plain, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                              stderr=subprocess.STDOUT)))
        objs.append(obj)
    for src, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, "%s:\n%s" % (src, out.decode(errors="replace")[-3000:])
    exe = os.path.join(build, "abi_sanitize")
    link = [HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
            "-fsanitize=undefined", "-o", exe] + objs + ["-pthread"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "sanitize ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
