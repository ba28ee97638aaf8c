"""The host-side checks of the C ABI (tests/test_abi.py) run again against a build whose host
code is compiled with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only; the device
code is built as usual and never runs here).  Argument validation, the size arithmetic of the
workspace queries and the chunk planner must be free of out-of-bounds accesses, signed
overflow and other undefined behaviour for every argument the tests pass, including the
huge dimensions that must be rejected.

The sanitized library is built once into triangular_attention_amd/_build/sanitize/ (rebuilt
when a source changes) and loaded by a child Python process with the sanitizer runtime
preloaded."""
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "triangular_attention_amd", "csrc")
OUT = os.path.join(ROOT, "triangular_attention_amd", "_build", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
sys.path.insert(0, ROOT)
from triangular_attention_amd.build import SOURCES  # noqa: E402  (the library's own source list)
# each sanitizer flag applies to the host pass only
HOST_SANITIZE = ["-Xarch_host -fsanitize=address", "-Xarch_host -fsanitize=undefined",
                 "-Xarch_host -fno-sanitize-recover=undefined", "-Xarch_host -fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-result"]


def _runtime():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return rt[-1] if rt else None


def _sources_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        h.update(f.encode() + open(os.path.join(CSRC, f), "rb").read())
    h.update(" ".join(FLAGS + HOST_SANITIZE + list(SOURCES)).encode())
    return h.hexdigest()[:16]


def _build():
    lib = os.path.join(OUT, "libtri_attn.so")
    stamp = os.path.join(OUT, "sources.hash")
    want = _sources_hash()
    if os.path.exists(lib) and os.path.exists(stamp) and open(stamp).read() == want:
        return lib
    os.makedirs(OUT, exist_ok=True)
    flags = FLAGS + [w for f in HOST_SANITIZE for w in f.split()]
    procs, objs = [], []
    for s in SOURCES:
        o = os.path.join(OUT, s.replace(".hip", ".o"))
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", o],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p, s in zip(procs, SOURCES):
        out, _ = p.communicate()
        assert p.returncode == 0, f"hipcc failed for {s}:\n{out[-3000:]}"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SANITIZE[0].split(), *HOST_SANITIZE[1].split(),
            *objs, "-o", lib]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    open(stamp, "w").write(want)
    return lib


@pytest.mark.timeout(900)
def test_abi_checks_under_address_and_undefined_behaviour_sanitizers():
    rt = _runtime()
    if not (os.path.exists(HIPCC) and rt and shutil.which("objcopy")):
        pytest.skip("ROCm compiler or sanitizer runtime not available")
    lib = _build()
    env = dict(os.environ)
    env.update({"TRI_ATTN_LIBRARY": lib, "LD_PRELOAD": rt,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "HIP_VISIBLE_DEVICES": "", "ROCR_VISIBLE_DEVICES": ""})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
