"""The C ABI's host-side argument checks under AddressSanitizer.

Builds a copy of libw4a8.so whose host code is instrumented (the kernels are
compiled as usual and never run here), then runs tests/test_abi_cpu.py
against it in a child interpreter with the sanitizer runtime preloaded: every
rejection path, workspace query and plan computation of abi.hip executes
under ASan.  CPU only; the build goes to _build/asan and is redone only when
a source is newer than it."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libw4a8_asan.so")
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


def _sources():
    return (sorted(glob.glob(os.path.join(ROOT, "bit_quantized_amd", "csrc", "*.hip"))) +
            sorted(glob.glob(os.path.join(ROOT, "bit_quantized_amd", "csrc", "*.h"))) +
            sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))


def _build():
    sys.path.insert(0, ROOT)
    from bit_quantized_amd import build as B
    srcs = [s for s in _sources() if s.endswith(".hip")]
    if os.path.exists(LIB) and os.path.getmtime(LIB) > max(os.path.getmtime(s) for s in _sources()):
        return
    os.makedirs(OUT, exist_ok=True)
    # host code only is instrumented: each -fsanitize= follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    procs, objs = [], []
    for s in srcs:
        obj = os.path.join(OUT, os.path.basename(s) + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen([B.HIPCC, *B.FLAGS, *san, "-c", s, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-3000:]
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *san, *objs,
                        "-o", LIB + ".tmp"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    os.replace(LIB + ".tmp", LIB)


@pytest.mark.skipif(not RUNTIME, reason="no AddressSanitizer runtime in this ROCm")
def test_abi_host_checks_under_asan():
    _build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join([RUNTIME[-1]] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:exitcode=86"
    env["W4A8_LIB_PATH"] = LIB
    # the child loads the instrumented build, which calls into the sanitizer
    probe = subprocess.run([sys.executable, "-c", "from bit_quantized_amd import _lib; "
                            "print(_lib.load()._name)"], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip() == LIB, probe.stdout + probe.stderr
    syms = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True)
    assert "__asan_report_load" in syms.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in r.stdout
