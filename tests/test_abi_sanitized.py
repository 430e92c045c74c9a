"""The host-side checks of test_abi.py again, against a build of the C ABI layer
(csrc/tsa_api.cpp) instrumented with the host AddressSanitizer and
UndefinedBehaviorSanitizer (signed overflow, shifts, out-of-bounds indexing and
the like abort the run).  The HIP kernel objects are linked in unchanged; no
GPU call is made.  Runs on any host with g++ and its sanitizer runtimes.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_sparse_causal_amd")
CSRC = os.path.join(PKG, "csrc")


def _kernel_sources():
    """The HIP sources of the library, as its build script lists them."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("_tsa_build_sources", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [s for s in mod.SOURCES if s.endswith(".hip")]


KERNEL_SOURCES = _kernel_sources()


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None,
                    reason="g++ with the host sanitizer runtimes is needed")
def test_abi_checks_under_host_sanitizers(tmp_path):
    objs = [os.path.join(PKG, "_build", src + ".o") for src in KERNEL_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        import importlib.util

        spec = importlib.util.spec_from_file_location("_tsa_build", os.path.join(PKG, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(verbose=False)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    api = str(tmp_path / "tsa_api.o")
    lib = str(tmp_path / "libtsa_sanitized.so")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]
    subprocess.run(["g++", *flags, "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include", f"-I{os.path.join(ROOT, 'include')}",
                    f"-I{CSRC}", "-c", os.path.join(CSRC, "tsa_api.cpp"), "-o", api], check=True)
    subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", api, *objs, f"-L{rocm}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{rocm}/lib", "-o", lib], check=True)
    env = dict(os.environ)
    env.update({
        "TSA_ABI_LIBRARY": lib,
        "LD_PRELOAD": " ".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p),
        "ASAN_OPTIONS": "detect_leaks=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=600)
    tail = (proc.stdout + proc.stderr)[-4000:]
    assert proc.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
