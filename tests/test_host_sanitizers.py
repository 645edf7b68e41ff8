"""The library's host code (argument checks, workspace layout, error paths)
under AddressSanitizer and UndefinedBehaviorSanitizer: a build of the same
sources with sanitized host code runs the C-ABI validation tests in a child
process with the ASan runtime preloaded. No GPU is needed: every call in those
tests returns from host-side validation."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers(tmp_path):
    from attention_lm_amd import build as B
    try:
        B.hipcc()
        rt = B.sanitizer_runtime_dir()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_host_sanitized(str(tmp_path / "hostsan"))
    log = tmp_path / "sanitizer.log"
    env = dict(os.environ)
    env.update({
        "HYMBA_MIXER_LIB": lib,
        "LD_PRELOAD": os.path.join(rt, "libclang_rt.asan-x86_64.so"),
        "LD_LIBRARY_PATH": rt + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else ""),
        # the interpreter itself is not instrumented: leaks at exit are not the library's
        "ASAN_OPTIONS": f"detect_leaks=0:abort_on_error=1:log_path={log}",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={log}",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path)
                      if f.startswith("sanitizer.log"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], reports[-3000:])
    assert " passed" in r.stdout
