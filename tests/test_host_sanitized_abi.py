"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/test_abi.py runs in a child process against
the sanitized build of the library (host code instrumented, device code
compiled but never launched), with the sanitizer runtime preloaded into that
Python process.  Any sanitizer report fails the test.  No GPU is used."""
import os
import subprocess
import sys

from tree_causal_attention_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env["JT_LIBRARY"] = lib
    # the sanitizer runtime must come first; anything already preloaded stays
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = build.asan_runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={tmp_path}/asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=900)
    reports = {p.name: p.read_text() for p in tmp_path.iterdir() if "san" in p.name}
    assert not reports, "sanitizer reports:\n" + "\n".join(reports.values())[:4000]
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
