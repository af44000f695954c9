"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
called from two threads at once (runs without a GPU).

The library is rebuilt with both sanitizers on its host code (argument checks,
overflow-checked size arithmetic, workspace layout, launchers) into a
temporary directory, loaded into a child Python process that has the clang
ASan runtime preloaded, and every host validation case of
``test_capi_host.py`` runs there on two threads concurrently, many times over.
Every case fails validation before any HIP call, so no kernel is launched (on
any machine).  Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

from gemm_block_q4_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, threading, traceback
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from gemm_block_q4_amd import _binding
lib = _binding.load_library({lib!r}, share_torch_runtime=False)
import test_capi_host as T
cases = [getattr(T, n) for n in sorted(dir(T)) if n.startswith("test_") and n != "test_exports_every_declared_function"]
errors = []
def worker():
    try:
        for _ in range(50):
            for c in cases:
                c(lib)
    except BaseException:
        errors.append(traceback.format_exc())
threads = [threading.Thread(target=worker) for _ in range(2)]
for t in threads: t.start()
for t in threads: t.join()
if errors:
    print(errors[0]); sys.exit(3)
print("SANITIZED_OK", len(cases))
"""


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if B.asan_runtime() is None:
        pytest.fail("no clang ASan runtime found next to hipcc")
    out = str(tmp_path_factory.mktemp("asan") / "libq4k_asan.so")
    return B.build(sanitize=True, out=out)


def test_validation_layer_under_asan_ubsan_two_threads(sanitized_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = B.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # no device is touched; keep a GPU machine's devices out of the child anyway
    env["HIP_VISIBLE_DEVICES"] = ""
    script = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=sanitized_lib)
    res = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                         timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "SANITIZED_OK" in res.stdout, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
