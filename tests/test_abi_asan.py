"""Host AddressSanitizer over the C ABI's host code (argument checks, workspace sizing and
carving, launch policies): the library is rebuilt with its host code sanitized
(build(asan=True); the GPU code is compiled as usual) and test_abi.py runs against that copy in
a child process that preloads the sanitizer's runtime. A probe library built the same way with
a planted heap overflow must be reported, so that a clean run means the sanitizer was live.
CPU only: no call here reaches the GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "deepseek_sparse_attention_indexer_amd"))
import build  # noqa: E402

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")

PROBE = """#include <stdlib.h>
extern "C" int probe_overflow(int n) {
  int* p = (int*)malloc(n * sizeof(int));
  p[n] = 1;   // one past the end
  int v = p[0];
  free(p);
  return v;
}
"""


def _env(lib=None):
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""          # nothing here may reach a GPU
    if lib:
        env["DSA_LIBRARY"] = lib
    return env


def test_sanitizer_is_live(tmp_path):
    src = tmp_path / "probe.cpp"
    src.write_text(PROBE)
    so = tmp_path / "probe.so"
    subprocess.run(["hipcc", "-x", "c++", "-shared", "-fPIC", *build.ASAN_HOST_FLAGS, str(src), "-o", str(so)],
                   check=True, capture_output=True, timeout=300)
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).probe_overflow(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "AddressSanitizer: heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_abi_tests_pass_under_host_asan(tmp_path):
    lib = build.build(out=str(tmp_path / "libdsa_asan.so"), asan=True)
    which = subprocess.run([sys.executable, "-c", "from deepseek_sparse_attention_indexer_amd import _binding as B; "
                            "print(B.lib_path())"], env=_env(lib), capture_output=True, text=True, timeout=300,
                           cwd=ROOT)
    assert which.returncode == 0 and which.stdout.strip() == lib, which.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       env=_env(lib), capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in r.stdout, out[-4000:]
