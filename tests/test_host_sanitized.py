"""The host-side tests of the C-ABI library (test_host_lib.py) again, on the library's
host-checking variant: AddressSanitizer and UndefinedBehaviorSanitizer on every line of
host code (argument validation, alias and extent checks, step planning, scalar and RNG
helpers), in a child process with the sanitizer runtime loaded first. A report aborts
the child and fails the test. A control library built with the same flags, holding a
heap overflow and a signed overflow, shows that both sanitizers are live in that set-up.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CONTROL = r"""
#include <hip/hip_runtime.h>
#include <climits>
extern "C" int heap_overflow(int n) {
  int* p = new int[4];
  for (int i = 0; i < 4; ++i) p[i] = i;
  int r = p[n];
  delete[] p;
  return r;
}
extern "C" int add_overflow(int a) { return a + INT_MAX; }
"""


def _env(b, lib):
    return dict(os.environ, FORGE_LIB=lib, LD_PRELOAD=b.sanitizer_runtime(), ASAN_OPTIONS="detect_leaks=0",
                UBSAN_OPTIONS="print_stacktrace=1", PYTHONPATH=ROOT)


def _run(args, env, timeout=900):
    return subprocess.run([sys.executable, *args], env=env, cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_sanitizers_are_live(host_checked_build, tmp_path):
    b, lib, _ = host_checked_build
    src = tmp_path / "control.hip"
    src.write_text(CONTROL)
    so = str(tmp_path / "libcontrol.so")
    r = subprocess.run([b._hipcc(), *b.CFLAGS, *b.SAN_HOST, "-shared", *b.SAN_LINK, "-o", so, str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = _env(b, lib)
    ok = _run(["-c", f"import ctypes; print(ctypes.CDLL({so!r}).heap_overflow(3))"], env)
    assert ok.returncode == 0 and ok.stdout.strip() == "3", ok.stderr[-2000:]
    heap = _run(["-c", f"import ctypes; ctypes.CDLL({so!r}).heap_overflow(4)"], env)
    assert heap.returncode != 0 and "heap-buffer-overflow" in heap.stderr, heap.stderr[-2000:]
    ub = _run(["-c", f"import ctypes; ctypes.CDLL({so!r}).add_overflow(1)"], env)
    assert ub.returncode != 0 and "signed integer overflow" in ub.stderr, ub.stderr[-2000:]


def test_host_lib_under_sanitizers(host_checked_build):
    b, lib, _ = host_checked_build
    env = _env(b, lib)
    probe = _run(["-c", "import optimizer_gemm_amd as f; print(f.forge.LIB_PATH); print(open('/proc/self/maps').read())"],
                 env)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.splitlines()[0] == lib
    assert "libforge_san.so" in probe.stdout and "libclang_rt.asan" in probe.stdout
    r = _run(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_host_lib.py")],
             env)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, report
    assert " passed" in r.stdout, report
