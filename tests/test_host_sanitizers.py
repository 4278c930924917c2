"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The page pool, the argument checks and the work planning of libpa are host
C++.  This test builds them with ASan + UBSan (paged_kv_cache_185_amd.build.
build_host_sanitized: clang, host code only, UBSan errors fatal) and runs the
library's host tests (tests/test_library.py: random pool scripts against the
allocator model, the prefix cache, swap and compaction, workspace sizing,
argument validation and the host range checks) against that build in a child
process with the sanitizer runtime loaded first.  Any sanitizer report fails
the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

build = pytest.importorskip("paged_kv_cache_185_amd.build")


def _sanitized_env():
    try:
        lib = build.build_host_sanitized()
        rt = build.sanitizer_runtime()
    except RuntimeError as e:            # no clang or no sanitizer runtime in this image
        pytest.skip(f"host sanitizer build unavailable: {e}")
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env.update(PA_LIB_PATH=lib, LD_PRELOAD=rt + (":" + pre if pre else ""),
               # the interpreter itself is not instrumented and keeps memory
               # until exit by design: leak reports would be about it
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return lib, env


def test_host_code_is_clean_under_asan_and_ubsan():
    lib, env = _sanitized_env()
    # the child really maps the instrumented library and the runtime
    probe = ("import paged_kv_cache_185_amd as pa\n"
             "p = pa.Pool(8, 16); s = p.seq_new(); p.seq_append(s, 20)\n"
             "print('\\n'.join(l.split()[-1] for l in open('/proc/self/maps') if '/' in l))\n")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    maps = r.stdout.splitlines()
    assert any(m == lib for m in maps), "the sanitizer build was not loaded"
    assert any("libclang_rt.asan" in m for m in maps), "the sanitizer runtime was not loaded"
    assert not any(m.endswith("paged_kv_cache_185_amd/libpa.so") for m in maps)

    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_library.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in text and "runtime error:" not in text, text[-5000:]
    assert r.returncode == 0, text[-5000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-2000:]
