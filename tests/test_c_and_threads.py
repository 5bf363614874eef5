"""The C ABI from C and C++ programs, per-thread error state, and sanitizer builds.

Nothing here launches a kernel: the programs use empty batches (rows = 0), which apply the
state transitions without touching a device.
"""
import ctypes
import os
import subprocess
import sys
import threading

import pytest

import reduce_residual_rmsnorm_bnd_amd as bnd
from reduce_residual_rmsnorm_bnd_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(_build.LIB_PATH)

C_PROGRAM = r"""
#include "boundary.h"
#include <stdio.h>
#include <string.h>

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("line %d: %s\n", __LINE__, #cond); ++fails; } } while (0)

int main(void) {
  bnd_stream* s = NULL;
  bnd_owed owed = BND_OWED_NONE, again = BND_OWED_NONE;
  const void* parts[2] = {NULL, NULL};
  EXPECT(bnd_stream_create(&s, 0, 4096, 0, 0, NULL, 4096) == BND_OK);
  EXPECT(bnd_stream_state(s) == BND_INITIAL);
  EXPECT(bnd_fold_norm(s, BND_OWED_NONE, NULL, 1e-6f, NULL, 4096, NULL) == BND_ERR_NOT_STARTED);
  EXPECT(strlen(bnd_last_error()) > 0);
  EXPECT(bnd_publish_partials(s, parts, 2, 4096, &owed) == BND_OK);
  EXPECT(bnd_stream_state(s) == BND_PENDING && bnd_stream_pending_kind(s) == BND_KIND_PARTIALS);
  EXPECT(bnd_publish_partials(s, parts, 2, 4096, &again) == BND_ERR_PENDING);
  EXPECT(bnd_fold_norm(s, owed, NULL, 1e-6f, NULL, 4096, NULL) == BND_OK);
  EXPECT(bnd_stream_state(s) == BND_WRITTEN && bnd_stream_has_residual(s) == 1);
  EXPECT(bnd_fold_norm(s, owed, NULL, 1e-6f, NULL, 4096, NULL) == BND_ERR_FOREIGN_OUTPUT);
  EXPECT(bnd_stream_set_norm_form(s, BND_NORM_GEMMA) == BND_OK);
  EXPECT(bnd_take_output(s) == BND_OK && bnd_stream_state(s) == BND_INITIAL);
  EXPECT(strcmp(bnd_status_str(BND_ERR_WRONG_KIND), "BND_ERR_WRONG_KIND") == 0);
  {
    int64_t counts[3] = {5, 0, 7};
    int64_t begin = -1, rows = -1, total = -1;
    EXPECT(bnd_rsv_share(counts, 3, 2, &begin, &rows, &total) == BND_OK);
    EXPECT(begin == 5 && rows == 7 && total == 12);
  }
  EXPECT(bnd_stream_destroy(s) == BND_OK);
  printf("%s: %d failures\n", bnd_version(), fails);
  return fails ? 1 : 0;
}
"""


def _compile_and_run(tmp_path, compiler, std, suffix):
    src = tmp_path / f"abi_test.{suffix}"
    src.write_text(C_PROGRAM)
    exe = tmp_path / f"abi_test_{suffix}"
    cmd = [compiler, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE,
           str(src), "-o", str(exe), "-L", LIBDIR, "-lboundary", f"-Wl,-rpath,{LIBDIR}",
           "-Wl,-rpath-link,/opt/rocm/lib"]
    subprocess.check_call(cmd)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 failures" in out.stdout


@pytest.fixture(scope="module", autouse=True)
def _lib_name():
    # the library file is libboundary.so, linkable as -lboundary
    assert os.path.basename(_build.LIB_PATH) == "libboundary.so"


def test_header_is_plain_c(tmp_path):
    _compile_and_run(tmp_path, "gcc", "c99", "c")


def test_header_is_valid_cpp(tmp_path):
    _compile_and_run(tmp_path, "g++", "c++17", "cpp")


def test_last_error_is_per_thread():
    L = bnd.lib()
    results = {}
    barrier = threading.Barrier(2)

    def failing():
        h = ctypes.c_void_p()
        barrier.wait()
        st = L.bnd_stream_create(ctypes.byref(h), -1, 4096, 0, 0, None, 4096)
        barrier.wait()
        results["failing"] = (st, L.bnd_last_error())

    def succeeding():
        h = ctypes.c_void_p()
        barrier.wait()
        st = L.bnd_stream_create(ctypes.byref(h), 4, 4096, 0, 0, None, 4096)
        barrier.wait()
        results["succeeding"] = (st, L.bnd_last_error())
        L.bnd_stream_destroy(h)

    ts = [threading.Thread(target=failing), threading.Thread(target=succeeding)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert results["failing"][0] == bnd.BND_ERR_INVALID_ARG and results["failing"][1]
    assert results["succeeding"] == (bnd.BND_OK, b"")


def test_independent_streams_in_threads():
    """Microbatches on separate threads, each with its own stream (no shared state)."""
    L = bnd.lib()
    errors = []

    def worker(i):
        h = ctypes.c_void_p()
        if L.bnd_stream_create(ctypes.byref(h), 0, 1024, 0, 0, None, 1024):
            errors.append(i)
            return
        owed = ctypes.c_uint64()
        for _ in range(2000):
            ok = (L.bnd_publish_partials(h, (ctypes.c_void_p * 1)(None), 1, 1024, ctypes.byref(owed)) == 0
                  and L.bnd_fold_norm(h, owed.value, None, 1e-6, None, 1024, None) == 0)
            if not ok:
                errors.append(i)
                break
        L.bnd_stream_destroy(h)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors


SANITIZED_PINS = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
o = oracle.Oracle(oracle.load({lib!r}))
for pin in oracle_pins.PINS:
    pin(o)
print("all pins ran clean")
"""


def test_oracle_and_generator_under_ubsan(tmp_path):
    """UBSan builds (aborting on the first report) of the oracle and the generator run the
    whole pin suite."""
    import oracle
    import workloads

    san = ["-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-static-libubsan", "-g"]
    lib = str(tmp_path / "liboracle_ubsan.so")
    oracle.build(out=lib, extra=san)
    gen = str(tmp_path / "libgen_ubsan.so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", *san, "-o", gen,
                           workloads._SRC, "-lm"])
    script = tmp_path / "run.py"
    body = SANITIZED_PINS.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    # route the generator through the sanitized build as well
    body = body.replace("import oracle, oracle_pins",
                        "import workloads\nworkloads._LIB_PATH = " + repr(gen) +
                        "\nimport oracle, oracle_pins")
    script.write_text(body)
    out = subprocess.run([sys.executable, str(script)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-4000:]
    assert "all pins ran clean" in out.stdout
