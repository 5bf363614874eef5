"""The host state machine under UBSan, including the legal rows > 0 paths.

host.cpp is compiled with g++ (host code only, undefined-behaviour sanitizer aborting on the
first report) and linked with launch functions that return success without launching, so
every call runs its full validation, argument packing and state transition on the CPU. A
subprocess loads that build in place of libboundary.so and runs the host test module's checks
plus a walk through every legal transition with non-empty slices and fake, never-dereferenced
device addresses.
"""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_residual_rmsnorm_bnd_amd", "csrc")

if torch.cuda.device_count() > 0:
    pytestmark = pytest.mark.skip(reason="host-only checks with fake device addresses")

STUB = r"""
#include <hip/hip_runtime.h>
#include "launch.h"
namespace bnd {
hipError_t launch_read(Source, int, bool, const RowArgs&, const Launch&, hipStream_t) { return hipSuccess; }
hipError_t launch_complete(Source, int, bool, const RowArgs&, const Launch&, hipStream_t) {
  return hipSuccess;
}
int wave_read_rows_per_cu(Source, bool, int vpt, bool deep) { return deep ? 8 : vpt == 8 ? 12 : 8; }
int wave_complete_rows_per_cu(Source, Tail, int vpt, bool deep) { return deep ? 8 : vpt == 8 ? 16 : 8; }
}  // namespace bnd
"""

SCRIPT = r"""
import ctypes, sys
sys.path[:0] = [{root!r}, {tests!r}]
from reduce_residual_rmsnorm_bnd_amd import boundary as B
B._lib = B._declare(ctypes.CDLL({lib!r}))
import test_abi_host as T
L = B._lib

def reset():
    for opt in (1, 2, 3, 4, 5):
        L.bnd_set_option(opt, 0)

n = 0
for name in dir(T):
    fn = getattr(T, name)
    if not name.startswith("test_") or not callable(fn):
        continue
    if name == "test_transition":
        for call, start in T.CASES:
            fn(call, start); reset(); n += 1
    else:
        fn(); reset(); n += 1

# legal paths with non-empty slices: every call validates, packs its launch and transitions
VP = ctypes.c_void_p
F = 0x7F0000000000
fake = lambda off: VP(F + off)
H, T_, rows, rb = 4096, 64, 24, 8
o, o2 = ctypes.c_uint64(), ctypes.c_uint64()
h = VP()
assert L.bnd_stream_create(ctypes.byref(h), T_, H, rb, rows, fake(0), H) == 0
w, y, q, sc, x = fake(1 << 20), fake(1 << 26), fake(1 << 27), fake(1 << 28), fake(1 << 29)
parts = (VP * 8)(*[fake((2 + p) << 30) for p in range(8)])
assert L.bnd_enter_norm(h, x, H, w, 1e-6, y, H, None) == 0, L.bnd_last_error()
assert L.bnd_publish_partials(h, parts, 8, H, ctypes.byref(o)) == 0
assert L.bnd_snapshot(h, o.value, y, H, None) == 0, L.bnd_last_error()
assert L.bnd_fold_norm(h, o.value, w, 1e-6, y, H, None) == 0, L.bnd_last_error()
assert L.bnd_publish_partials(h, parts, 8, H, ctypes.byref(o)) == 0
assert L.bnd_fold_norm_quant_fp8(h, o.value, w, 1e-6, q, H, sc, None) == 0, L.bnd_last_error()
assert L.bnd_publish_partials(h, parts, 8, H, ctypes.byref(o)) == 0
assert L.bnd_add_to_output(h, o.value, fake(12 << 30), H, fake(13 << 30), H, ctypes.byref(o2), None) == 0
assert L.bnd_complete_only(h, o2.value, fake(14 << 30), H, ctypes.byref(o), None) == 0
assert L.bnd_fold_norm(h, o.value, w, 1e-6, y, H, None) == 0, L.bnd_last_error()
assert L.bnd_publish_moe(h, fake(15 << 30), 512, H, fake(16 << 30), fake(17 << 30), 8, ctypes.byref(o)) == 0
assert L.bnd_moe_finalize_fold_norm(h, o.value, w, 1e-6, y, H, None) == 0, L.bnd_last_error()
assert L.bnd_stream_set_norm_form(h, 1) == 0
assert L.bnd_publish_moe(h, fake(15 << 30), 512, H, fake(16 << 30), fake(17 << 30), 8, ctypes.byref(o)) == 0
assert L.bnd_complete_only(h, o.value, fake(14 << 30), H, ctypes.byref(o2), None) == 0
assert L.bnd_fold_norm(h, o2.value, w, 1e-6, y, H, None) == 0
far = lambda k: fake(k << 36)  # 64 GiB apart: no region overlaps another
parts2 = (VP * 8)(*[far(4 + p) for p in range(8)])
for H2 in (8, 264, 4096, 7168, 16384, 32768):  # every launch-shape branch
    for rows2 in (1, 300, 2048, 4096):  # 2048 x 4096: one wavefront per row
        h2 = VP()
        assert L.bnd_stream_create(ctypes.byref(h2), 4096, H2, 0, rows2, far(0), H2) == 0
        assert L.bnd_publish_partials(h2, parts2, 8, H2, ctypes.byref(o)) == 0
        assert L.bnd_fold_norm(h2, o.value, far(1), 1e-6, far(2), H2, None) == 0, (H2, L.bnd_last_error())
        L.bnd_stream_destroy(h2)
h3 = VP()  # the one-wavefront rows forced, for a MoE finalize and an fp8 fold
assert L.bnd_set_option(3, 8) == 0
assert L.bnd_stream_create(ctypes.byref(h3), 4096, 4096, 0, 100, far(0), 4096) == 0
assert L.bnd_publish_moe(h3, far(10), 512, 4096, far(11), far(12), 8, ctypes.byref(o)) == 0
assert L.bnd_moe_finalize_fold_norm(h3, o.value, far(1), 1e-6, far(2), 4096, None) == 0, L.bnd_last_error()
assert L.bnd_publish_partials(h3, parts2, 8, 4096, ctypes.byref(o)) == 0
assert L.bnd_fold_norm_quant_fp8(h3, o.value, far(1), 1e-6, far(2), 4096, far(3), None) == 0, L.bnd_last_error()
assert L.bnd_stream_destroy(h3) == 0
reset()
assert L.bnd_take_output(h) == 0 and L.bnd_stream_destroy(h) == 0
print(f"ran {{n}} host checks and the legal-path walk clean")
"""


def test_host_state_machine_under_ubsan(tmp_path):
    stub = tmp_path / "stub_launch.cpp"
    stub.write_text(STUB)
    lib = str(tmp_path / "libboundary_host_ubsan.so")
    subprocess.check_call([
        "g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-static-libubsan",
        "-g", "-O1", "-shared", "-fPIC", "-o", lib, os.path.join(CSRC, "host.cpp"), str(stub),
        "-L/opt/rocm/lib", "-lamdhip64"])
    script = tmp_path / "run.py"
    script.write_text(SCRIPT.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib))
    out = subprocess.run([sys.executable, str(script)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout[-3000:] + out.stderr[-5000:]
    assert "clean" in out.stdout
