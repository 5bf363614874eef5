"""AddressSanitizer builds (host code only, g++/gcc) of the state machine and the oracle.

Two standalone programs, so no sanitizer runtime has to be injected into Python:

* the host state machine (host.cpp) linked with launch functions that return success without
  launching, driven through every legal transition with non-empty slices and fake,
  never-dereferenced device addresses, plus the refused calls;
* the oracle (oracle.c) on small rows held in heap buffers of exactly the sizes its callers
  pass, so any read or write past an operand is reported.

Both abort on the first report (and on undefined behaviour).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_residual_rmsnorm_bnd_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")

HOST_DRIVER = r"""
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdint.h>
#include "boundary.h"
#include "launch.h"

namespace bnd {
hipError_t launch_read(Source, int, bool, const RowArgs&, const Launch&, hipStream_t) { return hipSuccess; }
hipError_t launch_complete(Source, int, bool, const RowArgs&, const Launch&, hipStream_t) { return hipSuccess; }
int wave_read_rows_per_cu(Source, bool, int vpt, bool deep) { return deep ? 8 : vpt == 8 ? 12 : 8; }
int wave_complete_rows_per_cu(Source, Tail, int vpt, bool deep) { return deep ? 8 : vpt == 8 ? 16 : 8; }
}  // namespace bnd

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { printf("line %d: %s: %s\n", __LINE__, #c, bnd_last_error()); ++fails; } } while (0)
static void* fake(uint64_t k) { return (void*)(uintptr_t)(0x7F0000000000ull + (k << 36)); }

// The automatic launch shape of a two-partial fold (or complete_only) over `rows` rows of H:
// the one-wavefront width, 0 for a multi-wave shape, -1 on an error. With the stubs above a
// round is 12 rows per CU at 8 vectors per lane and 8 elsewhere for the reads, 16 and 8 for
// the completes, on the 256 CUs assumed without a device.
static int auto_width(int64_t H, int64_t rows, bool complete, int* depth = nullptr) {
  bnd_stream* s = nullptr;
  bnd_owed o = BND_OWED_NONE, o2 = BND_OWED_NONE;
  const void* parts[2] = {fake(4), fake(5)};
  if (bnd_stream_create(&s, rows, H, 0, rows, fake(0), H) != BND_OK) return -1;
  int rc = bnd_written(s, fake(0), H) | bnd_publish_partials(s, parts, 2, H, &o);
  rc |= complete ? bnd_complete_only(s, o, fake(25), H, &o2, nullptr)
                 : bnd_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr);
  bnd_stream_destroy(s);
  int64_t r = 0; int th = 0, v = 0, one = 0;
  if (rc != BND_OK || bnd_last_launch_shape(&r, &th, &v, &one) != BND_OK || r != rows) return -1;
  if (depth && bnd_last_launch_ring_depth(depth) != BND_OK) return -1;
  return one ? v : 0;
}

// The same for a MoE finalize (k = 2 picks per row).
static int auto_width_moe(int64_t H, int64_t rows) {
  bnd_stream* s = nullptr;
  bnd_owed o = BND_OWED_NONE;
  if (bnd_stream_create(&s, rows, H, 0, rows, fake(0), H) != BND_OK) return -1;
  int rc = bnd_written(s, fake(0), H);
  rc |= bnd_publish_moe(s, fake(26), 2 * rows, H, (const int32_t*)fake(27), (const float*)fake(28), 2, &o);
  rc |= bnd_moe_finalize_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr);
  bnd_stream_destroy(s);
  int64_t r = 0; int th = 0, v = 0, one = 0;
  if (rc != BND_OK || bnd_last_launch_shape(&r, &th, &v, &one) != BND_OK || r != rows) return -1;
  return one ? v : 0;
}

// Any automatic launch shape covers its row with a shape some kernel has: one wavefront per row at
// the narrowest even width that covers H (up to 14 for the reads, 16 for the completes), with a
// ring of 2 or the deep ring of its own width (4 .. 8); otherwise whole wavefronts of 1, 2 or 4
// vectors per thread. kind: 0 fold, 1 fp8 fold, 2 complete_only, 3 MoE finalize.
static bool auto_shape_valid(int64_t H, int64_t rows, int kind) {
  bnd_stream* s = nullptr;
  bnd_owed o = BND_OWED_NONE, o2 = BND_OWED_NONE;
  const void* parts[3] = {fake(4), fake(5), fake(6)};
  if (bnd_stream_create(&s, rows, H, 0, rows, fake(0), H) != BND_OK) return false;
  int rc = bnd_written(s, fake(0), H);
  if (kind == 3)
    rc |= bnd_publish_moe(s, fake(26), 2 * rows, H, (const int32_t*)fake(27), (const float*)fake(28), 2, &o);
  else
    rc |= bnd_publish_partials(s, parts, 3, H, &o);
  if (kind == 0) rc |= bnd_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr);
  if (kind == 1)
    rc |= bnd_fold_norm_quant_fp8(s, o, (const float*)fake(1), 1e-6f, (uint8_t*)fake(21), H, (float*)fake(22), nullptr);
  if (kind == 2) rc |= bnd_complete_only(s, o, fake(25), H, &o2, nullptr);
  if (kind == 3) rc |= bnd_moe_finalize_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr);
  bnd_stream_destroy(s);
  int64_t r = 0; int th = 0, v = 0, one = 0, depth = -1;
  if (rc != BND_OK || bnd_last_launch_shape(&r, &th, &v, &one) != BND_OK ||
      bnd_last_launch_ring_depth(&depth) != BND_OK || r != rows)
    return false;
  if (one) {
    const int widest = kind == 2 ? 16 : 14;
    return th == 64 && v % 2 == 0 && v >= 2 && v <= widest && (int64_t)v * 64 * 8 >= H &&
           (v == 2 || (int64_t)(v - 2) * 64 * 8 < H) && (depth == 2 || (depth == v && v >= 4 && v <= 8));
  }
  return th % 64 == 0 && th >= 64 && th <= 1024 && (v == 1 || v == 2 || v == 4) && (int64_t)th * v * 8 >= H &&
         depth == 0;
}

int main() {
  uint64_t lcg = 0x9E3779B97F4A7C15ull;
  auto next = [&lcg](uint64_t n) { lcg = lcg * 6364136223846793005ull + 1442695040888963407ull; return (lcg >> 33) % n; };
  for (int c = 0; c < 400; ++c) {
    const int64_t Hc = 8 * (int64_t)(1 + next(c % 2 ? 1024 : 4096));  // half the cases at H <= 8192
    const int64_t rows = 1 + (int64_t)next(c % 3 ? 4096 : 40000);
    const int kind = c % 4;
    if (!auto_shape_valid(Hc, rows, kind)) {
      printf("automatic shape invalid: H=%lld rows=%lld kind=%d: %s\n", (long long)Hc, (long long)rows, kind,
             bnd_last_error());
      ++fails;
    }
  }
  const int64_t H = 4096;
  bnd_owed o = BND_OWED_NONE, o2 = BND_OWED_NONE;
  const void* parts[8];
  for (int p = 0; p < 8; ++p) parts[p] = fake(4 + p);
  for (int64_t rows : {0, 1, 300, 2048}) {
    bnd_stream* s = nullptr;
    EXPECT(bnd_stream_create(&s, 4096, H, 0, rows, fake(0), H) == BND_OK);
    EXPECT(bnd_fold_norm(s, BND_OWED_NONE, (const float*)fake(1), 1e-6f, fake(2), H, nullptr) == BND_ERR_NOT_STARTED);
    EXPECT(bnd_enter_norm(s, fake(3), H, (const float*)fake(1), 1e-6f, fake(2), H, nullptr) == BND_OK);
    EXPECT(bnd_publish_partials(s, parts, 8, H, &o) == BND_OK);
    EXPECT(bnd_take_output(s) == BND_ERR_PENDING);
    EXPECT(bnd_snapshot(s, o, fake(20), H, nullptr) == BND_OK);
    EXPECT(bnd_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr) == BND_OK);
    EXPECT(bnd_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr) == BND_ERR_FOREIGN_OUTPUT);
    EXPECT(bnd_publish_partials(s, parts, 8, H, &o) == BND_OK);
    EXPECT(bnd_fold_norm_quant_fp8(s, o, (const float*)fake(1), 1e-6f, (uint8_t*)fake(21), H, (float*)fake(22),
                                   nullptr) == BND_OK);
    EXPECT(bnd_publish_partials(s, parts, 8, H, &o) == BND_OK);
    EXPECT(bnd_add_to_output(s, o, fake(23), H, fake(24), H, &o2, nullptr) == BND_OK);
    EXPECT(bnd_complete_only(s, o2, fake(25), H, &o, nullptr) == BND_OK);
    EXPECT(bnd_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr) == BND_OK);
    EXPECT(bnd_publish_moe(s, fake(26), 16384, H, (const int32_t*)fake(27), (const float*)fake(28), 8, &o) == BND_OK);
    EXPECT(bnd_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr) == BND_ERR_WRONG_KIND);
    EXPECT(bnd_stream_set_norm_form(s, BND_NORM_GEMMA) == BND_OK);
    EXPECT(bnd_moe_finalize_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), H, nullptr) == BND_OK);
    EXPECT(bnd_written(s, fake(0), H) == BND_OK);
    EXPECT(bnd_take_output(s) == BND_OK);
    EXPECT(bnd_stream_destroy(s) == BND_OK);
  }
  for (int64_t Hs : {8, 264, 7168, 16384, 32768}) {  // the other launch-shape branches
    bnd_stream* s = nullptr;
    EXPECT(bnd_stream_create(&s, 2048, Hs, 0, 2048, fake(0), Hs) == BND_OK);
    EXPECT(bnd_publish_partials(s, parts, 8, Hs, &o) == BND_OK);
    EXPECT(bnd_fold_norm(s, o, (const float*)fake(1), 1e-6f, fake(2), Hs, nullptr) == BND_OK);
    EXPECT(bnd_stream_destroy(s) == BND_OK);
  }
  int64_t counts[4] = {3, 0, 5, 2}, b = 0, n = 0, t = 0;
  EXPECT(bnd_rsv_share(counts, 4, 2, &b, &n, &t) == BND_OK && b == 3 && n == 5 && t == 10);
  int64_t r = 0; int th = 0, v = 0, one = 0;
  EXPECT(bnd_last_launch_shape(&r, &th, &v, &one) == BND_OK && r == 2048);
  // one wavefront per row from 6 rows per CU, over one round or a last round full enough
  int depth = -1;
  EXPECT(auto_width(4096, 1023, false) == 0);     // under 4 rows per CU
  EXPECT(auto_width(4096, 1024, false, &depth) == 8 && depth == 8);  // 4 .. 7 per CU: the deep ring
  EXPECT(auto_width(4096, 2047, true, &depth) == 8 && depth == 8);
  EXPECT(auto_width(4096, 1535, false) == 8);
  EXPECT(auto_width(4096, 2048, false, &depth) == 8 && depth == 2);  // from 8 rows per CU: two in flight
  EXPECT(auto_width(2048, 1024, false, &depth) == 0 && depth == 0);  // widths 4 and 6: from 6 rows per CU
  EXPECT(auto_width(2048, 1535, false) == 0);
  EXPECT(auto_width(2048, 1536, false, &depth) == 4 && depth == 4);  // 6 .. 7 per CU: the deep ring
  EXPECT(auto_width(3072, 2047, true, &depth) == 6 && depth == 6);
  EXPECT(auto_width(3072, 2048, false, &depth) == 6 && depth == 2);
  EXPECT(auto_width(6144, 1536, false, &depth) == 12 && depth == 2);  // none for the wider rows
  EXPECT(auto_width(4096, 1536, false) == 8);
  EXPECT(auto_width(4096, 3072, false) == 8);     // one round of 3072
  EXPECT(auto_width(4096, 4096, false) == 0);     // last round 1/3 full
  EXPECT(auto_width(4096, 5375, false) == 0);     // just under 3/4
  EXPECT(auto_width(4096, 5376, false) == 8);     // 3/4
  EXPECT(auto_width(4096, 6144, false) == 8);     // two whole rounds
  EXPECT(auto_width(7168, 3072, false) == 0);     // rounds of 2048: half full
  EXPECT(auto_width(7168, 4096, false) == 14);
  EXPECT(auto_width(2048, 2048, false) == 4);     // the narrowest width that covers the row
  EXPECT(auto_width(5120, 2048, false) == 10);
  EXPECT(auto_width(1536, 2048, false) == 0);     // 192 vectors: three per lane, too short
  EXPECT(auto_width(8192, 2048, false) == 0);     // longer than 14 vectors per lane
  EXPECT(auto_width(4096, 5461, true) == 0);      // complete rounds of 4096: just under 1/3
  EXPECT(auto_width(4096, 5462, true) == 8);      // 1/3
  EXPECT(auto_width(7168, 2560, true) == 0);      // rounds of 2048, 1/4 full
  EXPECT(auto_width(7168, 2048 + 682, true) == 0);
  EXPECT(auto_width(7168, 2048 + 683, true) == 14);
  // width 2 (rounds of 2048 with the stubs): rows of 97..128 vectors, from 12 rows per CU
  EXPECT(auto_width(1024, 3071, false) == 0);     // under 12 rows per CU
  EXPECT(auto_width(1024, 4096, false) == 2);     // two whole rounds
  EXPECT(auto_width(1024, 3072, false) == 0);     // last round half full
  EXPECT(auto_width(776, 4096, false) == 2);      // 97 vectors
  EXPECT(auto_width(768, 4096, false) == 0);      // 96 vectors: three quarters of the lanes
  EXPECT(auto_width(1024, 4096, true) == 2);
  EXPECT(auto_width(1032, 4096, false) == 0);     // 129 vectors: width 4, too few to fill it
  EXPECT(auto_width(8192, 2048, true) == 16);     // the completes go to 16 vectors per lane
  EXPECT(auto_width(8200, 2048, true) == 0);
  EXPECT(auto_width_moe(1024, 4096) == 0);        // width 2 is not taken for MoE picks
  EXPECT(auto_width_moe(4096, 2048) == 8);
  EXPECT(auto_width_moe(4096, 1024) == 8 && bnd_last_launch_ring_depth(&depth) == BND_OK && depth == 8);
  EXPECT(auto_width_moe(2048, 1536) == 4 && bnd_last_launch_ring_depth(&depth) == BND_OK && depth == 4);
  EXPECT(auto_width_moe(3072, 1024) == 0);        // the deep ring at width 6: from 6 rows per CU
  printf("host walk: %d failures\n", fails);
  return fails ? 1 : 0;
}
"""

ORACLE_DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include "oracle.c"

/* every operand in its own heap block of exactly the bytes the call may touch */
static void* take(size_t bytes) { void* p = malloc(bytes ? bytes : 1); if (p) memset(p, 0, bytes); return p; }

int main(void) {
  const int64_t T = 5, H = 24, rows = 3, rb = 2, ld = 32;  /* padded rows: ld > H */
  enum { P = 3, K = 2, NE = 7 };
  uint16_t* parts[P];
  for (int p = 0; p < P; ++p) {
    parts[p] = take(((T - 1) * ld + H) * 2);
    for (int64_t i = 0; i < (T - 1) * ld + H; ++i) parts[p][i] = orc_bf16_round((double)((i * 7 + p) % 13) - 6.0);
  }
  uint16_t* res = take(((rows - 1) * ld + H) * 2);
  for (int64_t i = 0; i < (rows - 1) * ld + H; ++i) res[i] = orc_bf16_round(0.25 * (double)(i % 9));
  float* w = take(H * 4);
  for (int64_t h = 0; h < H; ++h) w[h] = 1.0f + 0.01f * (float)h;
  uint16_t* res_out = take(((rows - 1) * ld + H) * 2);
  uint16_t* y = take(((rows - 1) * ld + H) * 2);
  uint8_t* q = take((rows - 1) * ld + H);
  float* scale = take(rows * 4);
  double* xe = take(rows * H * 8);
  double* ye = take(rows * H * 8);
  double* mag = take(rows * H * 8);
  int rc = 0;
  rc |= orc_fold_norm(rows, H, rb, P, (const uint16_t* const*)parts, ld, res, ld, w, 1e-6f, 0, res_out, ld, y,
                      ld, NULL, 0, NULL, xe, ye, mag);
  rc |= orc_fold_norm(rows, H, rb, P, (const uint16_t* const*)parts, ld, NULL, 0, w, 1e-6f, 1, res_out, ld, NULL,
                      0, q, ld, scale, xe, ye, mag);
  rc |= orc_enter_norm(rows, H, res, ld, w, 1e-6f, 0, res_out, ld, y, ld, ye);
  rc |= orc_written_norm(rows, H, res, ld, w, 0.0f, 1, y, ld, ye);
  uint16_t* extra = take(((T - 1) * ld + H) * 2);
  rc |= orc_complete_partials(rows, H, rb, P, (const uint16_t* const*)parts, ld, extra, ld, y, ld, xe, mag);
  rc |= orc_snapshot(rows, H, rb, P, (const uint16_t* const*)parts, ld, res, ld, y, ld, xe, mag);
  rc |= orc_snapshot(rows, H, 0, 0, NULL, ld, res, ld, y, ld, xe, mag);
  uint16_t* E = take(((NE - 1) * ld + H) * 2);
  for (int64_t i = 0; i < (NE - 1) * ld + H; ++i) E[i] = orc_bf16_round(0.5 * (double)(i % 5));
  int32_t* idx = take(T * K * 4);
  float* gate = take(T * K * 4);
  for (int i = 0; i < T * K; ++i) { idx[i] = (i * 3) % (NE + 2) - 1; gate[i] = 0.5f; }  /* some out of range */
  rc |= orc_moe_fold_norm(rows, H, rb, K, E, ld, NE, idx, gate, res, ld, w, 1e-6f, 0, res_out, ld, y, ld, NULL, 0,
                          NULL, xe, ye, mag);
  rc |= orc_moe_fold_norm(rows, H, rb, K, E, ld, NE, idx, gate, NULL, 0, w, 1e-6f, 0, res_out, ld, NULL, 0, q, ld,
                          scale, xe, ye, mag);
  rc |= orc_complete_moe(rows, H, rb, K, E, ld, NE, idx, gate, extra, ld, y, ld, xe, mag);
  for (int c = 0; c < 256; ++c)
    if ((c & 0x7F) != 0x7F) rc |= orc_e4m3_round(orc_e4m3_value((uint8_t)c)) != (uint8_t)c && (c & 0x7F) != 0;
  for (int p = 0; p < P; ++p) free(parts[p]);
  free(res); free(w); free(res_out); free(y); free(q); free(scale); free(xe); free(ye); free(mag);
  free(extra); free(E); free(idx); free(gate);
  printf("oracle walk: rc %d\n", rc);
  return rc ? 1 : 0;
}
"""


def _run(exe):
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=ENV)
    assert out.returncode == 0, out.stdout[-3000:] + out.stderr[-6000:]
    return out.stdout


def test_host_state_machine_under_asan(tmp_path):
    src = tmp_path / "host_walk.cpp"
    src.write_text(HOST_DRIVER)
    exe = tmp_path / "host_walk"
    subprocess.check_call(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", INCLUDE,
                           "-I", CSRC, *SAN, "-o", str(exe), str(src), os.path.join(CSRC, "host.cpp"),
                           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    assert "host walk: 0 failures" in _run(exe)


def test_oracle_under_asan(tmp_path):
    src = tmp_path / "oracle_walk.c"
    src.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_walk"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.dirname(ORACLE_SRC), *SAN, "-o", str(exe), str(src),
                           "-lm"])
    assert "oracle walk: rc 0" in _run(exe)
