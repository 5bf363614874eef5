"""Register budgets of the fold kernels, read from the compiler (no GPU needed).

The launch heuristic gives a row one vector per thread when all rows fit on the chip at once,
counting 32 resident waves per CU, i.e. 8 per SIMD. A wave holds 512 / 8 = 64 VGPRs at that
occupancy, so the fold and read kernels with one or two vectors per thread and up to eight
partial sources must stay within 64 VGPRs and never use scratch. A data-dependent branch around
the Gemma weight offset once pushed the P = 8 fold to 100 VGPRs (half the resident rows, about
a microsecond on the prefill boundary); this test fails on such a change before it reaches a
benchmark. The one-wavefront-per-row read and complete kernels (2 to 14 and 2 to 16 vectors per lane, even,
the source count a runtime argument) are chosen from their occupancy (rows resident at once);
they must keep at least two waves per SIMD (at most 256 VGPRs), also without scratch. No kernel of
either library (every source file, the completes, the MoE reads and the measurement kernels
included) may use scratch: a spill once serialised the 16-source snapshot with four vectors per
thread (636 bytes per lane, a wait on every load), and another made the gathering stream's
eight-vector shape a measure of spilling rather than of memory.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_residual_rmsnorm_bnd_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

# same device flags as the library build
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"),
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--offload-device-only",
         "-Rpass-analysis=kernel-resource-usage"]

NAME = re.compile(r"Function Name: _ZN3bnd11read_kernelILNS_6SourceE(\d)ELi(\d+)ELi(\d)ELb([01])ELb([01])E")
COMPLETE_NAME = re.compile(r"Function Name: _ZN3bnd15complete_kernelILNS_6SourceE(\d)ELi(\d+)ELi(\d)ELb([01])E")
WAVE_NAME = re.compile(r"Function Name: _ZN3bnd16wave_read_kernelILNS_6SourceE(\d)ELi(\d+)ELb([01])ELi(\d+)E")
WAVE_COMPLETE_NAME = re.compile(
    r"Function Name: _ZN3bnd20wave_complete_kernelILNS_6SourceE(\d)ELi(\d+)ELNS_4TailE(\d)ELi(\d+)E")
ANY_NAME = re.compile(r"Function Name: (\S+)")
TAILS = {0: "None", 1: "Extra", 2: "Residual"}
FIELD = re.compile(r"remark: +(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)")
SOURCES = {0: "Partials", 1: "Moe", 2: "Input", 3: "Residual"}


def _resources(tmp_path, files):
    procs = {f: subprocess.Popen([HIPCC, *FLAGS, "-c", os.path.join(CSRC, f), "-o", str(tmp_path / (f + ".o"))],
                                 cwd=CSRC, stderr=subprocess.PIPE, text=True) for f in files}
    table = {}
    for f, p in procs.items():
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-3000:]
        current = None
        for line in err.splitlines():
            m = NAME.search(line)
            if m:  # (kind, sources, vectors per thread, fp8); kind ends in "Nt" for non-temporal stores
                kind = SOURCES[int(m.group(1))] + ("Nt" if m.group(5) == "1" else "")
                current = (kind, int(m.group(2)), int(m.group(3)), m.group(4) == "1")
                table[current] = {}
                continue
            m = COMPLETE_NAME.search(line)
            if m:  # several wavefronts per row: (kind, sources, vectors per thread, False); "Fold": snapshot
                kind = "Complete" + SOURCES[int(m.group(1))] + ("Fold" if m.group(4) == "1" else "")
                current = (kind, int(m.group(2)), int(m.group(3)), False)
                table[current] = {}
                continue
            m = WAVE_NAME.search(line)
            if m:  # one wavefront per row: (kind, ring depth, vectors per lane, fp8)
                current = ("Wave" + SOURCES[int(m.group(1))], int(m.group(4)), int(m.group(2)), m.group(3) == "1")
                table[current] = {}
                continue
            m = WAVE_COMPLETE_NAME.search(line)
            if m:  # one-wavefront complete: (kind, tail and ring depth, vectors per lane, False)
                current = ("WaveComplete" + SOURCES[int(m.group(1))], (TAILS[int(m.group(3))], int(m.group(4))),
                           int(m.group(2)), False)
                table[current] = {}
                continue
            m = ANY_NAME.search(line)
            if m:  # any other kernel (the measurement library's): only its scratch use is checked
                current = ("Other", m.group(1), 0, False)
                table[current] = {}
                continue
            m = FIELD.search(line)
            if m and current is not None and m.group(1) not in table[current]:
                table[current][m.group(1)] = int(m.group(2))
    return table


# every file with kernels: the boundary library's and the measurement library's
KERNEL_SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    return _resources(tmp_path_factory.mktemp("res"), KERNEL_SOURCES)


def test_every_kernel_source_compiled():
    assert KERNEL_SOURCES == ["ceiling.hip", "k_complete.hip", "k_moe.hip", "k_partials.hip", "k_read.hip",
                              "k_wave.hip", "k_wave_complete.hip"], KERNEL_SOURCES


def test_every_instance_reported(resources):
    # 16 source counts x 3 vector counts x bf16/fp8 for partials; 3 vector counts for the enter (bf16
    # only) and 3 x 2 for the read of a Written stream; with one vector per thread also with
    # non-temporal stores
    assert sum(1 for k in resources if k[0] == "Partials") == 96
    assert sum(1 for k in resources if k[0] == "PartialsNt") == 32
    assert sum(1 for k in resources if k[0] == "Input") == 3
    assert not any(k[0].startswith("Input") and k[3] for k in resources), "the enter has no fp8 form"
    assert sum(1 for k in resources if k[0] == "Residual") == 6
    assert sum(1 for k in resources if k[0] in ("InputNt", "ResidualNt")) == 3
    # MoE reads, bf16 only: 16 pick counts x 3 vector counts, and one vector with non-temporal stores
    assert sum(1 for k in resources if k[0] == "Moe") == 48
    assert sum(1 for k in resources if k[0] == "MoeNt") == 16
    # completes: partials, partials plus the residual (snapshot) and MoE picks, 16 x 3 each, and the
    # residual copy (a snapshot of a Written stream) at 3 vector counts
    for kind in ("CompletePartials", "CompletePartialsFold", "CompleteMoe"):
        assert sum(1 for k in resources if k[0] == kind) == 48, kind
    assert sum(1 for k in resources if k[0] == "CompleteResidualFold") == 3
    # the measurement library: mixed and gathering streams at 1, 2, 4, 8 vectors, two empty kernels
    assert sum(1 for k in resources if k[0] == "Other") == 10
    # one wavefront per row: partials bf16 and fp8, MoE bf16, at 2, 4, ..., 14 vectors per lane with
    # a ring of 2, and at 4, 6 and 8 vectors per lane also with the deep ring of as many
    waves = sorted((k[0], k[1], k[2], k[3]) for k in resources if k[0] in ("WavePartials", "WaveMoe"))
    kinds = (("WavePartials", False), ("WavePartials", True), ("WaveMoe", False))
    want = [(kind, 2, vpt, fp8) for vpt in range(2, 15, 2) for kind, fp8 in kinds]
    want += [(kind, vpt, vpt, fp8) for vpt in (4, 6, 8) for kind, fp8 in kinds]
    assert waves == sorted(want), waves


def test_one_wave_completes_reported(resources):
    # partials with no tail, the extra row or the residual; MoE picks with no tail or the extra row
    got = sorted((k[0], k[1], k[2]) for k in resources if k[0].startswith("WaveComplete"))
    kinds = (("WaveCompletePartials", "None"), ("WaveCompletePartials", "Extra"), ("WaveCompletePartials", "Residual"),
             ("WaveCompleteMoe", "None"), ("WaveCompleteMoe", "Extra"))
    want = [(kind, (tail, 2), vpt) for vpt in range(2, 17, 2) for kind, tail in kinds]
    want += [(kind, (tail, vpt), vpt) for vpt in (4, 6, 8) for kind, tail in kinds]  # the deep ring
    assert got == sorted(want), got


def test_one_wave_rows_keep_two_waves_per_simd(resources):
    low = {k: v["VGPRs"] for k, v in resources.items()
           if k[0].startswith("Wave") and (v["VGPRs"] > 256 or v["Occupancy [waves/SIMD]"] < 2)}
    assert not low, f"one-wavefront rows above 256 VGPRs: {low}"


def test_fold_kernels_fit_eight_waves_per_simd(resources):
    kinds = ("Partials", "PartialsNt", "Input", "InputNt", "Residual", "ResidualNt")
    over = {k: v["VGPRs"] for k, v in resources.items()
            if k[2] <= 2 and k[0] in kinds and (not k[0].startswith("Partials") or k[1] <= 8) and v["VGPRs"] > 64}
    assert not over, f"kernels above 64 VGPRs (fewer than 8 waves per SIMD): {over}"


def test_one_vector_moe_reads_fit_eight_waves_per_simd(resources):
    # one vector per thread is chosen when every row of the launch is resident at 8 waves per SIMD
    # (the 256-row share among them): up to eight picks that must hold
    over = {k: v["VGPRs"] for k, v in resources.items()
            if k[0] in ("Moe", "MoeNt") and k[2] == 1 and k[1] <= 8 and v["VGPRs"] > 64}
    assert not over, f"one-vector MoE reads above 64 VGPRs: {over}"


def test_two_vector_fold_register_use(resources):
    # the P = 8 fold with two vectors per thread, bf16 and fp8 outputs: prefill batches above
    # 8 rows per CU and rows up to H = 16384
    for fp8 in (False, True):
        r = resources[("Partials", 8, 2, fp8)]
        assert r["VGPRs"] <= 64 and r["Occupancy [waves/SIMD]"] == 8, r


def test_no_scratch(resources):
    spilled = {k: v["ScratchSize [bytes/lane]"] for k, v in resources.items() if v["ScratchSize [bytes/lane]"]}
    assert not spilled, f"kernels using scratch: {spilled}"
