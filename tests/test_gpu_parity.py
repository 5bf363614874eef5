"""The HIP path against the fp64 oracle, through the C ABI (gfx950 device).

Inputs come from the seeded generator; expected values come only from the
oracle run on those same inputs (chains of calls are replayed by the oracle on
its own outputs). bf16 outputs must lie within 2 bf16 ulp (plus the fp32
accumulation term under cancellation) of the exact value; fp8 codes must match
except <= 0.1% off by one step. Every output buffer is surrounded by guard rows
and padding columns filled with a canary pattern that must survive each call.
"""
import numpy as np
import pytest
import torch

import oracle
import tolerance
import workloads
import reduce_residual_rmsnorm_bnd_amd as bnd

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
CANARY16 = -23131  # 0xA5A5 as int16
CANARY8 = 0xA5
GUARD = 3


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    for opt in (bnd.BND_OPT_FUSED_UNAVAILABLE, bnd.BND_OPT_THREADS_PER_ROW,
                bnd.BND_OPT_VECTORS_PER_THREAD, bnd.BND_OPT_ONE_WAVEFRONT, bnd.BND_OPT_RING_DEPTH):
        bnd.set_option(opt, 0)


def bits(t):
    return workloads.bf16_bits(t.detach().cpu().contiguous())


class forced_shape:
    """Pin the launch shape (threads per row, vectors per thread) for a block of calls; with
    one_wave, the one-wavefront mode instead (ALWAYS: the narrowest one-wavefront kernel that
    covers H, which is how the 4-vector kernel is reached).

    No result depends on the launch shape: the residual is elementwise, and every kernel reduces
    a row's sum of squares in the same order, so y, the fp8 codes and scales are bitwise the same
    under every shape (test_every_launch_shape_gives_the_same_bits)."""

    def __init__(self, threads, vpt, one_wave=bnd.BND_ONE_WAVEFRONT_AUTO, depth=0):
        self.threads, self.vpt, self.one_wave, self.depth = threads, vpt, one_wave, depth

    def __enter__(self):
        bnd.set_option(bnd.BND_OPT_THREADS_PER_ROW, self.threads)
        bnd.set_option(bnd.BND_OPT_VECTORS_PER_THREAD, self.vpt)
        bnd.set_option(bnd.BND_OPT_ONE_WAVEFRONT, self.one_wave)
        bnd.set_option(bnd.BND_OPT_RING_DEPTH, self.depth)

    def __exit__(self, *exc):
        bnd.set_option(bnd.BND_OPT_THREADS_PER_ROW, 0)
        bnd.set_option(bnd.BND_OPT_VECTORS_PER_THREAD, 0)
        bnd.set_option(bnd.BND_OPT_ONE_WAVEFRONT, bnd.BND_ONE_WAVEFRONT_AUTO)
        bnd.set_option(bnd.BND_OPT_RING_DEPTH, 0)


def forced_wave(vpt, depth=2):
    """The one-wavefront kernel of `vpt` vectors per lane (2 .. 16, even): under the ALWAYS mode a
    forced count names the one-wavefront width; a depth of 4, 6 or 8 takes that width's deep ring."""
    return forced_shape(64, vpt, bnd.BND_ONE_WAVEFRONT_ALWAYS, depth)


class Guarded:
    """A [rows, H] view inside a canary-filled buffer with guard rows and padded columns."""

    def __init__(self, rows, H, dtype=torch.bfloat16, pad=0):
        self.rows, self.H, self.pad = rows, H, pad
        self.buf = torch.empty(rows + 2 * GUARD, H + pad, dtype=dtype, device=DEV)
        if dtype == torch.bfloat16:
            self.buf.view(torch.int16).fill_(CANARY16)
        elif dtype == torch.uint8:
            self.buf.fill_(CANARY8)
        else:
            self.buf.view(torch.int32).fill_(-1515870811)
        self.view = self.buf[GUARD:GUARD + rows, :H]

    def from_host(self, t):
        self.view.copy_(t.to(DEV))
        return self

    def check_guards(self, what):
        b = self.buf.cpu()
        if b.dtype == torch.bfloat16:
            b, c = b.view(torch.int16), CANARY16
        elif b.dtype == torch.uint8:
            c = CANARY8
        else:
            b, c = b.view(torch.int32), -1515870811
        outside = torch.ones_like(b, dtype=torch.bool)
        outside[GUARD:GUARD + self.rows, :self.H] = False
        assert torch.all(b[outside] == c), f"{what}: a write landed outside the output"


def check_fold(ref, res_bits, y_bits, w, eps, what):
    a = tolerance.check_bf16(res_bits, ref["x_exact"], ref["mag"], f"{what} residual")
    b = tolerance.check_bf16(y_bits, ref["y_exact"],
                             tolerance.read_s_term(ref["x_exact"], ref["mag"], w, eps), f"{what} y")
    print(f"\n  {what}: residual max {a['max_err_ulp']:.3f} ulp ({a['over_half_ulp']} > 0.5 ulp), "
          f"y max {b['max_err_ulp']:.3f} ulp ({b['over_half_ulp']} > 0.5 ulp) over {a['n']} elements",
          flush=True)


def run_fold(d, *, row_begin=0, rows=None, fp8=False, pad=0, with_residual=True, partials=None,
             gemma=False):
    """One fold through the library; returns host results and the guarded buffers."""
    T, H = d["T"], d["H"]
    rows = T - row_begin if rows is None else rows
    parts = partials if partials is not None else [c.to(DEV) for c in d["partials"]]
    res = Guarded(rows, H, pad=pad)
    if with_residual:
        res.from_host(d["residual"][row_begin:row_begin + rows])
    w = d["weight"].to(DEV)
    s = bnd.bnd_stream_create(T, H, res.view, row_begin, rows)
    if gemma:
        bnd.bnd_stream_set_norm_form(s, bnd.BND_NORM_GEMMA)
    if with_residual:
        bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_partials(s, parts)
    out = {"res": res}
    if fp8:
        q = Guarded(rows, H, torch.uint8, pad=pad)
        sc = torch.full((rows + 2,), -1.0, dtype=torch.float32, device=DEV)
        bnd.bnd_fold_norm_quant_fp8(s, owed, w, d["eps"], q.view, sc[1:rows + 1])
        out.update(q=q, scale_buf=sc)
    else:
        y = Guarded(rows, H, pad=pad)
        bnd.bnd_fold_norm(s, owed, w, d["eps"], y.view)
        out["y"] = y
    torch.cuda.synchronize()
    assert s.state == bnd.BND_WRITTEN and s.has_residual
    out["stream"] = s
    return out


def oracle_fold(orc, d, *, row_begin=0, rows=None, fp8=False, with_residual=True, gemma=False):
    T = d["T"]
    rows = T - row_begin if rows is None else rows
    res = bits(d["residual"][row_begin:row_begin + rows]) if with_residual else None
    return orc.fold_norm([bits(c) for c in d["partials"]], res, d["weight"].numpy(), d["eps"],
                         row_begin=row_begin, rows=rows, fp8=fp8, gemma=gemma)


def assert_fold_matches(orc, d, what, **kw):
    fp8 = kw.get("fp8", False)
    got = run_fold(d, **kw)
    okw = {k: v for k, v in kw.items() if k in ("row_begin", "rows", "fp8", "with_residual", "gemma")}
    ref = oracle_fold(orc, d, **okw)
    w = d["weight"].numpy()
    if kw.get("gemma"):
        w = 1.0 + w.astype(np.float64)  # the read's effective weight, for the tolerance
    got["res"].check_guards(f"{what} residual")
    res_bits = bits(got["res"].view)
    if fp8:
        got["q"].check_guards(f"{what} q")
        sc = got["scale_buf"].cpu().numpy()
        assert sc[0] == -1.0 and sc[-1] == -1.0, "scale written outside its rows"
        tolerance.check_bf16(res_bits, ref["x_exact"], ref["mag"], f"{what} residual")
        f = tolerance.check_fp8(got["q"].view.cpu().numpy(), ref["q"], f"{what} q")
        s = tolerance.check_scale(sc[1:-1], ref["scale"], f"{what} scale")
        print(f"\n  {what}: fp8 off-by-one {f['off_by_one']}/{f['n']}, scale max rel "
              f"{s['max_rel']:.3g}", flush=True)
    else:
        got["y"].check_guards(f"{what} y")
        check_fold(ref, res_bits, bits(got["y"].view), w, d["eps"], what)
    return got, ref


# ------------------------------------------------------------------ the five workloads

def test_tiny_fold(orc):
    assert_fold_matches(orc, workloads.tiny(), "tiny T=16 H=256 P=2")


def test_tiny_enter_and_written_read(orc):
    d = workloads.tiny()
    T, H = d["T"], d["H"]
    res = Guarded(T, H)
    y = Guarded(T, H)
    w = d["weight"].to(DEV)
    s = bnd.bnd_stream_create(T, H, res.view)
    bnd.bnd_enter_norm(s, d["x_in"].to(DEV), w, d["eps"], y.view)
    torch.cuda.synchronize()
    assert s.state == bnd.BND_WRITTEN
    ref = orc.enter_norm(bits(d["x_in"]), w.cpu().numpy(), d["eps"])
    res.check_guards("enter residual")
    y.check_guards("enter y")
    assert np.array_equal(bits(res.view), ref["residual"]), "enter must copy x into the residual"
    zero = np.zeros((T, H))
    tolerance.check_bf16(bits(y.view), ref["y_exact"], zero, "enter y")
    # a stack-entry read of a Written stream skips the enter: y = norm(residual)
    y2 = Guarded(T, H)
    bnd.bnd_enter_norm(s, None, w, d["eps"], y2.view)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y2.view), bits(y.view))
    # the same read through fold_norm with nothing owed, and its fp8 form
    y3 = Guarded(T, H)
    bnd.bnd_fold_norm(s, bnd.BND_OWED_NONE, w, d["eps"], y3.view)
    q = Guarded(T, H, torch.uint8)
    sc = torch.empty(T, dtype=torch.float32, device=DEV)
    bnd.bnd_fold_norm_quant_fp8(s, bnd.BND_OWED_NONE, w, d["eps"], q.view, sc)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y3.view), bits(y.view))
    assert np.array_equal(bits(res.view), ref["residual"]), "a Written read must not update"
    rq = orc.fold_norm([np.zeros((T, H), np.uint16)], ref["residual"], w.cpu().numpy(), d["eps"],
                       fp8=True)
    tolerance.check_fp8(q.view.cpu().numpy(), rq["q"], "written fp8 q")
    tolerance.check_scale(sc.cpu().numpy(), rq["scale"], "written fp8 scale")


def test_prefill_full(orc):
    d = workloads.prefill()
    got, _ = assert_fold_matches(orc, d, "prefill T=2048 H=4096 P=8")
    again = run_fold(d)
    assert torch.equal(again["y"].buf, got["y"].buf), "run-to-run results must be bitwise equal"
    assert torch.equal(again["res"].buf, got["res"].buf)


def test_quantised_full(orc):
    assert_fold_matches(orc, workloads.quantised(), "fp8 T=2048 H=7168 P=8 outliers", fp8=True)


def _moe_device(d):
    return (d["expert_rows"].to(DEV), d["idx"].to(DEV), d["gate"].to(DEV))


def run_moe(orc, d, row_begin, rows, what, gemma=False, terminal=False):
    T, H, k = d["T"], d["H"], d["k"]
    E, idx, gate = _moe_device(d)
    res = Guarded(rows, H).from_host(d["residual"][row_begin:row_begin + rows])
    y = Guarded(rows, H)
    w = d["weight"].to(DEV)
    s = bnd.bnd_stream_create(T, H, res.view, row_begin, rows)
    if gemma:
        bnd.bnd_stream_set_norm_form(s, bnd.BND_NORM_GEMMA)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_moe(s, E, idx, gate, k)
    bnd.bnd_moe_finalize_fold_norm(s, owed, w, d["eps"], y.view)
    if terminal:  # the final norm releases the stream after handing on its output
        bnd.bnd_take_output(s)
    torch.cuda.synchronize()
    assert s.state == (bnd.BND_INITIAL if terminal else bnd.BND_WRITTEN)
    ref = orc.moe_fold_norm(bits(d["expert_rows"]), d["idx"].numpy(), d["gate"].numpy(), k,
                            bits(d["residual"][row_begin:row_begin + rows]), d["weight"].numpy(),
                            d["eps"], row_begin=row_begin, rows=rows, gemma=gemma)
    res.check_guards(f"{what} residual")
    y.check_guards(f"{what} y")
    w_eff = d["weight"].numpy().astype(np.float64) + (1.0 if gemma else 0.0)
    check_fold(ref, bits(res.view), bits(y.view), w_eff, d["eps"], what)
    return res, y


def test_moe_full_and_slice(orc):
    d = workloads.moe()
    full_res, full_y = run_moe(orc, d, 0, d["T"], "MoE T=2048 H=4096 k=8")
    rb, rows = workloads.MOE_SLICE
    full_shape = bnd.last_launch_shape()
    sl_res, sl_y = run_moe(orc, d, rb, rows, "MoE slice rows 768..1023")
    slice_shape = bnd.last_launch_shape()
    print(f"\n  MoE launch shapes: full {full_shape}, slice {slice_shape}", flush=True)
    # the share stores exactly the rows of the full call, each under the library's own launch
    # choice (which differs between the two)
    assert torch.equal(sl_res.view, full_res.view[rb:rb + rows])
    assert torch.equal(sl_y.view, full_y.view[rb:rb + rows])


@pytest.mark.parametrize("T", [1, 8, 32, 128])
def test_decode_chain(orc, T):
    """1 enter + 96 folds (2 boundaries x 48 layers), each boundary with fresh partials."""
    H, P, n_b = 4096, 4, 96
    start = workloads.decode_start(T, H)
    res = Guarded(T, H)
    y = Guarded(T, H)
    s = bnd.bnd_stream_create(T, H, res.view)
    w0 = start["weight"].to(DEV)
    bnd.bnd_enter_norm(s, start["x_in"].to(DEV), w0, 1e-6, y.view)
    ref = orc.enter_norm(bits(start["x_in"]), start["weight"].numpy(), 1e-6)
    o_res = ref["residual"]
    torch.cuda.synchronize()
    tolerance.check_bf16(bits(y.view), ref["y_exact"], np.zeros((T, H)), f"decode T={T} enter")
    worst_res = worst_y = 0.0
    for b in range(n_b):
        d = workloads.decode_boundary(T, b, P, H)
        parts = [c.to(DEV) for c in d["partials"]]
        owed = bnd.bnd_publish_partials(s, parts)
        bnd.bnd_fold_norm(s, owed, d["weight"].to(DEV), d["eps"], y.view)
        torch.cuda.synchronize()
        r = orc.fold_norm([bits(c) for c in d["partials"]], o_res, d["weight"].numpy(), d["eps"])
        a = tolerance.check_bf16(bits(res.view), r["x_exact"], r["mag"], f"decode T={T} b={b} residual")
        c = tolerance.check_bf16(bits(y.view), r["y_exact"],
                                 tolerance.read_s_term(r["x_exact"], r["mag"], d["weight"].numpy(),
                                                       d["eps"]), f"decode T={T} b={b} y")
        worst_res = max(worst_res, a["max_err_ulp"])
        worst_y = max(worst_y, c["max_err_ulp"])
        o_res = r["residual"]
    res.check_guards("decode residual")
    y.check_guards("decode y")
    print(f"\n  decode T={T}: 96 folds, worst residual {worst_res:.3f} ulp, worst y {worst_y:.3f} ulp",
          flush=True)


# ------------------------------------------------------------------ shapes and edge cases

SHAPES = [  # T, H, P, pad, row_begin, rows
    (1, 8, 1, 0, 0, None),
    (3, 264, 3, 8, 0, None),
    (37, 4104, 8, 0, 0, None),
    (6, 7168, 16, 16, 1, 4),
    (2, 32768, 2, 0, 0, None),
    (64, 512, 5, 0, 0, None),
    (5, 16384, 9, 0, 0, None),
    (9, 1016, 13, 0, 0, None),
]


@pytest.mark.parametrize("T,H,P,pad,rb,rows", SHAPES)
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_shapes(orc, T, H, P, pad, rb, rows, fp8):
    d = workloads.fold_inputs(100 + T + H + P, T, H, P)
    assert_fold_matches(orc, d, f"T={T} H={H} P={P} pad={pad} slice={rb}+{rows}", fp8=fp8, pad=pad,
                        row_begin=rb, rows=rows)


@pytest.mark.parametrize("threads,vpt", [(128, 4), (256, 2), (256, 4), (512, 1), (1024, 1),
                                         (320, 2), (192, 4)])
def test_launch_shapes(orc, threads, vpt):
    bnd.set_option(bnd.BND_OPT_THREADS_PER_ROW, threads)
    bnd.set_option(bnd.BND_OPT_VECTORS_PER_THREAD, vpt)
    d = workloads.fold_inputs(7, 33, 4096, 8)
    assert_fold_matches(orc, d, f"launch {threads}x{vpt}")
    assert_fold_matches(orc, d, f"launch {threads}x{vpt} fp8", fp8=True)


@pytest.mark.parametrize("mode", [bnd.BND_ONE_WAVEFRONT_NEVER, bnd.BND_ONE_WAVEFRONT_ALWAYS],
                         ids=["multi_wave", "one_wave"])
def test_many_rows(orc, mode):
    """More rows than a 16-bit grid dimension holds (70001 rows of H = 64), under both launch
    forms, against the oracle on every row: folds with bf16 and fp8 output and a MoE finalize."""
    one = mode == bnd.BND_ONE_WAVEFRONT_ALWAYS
    bnd.set_option(bnd.BND_OPT_ONE_WAVEFRONT, mode)
    d = workloads.fold_inputs(430, 70001, 64, 2)
    for fp8 in (False, True):
        assert_fold_matches(orc, d, f"T=70001 H=64 P=2 {'fp8' if fp8 else 'bf16'} one_wave={one}", fp8=fp8)
        rows, _, _, got_one = bnd.last_launch_shape()
        assert rows == 70001 and got_one == one
    dm = workloads.moe_inputs(431, 70001, 64, 8, 2)
    run_moe(orc, dm, 0, 70001, f"MoE T=70001 H=64 k=2 one_wave={one}")
    assert bnd.last_launch_shape()[3] == one


def test_pending_without_residual(orc):
    d = workloads.fold_inputs(8, 12, 1024, 3)
    assert_fold_matches(orc, d, "no residual", with_residual=False)


def test_outlier_and_zero_rows(orc):
    d = workloads.fold_inputs(9, 6, 2048, 2)
    z = torch.zeros(6, 2048, dtype=torch.bfloat16)
    d["residual"] = d["residual"].clone()
    d["residual"][2] = 0
    d["partials"] = [c.clone() for c in d["partials"]]
    for c in d["partials"]:
        c[2] = 0
        c[4, 100] = 3.0e4
    d["residual"][4, 101] = -2.5e-6
    assert_fold_matches(orc, d, "zero and outlier rows", fp8=True)
    assert_fold_matches(orc, d, "zero and outlier rows bf16")
    del z


def test_moe_edge_cases(orc):
    d = workloads.moe_inputs(11, 40, 1024, 16, 16)  # k = 16 of 16 experts
    idx = d["idx"].clone()
    idx[5] = -1                         # a corrupt index contributes nothing
    idx[17] = d["expert_rows"].shape[0]
    d["idx"] = idx
    run_moe(orc, d, 0, 40, "MoE k=16 with out-of-range indices")
    # nothing, whatever the dropped pick's gate holds
    gate = d["gate"].clone()
    gate[5] = float("nan")
    gate[17] = float("inf")
    d["gate"] = gate
    for shape in ((256, 1), (64, 2, bnd.BND_ONE_WAVEFRONT_ALWAYS)):
        with forced_shape(*shape):
            res, y = run_moe(orc, d, 0, 40, f"MoE k=16, dropped picks with NaN and inf gates, {shape}")
        assert torch.isfinite(y.view.float()).all() and torch.isfinite(res.view.float()).all()
    d1 = workloads.moe_inputs(12, 9, 264, 4, 1)  # k = 1, ragged H
    run_moe(orc, d1, 3, 5, "MoE k=1 slice")


# ------------------------------------------------------------------ invariants on device

def test_invariant_zero_contribution_is_enter(orc):
    d = workloads.fold_inputs(21, 10, 4096, 1)
    T, H = 10, 4096
    zero = [torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)]
    a = run_fold(d, partials=zero)
    res = Guarded(T, H)
    y = Guarded(T, H)
    s = bnd.bnd_stream_create(T, H, res.view)
    bnd.bnd_enter_norm(s, d["residual"].to(DEV), d["weight"].to(DEV), d["eps"], y.view)
    torch.cuda.synchronize()
    assert torch.equal(a["y"].view, y.view) and torch.equal(a["res"].view, res.view)


def test_invariant_written_fold_applies_no_second_update(orc):
    d = workloads.fold_inputs(22, 16, 4096, 4)
    got = run_fold(d)
    s = got["stream"]
    before = got["res"].view.clone()
    y2 = Guarded(16, 4096)
    bnd.bnd_fold_norm(s, bnd.BND_OWED_NONE, d["weight"].to(DEV), d["eps"], y2.view)
    torch.cuda.synchronize()
    assert torch.equal(got["res"].view, before), "a second read must not fold again"
    ref = oracle_fold(orc, d)
    again = orc.written_norm(ref["residual"], d["weight"].numpy(), d["eps"])
    tolerance.check_bf16(bits(y2.view), again["y_exact"], np.zeros((16, 4096)), "written read y")


def test_invariant_moe_over_stacked_partials_is_fold(orc):
    d = workloads.fold_inputs(23, 24, 2048, 4)
    T, H, P = 24, 2048, 4
    a = run_fold(d)
    E = torch.cat([c for c in d["partials"]], 0).to(DEV)
    idx = torch.tensor([[p * T + t for p in range(P)] for t in range(T)], dtype=torch.int32,
                       device=DEV).reshape(-1)
    gate = torch.ones(T * P, dtype=torch.float32, device=DEV)
    res = Guarded(T, H).from_host(d["residual"])
    y = Guarded(T, H)
    s = bnd.bnd_stream_create(T, H, res.view)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_moe(s, E, idx, gate, P)
    bnd.bnd_moe_finalize_fold_norm(s, owed, d["weight"].to(DEV), d["eps"], y.view)
    torch.cuda.synchronize()
    assert torch.equal(y.view, a["y"].view) and torch.equal(res.view, a["res"].view)


def test_invariant_slice_equals_full_rows(orc):
    """A share's rows are bitwise the full call's rows, under the automatic shapes and with the
    full call and the shares under different forced shapes."""
    d = workloads.fold_inputs(24, 64, 4096, 8)
    full = run_fold(d)
    full_fp8 = run_fold(d, fp8=True)
    for shape in (None, (256, 2), (512, 1), (64, 8, bnd.BND_ONE_WAVEFRONT_ALWAYS)):
        for rb, rows in ((0, 8), (24, 16), (56, 8), (63, 1)):
            if shape is None:
                part = run_fold(d, row_begin=rb, rows=rows)
                part_fp8 = run_fold(d, row_begin=rb, rows=rows, fp8=True)
            else:
                with forced_shape(*shape):
                    part = run_fold(d, row_begin=rb, rows=rows)
                    part_fp8 = run_fold(d, row_begin=rb, rows=rows, fp8=True)
            assert torch.equal(part["y"].view, full["y"].view[rb:rb + rows]), (shape, rb, rows)
            assert torch.equal(part["res"].view, full["res"].view[rb:rb + rows])
            assert torch.equal(part_fp8["q"].view, full_fp8["q"].view[rb:rb + rows]), (shape, rb, rows)
            assert torch.equal(part_fp8["scale_buf"][1:rows + 1], full_fp8["scale_buf"][1 + rb:1 + rb + rows])


MULTI_WAVE_SHAPES = [(64, 1), (128, 1), (256, 1), (512, 1), (1024, 1), (64, 2), (128, 2), (256, 2),
                     (320, 2), (512, 2), (64, 4), (128, 4), (192, 4), (256, 4)]


def _launch_shapes(H):
    """Every multi-wave shape and one-wavefront width (ring of two, and the deep ring where it is
    built) that covers a row of H elements: (label, forced_shape arguments, multi-wave?)."""
    nvec = H // 8
    out = [("auto", None, True)]
    out += [(f"{t}x{v}", (t, v), True) for t, v in MULTI_WAVE_SHAPES if t * v >= nvec]
    for w in range(2, 15, 2):
        if 64 * w >= nvec:
            out.append((f"wave{w}", (64, w, bnd.BND_ONE_WAVEFRONT_ALWAYS), False))
            if w in (4, 6, 8):
                out.append((f"wave{w}deep", (64, w, bnd.BND_ONE_WAVEFRONT_ALWAYS, w), False))
    return out


@pytest.mark.parametrize("H", [1016, 3600, 4096, 7168])
def test_every_launch_shape_gives_the_same_bits(orc, H):
    """Every kernel reduces a row's sum of squares in one order, so the residual, y, the fp8 codes
    and their scales are bitwise the same under every launch shape: folds with bf16 and fp8 output,
    the MoE finalize, enter and the read of a Written stream. The automatic shape's results are
    also checked against the oracle."""
    T = 37
    d = workloads.fold_inputs(600 + H, T, H, 8)
    dm = workloads.moe_inputs(700 + H, T, H, 16, 8)

    def call(kind):
        if kind == "fold":
            g = run_fold(d)
            return g["res"].view, g["y"].view
        if kind == "fp8":
            g = run_fold(d, fp8=True)
            return g["res"].view, g["q"].view, g["scale_buf"][1:T + 1]
        if kind == "moe":
            res, y = _moe_only(dm, 0, T)
            return res.view, y.view
        # enter, then the reads of the Written stream it leaves, bf16 and fp8
        res, y, y2, q = Guarded(T, H), Guarded(T, H), Guarded(T, H), Guarded(T, H, torch.uint8)
        sc = torch.full((T,), -1.0, dtype=torch.float32, device=DEV)
        st = bnd.bnd_stream_create(T, H, res.view)
        bnd.bnd_enter_norm(st, d["residual"].to(DEV), d["weight"].to(DEV), d["eps"], y.view)
        bnd.bnd_fold_norm(st, bnd.BND_OWED_NONE, d["weight"].to(DEV), d["eps"], y2.view)
        bnd.bnd_fold_norm_quant_fp8(st, bnd.BND_OWED_NONE, d["weight"].to(DEV), d["eps"], q.view, sc)
        torch.cuda.synchronize()
        q.check_guards("written fp8 read")
        return res.view, y.view, y2.view, q.view, sc

    assert_fold_matches(orc, d, f"H={H} automatic shape")
    assert_fold_matches(orc, d, f"H={H} automatic shape fp8", fp8=True)
    run_moe(orc, dm, 0, T, f"MoE H={H} automatic shape")
    # enter and the Written reads at the automatic shape against the oracle
    res, y, y2, q, sc = call("enter")
    w = d["weight"].numpy()
    ref = orc.enter_norm(bits(d["residual"]), w, d["eps"])
    assert np.array_equal(bits(res), ref["residual"]), "enter must copy x into the residual"
    tolerance.check_bf16(bits(y), ref["y_exact"], np.zeros((T, H)), f"H={H} enter y")
    assert torch.equal(y2, y), "the Written read is the enter's read"
    rq = orc.fold_norm([np.zeros((T, H), np.uint16)], ref["residual"], w, d["eps"], fp8=True)
    tolerance.check_fp8(q.cpu().numpy(), rq["q"], f"H={H} written fp8 q")
    tolerance.check_scale(sc.cpu().numpy(), rq["scale"], f"H={H} written fp8 scale")
    base = {}
    checked = 0
    for label, shape, multi in _launch_shapes(H):
        for kind in ("fold", "fp8", "moe") + (("enter",) if multi else ()):
            if shape is None:
                got = call(kind)
            else:
                with forced_shape(*shape):
                    got = call(kind)
            if kind not in base:
                base[kind] = got
                continue
            for a, b in zip(got, base[kind]):
                assert torch.equal(a, b), f"{kind} under {label} differs from the automatic shape"
            checked += 1
    print(f"\n  H={H}: {checked} calls under forced shapes bitwise equal to the automatic shape", flush=True)


def _moe_only(d, row_begin, rows):
    """The MoE finalize through the library without the oracle: (residual, y) guarded buffers."""
    T, H, k = d["T"], d["H"], d["k"]
    E, idx, gate = _moe_device(d)
    res = Guarded(rows, H).from_host(d["residual"][row_begin:row_begin + rows])
    y = Guarded(rows, H)
    s = bnd.bnd_stream_create(T, H, res.view, row_begin, rows)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_moe(s, E, idx, gate, k)
    bnd.bnd_moe_finalize_fold_norm(s, owed, d["weight"].to(DEV), d["eps"], y.view)
    torch.cuda.synchronize()
    return res, y


# ------------------------------------------------------------------ unfused fallback

def test_complete_only_then_one_source_fold(orc):
    d = workloads.fold_inputs(31, 20, 4096, 8)
    T, H = 20, 4096
    bnd.set_option(bnd.BND_OPT_FUSED_UNAVAILABLE, 1)
    res = Guarded(T, H).from_host(d["residual"])
    y = Guarded(T, H)
    out = Guarded(T, H)
    w = d["weight"].to(DEV)
    s = bnd.bnd_stream_create(T, H, res.view)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_partials(s, [c.to(DEV) for c in d["partials"]])
    with pytest.raises(bnd.BoundaryError) as e:
        bnd.bnd_fold_norm(s, owed, w, d["eps"], y.view)
    assert e.value.status == bnd.BND_ERR_UNAVAILABLE
    owed2 = bnd.bnd_complete_only(s, owed, out.view)
    assert s.state == bnd.BND_PENDING
    bnd.bnd_fold_norm(s, owed2, w, d["eps"], y.view)
    torch.cuda.synchronize()
    for g in (res, y, out):
        g.check_guards("fallback")
    c = orc.complete_partials([bits(p) for p in d["partials"]])
    tolerance.check_bf16(bits(out.view), c["s_exact"], c["mag"], "complete_only out")
    ref = orc.fold_norm([c["out"]], bits(d["residual"]), d["weight"].numpy(), d["eps"])
    check_fold(ref, bits(res.view), bits(y.view), d["weight"].numpy(), d["eps"], "unfused fallback")


def test_moe_complete_only(orc):
    d = workloads.moe_inputs(32, 48, 2048, 32, 8)
    T, H, k = 48, 2048, 8
    E, idx, gate = _moe_device(d)
    rb, rows = 16, 24
    res = Guarded(rows, H).from_host(d["residual"][rb:rb + rows])
    out = Guarded(rows, H)
    y = Guarded(rows, H)
    s = bnd.bnd_stream_create(T, H, res.view, rb, rows)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_moe(s, E, idx, gate, k)
    owed2 = bnd.bnd_complete_only(s, owed, out.view)
    assert s.pending_kind == bnd.BND_KIND_PARTIALS
    bnd.bnd_fold_norm(s, owed2, d["weight"].to(DEV), d["eps"], y.view)
    torch.cuda.synchronize()
    c = orc.complete_moe(bits(d["expert_rows"]), d["idx"].numpy(), d["gate"].numpy(), k,
                         row_begin=rb, rows=rows)
    tolerance.check_bf16(bits(out.view), c["s_exact"], c["mag"], "MoE complete_only out")
    ref = orc.fold_norm([c["out"]], bits(d["residual"][rb:rb + rows]), d["weight"].numpy(),
                        d["eps"])
    check_fold(ref, bits(res.view), bits(y.view), d["weight"].numpy(), d["eps"], "MoE unfused")


# ------------------------------------------------------------------ errors and empty batches

def test_refused_call_writes_nothing(orc):
    d = workloads.fold_inputs(41, 8, 1024, 2)
    res = Guarded(8, 1024).from_host(d["residual"])
    y = Guarded(8, 1024)
    s = bnd.bnd_stream_create(8, 1024, res.view)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_partials(s, [c.to(DEV) for c in d["partials"]])
    res_before = res.buf.clone()
    y_before = y.buf.clone()
    w = d["weight"].to(DEV)
    bad_y = y.buf.view(-1)[1:1 + 8 * 1024].view(8, 1024)  # misaligned by one element
    for call in (lambda: bnd.bnd_fold_norm(s, owed + 1, w, d["eps"], y.view),
                 lambda: bnd.bnd_fold_norm(s, owed, w, -1.0, y.view),
                 lambda: bnd.bnd_fold_norm(s, owed, w, d["eps"], bad_y),
                 lambda: bnd.bnd_fold_norm(s, owed, w, d["eps"], res.view),
                 lambda: bnd.bnd_moe_finalize_fold_norm(s, owed, w, d["eps"], y.view)):
        with pytest.raises(bnd.BoundaryError):
            call()
    torch.cuda.synchronize()
    assert torch.equal(res.buf, res_before) and torch.equal(y.buf, y_before)
    assert s.state == bnd.BND_PENDING
    bnd.bnd_fold_norm(s, owed, w, d["eps"], y.view)
    torch.cuda.synchronize()
    assert not torch.equal(y.buf, y_before)


def test_empty_batch_applies_transitions(orc):
    H = 4096
    s = bnd.bnd_stream_create(0, H, None)
    owed = bnd.bnd_publish_partials(s, [torch.empty(0, H, dtype=torch.bfloat16, device=DEV)] * 2)
    bnd.bnd_fold_norm(s, owed, torch.empty(H, device=DEV), 1e-6,
                      torch.empty(0, H, dtype=torch.bfloat16, device=DEV))
    assert s.state == bnd.BND_WRITTEN
    bnd.bnd_take_output(s)
    assert s.state == bnd.BND_INITIAL


def test_enter_aliasing_input_and_residual(orc):
    d = workloads.tiny()
    T, H = d["T"], d["H"]
    x = Guarded(T, H).from_host(d["x_in"])
    y = Guarded(T, H)
    s = bnd.bnd_stream_create(T, H, x.view)
    bnd.bnd_enter_norm(s, x.view, d["weight"].to(DEV), d["eps"], y.view)
    torch.cuda.synchronize()
    ref = orc.enter_norm(bits(d["x_in"]), d["weight"].numpy(), d["eps"])
    assert np.array_equal(bits(x.view), bits(d["x_in"]))
    tolerance.check_bf16(bits(y.view), ref["y_exact"], np.zeros((T, H)), "aliased enter y")


# ------------------------------------------------------------------ HIP graph replay

def test_graph_replay_matches_eager(orc):
    """A decode-style chain (enter + 4 folds) captured once and replayed several times, with
    eager library work and synchronisations in between; every replay must equal the eager run."""
    T, H, P, n_b = 8, 4096, 4, 4
    start = workloads.decode_start(T, H)
    bounds = [workloads.decode_boundary(T, b, P, H) for b in range(n_b)]
    x_in = start["x_in"].to(DEV)
    w0 = start["weight"].to(DEV)
    parts = [[c.to(DEV) for c in d["partials"]] for d in bounds]
    ws = [d["weight"].to(DEV) for d in bounds]

    def chain(res, y):
        s = bnd.bnd_stream_create(T, H, res)
        bnd.bnd_enter_norm(s, x_in, w0, 1e-6, y)
        for b in range(n_b):
            owed = bnd.bnd_publish_partials(s, parts[b])
            bnd.bnd_fold_norm(s, owed, ws[b], 1e-6, y)
        return s

    res_e = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    y_e = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    chain(res_e, y_e)
    torch.cuda.synchronize()

    res_g = torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)
    y_g = torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain(res_g, y_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        keep = chain(res_g, y_g)
    other_res = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    other_y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    for rep in range(4):
        res_g.zero_()
        y_g.zero_()
        g.replay()
        chain(other_res, other_y)  # eager library work between replays
        torch.cuda.synchronize()
        assert torch.equal(res_g, res_e), f"replay {rep}: residual differs from the eager run"
        assert torch.equal(y_g, y_e), f"replay {rep}: y differs from the eager run"
    del keep


# ------------------------------------------------------------------ Gemma-form weight

def _gemma_inputs(seed, T, H, P):
    d = workloads.fold_inputs(seed, T, H, P, w_mean=0.0, w_std=0.1)  # offsets from one
    return d


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_gemma_fold(orc, fp8):
    d = _gemma_inputs(71, 96, 4096, 8)
    assert_fold_matches(orc, d, f"Gemma weight fold {'fp8' if fp8 else 'bf16'}", fp8=fp8, gemma=True)
    d2 = _gemma_inputs(72, 7, 7168, 3)
    assert_fold_matches(orc, d2, "Gemma weight H=7168 slice", fp8=fp8, gemma=True, row_begin=2,
                        rows=4)


def test_gemma_enter(orc):
    d = _gemma_inputs(73, 12, 2048, 1)
    T, H = 12, 2048
    res = Guarded(T, H)
    y = Guarded(T, H)
    s = bnd.bnd_stream_create(T, H, res.view)
    bnd.bnd_stream_set_norm_form(s, bnd.BND_NORM_GEMMA)
    x = workloads.stack_input(73, T, H)
    bnd.bnd_enter_norm(s, x.to(DEV), d["weight"].to(DEV), d["eps"], y.view)
    torch.cuda.synchronize()
    ref = orc.enter_norm(bits(x), d["weight"].numpy(), d["eps"], gemma=True)
    assert np.array_equal(bits(res.view), ref["residual"])
    tolerance.check_bf16(bits(y.view), ref["y_exact"], np.zeros((T, H)), "Gemma enter y")


def test_gemma_terminal_moe_finalize(orc):
    """The terminal finalize of the guide: a deferred MoE handoff finalized, folded and
    normalised with a GemmaRMSNorm weight in one pass, then the stream is released."""
    d = workloads.moe_inputs(74, 512, 4096, 128, 8, w_mean=0.0, w_std=0.1)
    run_moe(orc, d, 0, 512, "terminal MoE finalize, Gemma weight", gemma=True, terminal=True)
    run_moe(orc, d, 192, 64, "terminal MoE finalize share, Gemma weight", gemma=True, terminal=True)


# ------------------------------------------------------------------ variable-size shares (RSv)

RSV_COUNTS = [300, 0, 511, 256, 257, 1, 400, 322]  # T = 2047, not a multiple of the rank count


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_rsv_shares_tile_the_batch(orc, fp8):
    T = sum(RSV_COUNTS)
    d = workloads.fold_inputs(81, T, 4096, 8)
    key = "q" if fp8 else "y"
    full = run_fold(d, fp8=fp8)
    for r in range(len(RSV_COUNTS)):
        rb, rows, t = bnd.bnd_rsv_share(RSV_COUNTS, r)
        assert t == T
        # each share under the library's own launch choice, which differs with its row count
        part = run_fold(d, row_begin=rb, rows=rows, fp8=fp8)
        assert torch.equal(part["res"].view, full["res"].view[rb:rb + rows])
        assert torch.equal(part[key].view, full[key].view[rb:rb + rows]), f"share {r}"
        if fp8:
            assert torch.equal(part["scale_buf"][1:rows + 1],
                               full["scale_buf"][1 + rb:1 + rb + rows])
    for r in (2, 5):
        rb, rows, _ = bnd.bnd_rsv_share(RSV_COUNTS, r)
        assert_fold_matches(orc, d, f"RSv share {r} ({rows} rows at {rb})", fp8=fp8, row_begin=rb,
                            rows=rows)


def test_rsv_moe_shares(orc):
    counts = [5, 17, 0, 42]
    d = workloads.moe_inputs(82, sum(counts), 2048, 32, 8)
    full_res, full_y = run_moe(orc, d, 0, sum(counts), "MoE RSv full")
    for r in range(len(counts)):
        rb, rows, _ = bnd.bnd_rsv_share(counts, r)
        res, y = run_moe(orc, d, rb, rows, f"MoE RSv share {r}")
        assert torch.equal(res.view, full_res.view[rb:rb + rows])
        assert torch.equal(y.view, full_y.view[rb:rb + rows])


# ------------------------------------------------------------------ add_to_output, snapshot

def test_add_to_output_then_fold(orc):
    T, H, P = 40, 4096, 8
    d = workloads.fold_inputs(83, T, H, P)
    extra = workloads.to_bf16(workloads.normal_f32(83, 12345, (T, H), 0.0, 0.25))
    rb, rows = 8, 24
    res = Guarded(rows, H).from_host(d["residual"][rb:rb + rows])
    out = Guarded(rows, H)
    y = Guarded(rows, H)
    w = d["weight"].to(DEV)
    s = bnd.bnd_stream_create(T, H, res.view, rb, rows)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_partials(s, [c.to(DEV) for c in d["partials"]])
    owed2 = bnd.bnd_add_to_output(s, owed, extra.to(DEV), out.view)
    assert s.state == bnd.BND_PENDING and s.pending_kind == bnd.BND_KIND_PARTIALS
    res_before = res.view.clone()
    bnd.bnd_fold_norm(s, owed2, w, d["eps"], y.view)
    torch.cuda.synchronize()
    for g in (res, out, y):
        g.check_guards("add_to_output")
    c = orc.complete_partials([bits(p) for p in d["partials"]], extra=bits(extra), row_begin=rb,
                              rows=rows)
    tolerance.check_bf16(bits(out.view), c["s_exact"], c["mag"], "add_to_output out")
    assert not torch.equal(res.view, res_before)
    ref = orc.fold_norm([c["out"]], bits(d["residual"][rb:rb + rows]), d["weight"].numpy(), d["eps"])
    check_fold(ref, bits(res.view), bits(y.view), d["weight"].numpy(), d["eps"], "add_to_output fold")


def test_add_to_output_on_moe_handoff(orc):
    d = workloads.moe_inputs(84, 33, 2048, 16, 4)
    T, H, k = 33, 2048, 4
    extra = workloads.to_bf16(workloads.normal_f32(84, 12345, (T, H), 0.0, 0.25))
    E, idx, gate = _moe_device(d)
    res = Guarded(T, H).from_host(d["residual"])
    out = Guarded(T, H)
    s = bnd.bnd_stream_create(T, H, res.view)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_moe(s, E, idx, gate, k)
    bnd.bnd_add_to_output(s, owed, extra.to(DEV), out.view)
    torch.cuda.synchronize()
    c = orc.complete_moe(bits(d["expert_rows"]), d["idx"].numpy(), d["gate"].numpy(), k,
                         extra=bits(extra))
    tolerance.check_bf16(bits(out.view), c["s_exact"], c["mag"], "MoE add_to_output out")


def test_snapshot_leaves_the_owed_work(orc):
    T, H, P = 64, 4096, 8
    d = workloads.fold_inputs(85, T, H, P)
    res = Guarded(T, H).from_host(d["residual"])
    snap = Guarded(T, H)
    y = Guarded(T, H)
    w = d["weight"].to(DEV)
    s = bnd.bnd_stream_create(T, H, res.view)
    bnd.bnd_written(s, res.view)
    owed = bnd.bnd_publish_partials(s, [c.to(DEV) for c in d["partials"]])
    before = res.view.clone()
    bnd.bnd_snapshot(s, owed, snap.view)
    torch.cuda.synchronize()
    assert torch.equal(res.view, before), "a snapshot must not touch the residual"
    assert s.state == bnd.BND_PENDING
    ref = orc.snapshot([bits(c) for c in d["partials"]], bits(d["residual"]))
    tolerance.check_bf16(bits(snap.view), ref["x_exact"], ref["mag"], "snapshot")
    bnd.bnd_fold_norm(s, owed, w, d["eps"], y.view)   # the same handle still folds
    torch.cuda.synchronize()
    assert torch.equal(snap.view, res.view), "the snapshot is the residual the fold stores"
    snap2 = Guarded(T, H)
    bnd.bnd_snapshot(s, bnd.BND_OWED_NONE, snap2.view)  # Written: a copy of the residual
    torch.cuda.synchronize()
    assert torch.equal(snap2.view, res.view)
    for g in (res, snap, snap2, y):
        g.check_guards("snapshot")
    # a MoE handoff is refused and left pending
    dm = workloads.moe_inputs(86, 8, 1024, 8, 2)
    E, idx, gate = _moe_device(dm)
    r2 = Guarded(8, 1024).from_host(dm["residual"])
    s2 = bnd.bnd_stream_create(8, 1024, r2.view)
    bnd.bnd_written(s2, r2.view)
    o2 = bnd.bnd_publish_moe(s2, E, idx, gate, 2)
    with pytest.raises(bnd.BoundaryError) as e:
        bnd.bnd_snapshot(s2, o2, Guarded(8, 1024).view)
    assert e.value.status == bnd.BND_ERR_WRONG_KIND and s2.state == bnd.BND_PENDING


# ------------------------------------------------------------------ one wavefront per row

WAVE = (64, 8)        # threads per row, vectors per thread: the one-wavefront read, H <= 4096
WAVE_WIDE = (64, 14)  # the same for rows of up to 7168 elements

WAVE_SHAPES = [  # vectors per lane, T, H, P, pad, row_begin, rows
    (8, 300, 4096, 8, 0, 0, None),
    (8, 77, 3600, 3, 8, 0, None),     # 450 vectors: the last lanes of the last vector idle
    (8, 5, 264, 16, 0, 0, None),      # 33 vectors: most lanes idle, sixteen sources
    (8, 3, 8, 1, 0, 0, None),         # one vector
    (8, 40, 4096, 2, 16, 7, 20),      # a slice of rows
    (14, 300, 7168, 8, 0, 0, None),
    (14, 61, 6680, 5, 8, 0, None),    # 835 vectors: ragged last vector
    (14, 9, 4104, 16, 0, 0, None),    # just above the narrow kernel's rows, sixteen sources
    (14, 3, 8, 1, 0, 0, None),
    (14, 40, 7168, 2, 16, 11, 25),
    (4, 33, 2048, 8, 0, 0, None),
    (4, 9, 1544, 3, 8, 2, 5),       # 193 vectors: one vector of the last lane column busy
    (4, 5, 8, 16, 0, 0, None),
    (6, 21, 3072, 5, 0, 0, None),
    (6, 7, 2056, 16, 8, 1, 4),      # 257 vectors
    (10, 15, 5120, 8, 0, 0, None),
    (10, 9, 4104, 4, 16, 2, 6),
    (12, 13, 6144, 8, 0, 0, None),
    (12, 5, 5128, 2, 0, 0, None),
    (2, 33, 1024, 8, 0, 0, None),
    (2, 9, 776, 3, 8, 2, 5),        # 97 vectors: one vector of the last lane column busy
    (2, 5, 8, 16, 0, 0, None),
]


@pytest.mark.parametrize("vpt,T,H,P,pad,rb,rows", WAVE_SHAPES)
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_wave_rows(orc, vpt, T, H, P, pad, rb, rows, fp8):
    d = workloads.fold_inputs(300 + T + H + P, T, H, P)
    with forced_wave(vpt):
        assert_fold_matches(orc, d, f"one wave per row x{vpt} T={T} H={H} P={P} slice={rb}+{rows}",
                            fp8=fp8, pad=pad, row_begin=rb, rows=rows)
    assert bnd.last_launch_shape()[1:] == (64, vpt, True)


DEEP_SHAPES = [  # vectors per lane, T, H, P, pad, row_begin, rows: the kernels with the deep ring
    (8, 300, 4096, 8, 0, 0, None),
    (8, 77, 3600, 3, 8, 0, None),
    (8, 9, 3080, 16, 0, 2, 5),      # 385 vectors: the narrowest rows of the 8-wide kernel
    (8, 3, 8, 1, 0, 0, None),
    (6, 150, 3072, 4, 0, 0, None),
    (6, 21, 2056, 16, 0, 3, 17),    # 257 vectors: the narrowest rows of the 6-wide kernel
    (4, 200, 2048, 8, 0, 0, None),
    (4, 31, 1544, 5, 8, 1, 29),     # 193 vectors
    (4, 3, 8, 1, 0, 0, None),
]


@pytest.mark.parametrize("vpt,T,H,P,pad,rb,rows", DEEP_SHAPES)
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_deep_ring_rows(orc, vpt, T, H, P, pad, rb, rows, fp8):
    """The deep ring (every vector of a source in flight) against the oracle, and bitwise against
    the ring of two: one wavefront sums every element in the same order whatever the depth."""
    d = workloads.fold_inputs(460 + T + P, T, H, P)
    with forced_wave(vpt, depth=vpt):
        a, _ = assert_fold_matches(orc, d, f"deep ring x{vpt} T={T} H={H} P={P} slice={rb}+{rows}", fp8=fp8,
                                   pad=pad, row_begin=rb, rows=rows)
        assert bnd.last_launch_shape()[1:] == (64, vpt, True) and bnd.last_launch_ring_depth() == vpt
    with forced_wave(vpt):
        b = run_fold(d, fp8=fp8, pad=pad, row_begin=rb, rows=rows)
        assert bnd.last_launch_ring_depth() == 2
    assert torch.equal(a["res"].buf, b["res"].buf)
    if fp8:
        assert torch.equal(a["q"].buf, b["q"].buf) and torch.equal(a["scale_buf"], b["scale_buf"])
    else:
        assert torch.equal(a["y"].buf, b["y"].buf)


@pytest.mark.parametrize("vpt", [8, 6, 4])
def test_deep_ring_moe_and_completes(orc, vpt):
    """The deep ring for the MoE finalize (out-of-range picks included) and the completes, against
    the oracle and bitwise against the ring of two."""
    H = vpt * 512
    d = workloads.moe_inputs(470 + vpt, 40, H, 16, 8)
    idx = d["idx"].clone()
    idx[9] = -1
    idx[30] = d["expert_rows"].shape[0]
    d["idx"] = idx
    with forced_wave(vpt, depth=vpt):
        ra, ya = run_moe(orc, d, 3, 30, f"deep ring x{vpt} MoE k=8")
        assert bnd.last_launch_ring_depth() == vpt
    with forced_wave(vpt):
        rb_, yb = run_moe(orc, d, 3, 30, f"ring of two x{vpt} MoE k=8")
    assert torch.equal(ra.buf, rb_.buf) and torch.equal(ya.buf, yb.buf)
    dp = workloads.fold_inputs(471 + vpt, 37, H, 8)
    extra = workloads.to_bf16(workloads.normal_f32(471 + vpt, 12345, (37, H), 0.0, 0.25))
    for kind in ("complete_only", "add_to_output", "snapshot"):
        ex = extra if kind == "add_to_output" else None
        with forced_wave(vpt, depth=vpt):
            a = _complete(dp, kind, row_begin=2, rows=33, extra=ex)
            assert bnd.last_launch_ring_depth() == vpt
        with forced_wave(vpt):
            b = _complete(dp, kind, row_begin=2, rows=33, extra=ex)
        e, mag = _oracle_complete(orc, dp, kind, row_begin=2, rows=33, extra=ex)
        tolerance.check_bf16(bits(a.view), e, mag, f"deep ring {kind}")
        assert torch.equal(a.buf, b.buf), kind


WAVE_WIDTHS = [(8, 4096), (14, 7168), (4, 2048), (6, 3072), (10, 5120), (12, 6144), (2, 1024)]
WAVE_COMPLETE_WIDTHS = WAVE_WIDTHS + [(16, 8192)]  # the completes go one width further


@pytest.mark.parametrize("vpt,H", WAVE_WIDTHS, ids=lambda v: str(v))
def test_wave_rows_edge_cases(orc, vpt, H):
    d = workloads.fold_inputs(31, 12, H, 3)
    d1 = workloads.fold_inputs(34, 12, H, 1)
    with forced_wave(vpt):
        assert_fold_matches(orc, d, "one wave per row, no residual", with_residual=False)
        assert_fold_matches(orc, d, "one wave per row, no residual fp8", with_residual=False, fp8=True)
        # one partial: the source after it is the (empty) residual
        assert_fold_matches(orc, d1, "one wave per row, one partial, no residual", with_residual=False)
        assert_fold_matches(orc, d1, "one wave per row, one partial, no residual fp8", with_residual=False, fp8=True)
        assert_fold_matches(orc, d, "one wave per row, Gemma weight", gemma=True)
        assert_fold_matches(orc, d, "one wave per row, Gemma weight fp8", gemma=True, fp8=True)
    # zero rows: y = 0, scale 0 and +0 codes; a large outlier row
    d["partials"] = [c.clone() for c in d["partials"]]
    d["residual"] = d["residual"].clone()
    for c in d["partials"]:
        c[2].zero_()
        c[5, 17] = 3.0e4
    d["residual"][2].zero_()
    with forced_wave(vpt):
        assert_fold_matches(orc, d, "one wave per row, zero and outlier rows")
        assert_fold_matches(orc, d, "one wave per row, zero and outlier rows fp8", fp8=True)


@pytest.mark.parametrize("vpt,H", WAVE_WIDTHS, ids=lambda v: str(v))
def test_wave_rows_residual_matches_other_shapes(orc, vpt, H):
    """One wavefront per row and the multi-wave shape give bitwise the same residual and y."""
    d = workloads.fold_inputs(32, 64, H, 8)
    with forced_wave(vpt):
        a = run_fold(d)
    with forced_shape(512, 2):
        b = run_fold(d)
    assert torch.equal(a["res"].view, b["res"].view)
    assert torch.equal(a["y"].view, b["y"].view)


def test_wave_rows_moe(orc):
    d = workloads.moe_inputs(33, 100, 4096, 16, 8)
    idx = d["idx"].clone()
    idx[9] = -1
    idx[30] = d["expert_rows"].shape[0]  # out of range: contributes nothing
    d["idx"] = idx
    with forced_shape(*WAVE):
        run_moe(orc, d, 0, 100, "one wave per row, MoE k=8 with out-of-range picks")
        run_moe(orc, d, 40, 33, "one wave per row, MoE slice", gemma=True)
    d16 = workloads.moe_inputs(34, 9, 3600, 16, 16)
    with forced_shape(*WAVE):
        run_moe(orc, d16, 0, 9, "one wave per row, MoE k=16 H=3600")
    dw = workloads.moe_inputs(37, 70, 7168, 16, 8)
    idx = dw["idx"].clone()
    idx[3] = -5
    dw["idx"] = idx
    with forced_shape(*WAVE_WIDE):
        run_moe(orc, dw, 0, 70, "one wave per row x14, MoE k=8 H=7168")
        run_moe(orc, dw, 21, 30, "one wave per row x14, MoE slice", gemma=True)
    dr = workloads.moe_inputs(38, 6, 5000, 8, 3)
    with forced_shape(*WAVE_WIDE):
        run_moe(orc, dr, 0, 6, "one wave per row x14, MoE k=3 H=5000")
    for vpt, H in ((4, 2048), (6, 2600), (10, 5120), (12, 6104), (2, 1016)):
        dv = workloads.moe_inputs(40 + vpt, 20, H, 16, 8)
        with forced_wave(vpt):
            run_moe(orc, dv, 3, 15, f"one wave per row x{vpt}, MoE k=8 H={H}")
        assert bnd.last_launch_shape()[1:] == (64, vpt, True)


def test_wave_rows_moe_over_stacked_partials_is_fold(orc):
    d = workloads.fold_inputs(35, 24, 4096, 4)
    T, H, P = 24, 4096, 4
    with forced_shape(*WAVE):
        a = run_fold(d)
        E = torch.cat([c for c in d["partials"]], 0).to(DEV)
        idx = torch.tensor([[p * T + t for p in range(P)] for t in range(T)], dtype=torch.int32,
                           device=DEV).reshape(-1)
        gate = torch.ones(T * P, dtype=torch.float32, device=DEV)
        res = Guarded(T, H).from_host(d["residual"])
        y = Guarded(T, H)
        s = bnd.bnd_stream_create(T, H, res.view)
        bnd.bnd_written(s, res.view)
        owed = bnd.bnd_publish_moe(s, E, idx, gate, P)
        bnd.bnd_moe_finalize_fold_norm(s, owed, d["weight"].to(DEV), d["eps"], y.view)
        torch.cuda.synchronize()
    assert torch.equal(y.view, a["y"].view) and torch.equal(res.view, a["res"].view)


def test_wave_rows_refused_where_no_kernel(orc):
    """One wavefront per row of a given width (2 to 14 vectors per lane, rows of up to 512 times
    the width) exists only for calls with owed work and rows it covers: a forced width that does
    not cover the row (8 for H = 4104, 14 for H = 7176) and a call without owed work are refused
    before anything is launched, and so is the ALWAYS mode for rows longer than 7168."""
    d = workloads.fold_inputs(36, 4, 4104, 2)
    with forced_shape(*WAVE):
        with pytest.raises(bnd.BoundaryError) as e:
            run_fold(d)
        assert e.value.status == bnd.BND_ERR_NO_PATH
    d = workloads.fold_inputs(39, 4, 7176, 2)
    with forced_shape(*WAVE_WIDE):
        with pytest.raises(bnd.BoundaryError) as e:
            run_fold(d)
        assert e.value.status == bnd.BND_ERR_NO_PATH
        res = Guarded(4, 4096)
        y = Guarded(4, 4096)
        s = bnd.bnd_stream_create(4, 4096, res.view)
        with pytest.raises(bnd.BoundaryError) as e:
            bnd.bnd_enter_norm(s, torch.zeros(4, 4096, dtype=torch.bfloat16, device=DEV),
                               torch.ones(4096, device=DEV), 1e-6, y.view)
        assert e.value.status == bnd.BND_ERR_NO_PATH
    torch.cuda.synchronize()
    res.check_guards("refused enter residual")
    y.check_guards("refused enter y")
    d = workloads.fold_inputs(41, 4, 7176, 2)
    with forced_shape(0, 0, bnd.BND_ONE_WAVEFRONT_ALWAYS):
        with pytest.raises(bnd.BoundaryError) as e:
            run_fold(d)
        assert e.value.status == bnd.BND_ERR_NO_PATH
    # the completes go to 8192 (16 vectors per lane) and no further
    d = workloads.fold_inputs(43, 4, 8200, 2)
    with forced_shape(0, 0, bnd.BND_ONE_WAVEFRONT_ALWAYS):
        with pytest.raises(bnd.BoundaryError) as e:
            _complete(d, "complete_only")
        assert e.value.status == bnd.BND_ERR_NO_PATH and "8192" in str(e.value)
    # NEVER keeps the multi-wave shapes even where the automatic choice takes one wavefront
    d = workloads.fold_inputs(42, 2048, 4096, 2)
    with forced_shape(0, 0, bnd.BND_ONE_WAVEFRONT_NEVER):
        run_fold(d)
    assert bnd.last_launch_shape()[3] is False


# ------------------------------------------------------------------ one wavefront per row: complete

def _complete(d, kind, *, row_begin=0, rows=None, extra=None, moe=False, with_residual=True):
    """complete_only / add_to_output / snapshot through the library under the current launch
    shape; checks that the residual is untouched and returns the guarded output buffer."""
    T, H = d["T"], d["H"]
    rows = T - row_begin if rows is None else rows
    res = Guarded(rows, H)
    if with_residual:
        res.from_host(d["residual"][row_begin:row_begin + rows])
    out = Guarded(rows, H)
    s = bnd.bnd_stream_create(T, H, res.view, row_begin, rows)
    if with_residual:
        bnd.bnd_written(s, res.view)
    if moe:
        E, idx, gate = _moe_device(d)
        owed = bnd.bnd_publish_moe(s, E, idx, gate, d["k"])
    else:
        owed = bnd.bnd_publish_partials(s, [c.to(DEV) for c in d["partials"]])
    before = res.view.clone()
    if kind == "complete_only":
        bnd.bnd_complete_only(s, owed, out.view)
    elif kind == "add_to_output":
        bnd.bnd_add_to_output(s, owed, extra.to(DEV), out.view)
    else:
        bnd.bnd_snapshot(s, owed, out.view)
    torch.cuda.synchronize()
    out.check_guards(f"{kind} out")
    res.check_guards(f"{kind} residual")
    assert torch.equal(res.view, before), f"{kind} must not touch the residual"
    return out


def _oracle_complete(orc, d, kind, *, row_begin=0, rows=None, extra=None, moe=False, with_residual=True):
    T = d["T"]
    rows = T - row_begin if rows is None else rows
    ex = None if extra is None else bits(extra)
    if moe:
        c = orc.complete_moe(bits(d["expert_rows"]), d["idx"].numpy(), d["gate"].numpy(), d["k"],
                             row_begin=row_begin, rows=rows, extra=ex)
        return c["s_exact"], c["mag"]
    parts = [bits(c) for c in d["partials"]]
    if kind == "snapshot":
        r = bits(d["residual"][row_begin:row_begin + rows]) if with_residual else None
        c = orc.snapshot(parts, r, row_begin=row_begin, rows=rows)
        return c["x_exact"], c["mag"]
    c = orc.complete_partials(parts, row_begin=row_begin, rows=rows, extra=ex)
    return c["s_exact"], c["mag"]


WAVE_COMPLETE_SHAPES = [  # vectors per lane, T, H, P, row_begin, rows
    (8, 50, 4096, 8, 0, None),
    (8, 21, 3600, 1, 3, 15),      # one source: the stored pass is the only pass; ragged rows
    (14, 30, 7168, 8, 0, None),
    (14, 17, 6680, 3, 5, 9),
    (4, 25, 2048, 8, 2, 20),
    (4, 9, 1000, 1, 0, None),
    (6, 11, 2600, 5, 0, None),
    (10, 13, 5120, 8, 1, 10),
    (12, 7, 6144, 2, 0, None),
    (2, 19, 1024, 8, 1, 16),
    (2, 6, 520, 1, 0, None),
    (16, 12, 8192, 8, 0, None),
    (16, 7, 7176, 3, 1, 5),       # 897 vectors: just past the reads' widest kernel
]


@pytest.mark.parametrize("vpt,T,H,P,rb,rows", WAVE_COMPLETE_SHAPES)
@pytest.mark.parametrize("kind", ["complete_only", "add_to_output", "snapshot"])
def test_wave_complete(orc, kind, vpt, T, H, P, rb, rows):
    """The one-wavefront complete against the oracle, and bitwise against the multi-wave shape
    (the sums run in the same order)."""
    d = workloads.fold_inputs(400 + T + P, T, H, P)
    extra = (workloads.to_bf16(workloads.normal_f32(400 + T, 12345, (T, H), 0.0, 0.25))
             if kind == "add_to_output" else None)
    what = f"one wave per row x{vpt} {kind} T={T} H={H} P={P} slice={rb}+{rows}"
    print(f"\n  {what}", flush=True)
    with forced_wave(vpt):
        a = _complete(d, kind, row_begin=rb, rows=rows, extra=extra)
    assert bnd.last_launch_shape()[1:] == (64, vpt, True)
    b = _complete(d, kind, row_begin=rb, rows=rows, extra=extra)  # the automatic shape
    ex, mag = _oracle_complete(orc, d, kind, row_begin=rb, rows=rows, extra=extra)
    tolerance.check_bf16(bits(a.view), ex, mag, what)
    assert torch.equal(a.view.view(torch.int16), b.view.view(torch.int16)), f"{what}: differs from the other shape"


@pytest.mark.parametrize("P", [8, 16])
def test_multi_wave_completes_every_shape(orc, P):
    """complete_only, add_to_output, snapshot and the MoE complete under every multi-wave shape that
    covers the row, four vectors per thread included (where the many-source snapshot kernels once
    spilled to scratch): each against the oracle, and bitwise equal to the automatic shape."""
    T, H = 37, 4096
    d = workloads.fold_inputs(900 + P, T, H, P)
    dm = workloads.moe_inputs(910 + P, T, H, P, P)
    extra = workloads.to_bf16(workloads.normal_f32(920 + P, 12345, (T, H), 0.0, 0.25))
    kinds = {"complete_only": (d, False, None), "add_to_output": (d, False, extra), "snapshot": (d, False, None),
             "moe complete_only": (dm, True, None)}
    exact = {}
    for kind, (inp, moe, ex) in kinds.items():
        exact[kind] = _oracle_complete(orc, inp, kind.split()[-1], extra=ex, moe=moe)
    shapes = [("auto", None)] + [(f"{t}x{v}", (t, v)) for t, v in MULTI_WAVE_SHAPES if t * v >= H // 8]
    base = {}

    def written_snapshot():
        # a snapshot of a Written stream: a copy of the residual
        res = Guarded(T, H).from_host(d["residual"])
        out = Guarded(T, H)
        s = bnd.bnd_stream_create(T, H, res.view)
        bnd.bnd_written(s, res.view)
        bnd.bnd_snapshot(s, bnd.BND_OWED_NONE, out.view)
        torch.cuda.synchronize()
        out.check_guards("written snapshot")
        assert torch.equal(out.view, res.view), "a snapshot of a Written stream is its residual"

    for label, shape in shapes:
        for kind, (inp, moe, ex) in kinds.items():
            if shape is None:
                out = _complete(inp, kind.split()[-1], extra=ex, moe=moe)
            else:
                with forced_shape(*shape):
                    out = _complete(inp, kind.split()[-1], extra=ex, moe=moe)
                assert bnd.last_launch_shape()[1:] == (shape[0], shape[1], False)
            what = f"{kind} P/k={P} under {label}"
            tolerance.check_bf16(bits(out.view), *exact[kind], what)
            if kind not in base:
                base[kind] = out.view.clone()
            else:
                assert torch.equal(out.view, base[kind]), f"{what} differs from the automatic shape"
        if shape is None:
            written_snapshot()
        else:
            with forced_shape(*shape):
                written_snapshot()
    print(f"\n  P/k={P}: {len(kinds) + 1} calls under {len(shapes)} shapes", flush=True)


@pytest.mark.parametrize("kind", ["fold", "fp8", "moe", "complete_only", "add_to_output", "snapshot",
                                  "moe complete_only"])
def test_every_multi_wave_instance(orc, kind):
    """Every multi-wave kernel instance the call can reach, each against the oracle: source counts
    1 .. 16 (partials or picks, each its own kernel) at one, two and four vectors per thread; the
    reads at one vector also with both store policies (5 rows, fewer than the CUs, take the
    non-temporal-store kernels; 260 rows the others)."""
    H = 4096
    cases = [(5, (512, 1)), (37, (256, 2)), (37, (128, 4))]
    if kind in ("fold", "fp8", "moe"):
        cases.append((260, (512, 1)))
    checked = 0
    for n in range(1, 17):
        for T, shape in cases:
            what = f"{kind} n={n} T={T} under {shape[0]}x{shape[1]}"
            seed = 1000 + 17 * n + T
            with forced_shape(*shape):
                if kind in ("fold", "fp8"):
                    assert_fold_matches(orc, workloads.fold_inputs(seed, T, H, n), what, fp8=kind == "fp8")
                elif kind == "moe":
                    run_moe(orc, workloads.moe_inputs(seed, T, H, max(n, 2), n), 0, T, what)
                else:
                    moe = kind.startswith("moe")
                    d = workloads.moe_inputs(seed, T, H, max(n, 2), n) if moe else workloads.fold_inputs(seed, T, H, n)
                    ex = (workloads.to_bf16(workloads.normal_f32(seed, 12345, (T, H), 0.0, 0.25))
                          if kind == "add_to_output" else None)
                    out = _complete(d, kind.split()[-1], extra=ex, moe=moe)
                    tolerance.check_bf16(bits(out.view), *_oracle_complete(orc, d, kind.split()[-1], extra=ex, moe=moe),
                                         what)
            assert bnd.last_launch_shape() == (T, shape[0], shape[1], False), what
            checked += 1
    print(f"\n  {kind}: {checked} instances against the oracle", flush=True)


@pytest.mark.parametrize("vpt,H", WAVE_COMPLETE_WIDTHS, ids=lambda v: str(v))
def test_wave_complete_moe(orc, vpt, H):
    d = workloads.moe_inputs(410, 40, H, 16, 8)
    idx = d["idx"].clone()
    idx[5] = -1
    idx[77] = d["expert_rows"].shape[0]
    d["idx"] = idx
    extra = workloads.to_bf16(workloads.normal_f32(410, 12345, (40, H), 0.0, 0.25))
    for kind, ex in (("complete_only", None), ("add_to_output", extra)):
        what = f"one wave per row x{vpt} MoE {kind} H={H}"
        with forced_wave(vpt):
            a = _complete(d, kind, row_begin=4, rows=30, extra=ex, moe=True)
        b = _complete(d, kind, row_begin=4, rows=30, extra=ex, moe=True)
        e, mag = _oracle_complete(orc, d, kind, row_begin=4, rows=30, extra=ex, moe=True)
        tolerance.check_bf16(bits(a.view), e, mag, what)
        assert torch.equal(a.view.view(torch.int16), b.view.view(torch.int16)), what
    d1 = workloads.moe_inputs(411, 6, H, 4, 1)  # one pick: the stored pass is the only pass
    with forced_wave(vpt):
        a = _complete(d1, "complete_only", moe=True)
    e, mag = _oracle_complete(orc, d1, "complete_only", moe=True)
    tolerance.check_bf16(bits(a.view), e, mag, "one wave per row MoE k=1 complete_only")


@pytest.mark.parametrize("vpt,H", WAVE_COMPLETE_WIDTHS, ids=lambda v: str(v))
def test_wave_complete_edge_cases(orc, vpt, H):
    d = workloads.fold_inputs(412, 12, H, 4)
    # signed zeros: sums of -0 store +0 under both shapes
    d["partials"] = [c.clone() for c in d["partials"]]
    for c in d["partials"]:
        c[3].fill_(-0.0)
    with forced_wave(vpt):
        a = _complete(d, "complete_only")
    b = _complete(d, "complete_only")
    assert torch.equal(a.view.view(torch.int16), b.view.view(torch.int16))
    assert int((a.view[3].view(torch.int16) != 0).sum()) == 0, "a sum of -0 stores +0"
    # a snapshot of a Pending stream without a residual is bf16(s), with four partials and with one
    d1 = workloads.fold_inputs(413, 12, H, 1)
    for dd, what in ((d, "snapshot without a residual"), (d1, "one-partial snapshot without a residual")):
        with forced_wave(vpt):
            a = _complete(dd, "snapshot", with_residual=False)
        e, mag = _oracle_complete(orc, dd, "snapshot", with_residual=False)
        tolerance.check_bf16(bits(a.view), e, mag, what)
    # a snapshot of a Written stream copies the residual: no one-wavefront kernel, refused
    res = Guarded(12, H).from_host(d["residual"])
    out = Guarded(12, H)
    s = bnd.bnd_stream_create(12, H, res.view)
    bnd.bnd_written(s, res.view)
    with forced_wave(vpt):
        with pytest.raises(bnd.BoundaryError) as e:
            bnd.bnd_snapshot(s, bnd.BND_OWED_NONE, out.view)
    assert e.value.status == bnd.BND_ERR_NO_PATH
    torch.cuda.synchronize()
    out.check_guards("refused snapshot")
    assert int((out.view.view(torch.int16) != CANARY16).sum()) == 0, "a refused call wrote its output"


def test_wave_rows_over_several_rounds(orc):
    """Launches for which the automatic shape takes one wavefront per row over more than one round
    of resident rows, against the oracle on every row: a fold, an fp8 fold and a MoE finalize over
    two whole rounds (4096 rows at H = 7168) and a complete_only whose last round is half full
    (6144 rows at H = 4096), as row counts of 16 and 24 per CU."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T = 16 * cus  # 4096 rows on 256 CUs
    d = workloads.fold_inputs(420, T, 7168, 3)
    assert_fold_matches(orc, d, f"fold T={T} H=7168 P=3, two rounds")
    assert bnd.last_launch_shape() == (T, 64, 14, True)
    assert_fold_matches(orc, d, f"fp8 fold T={T} H=7168 P=3, two rounds", fp8=True)
    assert bnd.last_launch_shape() == (T, 64, 14, True)
    dm = workloads.moe_inputs(422, T, 7168, 16, 4)
    run_moe(orc, dm, 0, T, f"MoE finalize T={T} H=7168 k=4, two rounds")
    assert bnd.last_launch_shape() == (T, 64, 14, True)
    del dm
    T = 24 * cus  # 6144 rows on 256 CUs
    d = workloads.fold_inputs(421, T, 4096, 3)
    out = _complete(d, "complete_only")
    assert bnd.last_launch_shape() == (T, 64, 8, True)
    ex, mag = _oracle_complete(orc, d, "complete_only")
    tolerance.check_bf16(bits(out.view), ex, mag, f"complete_only T={T} H=4096 P=3, 1.5 rounds")


def test_automatic_one_wave_at_its_shortest_rows(orc):
    """The shortest rows the automatic shape gives one wavefront (H = 1544: 193 vectors, so only
    lane 0 holds a fourth) and the longest it does not (H = 1536), at 6 rows per CU, against the
    oracle."""
    T = 6 * torch.cuda.get_device_properties(0).multi_processor_count
    for H, one in ((1544, True), (1536, False)):
        d = workloads.fold_inputs(424 + H, T, H, 3)
        for fp8 in (False, True):
            assert_fold_matches(orc, d, f"fold T={T} H={H} P=3 fp8={fp8}", fp8=fp8)
            assert bnd.last_launch_shape()[3] is one
            if one:
                assert bnd.last_launch_shape()[2] == 4


def test_automatic_launch_shapes():
    """The launch shapes the library picks: one wavefront per row from 6 rows per CU where a
    launch's rows fit on the chip in one round, or where its last round of resident rows is full
    enough (3/4 for the reads, 1/3 for the completes). Row counts are written for the 256 CUs of
    an MI355X and scaled to the device's CU count (c)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def c(n):
        return n * cus // 256
    w = torch.ones(8192, device=DEV)

    def fold(T, H, P, fp8=False, kind="fold"):
        res = torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)
        parts = [torch.zeros(T, H, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
        s = bnd.bnd_stream_create(T, H, res)
        bnd.bnd_written(s, res)
        owed = bnd.bnd_publish_partials(s, parts)
        if kind == "complete_only":
            bnd.bnd_complete_only(s, owed, torch.empty(T, H, dtype=torch.bfloat16, device=DEV))
        elif kind == "snapshot":
            bnd.bnd_snapshot(s, owed, torch.empty(T, H, dtype=torch.bfloat16, device=DEV))
        elif fp8:
            bnd.bnd_fold_norm_quant_fp8(s, owed, w[:H], 1e-6, torch.empty(T, H, dtype=torch.uint8, device=DEV),
                                        torch.empty(T, dtype=torch.float32, device=DEV))
        else:
            bnd.bnd_fold_norm(s, owed, w[:H], 1e-6, torch.empty(T, H, dtype=torch.bfloat16, device=DEV))
        torch.cuda.synchronize()
        return bnd.last_launch_shape()

    assert fold(c(2048), 4096, 8) == (c(2048), 64, 8, True)                   # prefill boundary
    assert fold(c(2048), 7168, 8, fp8=True) == (c(2048), 64, 14, True)        # quantised boundary
    assert fold(c(2048), 4096, 8, kind="complete_only") == (c(2048), 64, 8, True)
    assert fold(c(2048), 7168, 8, kind="snapshot") == (c(2048), 64, 14, True)
    assert fold(c(1536), 4096, 8) == (c(1536), 64, 8, True)                   # 6 rows per CU
    assert fold(c(2048), 2048, 8) == (c(2048), 64, 4, True)                   # other hidden sizes
    assert fold(c(2048), 5120, 8) == (c(2048), 64, 10, True)
    assert fold(c(2048), 6144, 8) == (c(2048), 64, 12, True)
    assert fold(c(4096), 7168, 8) == (c(4096), 64, 14, True)                  # two whole rounds of 2048
    assert fold(c(6144), 4096, 8) == (c(6144), 64, 8, True)                   # two whole rounds of 3072
    assert fold(c(3072), 7168, 8)[3] is False                              # last round half full
    assert fold(c(4096), 4096, 8)[3] is False                              # last round a third full
    assert fold(c(6144), 4096, 8, kind="complete_only") == (c(6144), 64, 8, True)  # rounds of 4096, 1/2
    assert fold(c(3584), 7168, 8, kind="complete_only")[3] is False        # rounds of 3072, 1/6
    assert fold(c(4096), 1024, 8) == (c(4096), 64, 2, True)                   # width 2 from 12 rows per CU
    assert fold(c(4096), 1024, 8, kind="complete_only") == (c(4096), 64, 2, True)
    assert fold(c(2048), 1024, 8)[3] is False                              # width 2: too few rows
    assert fold(c(4096), 768, 8)[3] is False                               # rows too short
    assert fold(c(2048), 8192, 8)[3] is False                              # rows too long for a read
    assert fold(c(2048), 8192, 8, kind="complete_only") == (c(2048), 64, 16, True)
    assert fold(c(2048), 8192, 8, kind="snapshot") == (c(2048), 64, 16, True)
    assert fold(c(1024), 4096, 8) == (c(1024), 64, 8, True)                   # 4 rows per CU: the deep ring
    assert bnd.last_launch_ring_depth() == 8
    assert fold(c(1536), 4096, 8, kind="complete_only") == (c(1536), 64, 8, True)
    assert bnd.last_launch_ring_depth() == 8
    assert fold(c(2048), 4096, 8) == (c(2048), 64, 8, True) and bnd.last_launch_ring_depth() == 2
    assert fold(c(1024) - 1, 4096, 8)[3] is False                              # too few rows per CU
    assert fold(c(1024), 2048, 8)[3] is False                              # widths 4, 6: from 6 rows per CU
    assert fold(c(1536), 2048, 8) == (c(1536), 64, 4, True) and bnd.last_launch_ring_depth() == 4
    assert fold(c(1792), 3072, 8, kind="complete_only") == (c(1792), 64, 6, True)
    assert bnd.last_launch_ring_depth() == 6
    assert fold(c(2048), 3072, 8) == (c(2048), 64, 6, True) and bnd.last_launch_ring_depth() == 2
    assert fold(128, 4096, 4)[3] is False                               # a decode boundary
    d = workloads.moe_inputs(5, c(2048), 4096, 16, 8)
    E, idx, gate = _moe_device(d)
    for rb, rows, shape in ((0, c(2048), (c(2048), 64, 8, True)), (c(768), c(256), (c(256), 512, 1, False))):
        res = torch.zeros(rows, 4096, dtype=torch.bfloat16, device=DEV)
        s = bnd.bnd_stream_create(c(2048), 4096, res, rb, rows)
        bnd.bnd_written(s, res)
        owed = bnd.bnd_publish_moe(s, E, idx, gate, 8)
        bnd.bnd_moe_finalize_fold_norm(s, owed, w[:4096], 1e-6, torch.empty(rows, 4096, dtype=torch.bfloat16,
                                                                             device=DEV))
        torch.cuda.synchronize()
        assert bnd.last_launch_shape() == shape, (rb, rows)
    # the width of 2 is never taken for MoE picks
    d = workloads.moe_inputs(6, c(4096), 1024, 16, 8)
    E, idx, gate = _moe_device(d)
    res = torch.zeros(c(4096), 1024, dtype=torch.bfloat16, device=DEV)
    s = bnd.bnd_stream_create(c(4096), 1024, res)
    bnd.bnd_written(s, res)
    bnd.bnd_moe_finalize_fold_norm(s, bnd.bnd_publish_moe(s, E, idx, gate, 8), w[:1024], 1e-6,
                                   torch.empty(c(4096), 1024, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert bnd.last_launch_shape()[3] is False
    # MoE picks at 6 rows per CU and H = 2048 take the 4-wide deep ring
    d = workloads.moe_inputs(7, 1536, 2048, 16, 8)
    E, idx, gate = _moe_device(d)
    res = torch.zeros(1536, 2048, dtype=torch.bfloat16, device=DEV)
    s = bnd.bnd_stream_create(1536, 2048, res)
    bnd.bnd_written(s, res)
    bnd.bnd_moe_finalize_fold_norm(s, bnd.bnd_publish_moe(s, E, idx, gate, 8), w[:2048], 1e-6,
                                   torch.empty(1536, 2048, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert bnd.last_launch_shape() == (c(1536), 64, 4, True) and bnd.last_launch_ring_depth() == 4


@pytest.mark.parametrize("mode", [bnd.BND_ONE_WAVEFRONT_NEVER, bnd.BND_ONE_WAVEFRONT_ALWAYS],
                         ids=["multi_wave", "one_wave"])
def test_fp8_codes_at_e4m3_midpoints(orc, mode):
    """Rows whose fp32 quotients y / scale fall exactly on e4m3 midpoints while the exact quotients
    lie just off them (the weights of the oracle's pinned case E8), on 64 rows x = 2^-32 .. 2^31
    that each normalise to y = w exactly: the device takes every code from the correctly rounded
    fp32 quotient, as the oracle does, so codes and scales match exactly, under both launch
    forms."""
    w = np.array([3.0, 0.007114955689758062, 0.01130022294819355, 0.012974330224096775,
                  -0.010463169775903225, 1.0, -3.0, 0.0], np.float32)
    T, H = 64, 8
    res = torch.tensor([[2.0 ** (r - 32)] * H for r in range(T)], dtype=torch.float32).to(torch.bfloat16)
    d = {"T": T, "H": H, "P": 1, "partials": [torch.zeros(T, H, dtype=torch.bfloat16)], "residual": res,
         "weight": torch.from_numpy(w), "eps": 0.0}
    bnd.set_option(bnd.BND_OPT_ONE_WAVEFRONT, mode)
    got = run_fold(d, fp8=True)
    assert bnd.last_launch_shape()[3] == (mode == bnd.BND_ONE_WAVEFRONT_ALWAYS)
    ref = oracle_fold(orc, d, fp8=True)
    got["q"].check_guards("midpoint q")
    q = got["q"].view.cpu().numpy()
    sc = got["scale_buf"].cpu().numpy()
    assert sc[0] == -1.0 and sc[-1] == -1.0, "scale written outside its rows"
    assert np.array_equal(sc[1:-1], ref["scale"]), (sc[1:-1], ref["scale"])
    assert np.array_equal(q, ref["q"]), [[hex(int(v)) for v in row] for row in q[:2]]


@pytest.mark.parametrize("shape", [(512, 2), (576, 1), (64, 14)], ids=["512x2", "576x1", "wave"])
def test_fp8_subnormal_scale(orc, shape):
    """A row whose scale is subnormal has no finite reciprocal; the kernels divide by such a
    scale instead of multiplying by 1/scale, which would give +-448 codes for every nonzero y
    and NaN (a -448 code) for zeros. Rows of 1, 0.5 and 0 with random signs, weights 2^-130
    and eps = 0 put the scale near 1800 * 2^-149; the oracle fixes the codes."""
    T, H, P = 6, 4104, 2
    d = workloads.fold_inputs(500, T, H, P)
    sign = torch.where(d["residual"] >= 0, 1.0, -1.0)
    mag = torch.tensor([1.0, 0.5, 0.0]).repeat(H // 3)
    d["residual"] = (sign * mag).to(torch.bfloat16)
    d["partials"] = [torch.zeros_like(c) for c in d["partials"]]
    d["weight"] = torch.full((H,), 2.0 ** -130, dtype=torch.float32)
    d["eps"] = 0.0
    assert float(d["weight"][0]) == 2.0 ** -130, "the host keeps the subnormal weight"
    with forced_shape(*shape):
        got, ref = assert_fold_matches(orc, d, f"subnormal scale {shape[0]}x{shape[1]}", fp8=True)
    assert np.all(ref["scale"] > 0) and np.all(ref["scale"] < np.float32(2.0 ** -126)), "scales are subnormal"
    q = got["q"].view.cpu().numpy()
    assert np.all(q[:, 2::3] == 0), "a zero element must give code +0"
    assert np.all(q[:, 1::3] & 0x7F != 0x7E), "half-size elements must not saturate"


# ------------------------------------------------------------------ seeded random cases

def _random_case(i):
    """Case i of the seeded sweep: kind, sizes, slice, launch shape (one the host accepts)."""
    rng = np.random.default_rng(7000 + i)
    kind = ["fold", "fp8", "moe", "complete_only", "add_to_output", "snapshot"][i % 6]
    H = int(rng.choice([8, 64, 264, 1000, 2048, 3600, 4096, 4104, 5000, 7168, 8192]))
    T = int(rng.integers(1, 97))
    rb = int(rng.integers(0, T))
    rows = int(rng.integers(1, T - rb + 1))
    P = int(rng.integers(1, 17))
    gemma = bool(rng.integers(0, 2)) and kind in ("fold", "fp8", "moe")
    nvec = H // 8
    shapes = [(0, 0)]
    for th, v in ((64, 8), (128, 4), (256, 2), (256, 4), (512, 1), (512, 2), (1024, 1), (1024, 2)):
        if th * v >= nvec:
            shapes.append((th, v))
    for w in (6, 8, 10, 12, 14):  # one wavefront per row, every width that covers the row
        if nvec <= 64 * w:
            shapes.append((64, w))
    if nvec <= 896:
        shapes.append((0, 0, bnd.BND_ONE_WAVEFRONT_ALWAYS))  # the narrowest width, 4 included
    shape = shapes[int(rng.integers(0, len(shapes)))]
    return kind, T, H, P, rb, rows, gemma, shape


@pytest.mark.parametrize("i", range(36))
def test_random_cases(orc, i):
    kind, T, H, P, rb, rows, gemma, shape = _random_case(i)
    mode = " one-wavefront always" if len(shape) == 3 else ""
    what = (f"case {i}: {kind} T={T} H={H} P/k={P} slice={rb}+{rows} gemma={gemma} "
            f"shape={shape[0]}x{shape[1]}{mode}")
    print(f"\n  {what}", flush=True)
    with forced_shape(*shape):
        if kind in ("fold", "fp8"):
            d = workloads.fold_inputs(8000 + i, T, H, P)
            assert_fold_matches(orc, d, what, fp8=kind == "fp8", row_begin=rb, rows=rows, gemma=gemma)
        elif kind == "moe":
            d = workloads.moe_inputs(8000 + i, T, H, max(P, 2), P)
            run_moe(orc, d, rb, rows, what, gemma=gemma)
        else:
            d = workloads.fold_inputs(8000 + i, T, H, P)
            extra = (workloads.to_bf16(workloads.normal_f32(8000 + i, 12345, (T, H), 0.0, 0.25))
                     if kind == "add_to_output" else None)
            a = _complete(d, kind, row_begin=rb, rows=rows, extra=extra)
            e, mag = _oracle_complete(orc, d, kind, row_begin=rb, rows=rows, extra=extra)
            tolerance.check_bf16(bits(a.view), e, mag, what)


def _auto_case(i):
    """Case i of the seeded sweep at batch sizes where the automatic launch shape chooses between
    one wavefront per row and several (1536 .. 4608 rows): kind, sizes and slice."""
    rng = np.random.default_rng(7500 + i)
    kind = ["fold", "fp8", "moe", "complete_only", "add_to_output", "snapshot"][i % 6]
    H = int(rng.choice([1536, 1544, 2048, 2600, 3072, 4096, 5000, 6144, 7168]))
    T = int(rng.integers(1536, 4609))
    full = bool(rng.integers(0, 2))
    rb = 0 if full else int(rng.integers(0, T // 4))
    rows = T - rb if full else int(rng.integers(T // 2, T - rb + 1))
    P = int(rng.integers(1, 9))
    return kind, T, H, P, rb, rows


@pytest.mark.parametrize("i", range(8))
def test_random_cases_automatic_shape(orc, i):
    kind, T, H, P, rb, rows = _auto_case(i)
    what = f"auto case {i}: {kind} T={T} H={H} P/k={P} slice={rb}+{rows}"
    if kind in ("fold", "fp8"):
        d = workloads.fold_inputs(8500 + i, T, H, P)
        assert_fold_matches(orc, d, what, fp8=kind == "fp8", row_begin=rb, rows=rows)
    elif kind == "moe":
        d = workloads.moe_inputs(8500 + i, T, H, max(P, 2), P)
        run_moe(orc, d, rb, rows, what)
    else:
        d = workloads.fold_inputs(8500 + i, T, H, P)
        extra = (workloads.to_bf16(workloads.normal_f32(8500 + i, 12345, (T, H), 0.0, 0.25))
                 if kind == "add_to_output" else None)
        a = _complete(d, kind, row_begin=rb, rows=rows, extra=extra)
        e, mag = _oracle_complete(orc, d, kind, row_begin=rb, rows=rows, extra=extra)
        tolerance.check_bf16(bits(a.view), e, mag, what)
    r, th, v, one = bnd.last_launch_shape()
    assert r == rows
    print(f"\n  {what}: launch {th}x{v}{' one wavefront' if one else ''}", flush=True)


def _deep_band_case(i):
    """Case i of the seeded sweep over the batches where the deep ring is chosen or just missed
    (1024 .. 2047 rows, H = 1544 .. 4096): kind, sizes and slice."""
    rng = np.random.default_rng(7700 + i)
    kind = ["fold", "fp8", "moe", "complete_only", "add_to_output", "snapshot"][i % 6]
    H = int(rng.choice([1544, 2048, 2056, 2600, 3072, 3080, 3600, 4096]))
    rows = int(rng.integers(1024, 2048))
    rb = int(rng.integers(0, 64))
    P = int(rng.integers(1, 9))
    return kind, rb + rows + int(rng.integers(0, 8)), H, P, rb, rows


@pytest.mark.parametrize("i", range(12))
def test_random_cases_deep_ring_band(orc, i):
    kind, T, H, P, rb, rows = _deep_band_case(i)
    what = f"deep band case {i}: {kind} T={T} H={H} P/k={P} slice={rb}+{rows}"
    if kind in ("fold", "fp8"):
        d = workloads.fold_inputs(8700 + i, T, H, P)
        assert_fold_matches(orc, d, what, fp8=kind == "fp8", row_begin=rb, rows=rows)
    elif kind == "moe":
        d = workloads.moe_inputs(8700 + i, T, H, max(P, 2), P)
        run_moe(orc, d, rb, rows, what)
    else:
        d = workloads.fold_inputs(8700 + i, T, H, P)
        extra = (workloads.to_bf16(workloads.normal_f32(8700 + i, 12345, (T, H), 0.0, 0.25))
                 if kind == "add_to_output" else None)
        a = _complete(d, kind, row_begin=rb, rows=rows, extra=extra)
        e, mag = _oracle_complete(orc, d, kind, row_begin=rb, rows=rows, extra=extra)
        tolerance.check_bf16(bits(a.view), e, mag, what)
    r, th, v, one = bnd.last_launch_shape()
    assert r == rows
    print(f"\n  {what}: launch {th}x{v}{' one wavefront' if one else ''}, ring {bnd.last_launch_ring_depth()}",
          flush=True)


def test_concurrent_threads_on_separate_streams(orc):
    """Four host threads fold their own batches concurrently, each on its own HIP stream (default
    priority), five times each: every result equals the same call made alone, bitwise, and the
    lone calls match the oracle. The launch-shape state is per thread and the device queries are
    made once, so the threads share nothing but the read-only kernel tables."""
    import threading

    ds = [workloads.fold_inputs(950 + i, 512 + 256 * i, 4096 - 1024 * (i % 2), 4) for i in range(4)]
    alone = []
    for i, d in enumerate(ds):
        got, _ = assert_fold_matches(orc, d, f"thread batch {i} alone")
        alone.append((bits(got["res"].view), bits(got["y"].view), bnd.last_launch_shape()))
    torch.cuda.synchronize()
    barrier = threading.Barrier(4)
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                barrier.wait()
                for rep in range(5):
                    got = run_fold(ds[i])
                    res, y = bits(got["res"].view), bits(got["y"].view)
                    if not (np.array_equal(res, alone[i][0]) and np.array_equal(y, alone[i][1])):
                        errors.append(f"thread {i} rep {rep}: differs from the call made alone")
                    if bnd.last_launch_shape() != alone[i][2]:
                        errors.append(f"thread {i} rep {rep}: launch shape {bnd.last_launch_shape()}")
        except Exception as e:  # reported below, after every thread has ended
            errors.append(f"thread {i}: {e!r}")

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a worker thread did not finish"
    assert not errors, errors


def test_graph_replay_of_every_hot_call():
    """enter, a fold, an fp8 fold, a MoE finalize, complete_only and a one-partial fold, all at
    2048 x 4096 (the one-wavefront kernels), captured once into a HIP graph and replayed several
    times with eager library work in between; every replay must equal the eager run bitwise."""
    T, H, P, k = 2048, 4096, 8, 8
    d = workloads.fold_inputs(900, T, H, P)
    m = workloads.moe_inputs(901, T, H, 64, k)
    x_in = workloads.stack_input(902, T, H).to(DEV)
    parts = [c.to(DEV) for c in d["partials"]]
    w = d["weight"].to(DEV)
    E, idx, gate = _moe_device(m)

    def chain(res, y, q, sc, out):
        s = bnd.bnd_stream_create(T, H, res)
        bnd.bnd_enter_norm(s, x_in, w, 1e-6, y[0])
        bnd.bnd_fold_norm(s, bnd.bnd_publish_partials(s, parts), w, 1e-6, y[1])
        bnd.bnd_fold_norm_quant_fp8(s, bnd.bnd_publish_partials(s, parts), w, 1e-6, q, sc)
        bnd.bnd_moe_finalize_fold_norm(s, bnd.bnd_publish_moe(s, E, idx, gate, k), w, 1e-6, y[2])
        owed = bnd.bnd_complete_only(s, bnd.bnd_publish_partials(s, parts), out)
        bnd.bnd_fold_norm(s, owed, w, 1e-6, y[3])
        return s

    def buffers():
        z = lambda dt=torch.bfloat16: torch.zeros(T, H, dtype=dt, device=DEV)
        return z(), [z() for _ in range(4)], z(torch.uint8), torch.zeros(T, device=DEV), z()

    eager = buffers()
    chain(*eager)
    torch.cuda.synchronize()
    assert bnd.last_launch_shape() == (T, 64, 8, True), "the chain runs the one-wavefront kernels"
    graph = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain(*graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        keep = chain(*graph)
    other = buffers()
    flat = lambda b: [b[0], *b[1], b[2], b[3], b[4]]
    for rep in range(3):
        for t in flat(graph):
            t.zero_()
        g.replay()
        chain(*other)  # eager library work between replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(flat(graph), flat(eager))):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"
    del keep
