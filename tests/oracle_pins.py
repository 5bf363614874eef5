"""Pins of the oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something fixed independently of it: closed forms of the
RMSNorm read (tests/golden/closed_forms.json), exact rational brute force on
tiny inputs (tests/exact.py), torch's bf16 / float8_e4m3fn casts for the
number formats, and invariants the definition implies. The same pins run
against deliberately broken copies of the oracle in test_oracle_mutants.py, so
each plausible mistake (a dropped term, a wrong sign or index, eps outside the
root, the wrong fp8 maximum) is shown to fail at least one of them.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

import exact
import tolerance
import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))
CASES = GOLDEN["cases"]


def bits(vals) -> np.ndarray:
    t = torch.tensor(vals, dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
    return workloads.bf16_bits(t).copy()


def bval(b) -> np.ndarray:
    return tolerance.bf16_to_f64(b)


def f32(vals) -> np.ndarray:
    return np.asarray(vals, dtype=np.float32)


# ---------------------------------------------------------------- closed forms

def pin_e1_closed_form(o):
    c = CASES["E1_closed_form"]
    res = bits([c["residual"]])
    w = f32(c["weight"])
    for out in (o.written_norm(res, w, c["eps"]), o.enter_norm(res, w, c["eps"])):
        inv = out["y_exact"][0, 0]
        assert abs(inv - c["expect_inv"]) <= 1e-15 * inv, inv
        assert list(bval(out["y"])[0]) == c["expect_y_bf16"], bval(out["y"])[0]


def pin_e2_fold(o):
    c = CASES["E2_fold_two_partials"]
    res = bits([c["residual"]])
    parts = [bits([p]) for p in c["partials"]]
    out = o.fold_norm(parts, res, f32(c["weight"]), c["eps"])
    assert list(bval(out["residual"])[0]) == c["expect_residual"]
    assert list(out["x_exact"][0]) == c["expect_residual"]
    assert list(bval(out["y"])[0]) == c["expect_y_bf16"], bval(out["y"])[0]
    x, y, w = out["x_exact"][0], out["y_exact"][0], f32(c["weight"])
    h = 2  # x = 1.5, w = 2
    assert abs(y[h] / (x[h] * w[h]) - c["expect_inv"]) <= 1e-15 * c["expect_inv"]


def pin_e3_eps_inside_root(o):
    c = CASES["E3_eps_inside_sqrt"]
    res = bits([[c["value"]] * c["H"]])
    out = o.written_norm(res, np.ones(c["H"], np.float32), c["eps"])
    assert np.all(bval(out["y"]) == c["expect_y_bf16"]), bval(out["y"])


def pin_e4_one_hot(o):
    c = CASES["E4_one_hot"]
    x = [0.0] * c["H"]
    x[c["hot_index"]] = c["hot_value"]
    out = o.enter_norm(bits([x]), np.ones(c["H"], np.float32), c["eps"])
    y = bval(out["y"])[0]
    assert y[c["hot_index"]] == c["expect_hot_y_bf16"]
    assert np.count_nonzero(y) == 1
    assert np.array_equal(out["residual"], bits([x]))


def pin_e5_fp8(o):
    c = CASES["E5_fp8_per_token"]
    H = len(c["weight"])
    out = o.fold_norm([bits([[0.0] * H])], bits([[1.0] * H]), f32(c["weight"]), c["eps"], fp8=True)
    assert float(out["scale"][0]) == c["expect_scale"], out["scale"]
    assert list(out["q"][0]) == c["expect_codes"], [hex(v) for v in out["q"][0]]


def pin_e8_fp8_decided_in_fp32(o):
    """Codes of fp32 quotients that fall exactly on e4m3 midpoints, whose exact quotients lie
    just off them: the decision is taken in fp32, as on the device."""
    c = CASES["E8_fp8_decided_in_fp32"]
    H = len(c["weight"])
    out = o.fold_norm([bits([[0.0] * H])], bits([[1.0] * H]), f32(c["weight"]), c["eps"], fp8=True)
    assert float(out["scale"][0]) == c["expect_scale"], out["scale"]
    assert list(out["q"][0]) == c["expect_codes"], [hex(v) for v in out["q"][0]]
    assert c["expect_codes"] != c["exact_quotient_codes"]


def pin_e9_moe_finalize(o):
    """A MoE finalize fold derived by hand: gate-weighted picks, an out-of-range pick with a large
    gate that contributes nothing, rows whose mean square is exactly 4."""
    c = CASES["E9_moe_finalize"]
    w = f32(c["weight"])
    out = o.moe_fold_norm(bits(c["expert_rows"]), np.asarray(c["idx"], np.int32), f32(c["gate"]), c["k"],
                          bits(c["residual"]), w, c["eps"])
    assert out["x_exact"].tolist() == c["expect_x"], out["x_exact"]
    assert bval(out["residual"]).tolist() == c["expect_x"], bval(out["residual"])
    assert bval(out["y"]).tolist() == c["expect_y_bf16"], bval(out["y"])
    # inv from every nonzero element: y_exact = x w inv
    x, y = out["x_exact"], out["y_exact"]
    nz = x * w[None, :] != 0
    inv2 = 2.0 * y[nz] / (x * w[None, :])[nz]
    assert np.all(np.abs(inv2 - c["expect_inv_times_2"]) <= 1e-15), inv2


def pin_e6_zero_row(o):
    c = CASES["E6_zero_row"]
    H = c["H"]
    z = bits([[0.0] * H])
    w = workloads.normal_f32(6, 1, (H,), 1.0, 0.1)
    a = o.fold_norm([z, z], z, w, c["eps"], fp8=True)
    assert float(a["scale"][0]) == c["expect_scale"]
    assert np.all(a["q"] == c["expect_code"])
    b = o.fold_norm([z], z, w, c["eps"])
    assert np.all(bval(b["y"]) == c["expect_y_bf16"])


def pin_e7_gemma(o):
    c = CASES["E7_gemma_weight"]
    res = bits([c["residual"]])
    w = f32(c["weight"])
    out = o.written_norm(res, w, c["eps"], gemma=True)
    assert list(bval(out["y"])[0]) == c["expect_y_bf16"], bval(out["y"])[0]
    # the Gemma form with w = 0 is the plain read with a unit weight, exactly
    d = workloads.fold_inputs(61, 3, 64, 2)
    parts = [workloads.bf16_bits(p).copy() for p in d["partials"]]
    r = workloads.bf16_bits(d["residual"]).copy()
    a = o.fold_norm(parts, r, np.zeros(64, np.float32), 1e-6, gemma=True)
    b = o.fold_norm(parts, r, np.ones(64, np.float32), 1e-6)
    assert np.array_equal(a["y_exact"], b["y_exact"]) and np.array_equal(a["y"], b["y"])
    # and a plain weight w equals the Gemma weight w - 1 (exact for these fp32 values)
    wp = d["weight"].numpy()
    g = o.fold_norm(parts, r, (wp.astype(np.float64) - 1.0).astype(np.float32), 1e-6, gemma=True,
                    fp8=True)
    p = o.fold_norm(parts, r, wp, 1e-6, fp8=True)
    assert np.allclose(g["y_exact"], p["y_exact"], rtol=1e-7, atol=0)
    # the Gemma form through the MoE finalize
    E, idx, gate, rm, wm = _tiny_moe_case(62, 3, 16, 4, 2)
    m = o.moe_fold_norm(E, idx, gate, 2, rm, wm, 1e-6, gemma=True)
    for i in range(3):
        s = _exact_contrib_moe(E, idx, gate, 2, i, 16)
        x, inv, _ = exact.boundary_row(rm[i], s, list(wm), 1e-6)
        for h in range(16):
            yv = x[h] * inv * (1 + exact.f32_value(float(wm[h])))
            yb, tie = exact.bf16_round(yv)
            if tie > abs(yv) * Fraction(1, 10**12):
                assert int(m["y"][i, h]) == yb, (i, h)


# ---------------------------------------------------------------- brute force

def _tiny_fold_case(seed, T, H, P, wide):
    d = workloads.fold_inputs(seed, T, H, P, c_std=0.5, r_std=1.0)
    parts = [workloads.bf16_bits(c).copy() for c in d["partials"]]
    res = workloads.bf16_bits(d["residual"]).copy()
    if wide:  # spread exponents over ~2^-20 .. 2^20 to exercise the sums
        sc = workloads.uniform_f64(seed, 999, (P + 1, T, H))
        shifts = np.floor(sc * 41 - 20).astype(np.int32)
        for p in range(P):
            v = bval(parts[p]) * np.exp2(shifts[p])
            parts[p] = bits(v)
        res = bits(bval(res) * np.exp2(shifts[P]))
    return parts, res, d["weight"].numpy()


def _exact_contrib_partials(parts, t, H):
    return [sum((exact.bf16_value(int(p[t, h])) for p in parts), Fraction(0)) for h in range(H)]


def pin_bruteforce_fold(o):
    eps = 1e-6
    for seed, T, H, P, wide, with_res, rb in [(11, 3, 8, 1, False, True, 0),
                                              (12, 3, 16, 2, False, True, 1),
                                              (13, 2, 16, 3, True, True, 0),
                                              (14, 3, 8, 2, True, False, 0),
                                              (15, 4, 16, 4, False, True, 2)]:
        parts, res_full, w = _tiny_fold_case(seed, T, H, P, wide)
        rows = T - rb
        res = res_full[rb:].copy() if with_res else None
        out = o.fold_norm(parts, res, w, eps, row_begin=rb, rows=rows)
        for i in range(rows):
            s = _exact_contrib_partials(parts, rb + i, H)
            x, inv, y = exact.boundary_row(res[i] if with_res else None, s, list(w), eps)
            for h in range(H):
                assert Fraction(out["x_exact"][i, h]) == x[h], (seed, i, h)
                rb_bits, _ = exact.bf16_round(x[h])
                assert int(out["residual"][i, h]) == rb_bits, (seed, i, h)
                yb, tie = exact.bf16_round(y[h])
                if tie > abs(y[h]) * Fraction(1, 10**12):
                    assert int(out["y"][i, h]) == yb, (seed, i, h, float(y[h]))
                assert abs(out["y_exact"][i, h] - float(y[h])) <= 1e-14 * abs(float(y[h])) + 1e-300


def pin_bruteforce_fp8(o):
    eps = 1e-6
    checked = 0
    for seed, T, H, P in [(21, 3, 16, 2), (22, 2, 8, 3), (23, 4, 16, 1), (24, 3, 16, 2)]:
        parts, res, w = _tiny_fold_case(seed, T, H, P, wide=(seed == 22))
        if seed == 24:  # subnormal weights: the scale is subnormal too (below 2^-128)
            w = (w * np.float32(2.0 ** -130)).astype(np.float32)
        out = o.fold_norm(parts, res, w, eps, fp8=True)
        if seed == 24:
            assert np.all((out["scale"] > 0) & (out["scale"] < np.float32(2.0 ** -128))), out["scale"]
        for i in range(T):
            s = _exact_contrib_partials(parts, i, H)
            _, _, y = exact.boundary_row(res[i], s, list(w), eps)
            scale, codes, tie = exact.fp8_row(y)
            # the oracle's fp64 y sits within ~1e-13 of the exact y: away from an fp32 rounding
            # tie both round y to the same fp32 value, and from there every step is the same
            # fp32 arithmetic, so scale and codes agree exactly
            if tie > Fraction(1, 10**4):
                assert float(out["scale"][i]) == scale, (seed, i, out["scale"][i], scale)
                assert list(out["q"][i]) == codes, (seed, i)
                checked += 1
    assert checked >= 10, checked


def _tiny_moe_case(seed, T, H, n_experts, k):
    d = workloads.moe_inputs(seed, T, H, n_experts, k)
    return (workloads.bf16_bits(d["expert_rows"]).copy(), d["idx"].numpy().copy(),
            d["gate"].numpy().copy(), workloads.bf16_bits(d["residual"]).copy(),
            d["weight"].numpy())


def _exact_contrib_moe(E, idx, gate, k, t, H):
    s = [Fraction(0)] * H
    for j in range(k):
        e = int(idx[t * k + j])
        if not 0 <= e < E.shape[0]:
            continue
        g = Fraction(float(gate[t * k + j]))
        for h in range(H):
            s[h] += g * exact.bf16_value(int(E[e, h]))
    return s


def pin_bruteforce_moe(o):
    eps = 1e-6
    for seed, T, H, ne, k, rb in [(31, 3, 8, 6, 2, 0), (32, 4, 16, 8, 3, 1), (33, 2, 8, 4, 4, 0)]:
        E, idx, gate, res_full, w = _tiny_moe_case(seed, T, H, ne, k)
        if seed == 33:
            idx[1] = E.shape[0] + 5   # an index outside the buffer contributes nothing,
            gate[1] = np.float32("nan")  # whatever its gate holds
        rows = T - rb
        out = o.moe_fold_norm(E, idx, gate, k, res_full[rb:].copy(), w, eps, row_begin=rb,
                              rows=rows)
        for i in range(rows):
            s = _exact_contrib_moe(E, idx, gate, k, rb + i, H)
            x, _, y = exact.boundary_row(res_full[rb + i], s, list(w), eps)
            for h in range(H):
                assert abs(out["x_exact"][i, h] - float(x[h])) <= 2.0 ** -52 * abs(float(x[h]))
                xb, tie = exact.bf16_round(x[h])
                if tie > abs(x[h]) * Fraction(1, 10**12):
                    assert int(out["residual"][i, h]) == xb, (seed, i, h)
                yb, tie = exact.bf16_round(y[h])
                if tie > abs(y[h]) * Fraction(1, 10**12):
                    assert int(out["y"][i, h]) == yb, (seed, i, h)


def pin_bruteforce_complete(o):
    parts, _, _ = _tiny_fold_case(41, 3, 16, 3, wide=True)
    out = o.complete_partials(parts)
    for t in range(3):
        s = _exact_contrib_partials(parts, t, 16)
        for h in range(16):
            assert int(out["out"][t, h]) == exact.bf16_round(s[h])[0]
            assert Fraction(out["s_exact"][t, h]) == s[h]
    E, idx, gate, _, _ = _tiny_moe_case(42, 3, 8, 5, 2)
    out = o.complete_moe(E, idx, gate, 2)
    for t in range(3):
        s = _exact_contrib_moe(E, idx, gate, 2, t, 8)
        for h in range(8):
            b, tie = exact.bf16_round(s[h])
            if tie > abs(s[h]) * Fraction(1, 10**12):
                assert int(out["out"][t, h]) == b


def pin_add_to_output(o):
    """Complete, then add the extra once: exact brute force, and a zero extra is complete_only."""
    parts, _, _ = _tiny_fold_case(43, 3, 16, 3, wide=True)
    extra = bits(bval(_tiny_fold_case(44, 3, 16, 1, wide=True)[0][0]))
    out = o.complete_partials(parts, extra=extra, row_begin=1, rows=2)
    for i in range(2):
        s = _exact_contrib_partials(parts, 1 + i, 16)
        for h in range(16):
            v = s[h] + exact.bf16_value(int(extra[1 + i, h]))
            assert Fraction(out["s_exact"][i, h]) == v
            assert int(out["out"][i, h]) == exact.bf16_round(v)[0]
    z = o.complete_partials(parts, extra=np.zeros_like(parts[0]))
    assert np.array_equal(z["out"], o.complete_partials(parts)["out"])
    E, idx, gate, _, _ = _tiny_moe_case(45, 3, 8, 5, 2)
    ex = workloads.bf16_bits(workloads.to_bf16(workloads.normal_f32(45, 9, (3, 8)))).copy()
    m = o.complete_moe(E, idx, gate, 2, extra=ex)
    for t in range(3):
        s = _exact_contrib_moe(E, idx, gate, 2, t, 8)
        for h in range(8):
            v = s[h] + exact.bf16_value(int(ex[t, h]))
            b, tie = exact.bf16_round(v)
            if tie > abs(v) * Fraction(1, 10**12):
                assert int(m["out"][t, h]) == b


def pin_snapshot(o):
    """bf16(r + s) on the side: exact brute force, equal to the fold's stored residual, and a
    plain copy when nothing is owed."""
    parts, res_full, w = _tiny_fold_case(46, 4, 16, 3, wide=True)
    snap = o.snapshot(parts, res_full[1:].copy(), row_begin=1, rows=3)
    for i in range(3):
        s = _exact_contrib_partials(parts, 1 + i, 16)
        for h in range(16):
            x = exact.bf16_value(int(res_full[1 + i, h])) + s[h]
            assert Fraction(snap["x_exact"][i, h]) == x
            assert int(snap["out"][i, h]) == exact.bf16_round(x)[0]
    fold = o.fold_norm(parts, res_full[1:].copy(), w, 1e-6, row_begin=1, rows=3)
    assert np.array_equal(snap["out"], fold["residual"])
    nores = o.snapshot(parts, None)
    assert np.array_equal(nores["out"], o.complete_partials(parts)["out"])
    copy = o.snapshot([], res_full)
    assert np.array_equal(copy["out"], res_full)


# ---------------------------------------------------------------- number formats

def pin_bf16_codec(o):
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = every[((every >> 7) & 0xFF) != 0xFF]
    ref = bval(finite)
    for b, v in zip(finite, ref):
        assert o.bf16_value(int(b)) == v
        assert o.bf16_round(float(v)) == int(b)
    # fp32 inputs: compare with torch's fp32 -> bf16 cast (round to nearest even)
    rng = workloads.uniform_f64(7, 7, (6000,))
    u = (rng * (0x7F000000)).astype(np.uint32)           # positive finite fp32 patterns
    mids = (finite[(finite & 0x7FFF) < 0x7F00].astype(np.uint32) << 16) | 0x8000  # exact ties
    pats = np.concatenate([u, u | 0x80000000, mids[::23], mids[::29] + 1, mids[::31] - 1])
    f = pats.view(np.float32)
    want = workloads.bf16_bits(torch.from_numpy(f.copy()).to(torch.bfloat16))
    for v, wb in zip(f, want):
        assert o.bf16_round(float(v)) == int(wb), (float(v), hex(int(wb)))
    # one rounding from the exact value, not two
    assert o.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81


def pin_e4m3_codec(o):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    for c, v in zip(codes, ref):
        assert o.e4m3_value(int(c)) == v, (hex(int(c)), v)
        assert o.e4m3_round(float(v)) == int(c), (hex(int(c)), v)
    # midpoints between neighbours and their fp32 neighbours, plus a dense sweep
    pos = np.sort(ref[(ref > 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    m32 = mids.astype(np.float32)
    pts = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                          (workloads.uniform_f64(8, 8, (4000,)) * 448).astype(np.float32),
                          (workloads.uniform_f64(8, 9, (2000,)) * 0.02).astype(np.float32)])
    pts = np.concatenate([pts, -pts])
    want = torch.from_numpy(pts.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, wc in zip(pts, want):
        assert o.e4m3_round(float(v)) == int(wc), (float(v), hex(int(wc)))


# ---------------------------------------------------------------- invariants

def pin_invariants(o):
    eps = 1e-6
    d = workloads.fold_inputs(51, 5, 64, 3)
    parts = [workloads.bf16_bits(c).copy() for c in d["partials"]]
    res = workloads.bf16_bits(d["residual"]).copy()
    w = d["weight"].numpy()
    full = o.fold_norm(parts, res, w, eps)

    # I1: a fold of one zero contribution is the Initial-state enter read
    z = np.zeros_like(res)
    a = o.fold_norm([z], res, w, eps)
    b = o.enter_norm(res, w, eps)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["residual"], b["residual"])

    # I6: the contribution is a sum: any order of the partials gives the same result
    p2 = o.fold_norm([parts[2], parts[0], parts[1]], res, w, eps)
    assert np.array_equal(p2["y"], full["y"]) and np.array_equal(p2["residual"], full["residual"])

    # I4: a row slice computes the same rows as the full call
    sl = o.fold_norm(parts, res[1:4].copy(), w, eps, row_begin=1, rows=3)
    assert np.array_equal(sl["y"], full["y"][1:4])
    assert np.array_equal(sl["residual"], full["residual"][1:4])

    # I5: a MoE handoff with unit gates over stacked partials is the plain fold
    T, H, P = 5, 64, 3
    E = np.concatenate(parts, axis=0)                      # row p*T + t
    idx = np.array([[p * T + t for p in range(P)] for t in range(T)], np.int32).ravel()
    gate = np.ones(T * P, np.float32)
    m = o.moe_fold_norm(E, idx, gate, P, res, w, eps)
    assert np.array_equal(m["y"], full["y"]) and np.array_equal(m["residual"], full["residual"])

    # I3: complete_output then a one-source fold differs from the fused fold only by the
    # bf16 rounding of the completed sum (at most half a bf16 ulp of s per element)
    c = o.complete_partials(parts)
    assert np.array_equal(c["out"], np.array([[o.bf16_round(v) for v in row]
                                              for row in c["s_exact"]], np.uint16))
    two = o.fold_norm([c["out"]], res, w, eps)
    dx = np.abs(two["x_exact"] - full["x_exact"])
    assert np.array_equal(dx, np.abs(bval(c["out"]) - c["s_exact"]))
    assert np.all(dx <= 0.5 * tolerance.ulp_bf16(c["s_exact"]))

    # I7: with a unit weight, mean(y^2) = ms / (ms + eps)
    ones = np.ones(H, np.float32)
    u = o.fold_norm(parts, res, ones, eps)
    ms = np.mean(u["x_exact"] ** 2, axis=1)
    e32 = float(np.float32(eps))
    assert np.allclose(np.mean(u["y_exact"] ** 2, axis=1), ms / (ms + e32), rtol=1e-12, atol=0)

    # I8: with eps = 0 the read is scale invariant: y(2^m x) = y(x) exactly
    r0 = o.written_norm(res, w, 0.0)
    r1 = o.written_norm(bits(bval(res) * 2.0 ** 5), w, 0.0)
    assert np.array_equal(r0["y_exact"], r1["y_exact"]) and np.array_equal(r0["y"], r1["y"])


PINS = [pin_e1_closed_form, pin_e2_fold, pin_e3_eps_inside_root, pin_e4_one_hot, pin_e5_fp8,
        pin_e8_fp8_decided_in_fp32,
        pin_e6_zero_row, pin_e7_gemma, pin_e9_moe_finalize, pin_bruteforce_fold, pin_bruteforce_fp8, pin_bruteforce_moe,
        pin_bruteforce_complete, pin_add_to_output, pin_snapshot, pin_bf16_codec, pin_e4m3_codec, pin_invariants]
