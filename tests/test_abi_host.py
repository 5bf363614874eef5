"""libboundary on the host: exports, the stream state machine and argument validation.

Nothing here launches a kernel. Legal transitions run on empty slices (rows = 0
launches nothing but still applies the transition); refused calls use fake,
never-dereferenced device addresses and must fail before any launch. As a
guard against a validation bug turning into a launch with a fake address,
this module skips itself on a machine with a GPU.
"""
import ctypes
import json
import os
import re

import pytest
import torch

import reduce_residual_rmsnorm_bnd_amd as bnd
from reduce_residual_rmsnorm_bnd_amd import boundary as B

if torch.cuda.device_count() > 0:
    pytestmark = pytest.mark.skip(reason="host-only checks with fake device addresses")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "boundary.h")
TABLE = json.load(open(os.path.join(ROOT, "tests", "golden", "stream_transitions.json")))

STATUS = {"OK": B.BND_OK, "INVALID_ARG": B.BND_ERR_INVALID_ARG, "NOT_STARTED": B.BND_ERR_NOT_STARTED,
          "FOREIGN_OUTPUT": B.BND_ERR_FOREIGN_OUTPUT, "PENDING": B.BND_ERR_PENDING,
          "WRONG_KIND": B.BND_ERR_WRONG_KIND, "NO_PATH": B.BND_ERR_NO_PATH,
          "UNAVAILABLE": B.BND_ERR_UNAVAILABLE, "HIP": B.BND_ERR_HIP}
STATE = {"INITIAL": B.BND_INITIAL, "WRITTEN": B.BND_WRITTEN, "PENDING": B.BND_PENDING}

L = bnd.lib()
VP = ctypes.c_void_p
FAKE = 0x7F0000000000  # 4 KiB aligned, never dereferenced
H = 4096


def fake(off=0):
    return VP(FAKE + off)


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    for opt in (B.BND_OPT_FUSED_UNAVAILABLE, B.BND_OPT_THREADS_PER_ROW, B.BND_OPT_VECTORS_PER_THREAD,
                B.BND_OPT_ONE_WAVEFRONT, B.BND_OPT_RING_DEPTH):
        L.bnd_set_option(opt, 0)


def create(T=8, rows=0, row_begin=0, residual=None, ld=H, Hh=H):
    h = VP()
    st = L.bnd_stream_create(ctypes.byref(h), T, Hh, row_begin, rows,
                             residual if residual is not None else (fake() if rows else None), ld)
    assert st == B.BND_OK, L.bnd_last_error()
    return h


def owed_out():
    return ctypes.c_uint64()


# ------------------------------------------------------------------ exports

def test_library_exports_every_declared_symbol():
    decl = re.findall(r"^BND_API\s+[\w\s\*]+?\b(bnd_\w+)\s*\(", open(HEADER).read(), flags=re.M)
    assert len(decl) == len(set(decl)) == 26
    assert sorted(decl) == sorted(B.SYMBOLS)
    for name in decl:
        assert hasattr(L, name), name
    assert L.bnd_version().startswith(b"libboundary")


def test_status_strings():
    for name, code in STATUS.items():
        assert L.bnd_status_str(code).decode() == "BND_" + ("OK" if name == "OK" else "ERR_" + name)


# ------------------------------------------------------------------ state table

def _to_state(h, start):
    """Bring an empty-slice stream into one of the table's starting states."""
    o = owed_out()
    if start == "INITIAL":
        return None
    assert L.bnd_written(h, None, H) == 0
    if start == "WRITTEN":
        return None
    if start == "PENDING_PARTIALS":
        arr = (VP * 2)(None, None)
        assert L.bnd_publish_partials(h, arr, 2, H, ctypes.byref(o)) == 0
        return o.value
    if start == "PENDING_MOE":
        assert L.bnd_publish_moe(h, None, 0, H, None, None, 8, ctypes.byref(o)) == 0
        return o.value
    raise AssertionError(start)


def _call(h, call, owed):
    o = owed_out()
    w = None
    if call == "enter_norm":
        return L.bnd_enter_norm(h, None, H, w, 1e-6, None, H, None)
    if call == "fold_norm":
        return L.bnd_fold_norm(h, owed or 0, w, 1e-6, None, H, None)
    if call == "fold_norm_quant_fp8":
        return L.bnd_fold_norm_quant_fp8(h, owed or 0, w, 1e-6, None, H, None, None)
    if call == "moe_finalize_fold_norm":
        return L.bnd_moe_finalize_fold_norm(h, owed or 0, w, 1e-6, None, H, None)
    if call == "complete_only":
        return L.bnd_complete_only(h, owed or 0, None, H, ctypes.byref(o), None)
    if call == "add_to_output":
        return L.bnd_add_to_output(h, owed or 0, None, H, None, H, ctypes.byref(o), None)
    if call == "snapshot":
        return L.bnd_snapshot(h, owed or 0, None, H, None)
    if call == "publish_partials":
        return L.bnd_publish_partials(h, (VP * 1)(None), 1, H, ctypes.byref(o))
    if call == "publish_moe":
        return L.bnd_publish_moe(h, None, 0, H, None, None, 4, ctypes.byref(o))
    if call == "take_output":
        return L.bnd_take_output(h)
    if call == "written":
        return L.bnd_written(h, None, H)
    raise AssertionError(call)


CASES = [(c, s) for c in TABLE["table"] for s in TABLE["states"]]


@pytest.mark.parametrize("call,start", CASES, ids=[f"{c}-{s}" for c, s in CASES])
def test_transition(call, start):
    h = create()
    owed = _to_state(h, start)
    before = (L.bnd_stream_state(h), L.bnd_stream_pending_kind(h), L.bnd_stream_has_residual(h))
    want_status, want_state = TABLE["table"][call][start]
    st = _call(h, call, owed)
    assert st == STATUS[want_status], (call, start, L.bnd_last_error())
    assert L.bnd_stream_state(h) == STATE[want_state]
    if st != B.BND_OK:  # a refused call changes nothing
        assert (L.bnd_stream_state(h), L.bnd_stream_pending_kind(h),
                L.bnd_stream_has_residual(h)) == before
        assert L.bnd_last_error() != b""
    else:
        assert L.bnd_last_error() == b""
    L.bnd_stream_destroy(h)


def _call_owed(h, call, owed):
    """_call, returning (status, the new owed handle of a call that publishes or completes)."""
    o = owed_out()
    if call == "complete_only":
        return L.bnd_complete_only(h, owed or 0, None, H, ctypes.byref(o), None), o.value
    if call == "add_to_output":
        return L.bnd_add_to_output(h, owed or 0, None, H, None, H, ctypes.byref(o), None), o.value
    if call == "publish_partials":
        return L.bnd_publish_partials(h, (VP * 1)(None), 1, H, ctypes.byref(o)), o.value
    if call == "publish_moe":
        return L.bnd_publish_moe(h, None, 0, H, None, None, 4, ctypes.byref(o)), o.value
    return _call(h, call, owed), None


def test_random_call_sequences_follow_the_state_table():
    """Seeded random walks of every call over two empty-slice streams, against a model built from
    the state table alone: status and state after each call, the pending kind, a refused call
    changing nothing, and handles that are stale or belong to the other stream being refused."""
    import random

    rng = random.Random(2024)
    calls = sorted(TABLE["table"])
    kind_of = {"PENDING_PARTIALS": B.BND_KIND_PARTIALS, "PENDING_MOE": B.BND_KIND_MOE}
    checked = 0
    for walk in range(200):
        hs = [create(), create()]
        model = ["INITIAL", "INITIAL"]
        owed = [None, None]
        stale = [[], []]
        for _ in range(30):
            i = rng.randrange(2)
            h, st_model = hs[i], model[i]
            call = rng.choice(calls)
            handle = owed[i]
            forged = None
            if call in ("fold_norm", "fold_norm_quant_fp8", "moe_finalize_fold_norm", "complete_only",
                        "add_to_output", "snapshot") and rng.random() < 0.2:
                pool = stale[i] + ([owed[1 - i]] if owed[1 - i] else [])
                if st_model.startswith("PENDING") and pool:
                    forged = rng.choice(pool)
                elif st_model == "WRITTEN" and pool and call != "snapshot":
                    forged = rng.choice(pool)
            status, new = _call_owed(h, call, forged if forged is not None else handle)
            want_status, want_state = TABLE["table"][call][st_model]
            if forged is not None and want_status == "OK":
                want_status, want_state = "FOREIGN_OUTPUT", st_model
            assert status == STATUS[want_status], (walk, call, st_model, forged, L.bnd_last_error())
            if want_state == "PENDING":
                if status != B.BND_OK:
                    want_state = st_model
                elif call == "publish_moe":
                    want_state = "PENDING_MOE"
                elif call == "snapshot":
                    want_state = st_model
                else:  # publish_partials, or a complete that leaves one plain partial owed
                    want_state = "PENDING_PARTIALS"
            assert L.bnd_stream_state(h) == STATE[want_state.split("_")[0]], (walk, call, st_model)
            if want_state.startswith("PENDING"):
                assert L.bnd_stream_pending_kind(h) == kind_of[want_state]
            if status == B.BND_OK and want_state != st_model or new:
                if owed[i]:
                    stale[i].append(owed[i])
                owed[i] = new if new else (owed[i] if want_state.startswith("PENDING") and
                                           call == "snapshot" else None)
            model[i] = want_state
            checked += 1
        for h in hs:
            L.bnd_stream_destroy(h)
    assert checked == 200 * 30


def test_pending_without_residual_then_fold_writes_it():
    h = create()
    o = owed_out()
    assert L.bnd_publish_partials(h, (VP * 1)(None), 1, H, ctypes.byref(o)) == 0
    assert L.bnd_stream_state(h) == B.BND_PENDING and L.bnd_stream_has_residual(h) == 0
    assert L.bnd_fold_norm(h, o.value, None, 1e-6, None, H, None) == 0
    assert L.bnd_stream_state(h) == B.BND_WRITTEN and L.bnd_stream_has_residual(h) == 1


def test_owed_handles_are_per_stream_and_per_publication():
    a, b = create(), create()
    oa, ob = owed_out(), owed_out()
    for h, o in ((a, oa), (b, ob)):
        assert L.bnd_written(h, None, H) == 0
        assert L.bnd_publish_partials(h, (VP * 1)(None), 1, H, ctypes.byref(o)) == 0
    assert oa.value != ob.value and oa.value != 0
    # another microbatch's output
    assert L.bnd_fold_norm(a, ob.value, None, 1e-6, None, H, None) == B.BND_ERR_FOREIGN_OUTPUT
    assert L.bnd_fold_norm(a, 0, None, 1e-6, None, H, None) == B.BND_ERR_FOREIGN_OUTPUT
    # completing re-publishes: the old handle is stale
    new = owed_out()
    assert L.bnd_complete_only(a, oa.value, None, H, ctypes.byref(new), None) == 0
    assert new.value != oa.value
    assert L.bnd_fold_norm(a, oa.value, None, 1e-6, None, H, None) == B.BND_ERR_FOREIGN_OUTPUT
    assert L.bnd_stream_state(a) == B.BND_PENDING
    assert L.bnd_fold_norm(a, new.value, None, 1e-6, None, H, None) == 0
    # a Written stream owes nothing: any handle is foreign there
    assert L.bnd_fold_norm(a, new.value, None, 1e-6, None, H, None) == B.BND_ERR_FOREIGN_OUTPUT
    assert L.bnd_fold_norm(b, ob.value, None, 1e-6, None, H, None) == 0


def test_moe_complete_becomes_partials():
    h = create()
    o = _to_state(h, "PENDING_MOE")
    assert L.bnd_stream_pending_kind(h) == B.BND_KIND_MOE
    new = owed_out()
    assert L.bnd_complete_only(h, o, None, H, ctypes.byref(new), None) == 0
    assert L.bnd_stream_pending_kind(h) == B.BND_KIND_PARTIALS
    assert L.bnd_moe_finalize_fold_norm(h, new.value, None, 1e-6, None, H, None) == B.BND_ERR_WRONG_KIND
    assert L.bnd_fold_norm(h, new.value, None, 1e-6, None, H, None) == 0


# ------------------------------------------------------------------ validation (no launch)

def _pending(rows=4, T=8, P=2):
    h = create(T=T, rows=rows)
    o = owed_out()
    assert L.bnd_written(h, fake(), H) == 0
    arr = (VP * P)(*[fake((p + 1) << 24) for p in range(P)])
    assert L.bnd_publish_partials(h, arr, P, H, ctypes.byref(o)) == 0
    return h, o.value


def _unchanged(h, kind=B.BND_KIND_PARTIALS):
    assert L.bnd_stream_state(h) == B.BND_PENDING and L.bnd_stream_pending_kind(h) == kind


def test_create_validation():
    h = VP()
    assert L.bnd_stream_create(ctypes.byref(h), 8, 100, 0, 8, fake(), 104) == B.BND_ERR_NO_PATH
    assert L.bnd_stream_create(ctypes.byref(h), 8, 0, 0, 8, fake(), 8) == B.BND_ERR_NO_PATH
    assert L.bnd_stream_create(ctypes.byref(h), 8, 65536, 0, 8, fake(), 65536) == B.BND_ERR_NO_PATH
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 4, 5, fake(), H) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), -1, H, 0, 0, None, H) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 0, 8, None, H) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 0, 8, fake(2), H) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 0, 8, fake(), H - 8) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 0, 8, fake(), H + 4) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 0, 8, fake(), H + 8) == B.BND_OK
    L.bnd_stream_destroy(h)
    assert L.bnd_stream_create(None, 8, H, 0, 8, fake(), H) == B.BND_ERR_INVALID_ARG


def test_publish_validation():
    h = create(T=8, rows=8)
    assert L.bnd_written(h, fake(), H) == 0
    o = owed_out()
    for P in (0, 17):
        assert L.bnd_publish_partials(h, (VP * 17)(*[fake() for _ in range(17)]), P, H,
                                      ctypes.byref(o)) == B.BND_ERR_NO_PATH
    assert L.bnd_publish_partials(h, (VP * 2)(fake(), fake(8)), 2, H, ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_publish_partials(h, (VP * 2)(fake(), None), 2, H, ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_publish_partials(h, None, 2, H, ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_publish_partials(h, (VP * 1)(fake()), 1, H, None) == B.BND_ERR_INVALID_ARG
    for k in (0, 17):
        assert L.bnd_publish_moe(h, fake(), 64, H, fake(), fake(), k, ctypes.byref(o)) == B.BND_ERR_NO_PATH
    assert L.bnd_publish_moe(h, fake(), 64, H, fake(2), fake(), 8, ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_publish_moe(h, fake(), 64, H, fake(), None, 8, ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_publish_moe(h, fake(), -1, H, fake(), fake(), 8, ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_state(h) == B.BND_WRITTEN


def test_fold_validation_refuses_before_launch():
    h, o = _pending()
    y = fake(1 << 30)
    w = fake(1 << 31)
    cases = [
        (L.bnd_fold_norm, (h, o, None, 1e-6, y, H, None)),                # weight NULL
        (L.bnd_fold_norm, (h, o, fake((1 << 31) + 4), 1e-6, y, H, None)),  # weight misaligned
        (L.bnd_fold_norm, (h, o, w, -1.0, y, H, None)),                    # eps < 0
        (L.bnd_fold_norm, (h, o, w, float("nan"), y, H, None)),            # eps NaN
        (L.bnd_fold_norm, (h, o, w, float("inf"), y, H, None)),            # eps inf
        (L.bnd_fold_norm, (h, o, w, 1e-6, None, H, None)),                 # y NULL
        (L.bnd_fold_norm, (h, o, w, 1e-6, fake((1 << 30) + 8), H, None)),  # y misaligned
        (L.bnd_fold_norm, (h, o, w, 1e-6, y, H - 8, None)),                # ld_y < H
        (L.bnd_fold_norm, (h, o, w, 1e-6, fake(), H, None)),               # y is the residual
        (L.bnd_fold_norm, (h, o, w, 1e-6, fake((1 << 24) + 4096 * 2), H, None)),  # y inside partial 0
        (L.bnd_fold_norm_quant_fp8, (h, o, w, 1e-6, y, H, None, None)),    # scale NULL
        (L.bnd_fold_norm_quant_fp8, (h, o, w, 1e-6, fake((1 << 30) + 4), H, fake(1 << 29), None)),
        (L.bnd_fold_norm_quant_fp8, (h, o, w, 1e-6, y, H + 4, fake(1 << 29), None)),
        (L.bnd_fold_norm_quant_fp8, (h, o, w, 1e-6, y, H, y, None)),       # q overlaps scale
        (L.bnd_fold_norm, (h, o, w, 1e-6, fake((1 << 31) + 4096), H, None)),  # y overlaps the weight
        (L.bnd_fold_norm, (h, o, fake(8192), 1e-6, y, H, None)),           # the fold writes over the weight
        (L.bnd_fold_norm_quant_fp8, (h, o, w, 1e-6, fake(1 << 31), H, fake(1 << 29), None)),  # q is the weight
        (L.bnd_fold_norm_quant_fp8, (h, o, w, 1e-6, y, H, fake((1 << 31) + 64), None)),  # scale in the weight
    ]
    for fn, args in cases:
        st = fn(*args)
        assert st == B.BND_ERR_INVALID_ARG, (fn.__name__, args, st, L.bnd_last_error())
        _unchanged(h)


def test_fused_unavailable_refuses_multi_source_only():
    assert L.bnd_set_option(B.BND_OPT_FUSED_UNAVAILABLE, 1) == 0
    assert L.bnd_get_option(B.BND_OPT_FUSED_UNAVAILABLE) == 1
    o = owed_out()
    h = create()
    o2 = _to_state(h, "PENDING_PARTIALS")  # P = 2
    assert L.bnd_fold_norm(h, o2, None, 1e-6, None, H, None) == B.BND_ERR_UNAVAILABLE
    assert L.bnd_stream_state(h) == B.BND_PENDING
    # the fallback: complete_only, then a one-source fold
    assert L.bnd_complete_only(h, o2, None, H, ctypes.byref(o), None) == 0
    assert L.bnd_fold_norm(h, o.value, None, 1e-6, None, H, None) == 0
    m = create()
    om = _to_state(m, "PENDING_MOE")
    assert L.bnd_moe_finalize_fold_norm(m, om, None, 1e-6, None, H, None) == B.BND_ERR_UNAVAILABLE
    assert L.bnd_set_option(B.BND_OPT_FUSED_UNAVAILABLE, 0) == 0
    assert L.bnd_moe_finalize_fold_norm(m, om, None, 1e-6, None, H, None) == 0


def test_norm_form_validation():
    h = create()
    assert L.bnd_stream_set_norm_form(h, B.BND_NORM_GEMMA) == 0
    assert L.bnd_stream_set_norm_form(h, B.BND_NORM_PLAIN) == 0
    assert L.bnd_stream_set_norm_form(h, 2) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_set_norm_form(None, 0) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_state(h) == B.BND_INITIAL


def test_snapshot_keeps_the_owed_work():
    h = create()
    o = _to_state(h, "PENDING_PARTIALS")
    assert L.bnd_snapshot(h, o, None, H, None) == 0
    assert L.bnd_stream_state(h) == B.BND_PENDING and L.bnd_stream_pending_kind(h) == B.BND_KIND_PARTIALS
    assert L.bnd_fold_norm(h, o, None, 1e-6, None, H, None) == 0  # the same handle still folds
    assert L.bnd_snapshot(h, o, None, H, None) == B.BND_ERR_FOREIGN_OUTPUT  # Written: nothing owed
    assert L.bnd_snapshot(h, 0, None, H, None) == 0


def test_add_to_output_validation():
    h, o = _pending()
    new = owed_out()
    # extra required, aligned, and not overlapping the output
    assert L.bnd_add_to_output(h, o, None, H, fake(1 << 30), H, ctypes.byref(new), None) == B.BND_ERR_INVALID_ARG
    assert L.bnd_add_to_output(h, o, fake((1 << 29) + 2), H, fake(1 << 30), H, ctypes.byref(new), None) == B.BND_ERR_INVALID_ARG
    assert L.bnd_add_to_output(h, o, fake(1 << 30), H, fake(1 << 30), H, ctypes.byref(new), None) == B.BND_ERR_INVALID_ARG
    _unchanged(h)


def test_rsv_share():
    counts = [300, 0, 511, 256, 257, 1, 400, 322]
    T = sum(counts)
    begin = 0
    for r, c in enumerate(counts):
        b, n, t = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        assert L.bnd_rsv_share((ctypes.c_int64 * 8)(*counts), 8, r, ctypes.byref(b), ctypes.byref(n),
                               ctypes.byref(t)) == 0
        assert (b.value, n.value, t.value) == (begin, c, T)
        begin += c
    assert bnd.bnd_rsv_share(counts, 2) == (300, 511, T)
    b, n, t = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    arr = (ctypes.c_int64 * 3)(4, -1, 2)
    assert L.bnd_rsv_share(arr, 3, 0, ctypes.byref(b), ctypes.byref(n), ctypes.byref(t)) == B.BND_ERR_INVALID_ARG
    arr = (ctypes.c_int64 * 3)(4, 1, 2)
    assert L.bnd_rsv_share(arr, 3, 3, ctypes.byref(b), ctypes.byref(n), ctypes.byref(t)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_rsv_share(arr, 3, -1, ctypes.byref(b), ctypes.byref(n), ctypes.byref(t)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_rsv_share(None, 3, 0, ctypes.byref(b), ctypes.byref(n), ctypes.byref(t)) == B.BND_ERR_INVALID_ARG
    big = (ctypes.c_int64 * 2)(2**62, 2**62)
    assert L.bnd_rsv_share(big, 2, 1, ctypes.byref(b), ctypes.byref(n), ctypes.byref(t)) == B.BND_ERR_INVALID_ARG


def test_options_validation():
    for opt, bad in ((B.BND_OPT_FUSED_UNAVAILABLE, 2), (B.BND_OPT_THREADS_PER_ROW, 100),
                     (B.BND_OPT_THREADS_PER_ROW, 2048), (B.BND_OPT_VECTORS_PER_THREAD, 3),
                     (B.BND_OPT_VECTORS_PER_THREAD, 5), (B.BND_OPT_VECTORS_PER_THREAD, 18),
                     (B.BND_OPT_ONE_WAVEFRONT, 3), (B.BND_OPT_ONE_WAVEFRONT, -1),
                     (B.BND_OPT_RING_DEPTH, 1), (B.BND_OPT_RING_DEPTH, 3), (B.BND_OPT_RING_DEPTH, 10),
                     (B.BND_OPT_RING_DEPTH, 16), (B.BND_OPT_RING_DEPTH, 4 - 2**32),
                     (B.BND_OPT_VECTORS_PER_THREAD, 8 - 2**32), (B.BND_OPT_THREADS_PER_ROW, 256 - 2**32)):
        assert L.bnd_set_option(opt, bad) == B.BND_ERR_INVALID_ARG
    assert L.bnd_set_option(99, 0) == B.BND_ERR_INVALID_ARG
    assert L.bnd_set_option(B.BND_OPT_THREADS_PER_ROW, 256) == 0
    assert L.bnd_get_option(B.BND_OPT_THREADS_PER_ROW) == 256


def test_launch_shape_that_cannot_cover_the_row_is_refused():
    assert L.bnd_set_option(B.BND_OPT_THREADS_PER_ROW, 64) == 0
    assert L.bnd_set_option(B.BND_OPT_VECTORS_PER_THREAD, 1) == 0
    h, o = _pending()
    st = L.bnd_fold_norm(h, o, fake(1 << 31), 1e-6, fake(1 << 30), H, None)
    assert st == B.BND_ERR_NO_PATH, L.bnd_last_error()
    _unchanged(h)


def test_one_wave_rows_only_where_a_kernel_exists():
    # eight vectors per thread: one wavefront per row, for folds with H <= 4096 and 64 threads
    assert L.bnd_set_option(B.BND_OPT_VECTORS_PER_THREAD, 8) == 0
    assert L.bnd_get_option(B.BND_OPT_VECTORS_PER_THREAD) == 8
    h = create(T=8, rows=8)
    st = L.bnd_enter_norm(h, fake(1 << 28), H, fake(1 << 31), 1e-6, fake(1 << 30), H, None)
    assert st == B.BND_ERR_NO_PATH and b"wavefront" in L.bnd_last_error()
    assert L.bnd_stream_state(h) == B.BND_INITIAL
    wide = 4104
    h = create(T=8, rows=4, ld=wide, Hh=wide)
    assert L.bnd_written(h, fake(), wide) == 0
    o = owed_out()
    arr = (VP * 2)(*[fake((p + 1) << 24) for p in range(2)])
    assert L.bnd_publish_partials(h, arr, 2, wide, ctypes.byref(o)) == 0
    st = L.bnd_fold_norm(h, o.value, fake(1 << 31), 1e-6, fake(1 << 30), wide, None)
    assert st == B.BND_ERR_NO_PATH and b"H <=" in L.bnd_last_error()
    _unchanged(h)
    assert L.bnd_set_option(B.BND_OPT_THREADS_PER_ROW, 128) == 0
    h, o = _pending()
    st = L.bnd_fold_norm(h, o, fake(1 << 31), 1e-6, fake(1 << 30), H, None)
    assert st == B.BND_ERR_NO_PATH and b"64 threads" in L.bnd_last_error()
    _unchanged(h)


def test_wide_one_wave_rows_only_where_a_kernel_exists():
    # fourteen vectors per thread: one wavefront per row, for folds with H <= 7168
    assert L.bnd_set_option(B.BND_OPT_VECTORS_PER_THREAD, 14) == 0
    assert L.bnd_get_option(B.BND_OPT_VECTORS_PER_THREAD) == 14
    h = create(T=8, rows=8)
    st = L.bnd_enter_norm(h, fake(1 << 28), H, fake(1 << 31), 1e-6, fake(1 << 30), H, None)
    assert st == B.BND_ERR_NO_PATH and b"wavefront" in L.bnd_last_error()
    assert L.bnd_stream_state(h) == B.BND_INITIAL
    wide = 7176
    h = create(T=8, rows=4, ld=wide, Hh=wide)
    assert L.bnd_written(h, fake(), wide) == 0
    o = owed_out()
    arr = (VP * 2)(*[fake((p + 1) << 24) for p in range(2)])
    assert L.bnd_publish_partials(h, arr, 2, wide, ctypes.byref(o)) == 0
    st = L.bnd_fold_norm(h, o.value, fake(1 << 31), 1e-6, fake(1 << 30), wide, None)
    assert st == B.BND_ERR_NO_PATH and b"H <= 7168" in L.bnd_last_error()
    _unchanged(h)


def test_enter_validation():
    h = create(T=8, rows=8)
    w = fake(1 << 31)
    # x partly overlapping the residual storage
    assert L.bnd_enter_norm(h, fake(16), H, w, 1e-6, fake(1 << 30), H, None) == B.BND_ERR_INVALID_ARG
    # y overlapping x
    assert L.bnd_enter_norm(h, fake(1 << 28), H, w, 1e-6, fake(1 << 28), H, None) == B.BND_ERR_INVALID_ARG
    assert L.bnd_enter_norm(h, None, H, w, 1e-6, fake(1 << 30), H, None) == B.BND_ERR_INVALID_ARG
    # y overlapping the weight, and an entering copy that would write over the weight
    assert L.bnd_enter_norm(h, fake(1 << 28), H, w, 1e-6, fake((1 << 31) - 64), H, None) == B.BND_ERR_INVALID_ARG
    assert L.bnd_enter_norm(h, fake(1 << 28), H, fake(4096), 1e-6, fake(1 << 30), H, None) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_state(h) == B.BND_INITIAL


def test_binding_rejects_bad_tensors_before_the_library():
    with pytest.raises(ValueError):
        bnd.bnd_stream_create(4, 64, torch.zeros(4, 64, dtype=torch.bfloat16))  # host tensor
    with pytest.raises(TypeError):
        bnd.bnd_stream_create(4, 64, torch.zeros(4, 64, dtype=torch.float32))
    s = bnd.bnd_stream_create(4, 64, None, row_begin=4, rows=0)
    assert s.state == bnd.BND_INITIAL
    with pytest.raises(bnd.BoundaryError) as e:
        B._check(L.bnd_fold_norm(s.handle, 0, None, 1e-6, None, 64, None))
    assert e.value.status == bnd.BND_ERR_NOT_STARTED
    bnd.bnd_take_output(s)
    s.destroy()


def test_last_launch_shape_before_any_launch():
    # a fresh thread has launched nothing: all zero; NULL pointers are allowed
    import threading

    got = {}

    def probe():
        rows, threads, vpt, one = ctypes.c_int64(-1), ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_int(-1)
        got["st"] = L.bnd_last_launch_shape(ctypes.byref(rows), ctypes.byref(threads), ctypes.byref(vpt),
                                            ctypes.byref(one))
        got["shape"] = (rows.value, threads.value, vpt.value, one.value)
        got["null"] = L.bnd_last_launch_shape(None, None, None, None)

    t = threading.Thread(target=probe)
    t.start()
    t.join()
    assert got == {"st": 0, "shape": (0, 0, 0, 0), "null": 0}


def test_size_limits_without_overflow():
    """Rows, slices and leading dimensions at and past their limits are refused before any
    arithmetic on them can overflow (the sanitizer build runs this too)."""
    h = VP()
    big = 2**62
    max_rows = 2**31 - 1
    assert L.bnd_stream_create(ctypes.byref(h), 2**31, H, 0, 0, None, H) == B.BND_ERR_NO_PATH
    assert L.bnd_stream_create(ctypes.byref(h), 2**63 - 1, H, big, big, fake(), H) == B.BND_ERR_NO_PATH
    assert L.bnd_stream_create(ctypes.byref(h), max_rows, H, big, big, fake(), H) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), max_rows, H, max_rows, 1, fake(), H) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 0, 8, fake(), 2**31) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_create(ctypes.byref(h), 8, H, 0, 8, fake(), 2**31 - 8) == B.BND_OK
    L.bnd_stream_destroy(h)
    # the largest stream: a full slice of 2^31 - 1 rows at the largest leading dimension
    assert L.bnd_stream_create(ctypes.byref(h), max_rows, H, 0, max_rows, fake(), 2**31 - 8) == B.BND_OK
    assert L.bnd_written(h, fake(), 2**31 - 8) == B.BND_OK
    o = owed_out()
    arr = (VP * 2)(fake(1 << 44), fake(2 << 44))
    assert L.bnd_publish_partials(h, arr, 2, 2**31, ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_publish_moe(h, fake(1 << 44), 2**31, H, fake(3 << 44), fake(4 << 44), 8,
                             ctypes.byref(o)) == B.BND_ERR_INVALID_ARG
    assert L.bnd_stream_state(h) == B.BND_WRITTEN
    L.bnd_stream_destroy(h)


def test_launch_past_the_dispatch_work_item_count_is_refused():
    """A dispatch counts its grid in work-items with 32 bits: a call whose launch would need more
    (here 2^31 - 1 rows of H = 4096) is refused before the launch and keeps its state."""
    h = VP()
    rows = 2**31 - 1
    span = 1 << 45  # the operands' byte ranges (2^44 bytes each) do not overlap
    assert L.bnd_stream_create(ctypes.byref(h), rows, H, 0, rows, fake(), H) == B.BND_OK
    assert L.bnd_written(h, fake(), H) == B.BND_OK
    o = owed_out()
    arr = (VP * 2)(fake(span), fake(2 * span))
    assert L.bnd_publish_partials(h, arr, 2, H, ctypes.byref(o)) == B.BND_OK
    st = L.bnd_fold_norm(h, o, fake(7 * span), 1e-6, fake(3 * span), H, None)
    assert st == B.BND_ERR_NO_PATH, L.bnd_last_error()
    assert b"work-items" in L.bnd_last_error()
    assert L.bnd_stream_state(h) == B.BND_PENDING
    L.bnd_stream_destroy(h)


def test_one_wavefront_modes():
    assert L.bnd_get_option(B.BND_OPT_ONE_WAVEFRONT) == B.BND_ONE_WAVEFRONT_AUTO
    for v in (B.BND_ONE_WAVEFRONT_ALWAYS, B.BND_ONE_WAVEFRONT_NEVER, B.BND_ONE_WAVEFRONT_AUTO):
        assert L.bnd_set_option(B.BND_OPT_ONE_WAVEFRONT, v) == 0 and L.bnd_get_option(B.BND_OPT_ONE_WAVEFRONT) == v
    for v in (6, 10, 12):  # the other one-wavefront widths are accepted as vectors per thread
        assert L.bnd_set_option(B.BND_OPT_VECTORS_PER_THREAD, v) == 0
    assert L.bnd_set_option(B.BND_OPT_VECTORS_PER_THREAD, 0) == 0
    assert L.bnd_set_option(B.BND_OPT_ONE_WAVEFRONT, B.BND_ONE_WAVEFRONT_ALWAYS) == 0
    # ALWAYS: a call without a one-wavefront kernel, or rows longer than 7168, is refused
    h = create(T=8, rows=8)
    st = L.bnd_enter_norm(h, fake(1 << 28), H, fake(1 << 31), 1e-6, fake(1 << 30), H, None)
    assert st == B.BND_ERR_NO_PATH and b"wavefront" in L.bnd_last_error()
    assert L.bnd_stream_state(h) == B.BND_INITIAL
    wide = 7176
    h = create(T=8, rows=4, ld=wide, Hh=wide)
    assert L.bnd_written(h, fake(), wide) == 0
    o = owed_out()
    arr = (VP * 2)(*[fake((p + 1) << 24) for p in range(2)])
    assert L.bnd_publish_partials(h, arr, 2, wide, ctypes.byref(o)) == 0
    st = L.bnd_fold_norm(h, o.value, fake(1 << 31), 1e-6, fake(1 << 30), wide, None)
    assert st == B.BND_ERR_NO_PATH and b"H <= 7168" in L.bnd_last_error()
    _unchanged(h)
    # under ALWAYS a forced count names the width: an odd one is refused
    h = create(T=8, rows=4)
    assert L.bnd_written(h, fake(), H) == 0
    arr = (VP * 2)(*[fake((p + 1) << 24) for p in range(2)])
    assert L.bnd_publish_partials(h, arr, 2, H, ctypes.byref(o)) == 0
    assert L.bnd_set_option(B.BND_OPT_VECTORS_PER_THREAD, 1) == 0
    st = L.bnd_fold_norm(h, o.value, fake(1 << 31), 1e-6, fake(1 << 30), H, None)
    assert st == B.BND_ERR_NO_PATH and b"2 .. 14 (even)" in L.bnd_last_error()
    # under NEVER a one-wavefront count is refused
    assert L.bnd_set_option(B.BND_OPT_ONE_WAVEFRONT, B.BND_ONE_WAVEFRONT_NEVER) == 0
    assert L.bnd_set_option(B.BND_OPT_VECTORS_PER_THREAD, 8) == 0
    st = L.bnd_fold_norm(h, o.value, fake(1 << 31), 1e-6, fake(1 << 30), H, None)
    assert st == B.BND_ERR_NO_PATH and b"switched off" in L.bnd_last_error()
    assert L.bnd_stream_state(h) == B.BND_PENDING


def test_missing_library_raises():
    """Without the built library the binding raises on first use; nothing falls back to the CPU."""
    import subprocess
    import sys
    code = ("import reduce_residual_rmsnorm_bnd_amd.boundary as B\n"
            "B.LIB_PATH = '/nonexistent/libboundary.so'\n"
            "B._lib = None\n"
            "try:\n"
            "    B.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("raised:") and "is not built" in out.stdout



def test_ring_depth_option():
    """The ring depth takes 0 (automatic), 2, or 4, 6 or 8; a forced 8 needs a launch with one
    wavefront per row of 8 vectors per lane and is refused, before anything is launched, for any
    other."""
    for v in (2, 4, 6, 8, 0):
        assert L.bnd_set_option(B.BND_OPT_RING_DEPTH, v) == 0 and L.bnd_get_option(B.BND_OPT_RING_DEPTH) == v
    depth = ctypes.c_int(-1)
    assert L.bnd_last_launch_ring_depth(ctypes.byref(depth)) == 0 and depth.value in (0, 2, 4, 6, 8)
    assert L.bnd_last_launch_ring_depth(None) == 0
    assert L.bnd_set_option(B.BND_OPT_RING_DEPTH, 8) == 0
    o = owed_out()
    arr = (VP * 2)(*[fake((p + 1) << 24) for p in range(2)])
    for hh, ld in ((2048, 2048), (H, H)):  # a 4-wide one-wavefront row, then a multi-wave launch
        h = create(T=8, rows=4, ld=ld, Hh=hh)
        assert L.bnd_written(h, fake(), ld) == 0
        assert L.bnd_publish_partials(h, arr, 2, ld, ctypes.byref(o)) == 0
        if hh == 2048:
            assert L.bnd_set_option(B.BND_OPT_ONE_WAVEFRONT, B.BND_ONE_WAVEFRONT_ALWAYS) == 0
        else:
            assert L.bnd_set_option(B.BND_OPT_ONE_WAVEFRONT, B.BND_ONE_WAVEFRONT_NEVER) == 0
        st = L.bnd_fold_norm(h, o.value, fake(1 << 31), 1e-6, fake(1 << 30), ld, None)
        assert st == B.BND_ERR_NO_PATH and b"deep ring" in L.bnd_last_error()
        assert L.bnd_stream_state(h) == B.BND_PENDING
