"""C ABI and host planner (no GPU): the library loads and exports every entry
point the header declares; the planner's cut of the batch covers every KV row
exactly once and stage 2 merges exactly the pieces stage 1 leaves partial;
argument errors return status codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import mla_decode_split_amd as mla
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("mla_decode_plan", "mla_decode_run", "mla_decode_plan_destroy", "mla_status_string"):
        assert required in names


def test_library_exports_every_declared_function():
    lib = mla.library()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding exposes the same names
    assert all(hasattr(mla, n) for n in _declared_functions() if n != "mla_last_error_string")


def test_workgroup_timeline_only_in_the_measurement_build():
    """The product library carries no timeline: its entry point says so
    without touching the device."""
    with pytest.raises(mla.MlaError) as e:
        mla.mla_debug_wg_trace(None, clear=True)
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED


def test_status_strings():
    assert mla.mla_status_string(0) == "MLA_OK"
    assert mla.mla_status_string(2) == "MLA_ERR_UNSUPPORTED"


def _plan(bs, total_kv, kv="fp8", q="bf16", ind=None, rows=0, cus=256, **kw):
    prob = mla.make_problem(bs, total_kv, q, kv, num_cus=cus, **kw)
    opts = mla.mla_plan_options(rows, 0) if rows else None
    return mla.mla_decode_plan(prob, opts, ind)


def _indptr(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_plans_for_the_five_workloads(name):
    lengths = synth.workload_lengths(name)
    spec = synth.WORKLOADS[name]
    ind = _indptr(lengths)
    plan = _plan(len(lengths), int(ind[-1]), spec["kv_dtype"], spec["q_dtype"], ind)
    d = mla.mla_decode_plan_describe(plan)
    lo_last, _ = _range(d, d["num_splits"] - 1)
    assert _range(d, d["num_splits"] - 1)[1] >= ind[-1] > lo_last
    assert d["rows_per_split"] % d["tile_rows"] == 0
    assert d["partial_slots"] == 2 * d["num_splits"]
    assert d["lds_bytes"] * d["wgs_per_cu"] <= 160 * 1024  # that many workgroups fit a CU's LDS
    assert d["wgs_per_cu"] == (3 if spec["kv_dtype"] == "mxfp4" else 2)
    assert plan.workspace_bytes >= d["partial_slots"] * 16 * (512 * 2 + 4)  # bf16 O + fp32 LSE per head
    assert d["first_piece_table"] == 1  # stage 1 starts from the plan's first pieces
    _check_cut(plan, ind)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_first_piece_table_conditions(kv):
    """The first-piece table goes with the kernel arguments only when the plan
    has the host offsets, one query row per sequence and at most 768
    workgroups."""
    lengths = [300, 0, 1000, 7, 2048]
    ind = _indptr(lengths)
    total = int(ind[-1])
    desc = lambda plan: mla.mla_decode_plan_describe(plan)
    want = 1
    assert desc(_plan(len(lengths), total, kv, ind=ind, rows=64))["first_piece_table"] == want
    assert desc(_plan(len(lengths), total, kv, ind=None, rows=64))["first_piece_table"] == 0
    assert desc(_plan(len(lengths), total, kv, ind=ind, rows=64, kv_paged=1))["first_piece_table"] == want
    assert desc(_plan(len(lengths), total, kv, ind=ind, rows=64, kv_paged=16))["first_piece_table"] == want
    q2 = mla.make_problem(len(lengths), total, "bf16", kv, num_cus=256, total_q=2 * len(lengths), max_q_len=2)
    assert desc(mla.mla_decode_plan(q2, mla.mla_plan_options(64, 0), ind))["first_piece_table"] == 0
    # 768 workgroups fit the table, 769 do not
    many = [32] * 769
    assert desc(_plan(768, 768 * 32, kv, ind=_indptr(many[:768]), rows=32))["first_piece_table"] == want
    assert desc(_plan(769, 769 * 32, kv, ind=_indptr(many), rows=32))["first_piece_table"] == 0


def _range(d, g):
    """Rows [lo, hi) of workgroup g as the plan description states its cut."""
    R, R2, F = d["rows_per_split"], d["second_rows_per_split"], d["paired_splits"]
    if F == 0:
        return g * R, (g + 1) * R
    assert d["num_splits"] == 2 * F and R2 % d["tile_rows"] == 0 and 0 < R2 < R
    i = g if g < F else g - F
    J = d["xcd_group"]
    if J:  # workgroup slot i holds pair J (8 (k div J) + i mod 8) + k mod J, k = i div 8
        k = i // 8
        i = J * (8 * (k // J) + i % 8) + k % J
    lo = i * (R + R2) + (0 if g < F else R)
    return lo, lo + (R if g < F else R2)


def _check_cut(plan, ind):
    d = mla.mla_decode_plan_describe(plan)
    rec = mla.mla_decode_plan_pieces(plan, ind)
    bs = len(ind) - 1
    G = d["num_splits"]
    # the ranges tile the rows in order, each workgroup once
    bounds = sorted(_range(d, g) for g in range(G))
    assert bounds[0][0] == 0 and all(a[1] == b_[0] for a, b_ in zip(bounds, bounds[1:]))
    assert bounds[-1][1] >= ind[-1]
    covered = np.zeros(int(ind[-1]), dtype=np.int32)
    slots_of = {b: [] for b in range(bs)}
    used = set()
    for g, b, r0, r1, slot in rec:
        lo, hi = _range(d, g)
        assert ind[b] <= r0 < r1 <= ind[b + 1]
        assert lo <= r0 and r1 <= min(hi, ind[-1])
        covered[r0:r1] += 1
        if slot >= 0:
            assert slot < d["partial_slots"] and slot // 2 == g
            assert slot not in used
            used.add(int(slot))
            slots_of[b].append(int(slot))
        else:
            assert r0 == ind[b] and r1 == ind[b + 1]  # direct pieces are whole sequences
    assert np.all(covered == 1), "every KV row of every sequence exactly once"
    needs_merge = False
    for b in range(bs):
        merge = mla.mla_decode_plan_merge_slots(plan, ind, b)
        assert sorted(merge) == sorted(slots_of[b])
        assert len(merge) != 1
        needs_merge |= len(merge) > 0 or ind[b + 1] == ind[b]
    if not needs_merge:
        assert d["stage2"] == 0
    else:
        assert d["stage2"] == 1


@pytest.mark.parametrize("lengths,rows", [
    ([1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129], 32),
    ([1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129], 96),
    ([0, 5, 0, 0, 300, 0], 64),
    ([4096] * 3, 1024),
    ([1] * 200, 32),
    ([700, 1000, 33], 0),
])
def test_cut_properties(lengths, rows):
    ind = _indptr(lengths)
    plan = _plan(len(lengths), int(ind[-1]), ind=ind, rows=rows)
    _check_cut(plan, ind)


def test_random_ragged_cuts(rng):
    for trial in range(30):
        bs = int(rng.integers(1, 60))
        lengths = rng.integers(0, 3000, size=bs)
        lengths[rng.random(bs) < 0.1] = 0
        ind = _indptr(lengths)
        if ind[-1] == 0:
            continue
        rows = int(rng.choice([0, 32, 64, 96, 512, 2048]))
        plan = _plan(bs, int(ind[-1]) + int(rng.integers(0, 50)), ind=ind, rows=rows, cus=int(rng.choice([8, 256])))
        _check_cut(plan, ind)


def test_uniform_batch_without_host_indptr_keeps_stage2():
    plan = _plan(4, 4096)
    assert mla.mla_decode_plan_describe(plan)["stage2"] == 1


def test_single_split_batch_skips_stage2():
    ind = _indptr([100, 100, 100, 100])
    plan = _plan(4, 400, ind=ind, rows=128)
    d = mla.mla_decode_plan_describe(plan)
    # sequence 1 spans rows 100..200 across the 128-row boundary -> merge needed
    assert d["stage2"] == 1
    ind2 = _indptr([64, 64, 64, 64])
    d2 = mla.mla_decode_plan_describe(_plan(4, 256, ind=ind2, rows=128))
    assert d2["stage2"] == 0


def _status(fn, *args):
    try:
        fn(*args)
    except mla.MlaError as e:
        return e.status
    return mla.MLA_OK


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("max_q_len,tokens", [(0, 1), (1, 1), (2, 2), (3, 4), (4, 4)])
def test_plans_with_several_query_rows(kv_dtype, max_q_len, tokens):
    ind = _indptr([8192] * 64)
    total_q = 64 * max(max_q_len, 1)
    prob = mla.make_problem(64, int(ind[-1]), "bf16", kv_dtype, total_q=total_q, num_cus=256, max_q_len=max_q_len)
    plan = mla.mla_decode_plan(prob, None, ind)
    d = mla.mla_decode_plan_describe(plan)
    assert d["query_tokens"] == tokens
    assert d["lds_bytes"] * d["wgs_per_cu"] <= 160 * 1024
    if tokens == 1:
        assert d["wgs_per_cu"] == (3 if kv_dtype == "mxfp4" else 2)
    # every partial slot holds O and LSE of each of the workgroup's query tokens
    assert plan.workspace_bytes >= d["partial_slots"] * tokens * 16 * (512 * 2 + 4)
    _check_cut(plan, ind)


def test_several_query_rows_argument_errors():
    for bad_len in (5, 8, -1):
        prob = mla.make_problem(4, 100, total_q=4, num_cus=256, max_q_len=bad_len)
        assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_UNSUPPORTED, bad_len
    # more query rows than batch_size * max_q_len, or none at all
    for total_q in (9, 0):
        prob = mla.make_problem(4, 100, total_q=total_q, num_cus=256, max_q_len=2)
        assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_INVALID_ARG, total_q
    prob = mla.make_problem(4, 100, total_q=3, num_cus=256, max_q_len=2)  # some sequences with one row
    assert _status(mla.mla_decode_plan, prob) == mla.MLA_OK


def test_logit_cap_argument_errors():
    for bad in (-1.0, float("nan"), float("inf")):
        prob = mla.make_problem(4, 100, num_cus=256, logit_cap=bad)
        assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_INVALID_ARG, bad
    for ok in (0.0, 1e-3, 30.0):
        prob = mla.make_problem(4, 100, num_cus=256, logit_cap=ok)
        assert _status(mla.mla_decode_plan, prob) == mla.MLA_OK, ok


def test_plan_argument_errors():
    unsupported = [
        dict(num_heads=8), dict(qk_dim=512), dict(v_dim=576), dict(total_q=8),
    ]
    for kw in unsupported:
        prob = mla.make_problem(4, 100, num_cus=256, **kw)
        assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_UNSUPPORTED, kw
    prob = mla.make_problem(4, 100, q_dtype="mxfp4", num_cus=256)
    assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_UNSUPPORTED
    prob = mla.make_problem(0, 100, num_cus=256)
    assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_INVALID_ARG
    for bad in (0.0, -1.0 / 24, float("nan"), float("inf")):
        prob = mla.make_problem(4, 100, num_cus=256, sm_scale=bad)
        assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_INVALID_ARG, bad
    prob = mla.make_problem(3, 100, num_cus=256)
    assert _status(mla.mla_decode_plan, prob, None, np.array([0, 50, 40, 100], np.int32)) == mla.MLA_ERR_INVALID_ARG
    assert _status(mla.mla_decode_plan, prob, None, np.array([0, 50, 60, 101], np.int32)) == mla.MLA_ERR_INVALID_ARG
    assert mla.library().mla_decode_plan(None, None, None, None, None) == mla.MLA_ERR_INVALID_ARG


def test_run_argument_errors_before_any_launch():
    """Validation happens on the host before anything touches a device, so fake
    (never dereferenced) addresses are enough here."""
    plan = _plan(2, 64, kv="fp8", ind=_indptr([32, 32]))
    A = 1 << 20  # 16-byte aligned fake address
    ok = dict(q=A, q_scale=A, kv=A, kv_scale=A, qo=A, kvp=A, out=A, ws=A, n=plan.workspace_bytes)

    def run(**kw):
        a = dict(ok, **kw)
        return _status(mla.mla_decode_run, plan, a["q"], a["q_scale"], a["kv"], a["kv_scale"], a["qo"], a["kvp"],
                       a["out"], a["ws"], a["n"])

    assert run(q=None) == mla.MLA_ERR_INVALID_ARG
    assert run(kv_scale=None) == mla.MLA_ERR_INVALID_ARG      # fp8 KV needs its scale
    assert run(out=A + 2) == mla.MLA_ERR_INVALID_ARG          # misaligned
    assert run(n=plan.workspace_bytes - 1) == mla.MLA_ERR_INVALID_ARG
    assert run(ws=None) == mla.MLA_ERR_INVALID_ARG
    assert mla.library().mla_decode_run(None, A, A, A, A, A, A, A, A, 1 << 30, None) == mla.MLA_ERR_INVALID_ARG
    assert mla.library().mla_debug_decode(7, A, A, A, 10, None) == mla.MLA_ERR_UNSUPPORTED
    assert mla.library().mla_debug_decode(2, A, None, A, 10, None) == mla.MLA_ERR_INVALID_ARG
    assert mla.library().mla_debug_stream_read(A, 24, A, None) == mla.MLA_ERR_INVALID_ARG   # not 16-byte sized
    assert mla.library().mla_debug_stream_read(A + 8, 32, A, None) == mla.MLA_ERR_INVALID_ARG
    assert mla.library().mla_debug_stream_read(A, 32, None, None) == mla.MLA_ERR_INVALID_ARG
    assert mla.library().mla_debug_stream_read(A, 0, A, None) == mla.MLA_OK                 # nothing to launch
    ring = mla.library().mla_debug_stream_ring
    assert ring(A, 18432 + 16, 2, A, None) == mla.MLA_ERR_INVALID_ARG  # not whole 18 KB tiles
    assert ring(A + 8, 18432, 1, A, None) == mla.MLA_ERR_INVALID_ARG   # misaligned
    assert ring(A, 18432, 0, A, None) == mla.MLA_ERR_INVALID_ARG       # no workgroups
    assert ring(A, 18432, 1, None, None) == mla.MLA_ERR_INVALID_ARG
    assert ring(A, 18432 * (1 << 20), 1, A, None) == mla.MLA_ERR_INVALID_ARG  # a share past 32-bit offsets
    assert ring(A, 0, 4, A, None) == mla.MLA_OK                             # nothing to launch


@pytest.mark.parametrize("kv_dtype,q_len", [("fp8", 1), ("fp8", 2), ("fp8", 4), ("bf16", 1), ("bf16", 2),
                                            ("mxfp4", 1), ("mxfp4", 2), ("mxfp4", 4)])
def test_paged_plans(kv_dtype, q_len):
    ind = _indptr([8192] * 64)
    prob = mla.make_problem(64, int(ind[-1]), "bf16", kv_dtype, total_q=64 * q_len, num_cus=256, max_q_len=q_len,
                            kv_paged=1)
    plan = mla.mla_decode_plan(prob, None, ind)
    d = mla.mla_decode_plan_describe(plan)
    assert d["lds_bytes"] * d["wgs_per_cu"] <= 160 * 1024
    if kv_dtype != "bf16" and q_len < 4:
        # the index ring still leaves room for two workgroups (three for one-row MXFP4)
        assert d["wgs_per_cu"] == (3 if kv_dtype == "mxfp4" and q_len == 1 else 2)
    _check_cut(plan, ind)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
def test_page_sizes_share_the_paged_plan(kv_dtype):
    # pages of any power-of-two size run the page-size-1 kernels: same cut,
    # ring and residency
    ind = _indptr([700, 33, 4000, 1])
    base = mla.mla_decode_plan_describe(mla.mla_decode_plan(
        mla.make_problem(4, int(ind[-1]), "bf16", kv_dtype, num_cus=256, kv_paged=1), None, ind))
    for P in (2, 16, 64, 1024, 65536):
        plan = mla.mla_decode_plan(mla.make_problem(4, int(ind[-1]), "bf16", kv_dtype, num_cus=256, kv_paged=P),
                                   None, ind)
        assert mla.mla_decode_plan_describe(plan) == base
        _check_cut(plan, ind)


def test_paged_argument_errors_before_any_launch():
    """Every call below fails host-side validation (fake, never dereferenced addresses)."""
    for bad in (3, -1, 12, 1 << 17):  # page sizes: powers of two up to 65536
        prob = mla.make_problem(4, 100, num_cus=256, kv_paged=bad)
        assert _status(mla.mla_decode_plan, prob) == mla.MLA_ERR_INVALID_ARG
    A = 1 << 20
    ind = _indptr([32, 32])
    flat = _plan(2, 64, kv="fp8", ind=ind)
    paged = mla.mla_decode_plan(mla.make_problem(2, 64, "bf16", "fp8", num_cus=256, kv_paged=1), None, ind)
    n = paged.workspace_bytes

    def run_paged(plan, kv_rows=1000, kv_indices=A, kv_page_indptr=None):
        return _status(mla.mla_decode_run_paged, plan, A, A, A, A, kv_rows, kv_indices, kv_page_indptr, A, A, A, A, n)

    assert run_paged(flat) == mla.MLA_ERR_INVALID_ARG                    # contiguous plan
    assert run_paged(paged, kv_indices=None) == mla.MLA_ERR_INVALID_ARG
    assert run_paged(paged, kv_indices=A + 2) == mla.MLA_ERR_INVALID_ARG  # not 4-byte aligned
    assert run_paged(paged, kv_rows=0) == mla.MLA_ERR_INVALID_ARG
    assert run_paged(paged, kv_rows=1 << 23) == mla.MLA_ERR_UNSUPPORTED   # > 4 GB of fp8 rows
    assert _status(mla.mla_decode_run, paged, A, A, A, A, A, A, A, A, n) == mla.MLA_ERR_INVALID_ARG
    assert _status(mla.mla_decode_split, paged, A, A, A, A, A, A, A, A, n) == mla.MLA_ERR_INVALID_ARG
    assert _status(mla.mla_decode_split_paged, flat, A, A, A, A, 1000, A, None, A, A, A, A, n) == mla.MLA_ERR_INVALID_ARG
    assert run_paged(paged, kv_page_indptr=A) == mla.MLA_ERR_INVALID_ARG   # page lists with page size 1
    pages = mla.mla_decode_plan(mla.make_problem(2, 64, "bf16", "fp8", num_cus=256, kv_paged=16), None, ind)
    assert run_paged(pages) == mla.MLA_ERR_INVALID_ARG                       # page size 16 without page lists
    assert run_paged(pages, kv_page_indptr=A + 2) == mla.MLA_ERR_INVALID_ARG  # not 4-byte aligned
    assert _status(mla.mla_decode_split_paged, pages, A, A, A, A, 1000, A, None, A, A, A, A, n) == \
        mla.MLA_ERR_INVALID_ARG


def test_plan_destroy_accepts_null():
    mla.library().mla_decode_plan_destroy(None)


@pytest.mark.parametrize("skew", [0, -1, 25, 120, 500])
@pytest.mark.parametrize("lengths,rows,cus", [
    ([512] * 8, 256, 8),                       # uniform: pair boundaries on sequence boundaries
    ([4096] * 64, 1024, 128),                  # the bs64 x 4096 shape on 128 CUs
    ([700, 1000, 33, 1, 2500, 77, 300], 160, 0),
    ([700, 1000, 33, 1, 2500, 77, 300, 189], 150, 15),  # ragged, 30 ranges on 15 CUs
    ([1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129], 0, 4),
])
def test_paired_cut(lengths, rows, cus, skew):
    """With two workgroups per CU the first on each CU takes a longer range and
    the second the rest of their pair's rows; every KV row is still covered
    once and stage 2 merges exactly the partial pieces."""
    ind = _indptr(lengths)
    total = int(ind[-1])
    if cus == 0:  # as many CUs as make two workgroups each
        cus = ((total + rows - 1) // rows) // 2
    prob = mla.make_problem(len(lengths), total, "bf16", "fp8", num_cus=cus)
    opts = mla.mla_plan_options(rows, 0, skew)
    plan = mla.mla_decode_plan(prob, opts, ind)
    d = mla.mla_decode_plan_describe(plan)
    paired = d["num_splits"] == 2 * cus and skew != -1 and d["paired_splits"] > 0
    if skew == -1 or d["num_splits"] != 2 * cus:
        assert d["paired_splits"] == 0
    elif paired:
        assert d["paired_splits"] == cus and d["second_rows_per_split"] < d["rows_per_split"]
    _check_cut(plan, ind)


@pytest.mark.parametrize("seed", range(12))
def test_merge_batch_holds_the_longest_sequence(seed):
    """Stage 2 loads merge_batch slots at once: with host offsets the smallest
    of 2, 4, 8 and 16 that holds the most slots any sequence has (16 beyond
    that), from the stage-2 replay; without them 8."""
    rng = np.random.default_rng(9100 + seed)
    lengths = rng.integers(0, 3000, size=int(rng.integers(1, 40)))
    ind = _indptr(lengths)
    total = max(int(ind[-1]), 1)
    rows = int(rng.choice([32, 64, 96, 256, 1024]))
    plan = _plan(len(lengths), total, "fp8", ind=ind, rows=rows)
    most = 0
    for b in range(len(lengths)):
        slots = np.zeros(64, dtype=np.int32)
        cnt = ctypes.c_int32(0)
        st = mla.library().mla_decode_plan_merge_slots(plan.handle, ind.ctypes.data_as(ctypes.c_void_p), b,
                                                       slots.ctypes.data_as(ctypes.c_void_p), 64, ctypes.byref(cnt))
        assert st == mla.MLA_OK
        most = max(most, cnt.value)
    want = next((nb for nb in (2, 4, 8, 16) if most <= nb), 16)
    assert mla.mla_decode_plan_describe(plan)["merge_batch"] == want, (most, rows)
    assert mla.mla_decode_plan_describe(_plan(len(lengths), total, "fp8", rows=rows))["merge_batch"] == 8


@pytest.mark.parametrize("J", [1, 2, 4])
@pytest.mark.parametrize("lengths,rows,cus", [
    ([4096] * 64, 1024, 128),                                  # four pairs per sequence
    ([700, 1000, 33, 1, 2500, 77, 300, 189] * 4 + [1280], 160, 64),  # ragged, pieces crossing pairs
])
def test_xcd_grouped_pairs(lengths, rows, cus, J):
    """Paired ranges with J consecutive pairs on one XCD (consecutive workgroup
    slots go to consecutive XCDs): the cut still covers every row once and
    stage 2 merges exactly the partial pieces; pair p sits in a slot on XCD
    (p div J) mod 8."""
    ind = _indptr(lengths)
    prob = mla.make_problem(len(lengths), int(ind[-1]), "bf16", "fp8", num_cus=cus)
    plan = mla.mla_decode_plan(prob, mla.mla_plan_options(rows, 0, 0, J), ind)
    d = mla.mla_decode_plan_describe(plan)
    assert d["paired_splits"] == cus and d["xcd_group"] == J
    F, R, R2 = cus, d["rows_per_split"], d["second_rows_per_split"]
    for s in range(F):
        lo, _ = _range(d, s)
        p = lo // (R + R2)
        assert s % 8 == (p // J) % 8
        assert _range(d, F + s)[0] == lo + R  # the second workgroup of the pair shares the CU
    _check_cut(plan, ind)
    # without pairing (or a CU count that is not a multiple of 8 J) there is no grouping
    flat = mla.mla_decode_plan(prob, mla.mla_plan_options(rows, 0, -1, J), ind)
    assert mla.mla_decode_plan_describe(flat)["xcd_group"] == 0
