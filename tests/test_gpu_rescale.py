"""GPU parity where the online softmax must raise its running maximum after a
piece's first tile (MI355X only), and with zero fp8 scales.

Stage 1 keeps each query row's running maximum unless a later tile holds a
score more than 8 log2 units above it; then it rescales the accumulated output
and sum by alpha = 2^(m_old - m_new), recomputes the tile's probabilities and
exchanges them again.  N(0,1) inputs never reach that path, so these inputs do
(tests/rising_scores.py): a counter in the rope dims that makes scores climb
in steps along each sequence, a single spike above a plateau (so that the
rescaled older terms keep a large share of the result), and the steps reversed
as a control.  Each test first replays the rule on the host for the plan's own cut
and asserts that the input raises the maximum where it should (so the test
cannot pass vacuously), then compares the GPU output with the fp64 oracle
element by element (max-abs 2e-2, rel-L2 1e-2).  The softmax over the whole
sequence is the template's naive custom_kernel_bf16; the raise is the online
form of it that split-K stage 1 (submission 753817) computes."""
import numpy as np
import pytest
import torch

import mla_decode_split_amd as mla
import oracle
import synth
from mla_decode_split_amd import device as dev

import rising_scores as rs
from test_gpu_parity import COMBOS, EDGE_LENGTHS, _check_batch, _paged_equals_contiguous, _say

pytestmark = pytest.mark.gpu

LENGTHS = [700, 33, 1000, 1, 257, 64, 300]
ROWS = 160  # forced rows per split: pieces of 1 to 5 tiles, partial last tiles of every size


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _guard(w, plan, what):
    pieces = mla.mla_decode_plan_pieces(plan, w.kv_indptr)
    r = rs.piece_raises(w, pieces)
    _say(f"{what}: {int(r['raises'].sum())} later-tile raises over {len(r['raises'])} pieces, "
         f"per query row {r['by_row']}")
    return r


def _run_case(w, layout, what, rows=ROWS, page_size=16):
    """Oracle parity of `w` (contiguous) or of its paged copy (and then the
    paged output bitwise against the contiguous run with the same cut)."""
    if layout == "contig":
        (_, _), plan, _ = _check_batch(w, rows_per_split=rows, what=what)
        return plan
    pw = synth.page_workload(w, seed=4242, spare_rows=300 if layout == "paged" else 3 * page_size,
                             page_size=1 if layout == "paged" else page_size)
    (_, _), plan, _ = _check_batch(pw, rows_per_split=rows, what=what)
    _paged_equals_contiguous(w, pw, rows_per_split=rows, what=what)
    return plan


@pytest.mark.parametrize("layout", ["contig", "paged"])
@pytest.mark.parametrize("q_len", [1, 2, 4])
@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_max_raise_rising_steps(q_dtype, kv_dtype, q_len, layout):
    w = rs.make_steps(LENGTHS, q_dtype, kv_dtype, seed=31 + q_len, q_lens=[q_len] * len(LENGTHS))
    what = f"rising steps {q_dtype}/{kv_dtype} q_len {q_len} {layout}"
    plan = _run_case(w, layout, what)
    r = _guard(w, plan, what)
    # every piece long enough to reach the next step after its first tile raises
    long_enough = r["rows"] >= 72
    assert long_enough.any() and np.all(r["raises"][long_enough] >= 1), (r["rows"], r["raises"])
    assert r["partial_tile_raises"] >= 1  # also in a partial last tile (masked rows)
    if q_len == 4:
        assert r["by_row"].get(2, 0) >= 1  # the second row group's flags (rows 2 and 3)


@pytest.mark.parametrize("layout", ["contig", "paged"])
@pytest.mark.parametrize("q_len", [1, 4])
@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_max_raise_spike_over_plateau(q_dtype, kv_dtype, q_len, layout):
    w = rs.make_spike(LENGTHS, q_dtype, kv_dtype, seed=51 + q_len, q_lens=[q_len] * len(LENGTHS))
    what = f"spike over a plateau {q_dtype}/{kv_dtype} q_len {q_len} {layout}"
    plan = _run_case(w, layout, what)
    r = _guard(w, plan, what)
    assert int(r["raises"].sum()) >= 2  # spikes in a later tile of their piece
    assert all(r["by_row"].get(t, 0) >= 1 for t in range(0, q_len, 2))


@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_max_raise_falling_steps_control(q_dtype, kv_dtype):
    # the steps from the top down: the first tile holds each piece's largest scores
    w = rs.make_steps(LENGTHS, q_dtype, kv_dtype, seed=71, q_lens=[2] * len(LENGTHS), descend=True)
    what = f"falling steps {q_dtype}/{kv_dtype}"
    plan = _run_case(w, "contig", what)
    r = _guard(w, plan, what)
    multi = r["tiles"] >= 2
    assert multi.any() and float(r["max_excess"][multi].max()) < rs.SLACK - 0.5


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
def test_max_raise_pages_cap_four_rows(kv_dtype):
    # pages of 16 rows, a soft-cap of 30 (the climbing scores flatten near 30 /
    # ln 2 log2 units, so raises stop part way) and up to four query rows (two
    # row groups)
    w = rs.make_steps([700, 1000, 257, 64, 300], "bf16", kv_dtype, seed=91, q_lens=[4, 3, 4, 2, 4])
    w.logit_cap = 30.0
    what = f"rising steps, pages of 16, cap 30, q_len <= 4, kv={kv_dtype}"
    plan = _run_case(w, "pages", what, rows=224)
    r = _guard(w, plan, what)
    assert int(r["raises"].sum()) >= 5 and r["by_row"].get(2, 0) >= 1


def test_max_raise_full_size():
    # bs 64 x 8192, bf16 q, fp8 KV with rising steps, in the planner's own
    # launch configuration (the one the benchmark times); every sequence compared
    w = rs.make_steps([8192] * 64, "bf16", "fp8", seed=93)
    (_, _), plan, _ = _check_batch(w, poison=False, what="rising steps bs64 kv8192 fp8 (full size)")
    r = _guard(w, plan, "rising steps bs64 kv8192 fp8")
    assert np.all(r["raises"] >= 1)


# ------------------------------------------------------------- zero scales

@pytest.mark.parametrize("q_dtype,kv_dtype", [("bf16", "fp8"), ("fp8", "fp8"), ("fp8", "bf16"), ("fp8", "mxfp4")])
@pytest.mark.parametrize("which", ["kv", "q"])
def test_zero_scale(q_dtype, kv_dtype, which):
    """A per-tensor scale of 0 (an all-zero tensor's amax / 448): every score is
    0, so the output is the mean of V - or 0 when the zero scale is the KV's.
    Partial last tiles (masked rows) must stay finite."""
    if which == "kv" and kv_dtype != "fp8":
        pytest.skip("only fp8 KV has a per-tensor scale")
    if which == "q" and q_dtype != "fp8":
        pytest.skip("only fp8 q has a per-tensor scale")
    w = synth.make_batch(EDGE_LENGTHS, q_dtype, kv_dtype, seed=121, name="zero-scale")
    if which == "kv":
        w.kv_scale = np.float32(0.0)
    else:
        w.q_scale = np.float32(0.0)
    (_, _), plan, out = _check_batch(w, rows_per_split=96, what=f"{which} scale 0, {q_dtype}/{kv_dtype}")
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o))
    if which == "kv":
        assert np.all(o == 0.0)
