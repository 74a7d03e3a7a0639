"""The inputs of the running-maximum GPU tests do what those tests need (host
only): with the cut the planner makes for them, scores climbing in steps pass
the running maximum by more than the 8-log2-unit slack in a later tile of every
piece long enough to reach the next step (in both row groups at four query
rows, and in partial last tiles), falling steps never do, and a spike above a
plateau does while the plateau keeps a large share of the softmax.  The replay of
the rule (tests/rising_scores.py) is itself checked on a hand-made case."""
import numpy as np
import pytest

import synth

import rising_scores as rs

COMBOS = [("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8"), ("bf16", "mxfp4"), ("fp8", "bf16"), ("fp8", "mxfp4")]
LENGTHS = [700, 33, 1000, 1, 257, 64, 300]


@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_rising_steps_raise_in_every_long_piece(q_dtype, kv_dtype):
    for q_len in (1, 2, 4):
        w = rs.make_steps(LENGTHS, q_dtype, kv_dtype, seed=31 + q_len, q_lens=[q_len] * len(LENGTHS))
        r = rs.piece_raises(w, rs.plan_cut(160, w))
        long_enough = r["rows"] >= 72
        assert long_enough.sum() >= 10 and np.all(r["raises"][long_enough] >= 1)
        assert r["partial_tile_raises"] >= 1
        # odd query rows carry no counter: only even rows raise
        assert set(r["by_row"]) == set(range(0, q_len, 2))


@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_falling_steps_never_raise(q_dtype, kv_dtype):
    w = rs.make_steps(LENGTHS, q_dtype, kv_dtype, seed=71, q_lens=[2] * len(LENGTHS), descend=True)
    r = rs.piece_raises(w, rs.plan_cut(160, w))
    assert int(r["raises"].sum()) == 0
    assert float(r["max_excess"][r["tiles"] >= 2].max()) < rs.SLACK - 0.5


@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_spike_raises_and_plateau_keeps_its_share(q_dtype, kv_dtype):
    for q_len in (1, 4):
        w = rs.make_spike(LENGTHS, q_dtype, kv_dtype, seed=51 + q_len, q_lens=[q_len] * len(LENGTHS))
        r = rs.piece_raises(w, rs.plan_cut(160, w))
        assert int(r["raises"].sum()) >= 2  # spikes in a later tile of their piece
        assert all(r["by_row"].get(t, 0) >= 1 for t in range(0, q_len, 2))
    # the spike row's softmax weight, per head of the first query row of each
    # sequence of at least 300 rows, is between 5 % and 99 %, and below 90 %
    # on average over the heads: the rescaled plateau is a large part of the
    # output
    q, k = rs.decoded(w)
    for b, n in enumerate(LENGTHS):
        if n < 300:
            continue
        s0 = int(w.kv_indptr[b])
        sc = w.sm_scale * np.einsum("hd,jd->hj", q[int(w.qo_indptr[b])], k[s0:s0 + n])
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        share = p[:, int(0.7 * n)] / p.sum(axis=1)
        assert np.all((share > 0.05) & (share < 0.99)) and share.mean() < 0.9, share


def test_capped_steps_raise_in_both_row_groups():
    for kv_dtype in ("bf16", "fp8", "mxfp4"):
        w = rs.make_steps([700, 1000, 257, 64, 300], "bf16", kv_dtype, seed=91, q_lens=[4, 3, 4, 2, 4])
        w.logit_cap = 30.0
        r = rs.piece_raises(w, rs.plan_cut(224, w))
        assert int(r["raises"].sum()) >= 5 and r["by_row"].get(2, 0) >= 1


def test_counter_is_exact_in_every_format():
    # the counter dims decode to exactly a * bit (times the fp8 per-tensor
    # scale's rounding) and the query's to 2^d, so each even row's score
    # contribution is a constant times its step number
    for kv_dtype in ("bf16", "fp8", "mxfp4"):
        w = rs.make_steps([3000], "bf16", kv_dtype, seed=5)
        q, k = rs.decoded(w)
        c = k[:, rs.RAMP_DIM:rs.RAMP_DIM + rs.RAMP_BITS] @ q[0, 0, rs.RAMP_DIM:rs.RAMP_DIM + rs.RAMP_BITS]
        step = c[rs.STEP_ROWS] - c[0]
        assert step > 0
        assert np.allclose(c, step * (np.arange(3000) // rs.STEP_ROWS), rtol=0, atol=1e-9 * float(c.max()))


def test_full_size_steps_raise_in_every_piece():
    w = rs.make_steps([8192] * 64, "bf16", "fp8", seed=93)
    r = rs.piece_raises(w, rs.plan_cut(1024, w))
    assert len(r["raises"]) == 512 and np.all(r["raises"] >= 1)


def test_replay_on_a_hand_made_case():
    # one sequence of 96 rows, one query row whose score is 24 (log2 units)
    # on row 40 and 0 elsewhere: tile 1 (rows 32-63) raises the maximum by 24,
    # tile 2 does not; reversed (24 on row 5) nothing later raises
    class W:
        pass

    for row, expect in ((40, [1]), (5, [0])):
        w = W()
        w.q_dtype, w.kv_dtype, w.sm_scale, w.logit_cap = "bf16", "bf16", 1.0, 0.0
        w.qo_indptr = np.array([0, 1], dtype=np.int32)
        w.kv_indptr = np.array([0, 96], dtype=np.int32)
        w.total_q = 1
        qf = np.zeros((1, 16, 576), dtype=np.float32)
        qf[0, :, 0] = 1.0
        kf = np.zeros((96, 576), dtype=np.float32)
        kf[row, 0] = 24.0 / rs.LOG2E  # exact enough in bf16 for the test's margin
        w.q, w.kv = synth.bf16_bits(qf), synth.bf16_bits(kf)
        r = rs.piece_raises(w, np.array([[0, 0, 0, 96, -1]]))
        assert r["raises"].tolist() == expect
