"""Inputs whose softmax scores rise past a running maximum mid-piece, and a host
check that they really do.

The decode's stage 1 keeps, per query row and head, a running maximum of the
base-2 scores of the KV rows seen so far in its piece, and raises it (rescaling
the accumulated output and sum) only when a later 32-row tile holds a score
more than a slack of 8 log2 units above it.  N(0,1) inputs never get there, so
the inputs here are built so that they do.  A counter N_j per KV row lives in
the rope dims 544 + d (d < 8): K row j holds a * bit_d(N_j) there and every
even query row holds 2^d (odd query rows hold 0 and see N(0,1) scores only),
so an even row's raw score is its N(0,1) part plus exactly a * N_j.

  steps      N_j = (j - start) // 36: with a = 256 the score climbs about 15.4
             log2 units every 36 rows, so a later tile of every piece of more
             than about 68 rows raises the maximum; each step is flat, so the
             softmax spreads over the rows of the top step (no single row
             dominates the output)
  descend    the same steps from the top down: the control, where no later
             tile raises the maximum
  spike      N_j = 3 on one row per sequence (at 70 % of its length, for
             sequences of at least 96 rows) and 0 elsewhere, with a = 64: that
             row scores about 11.5 log2 units above the plateau, while the
             plateau's other rows keep a share of the softmax comparable to
             it, so the rescaled older terms matter to the result

The values go through synth.encode_batch, so every format holds them the way
it holds any input (every counter value is exact in each format); the oracle
decodes the stored bytes as always.

``piece_raises`` replays the rule on the decoded inputs in fp64 for the cut a
plan makes (mla_decode_plan_pieces), so each test can assert that its input
exercises the raise and cannot pass vacuously.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth

SLACK = 8.0       # log2 units
TILE = 32         # KV rows per tile
RAMP_DIM = 544    # first of the rope dims that carry the counter
RAMP_BITS = 8     # counter values < 256
STEP_ROWS = 36
LOG2E = 1.0 / math.log(2.0)


def _normals(seed, stream, n):
    return synth.bf16_to_f32(synth.normal_bf16(seed, stream, n))


def _steps(n, descend=False):
    pos = np.arange(n, dtype=np.int64)
    if descend:
        pos = n - 1 - pos
    return pos // STEP_ROWS


def _spike(n):
    c = np.zeros(n, dtype=np.int64)
    if n >= 96:
        c[int(0.7 * n)] = 3
    return c


def make_counter(lengths, q_dtype, kv_dtype, seed, counter, a, q_lens=None, name="counter"):
    """Batch of N(0,1) draws with the counter counter(n) (one value per KV row of
    a sequence of n rows) written into the rope dims."""
    lengths = np.asarray(lengths, dtype=np.int64)
    bs = lengths.shape[0]
    q_lens = np.ones(bs, dtype=np.int64) if q_lens is None else np.asarray(q_lens, dtype=np.int64)
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    ki = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total_q, total_kv = int(qo[-1]), int(ki[-1])
    q = _normals(seed, synth.STREAM_Q, total_q * 16 * 576).reshape(total_q, 16, 576).copy()
    kv = _normals(seed, synth.STREAM_KV, total_kv * 576).reshape(total_kv, 576).copy()
    bits = np.arange(RAMP_BITS)
    for b in range(bs):
        s, n = int(ki[b]), int(lengths[b])
        c = counter(n)
        if c.size and (c.min() < 0 or c.max() >= 1 << RAMP_BITS):
            raise ValueError("counter out of range")
        kv[s:s + n, RAMP_DIM:RAMP_DIM + RAMP_BITS] = a * ((c[:, None] >> bits[None, :]) & 1)
        for t in range(int(qo[b]), int(qo[b + 1])):
            q[t, :, RAMP_DIM:RAMP_DIM + RAMP_BITS] = (2.0 ** bits) if (t - int(qo[b])) % 2 == 0 else 0.0
    w = synth.encode_batch(q, kv, qo, ki, q_dtype, kv_dtype, name=name)
    w.meta.update(seed=seed, counter_a=a)
    return w


def make_steps(lengths, q_dtype, kv_dtype, seed, q_lens=None, descend=False):
    return make_counter(lengths, q_dtype, kv_dtype, seed, lambda n: _steps(n, descend), 256.0, q_lens,
                        name="falling steps" if descend else "rising steps")


def make_spike(lengths, q_dtype, kv_dtype, seed, q_lens=None):
    return make_counter(lengths, q_dtype, kv_dtype, seed, _spike, 64.0, q_lens, name="spike")


def decoded(w):
    """fp64 q [total_q, 16, 576] and K rows [total_kv, 576] in CSR order."""
    if w.q_dtype == "bf16":
        q = synth.bf16_to_f32(w.q).astype(np.float64)
    else:
        q = oracle.decode_fp8(w.q, float(w.q_scale))
    if w.kv_dtype == "bf16":
        k = synth.bf16_to_f32(w.kv).astype(np.float64)
    elif w.kv_dtype == "fp8":
        k = oracle.decode_fp8(w.kv, float(w.kv_scale))
    else:
        k = oracle.decode_mxfp4(w.kv, w.kv_scale)
    if getattr(w, "kv_indices", None) is not None:
        raise ValueError("replay the rule on the contiguous batch (the same CSR rows)")
    return q.reshape(w.total_q, 16, 576), k.reshape(-1, 576)


def piece_raises(w, pieces, margin=0.5):
    """Replay the running-maximum rule over the cut `pieces` ([n, 5] records
    (workgroup, sequence, row0, row1, slot)) in fp64.

    Returns a dict with, per piece, the number of later tiles (index >= 1)
    whose scores pass the running maximum by more than SLACK + margin for some
    query row and head ("clear raises"), the largest excess over the running
    maximum seen in any later tile, the piece's tiles and rows, the clear
    raises per query row index within the sequence, and how many clear raises
    fell in a partial last tile (the masked path)."""
    q, k = decoded(w)
    qo = np.asarray(w.qo_indptr, dtype=np.int64)
    cap = float(getattr(w, "logit_cap", 0.0))
    per_piece, max_excess, by_row, tiles, rows, partial = [], [], {}, [], [], 0
    for g, b, r0, r1, slot in np.asarray(pieces, dtype=np.int64):
        qs = q[qo[b]:qo[b + 1]]                         # [nq, 16, 576]
        if qs.shape[0] == 0:
            continue
        s = w.sm_scale * np.einsum("thd,jd->thj", qs, k[r0:r1])
        if cap > 0:
            s = cap * np.tanh(s / cap)
        s2 = s * LOG2E
        n = int(r1 - r0)
        nt = (n + TILE - 1) // TILE
        m = s2[:, :, :TILE].max(axis=2)                 # after tile 0: [nq, 16]
        raises, worst = 0, -np.inf
        for i in range(1, nt):
            tm = s2[:, :, i * TILE:(i + 1) * TILE].max(axis=2)
            ex = (tm - m).max(axis=1)                   # per query row
            worst = max(worst, float(ex.max()))
            flagged = ex > SLACK
            if np.any(ex > SLACK + margin):
                raises += 1
                partial += int(i == nt - 1 and n % TILE != 0)
                for t in np.flatnonzero(ex > SLACK + margin):
                    by_row[int(t)] = by_row.get(int(t), 0) + 1
            m[flagged] = np.maximum(m[flagged], tm[flagged])
        per_piece.append(raises)
        max_excess.append(worst)
        tiles.append(nt)
        rows.append(n)
    return {"raises": np.asarray(per_piece), "max_excess": np.asarray(max_excess), "tiles": np.asarray(tiles),
            "rows": np.asarray(rows), "by_row": by_row, "partial_tile_raises": partial}


def plan_cut(rows_per_split, w, num_cus=256):
    """The stage-1 cut for `w` with a forced split size, on the host (no GPU)."""
    import mla_decode_split_amd as mla

    prob = mla.make_problem(w.batch_size, w.total_kv, w.q_dtype, w.kv_dtype, total_q=w.total_q, num_cus=num_cus,
                            max_q_len=int(np.diff(w.qo_indptr).max(initial=0)), logit_cap=w.logit_cap)
    plan = mla.mla_decode_plan(prob, mla.mla_plan_options(rows_per_split, 0), w.kv_indptr)
    return mla.mla_decode_plan_pieces(plan, w.kv_indptr)
