"""Pins for the CPU fp64 oracle (no GPU).

The pages print no worked numeric example, so the oracle is pinned by things
that do not come from the oracle itself: the OCP format definitions and
torch's independent float8 casts for the decoders; closed forms (one KV row,
two KV rows, identical scores); brute force in exact / 60-digit decimal
arithmetic on tiny inputs; the split recombination identity; symmetries; and an
independent torch fp64 formulation (matmul + softmax + matmul) of the template
page's naive reference.
"""
from decimal import Decimal, getcontext
from fractions import Fraction
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H, D, V = 16, 576, 512
SM = 1.0 / math.sqrt(576.0)


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            rows.append((int(code, 16), float(val)))
    return rows


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


# ----------------------------------------------------------------- decoders

def test_e4m3fn_spot_values_from_format_definition():
    for code, val in _read_table("e4m3fn_values.txt"):
        assert _same(oracle.e4m3fn_value(code), val), hex(code)


def test_e4m3fn_all_codes_match_torch_cast():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.e4m3fn_value(c), float(ref[c])), hex(c)


def test_e2m1_table_from_format_definition():
    table = _read_table("e2m1_values.txt")
    assert len(table) == 16
    for nib, val in table:
        assert _same(oracle.e2m1_value(nib), val), hex(nib)


def test_e8m0_all_codes_match_torch_cast_and_definition():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.e8m0_value(c), float(ref[c])), hex(c)
    for code, val in _read_table("e8m0_values.txt"):
        assert _same(oracle.e8m0_value(code), val)


def test_fp8_decode_times_scale_is_exact_product(rng):
    codes = rng.integers(0, 256, size=4096, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11  # drop NaN codes
    scale = np.float32(0.0123456)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(scale)
    got = oracle.decode_fp8(codes, float(scale))
    assert np.array_equal(got, ref)


def test_mxfp4_nibble_order_and_block_scales():
    packed = np.zeros((1, 288), dtype=np.uint8)
    scales = np.full((1, 18), 127, dtype=np.uint8)
    packed[0, 0] = 0x21        # element 0 = nibble 0x1 (0.5), element 1 = nibble 0x2 (1.0)
    packed[0, 16] = 0xF7       # element 32 = 0x7 (6.0), element 33 = 0xF (-6.0); block 1
    scales[0, 1] = 130         # block 1 scaled by 2^3
    packed[0, 287] = 0x90      # element 574 = 0x0, element 575 = 0x9 (-0.5); block 17
    scales[0, 17] = 125        # 2^-2
    out = oracle.decode_mxfp4(packed, scales)
    assert out[0, 0] == 0.5 and out[0, 1] == 1.0
    assert out[0, 32] == 48.0 and out[0, 33] == -48.0
    assert out[0, 574] == 0.0 and out[0, 575] == -0.125
    assert np.count_nonzero(out) == 5


def test_mxfp4_decode_matches_definition_exhaustively():
    # every nibble in both positions, every finite scale code
    nibs = np.arange(16, dtype=np.uint8)
    byte_vals = (nibs[:, None] | (nibs[None, :] << 4)).reshape(-1)  # 256 bytes
    rows = 255
    packed = np.tile(np.concatenate([byte_vals, byte_vals[:32]]), (rows, 1)).astype(np.uint8)  # 288 bytes
    scales = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 18, axis=1)
    out = oracle.decode_mxfp4(packed, scales)
    e2m1 = np.array([oracle.e2m1_value(n) for n in range(16)])
    for r in (0, 1, 60, 127, 200, 254):
        s = math.ldexp(1.0, r - 127)
        exp_row = np.empty(576)
        exp_row[0::2] = e2m1[packed[r] & 0xF] * s
        exp_row[1::2] = e2m1[packed[r] >> 4] * s
        assert np.array_equal(out[r], exp_row)


# ----------------------------------------------------------------- helpers

def _bf16(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


def _f(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def _decode_ref_torch(q_bits, kv_bits, qo, kvp, sm=SM):
    """Independent formulation of the template page's naive reference in
    torch fp64: (q * sm_scale) @ k^T, softmax, @ v."""
    q = torch.from_numpy(q_bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    kv = torch.from_numpy(kv_bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    out = torch.empty(q.shape[0], q.shape[1], V, dtype=torch.float64)
    for b in range(len(kvp) - 1):
        k = kv[kvp[b]:kvp[b + 1]]
        for t in range(qo[b], qo[b + 1]):
            s = (q[t] * sm) @ k.T
            out[t] = torch.softmax(s, dim=-1) @ k[:, :V]
    return out.numpy()


def _rand_batch(rng, lengths, q_scale=1.0, kv_scale=1.0):
    bs = len(lengths)
    kvp = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    qo = np.arange(bs + 1, dtype=np.int32)
    q = _bf16(rng.standard_normal((bs, H, D)) * q_scale)
    kv = _bf16(rng.standard_normal((int(kvp[-1]), D)) * kv_scale)
    return q, kv, qo, kvp


# ----------------------------------------------------------------- closed forms

def test_single_kv_row_gives_that_row(rng):
    q, kv, qo, kvp = _rand_batch(rng, [1, 1, 1])
    out, lse = oracle.mla_decode(q, kv, qo, kvp)
    for b in range(3):
        row = _f(kv[b])
        for h in range(H):
            assert np.array_equal(out[b, h], row[:V])
            s = SM * float(np.dot(_f(q[b, h]), row))
            assert lse[b, h] == pytest.approx(s, rel=1e-13, abs=1e-13)


def test_identical_scores_give_mean_of_values(rng):
    # q = 0: every score is 0 -> uniform weights -> arithmetic mean of V rows.
    n = 37
    q = np.zeros((1, H, D), dtype=np.uint16)
    kv = _bf16(rng.standard_normal((n, D)))
    out, lse = oracle.mla_decode(q, kv, [0, 1], [0, n])
    vals = _f(kv)
    for v in range(0, V, 17):
        exact = sum(Fraction(float(x)) for x in vals[:, v]) / n
        assert out[0, 0, v] == pytest.approx(float(exact), rel=1e-14, abs=1e-15)
    assert np.allclose(lse[0], math.log(n), rtol=1e-14)


def test_identical_scores_through_rope_columns(rng):
    # q nonzero only in the rope columns (512..575), rope columns equal across
    # rows: scores are equal and nonzero -> still the mean of V.
    n = 9
    qf = np.zeros((1, H, D))
    qf[0, :, 512:] = rng.standard_normal((H, 64))
    kvf = rng.standard_normal((n, D))
    kvf[:, 512:] = kvf[0, 512:]
    q, kv = _bf16(qf), _bf16(kvf)
    out, _ = oracle.mla_decode(q, kv, [0, 1], [0, n])
    mean = _f(kv)[:, :V].mean(axis=0)
    for h in range(H):
        assert np.allclose(out[0, h], mean, rtol=1e-13, atol=1e-15)


def test_two_rows_closed_form(rng):
    q, kv, qo, kvp = _rand_batch(rng, [2])
    out, lse = oracle.mla_decode(q, kv, qo, kvp)
    k = _f(kv)
    for h in range(H):
        qq = _f(q[0, h])
        s1 = float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qq, k[0])) / 24)
        s2 = float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qq, k[1])) / 24)
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        assert np.allclose(out[0, h], w1 * k[0, :V] + w2 * k[1, :V], rtol=1e-13, atol=1e-14)
        assert lse[0, h] == pytest.approx(max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))), rel=1e-13)


# ----------------------------------------------------------------- logit soft-cap

def test_soft_capped_two_rows_closed_form(rng):
    # with a cap, the two weights are sigmoids of the difference of the capped scores
    cap = 0.75
    q, kv, qo, kvp = _rand_batch(rng, [2])
    out, lse = oracle.mla_decode(q, kv, qo, kvp, logit_cap=cap)
    k = _f(kv)
    for h in range(H):
        qq = _f(q[0, h])
        s1 = float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qq, k[0])) / 24)
        s2 = float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qq, k[1])) / 24)
        c1, c2 = cap * math.tanh(s1 / cap), cap * math.tanh(s2 / cap)
        w1 = 1.0 / (1.0 + math.exp(c2 - c1))
        assert np.allclose(out[0, h], w1 * k[0, :V] + (1.0 - w1) * k[1, :V], rtol=1e-12, atol=1e-13)
        assert lse[0, h] == pytest.approx(max(c1, c2) + math.log1p(math.exp(-abs(c1 - c2))), rel=1e-12)


def test_soft_cap_far_above_the_scores_changes_nothing(rng):
    # cap * tanh(s / cap) = s - s^3 / (3 cap^2) + ...: with |s| < 10 and cap 1e5
    # the scores move by < 4e-8 relative
    q, kv, qo, kvp = _rand_batch(rng, [5, 40])
    plain, lse0 = oracle.mla_decode(q, kv, qo, kvp)
    capped, lse1 = oracle.mla_decode(q, kv, qo, kvp, logit_cap=1e5)
    assert np.allclose(capped, plain, rtol=1e-7, atol=1e-9)
    assert np.allclose(lse1, lse0, rtol=1e-7)


def test_soft_cap_saturation_gives_mean_of_values(rng):
    # every score far above the cap: tanh saturates, the capped scores are all
    # equal (to cap up to ~1e-40), so the output is the mean of the V rows
    n = 11
    qf = np.zeros((1, H, D))
    qf[0, :, 512] = 64.0
    kvf = rng.standard_normal((n, D))
    kvf[:, 512] = 64.0 + rng.integers(0, 64, size=n)  # scores 64*[64, 128)/24 > 170
    q, kv = _bf16(qf), _bf16(kvf)
    out, lse = oracle.mla_decode(q, kv, [0, 1], [0, n], logit_cap=2.0)
    mean = _f(kv)[:, :V].mean(axis=0)
    for h in range(H):
        assert np.allclose(out[0, h], mean, rtol=1e-13, atol=1e-15)
    assert np.allclose(lse[0], 2.0 + math.log(n), rtol=1e-13)


def test_empty_sequence_gives_zero_and_minus_inf(rng):
    q, kv, qo, kvp = _rand_batch(rng, [3, 0, 2])
    out, lse = oracle.mla_decode(q, kv, qo, kvp)
    assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(out[[0, 2]]))


# ----------------------------------------------------------------- brute force

def test_brute_force_decimal_tiny_inputs(rng):
    """Direct softmax with no max subtraction, in 60-digit decimal arithmetic on
    exactly represented inputs (small dims: the oracle is dimension-generic)."""
    getcontext().prec = 60
    h, d, v = 2, 8, 4
    sm = 1.0 / math.sqrt(8.0)
    for n in range(1, 9):
        qf = rng.standard_normal((1, h, d)) * 2
        kf = rng.standard_normal((n, d)) * 2
        q, kv = _bf16(qf), _bf16(kf)
        out, lse = oracle.mla_decode(q, kv, [0, 1], [0, n], num_heads=h, qk_dim=d, v_dim=v, sm_scale=sm)
        qd, kd = _f(q), _f(kv)
        smd = Decimal(1) / Decimal(8).sqrt()
        for hh in range(h):
            s = [smd * sum(Decimal(float(qd[0, hh, i])) * Decimal(float(kd[j, i])) for i in range(d))
                 for j in range(n)]
            w = [x.exp() for x in s]
            tot = sum(w)
            for c in range(v):
                ref = sum(w[j] * Decimal(float(kd[j, c])) for j in range(n)) / tot
                assert out[0, hh, c] == pytest.approx(float(ref), rel=1e-12, abs=1e-14)
            assert lse[0, hh] == pytest.approx(float(tot.ln()), rel=1e-12, abs=1e-14)


# ----------------------------------------------------------------- identities

def _combine(outs, lses):
    """LSE-weighted recombination of per-piece results (test-side)."""
    finite = np.isfinite(lses)
    m = np.max(np.where(finite, lses, -np.inf), axis=0)
    w = np.where(finite, np.exp(lses - m), 0.0)
    return (w[:, :, None] * outs).sum(axis=0) / w.sum(axis=0)[:, None]


def test_split_recombination_equals_unsplit(rng):
    n = 300
    q, kv, qo, kvp = _rand_batch(rng, [n])
    full, full_lse = oracle.mla_decode(q, kv, qo, kvp)
    for trial in range(4):
        k = int(rng.integers(2, 9))
        cuts = np.sort(rng.integers(0, n + 1, size=k - 1))
        bounds = np.concatenate([[0], cuts, [n]]).astype(np.int32)   # may contain empty pieces
        qrep = np.repeat(q, k, axis=0)
        outs, lses = oracle.mla_decode(qrep, kv, np.arange(k + 1, dtype=np.int32), bounds)
        comb = _combine(outs, lses)
        assert np.allclose(comb, full[0], rtol=1e-12, atol=1e-14)
        # the combined LSE is log-sum-exp of the pieces'
        fin = np.isfinite(lses)
        m = np.max(np.where(fin, lses, -np.inf), axis=0)
        lse_c = m + np.log(np.where(fin, np.exp(lses - m), 0).sum(axis=0))
        assert np.allclose(lse_c, full_lse[0], rtol=1e-13)


def test_row_permutation_invariance(rng):
    q, kv, qo, kvp = _rand_batch(rng, [64])
    out, _ = oracle.mla_decode(q, kv, qo, kvp)
    perm = rng.permutation(64)
    out2, _ = oracle.mla_decode(q, kv[perm], qo, kvp)
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-15)


def test_score_shift_through_rope_column(rng):
    # Adding 1 to KV column 512 of every row adds q[h,512]*sm_scale to every
    # score of head h: the softmax, and so the output, is unchanged.
    qf = rng.standard_normal((1, H, D))
    kf = rng.standard_normal((50, D))
    kf[:, 512] = 0.0
    q = _bf16(qf)
    kv1 = _bf16(kf)
    kf2 = kf.copy()
    kf2[:, 512] = 1.0
    kv2 = _bf16(kf2)
    o1, l1 = oracle.mla_decode(q, kv1, [0, 1], [0, 50])
    o2, l2 = oracle.mla_decode(q, kv2, [0, 1], [0, 50])
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-15)
    assert np.allclose(l2 - l1, _f(q)[0, :, 512] * SM, rtol=1e-12, atol=1e-13)


def test_duplicated_heads_identical(rng):
    q, kv, qo, kvp = _rand_batch(rng, [40, 7])
    q[:, 5] = q[:, 3]
    out, lse = oracle.mla_decode(q, kv, qo, kvp)
    assert np.array_equal(out[:, 5], out[:, 3]) and np.array_equal(lse[:, 5], lse[:, 3])


def test_ragged_sequence_equals_sequence_alone(rng):
    lengths = [5, 130, 1, 77]
    q, kv, qo, kvp = _rand_batch(rng, lengths)
    out, _ = oracle.mla_decode(q, kv, qo, kvp)
    for b in range(4):
        alone, _ = oracle.mla_decode(q[b:b + 1], kv[kvp[b]:kvp[b + 1]], [0, 1], [0, lengths[b]])
        assert np.array_equal(alone[0], out[b])


def test_seq_subset_matches_full(rng):
    q, kv, qo, kvp = _rand_batch(rng, [12, 30, 3, 9])
    full, _ = oracle.mla_decode(q, kv, qo, kvp, threads=3)
    sub, _ = oracle.mla_decode(q, kv, qo, kvp, seq_ids=[3, 1])
    assert np.array_equal(sub[[1, 3]], full[[1, 3]])
    assert np.all(np.isnan(sub[[0, 2]]))


def test_matches_independent_torch_fp64(rng):
    lengths = [1, 2, 33, 250]
    q, kv, qo, kvp = _rand_batch(rng, lengths, q_scale=3.0, kv_scale=1.5)
    out, _ = oracle.mla_decode(q, kv, qo, kvp, threads=2)
    ref = _decode_ref_torch(q, kv, qo, kvp)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_multiple_query_rows_per_sequence(rng):
    # q_len > 1 through qo_indptr: every query row attends to all KV rows of
    # its sequence, with no mask.
    q = _bf16(rng.standard_normal((5, H, D)))
    kv = _bf16(rng.standard_normal((20, D)))
    qo = np.array([0, 3, 5], dtype=np.int32)
    kvp = np.array([0, 12, 20], dtype=np.int32)
    out, _ = oracle.mla_decode(q, kv, qo, kvp)
    ref = _decode_ref_torch(q, kv, qo, kvp)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------- paged KV (page size 1)

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
def test_paged_rows_equal_contiguous_rows(kv_dtype):
    # the same batch with its rows scattered over a larger buffer through a
    # random injective map gives exactly the contiguous result
    w = synth.make_batch([5, 0, 40, 17], "bf16", kv_dtype, seed=7, q_lens=[1, 2, 2, 1])
    pw = synth.page_workload(w, seed=8, spare_rows=30)
    assert pw.kv_rows == w.total_kv + 30 and not np.array_equal(pw.kv[: w.total_kv], w.kv)
    a, la = oracle.decode_workload(w)
    b, lb = oracle.decode_workload(pw)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_paged_identity_and_repeated_rows(rng):
    q, kv, qo, kvp = _rand_batch(rng, [6, 3])
    ident = np.arange(9, dtype=np.int32)
    assert np.array_equal(oracle.mla_decode(q, kv, qo, kvp, kv_indices=ident)[0], oracle.mla_decode(q, kv, qo, kvp)[0])
    # two CSR rows naming one physical row: the same as that row stored twice
    idx = np.array([0, 1, 2, 2, 4, 5, 6, 7, 8], dtype=np.int32)
    dup = kv[idx]
    assert np.array_equal(oracle.mla_decode(q, kv, qo, kvp, kv_indices=idx)[0], oracle.mla_decode(q, dup, qo, kvp)[0])


@pytest.mark.parametrize("page_size", [2, 16, 64])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
def test_pages_equal_contiguous_rows(kv_dtype, page_size):
    # pages of page_size rows: each sequence's rows are written page by page
    # (here, not by the generator) into pages drawn from a permutation of a
    # larger buffer; the oracle reading them through the page lists gives
    # exactly the contiguous result
    w = synth.make_batch([5, 0, 40, 17, 64, 1], "bf16", kv_dtype, seed=17, q_lens=[1, 2, 2, 1, 1, 1])
    P = page_size
    rng = np.random.default_rng(99 + P)
    lens = np.diff(np.asarray(w.kv_indptr, dtype=np.int64))
    starts = [0]
    for n in lens:
        starts.append(starts[-1] + (int(n) + P - 1) // P)
    npages = starts[-1] + 5
    page_ids = rng.permutation(npages)[: starts[-1]].astype(np.int32)
    kv = np.zeros((npages * P,) + w.kv.shape[1:], dtype=w.kv.dtype)
    ks = np.zeros((npages * P,) + w.kv_scale.shape[1:], dtype=np.uint8) if kv_dtype == "mxfp4" else w.kv_scale
    for b, n in enumerate(lens):
        for i in range(int(n)):
            dst = int(page_ids[starts[b] + i // P]) * P + i % P
            kv[dst] = w.kv[int(w.kv_indptr[b]) + i]
            if kv_dtype == "mxfp4":
                ks[dst] = w.kv_scale[int(w.kv_indptr[b]) + i]
    a, la = oracle.decode_workload(w)
    b_, lb = oracle.mla_decode(w.q, kv, w.qo_indptr, w.kv_indptr, q_dtype=w.q_dtype, kv_dtype=kv_dtype,
                               q_scale=w.q_scale, kv_scale=ks, sm_scale=w.sm_scale, kv_indices=page_ids,
                               kv_page_indptr=np.array(starts, dtype=np.int32), page_size=P)
    assert np.array_equal(a, b_, equal_nan=True) and np.array_equal(la, lb, equal_nan=True)
    # and the generator's paged layout reads back the same
    pw = synth.page_workload(w, seed=18, spare_rows=3 * P, page_size=P)
    assert pw.total_kv == w.total_kv and pw.kv_rows % P == 0
    c, lc = oracle.decode_workload(pw)
    assert np.array_equal(a, c, equal_nan=True) and np.array_equal(la, lc, equal_nan=True)


def test_pages_bigger_than_every_sequence(rng):
    # one page per sequence holding all its rows at its start: page p of P rows
    # is rows [p * P, p * P + len) of the buffer
    q, kv, qo, kvp = _rand_batch(rng, [6, 3])
    P = 8
    buf = np.zeros((3 * P,) + kv.shape[1:], dtype=kv.dtype)
    buf[2 * P: 2 * P + 6] = kv[0:6]
    buf[0:3] = kv[6:9]
    out, _ = oracle.mla_decode(q, buf, qo, kvp, kv_indices=np.array([2, 0], dtype=np.int32),
                               kv_page_indptr=np.array([0, 1, 2], dtype=np.int32), page_size=P)
    assert np.array_equal(out, oracle.mla_decode(q, kv, qo, kvp)[0])


# ----------------------------------------------------------------- quantised formats

def test_fp8_kv_folding_identity(rng):
    """fp8 codes with a power-of-two scale decode to bf16-representable values:
    the oracle on (codes, scale) equals the oracle on those values as bf16."""
    n = 70
    codes = rng.integers(0, 256, size=(n, D), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    scale = 0.25
    q = _bf16(rng.standard_normal((1, H, D)) * 0.05)
    o8, l8 = oracle.mla_decode(q, codes, [0, 1], [0, n], kv_dtype="fp8", kv_scale=scale)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale
    ob, lb = oracle.mla_decode(q, _bf16(dec), [0, 1], [0, n])
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_fp8_q_folding_identity(rng):
    n = 40
    qc = rng.integers(0, 256, size=(1, H, D), dtype=np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x22
    kv = _bf16(rng.standard_normal((n, D)))
    o8, _ = oracle.mla_decode(qc, kv, [0, 1], [0, n], q_dtype="fp8", q_scale=0.125)
    dec = torch.from_numpy(qc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 0.125
    ob, _ = oracle.mla_decode(_bf16(dec), kv, [0, 1], [0, n])
    assert np.array_equal(o8, ob)


def test_a8w8_scales_fold_into_scores(rng):
    """fp8 q and fp8 kv with arbitrary fp32 scales equal the independent torch
    formulation on the decoded tensors (the template page's fp8 reference
    multiplies scale_a * scale_b into the fp8 product)."""
    n = 90
    qc, qs = synth.encode_e4m3fn(rng.standard_normal((1, H, D)) * 40), 0.021
    kc, ks = synth.encode_e4m3fn(rng.standard_normal((n, D)) * 60), 0.017
    out, _ = oracle.mla_decode(qc, kc, [0, 1], [0, n], q_dtype="fp8", kv_dtype="fp8", q_scale=qs, kv_scale=ks)
    qd = torch.from_numpy(qc).view(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(qs))
    kd = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(ks))
    s = (qd[0] @ kd.T) * SM
    ref = torch.softmax(s, dim=-1) @ kd[:, :V]
    assert np.allclose(out[0], ref.numpy(), rtol=1e-11, atol=1e-13)


def test_mxfp4_kv_folding_identity(rng):
    n = 45
    packed, scales = synth.encode_mxfp4(rng.standard_normal((n, D)) * 3)
    q = _bf16(rng.standard_normal((1, H, D)) * 0.1)
    o4, l4 = oracle.mla_decode(q, packed, [0, 1], [0, n], kv_dtype="mxfp4", kv_scale=scales)
    dec = oracle.decode_mxfp4(packed, scales)
    ob, lb = oracle.mla_decode(q, _bf16(dec), [0, 1], [0, n])
    assert np.array_equal(o4, ob) and np.array_equal(l4, lb)
