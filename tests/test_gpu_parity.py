"""GPU parity of the HIP decode against the CPU fp64 oracle (MI355X only).

Every call goes through the C ABI (mla_decode_plan / mla_decode_run /
mla_debug_decode) via the ctypes binding.  Tolerances (bf16 output against the
fp64 oracle): max |gpu - oracle| <= 2e-2 and ||gpu - oracle||_2 / ||oracle||_2
<= 1e-2 over the compared outputs; the dequantisation check is bit-exact.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import mla_decode_split_amd as mla
from mla_decode_split_amd import device as dev

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 1e-2


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _bf16_out_to_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def _compare(got, ref, what):
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    _say(f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= MAX_ABS, f"{what}: max_abs {max_abs}"
    assert rel <= REL_L2, f"{what}: rel_l2 {rel}"
    return max_abs, rel


def _check_batch(w, rows_per_split=0, seq_ids=None, use_host_indptr=True, poison=True, what=""):
    _say(f"case {what or w.name}: bs={w.batch_size} total_kv={w.total_kv} q={w.q_dtype} kv={w.kv_dtype} "
         f"rows_per_split={rows_per_split}")
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=rows_per_split, use_host_indptr=use_host_indptr)
    ws = dev.workspace_for(plan, fill=float("nan") if poison else None)
    out = torch.full((b.total_q, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    dev.run(plan, b, out, ws)
    torch.cuda.synchronize()
    got = _bf16_out_to_f64(out)
    ref, _ = oracle.decode_workload(w, seq_ids=seq_ids, threads=_host_threads())
    if seq_ids is not None:
        rows = _query_rows(w, seq_ids)
        got, ref = got[rows], ref[rows]
    elif w.batch_size >= 32:
        _worst_sequence(w, got, ref, what or w.name)
    return _compare(got, ref, what or w.name), plan, out


def _host_threads():
    import os
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 8


def _worst_sequence(w, got, ref, what):
    """Print the worst per-sequence max-abs and rel-L2 (diagnostics; the bar is
    applied to the whole output)."""
    qo = np.asarray(w.qo_indptr, dtype=np.int64)
    worst_abs, worst_rel = (0.0, -1), (0.0, -1)
    for b in range(w.batch_size):
        g, r = got[qo[b]:qo[b + 1]], ref[qo[b]:qo[b + 1]]
        if g.size == 0:
            continue
        a = float(np.abs(g - r).max())
        rl = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
        worst_abs = max(worst_abs, (a, b))
        worst_rel = max(worst_rel, (rl, b))
    _say(f"{what}: worst sequence max_abs={worst_abs[0]:.3e} (b={worst_abs[1]}) "
         f"rel_l2={worst_rel[0]:.3e} (b={worst_rel[1]}) over {w.batch_size} sequences")


def _query_rows(w, seq_ids):
    """Output rows of the given sequences (several per sequence when q_len > 1)."""
    qo = np.asarray(w.qo_indptr, dtype=np.int64)
    return np.concatenate([np.arange(qo[b], qo[b + 1]) for b in seq_ids]).astype(np.int64)


# ------------------------------------------------------------- dequantisation

def test_fp8_decode_bit_exact():
    codes = np.arange(256, dtype=np.uint8)
    for scale in (1.0, 0.37, 2.0 ** -7):
        d_codes = torch.from_numpy(codes).cuda()
        d_scale = torch.tensor([scale], dtype=torch.float32, device="cuda")
        out = torch.empty(256, dtype=torch.float32, device="cuda")
        mla.mla_debug_decode("fp8", d_codes, d_scale, out, 256)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = (oracle.decode_fp8(codes, float(np.float32(scale)))).astype(np.float32)  # one rounding to fp32
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32)), f"scale {scale}"


def test_mxfp4_decode_bit_exact():
    # every byte value (both nibble positions) under every scale code 2..252,
    # where e2m1 * 2^(e-127) is a normal bf16/fp32 number
    rows = 251
    byte_vals = np.arange(256, dtype=np.uint8)
    packed = np.tile(np.concatenate([byte_vals, byte_vals[:32]]), (rows, 1))
    scales = np.repeat(np.arange(2, 253, dtype=np.uint8)[:, None], 18, axis=1)
    scales[::3, 5] = 127
    d_p = torch.from_numpy(packed).cuda()
    d_s = torch.from_numpy(np.concatenate([scales.reshape(-1), np.zeros(16, np.uint8)])).cuda()
    out = torch.empty((rows, 576), dtype=torch.float32, device="cuda")
    mla.mla_debug_decode("mxfp4", d_p, d_s, out, rows)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.decode_mxfp4(packed, scales).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_mxfp4_decode_extreme_scales_report():
    """Scale codes whose products leave the normal range: report what the
    hardware gives (recorded in the design notes); finite normal results must
    still be exact."""
    codes = np.array([0, 1, 253, 254], dtype=np.uint8)
    packed = np.tile(np.concatenate([np.arange(256, dtype=np.uint8), np.arange(32, dtype=np.uint8)]), (4, 1))
    scales = np.repeat(codes[:, None], 18, axis=1)
    d_p = torch.from_numpy(packed).cuda()
    d_s = torch.from_numpy(np.concatenate([scales.reshape(-1), np.zeros(16, np.uint8)])).cuda()
    out = torch.empty((4, 576), dtype=torch.float32, device="cuda")
    mla.mla_debug_decode("mxfp4", d_p, d_s, out, 4)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.decode_mxfp4(packed, scales)
    for r, c in enumerate(codes):
        exact = got[r] == ref[r]
        _say(f"e8m0={c}: {int(exact.sum())}/576 exact; sample got={got[r][:4]} ref={ref[r][:4]}")
        normal = (np.abs(ref[r]) >= 2.0 ** -126) & (np.abs(ref[r]) < 3.3e38)
        assert np.all(exact[normal])


def test_bf16_decode_passthrough():
    x = synth.normal_bf16(11, 1, 1000)
    out = torch.empty(1000, dtype=torch.float32, device="cuda")
    mla.mla_debug_decode("bf16", torch.from_numpy(x.view(np.int16)).cuda(), None, out, 1000)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), synth.bf16_to_f32(x))


# ------------------------------------------------------------- small batches, full comparison

EDGE_LENGTHS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257]
COMBOS = [("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8"), ("bf16", "mxfp4"), ("fp8", "bf16"), ("fp8", "mxfp4")]


@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_edge_lengths_all_formats(q_dtype, kv_dtype):
    w = synth.make_batch(EDGE_LENGTHS, q_dtype, kv_dtype, seed=101, name=f"edges-{q_dtype}-{kv_dtype}")
    _check_batch(w, what=f"edge lengths {q_dtype}/{kv_dtype}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("rows", [32, 96, 224, 512, 2048])
def test_forced_split_counts(kv_dtype, rows):
    # lengths 700, 1000, 33 -> splits per sequence range from 1 to 32
    w = synth.make_batch([700, 1000, 33], "bf16", kv_dtype, seed=202, name="forced")
    _check_batch(w, rows_per_split=rows, what=f"forced rows_per_split={rows} kv={kv_dtype}")


# (lengths, rows per split, the merge batch the plan picks): stage 2 loads 2,
# 4, 8 or 16 slots at once, from the most pieces one sequence has; 32-row
# ranges give up to 32 pieces, two batches of 16
MERGE_BATCH_CASES = [([300, 200, 60], 256, 2), ([520, 300], 256, 4), ([700, 1000, 33], 224, 8),
                     ([700, 1000, 33], 96, 16), ([700, 1000, 33], 32, 16)]


@pytest.mark.parametrize("q_len", [1, 2])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("lengths,rows,nb", MERGE_BATCH_CASES)
def test_merge_batch_sizes(lengths, rows, nb, kv_dtype, q_len):
    w = synth.make_batch(lengths, "bf16", kv_dtype, seed=212 + nb, name="merge-batch",
                         q_lens=None if q_len == 1 else [q_len] * len(lengths))
    (_, _), plan, _ = _check_batch(w, rows_per_split=rows, what=f"merge batch {nb}, rows {rows}, kv={kv_dtype}, q_len {q_len}")
    assert mla.mla_decode_plan_describe(plan)["merge_batch"] == nb


def test_empty_sequences_give_zero():
    w = synth.make_batch([0, 40, 0, 300, 0], "bf16", "fp8", seed=303, name="empties")
    (_, _), plan, out = _check_batch(w, rows_per_split=64, what="empty sequences")
    o = out.float().cpu().numpy()
    assert np.all(o[[0, 2, 4]] == 0.0)


def test_plan_without_host_indptr_matches():
    w = synth.make_batch([100, 7, 900, 64], "bf16", "fp8", seed=404, name="no-host-indptr")
    _check_batch(w, use_host_indptr=False, rows_per_split=128, what="plan without host indptr")
    _check_batch(w, use_host_indptr=True, rows_per_split=2048, what="single split per sequence (no stage 2)")


def test_many_short_sequences():
    # 1000 sequences (more than the merge kernel's argument table holds, and
    # several passes of the stage-1 sequence search), lengths 0..300 with a
    # few empty, two query rows each
    lengths = synth.uniform_lengths(77, synth.STREAM_LEN, 1000, 0, 300)
    w = synth.make_batch(lengths, "bf16", "fp8", seed=777, name="many", q_lens=[2] * 1000)
    (_, _), plan, out = _check_batch(w, what="1000 short sequences, two query rows")
    assert mla.mla_decode_plan_describe(plan)["stage2"] == 1
    o = out.float().cpu().numpy()
    for b in np.flatnonzero(lengths == 0)[:5]:
        assert np.all(o[2 * b:2 * b + 2] == 0.0)


def test_long_single_sequence():
    w = synth.make_batch([20000], "bf16", "fp8", seed=505, name="long")
    _check_batch(w, what="one sequence of 20000 rows")


def test_unaligned_mxfp4_scale_rows():
    # sequence starts at odd rows so tiles begin at scale offsets that are not 16-byte aligned
    w = synth.make_batch([1, 3, 5, 77, 129, 1000], "bf16", "mxfp4", seed=606, name="mx-unaligned")
    for rows in (32, 64, 160):
        _check_batch(w, rows_per_split=rows, what=f"mxfp4 unaligned starts rows={rows}")


# ------------------------------------------------------------- several query rows per sequence

@pytest.mark.parametrize("q_len", [2, 3, 4])
@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_multi_token_edge_lengths(q_dtype, kv_dtype, q_len):
    # every sequence has q_len query rows (multi-token prediction / speculative decoding)
    w = synth.make_batch(EDGE_LENGTHS, q_dtype, kv_dtype, seed=111 + q_len, name="mtp-edges",
                         q_lens=[q_len] * len(EDGE_LENGTHS))
    (_, _), plan, _ = _check_batch(w, what=f"q_len {q_len} edge lengths {q_dtype}/{kv_dtype}")
    assert mla.mla_decode_plan_describe(plan)["query_tokens"] == (4 if q_len == 3 else q_len)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("rows", [32, 96, 512])
def test_multi_token_ragged_rows_and_splits(kv_dtype, rows):
    # query rows 0..4 per sequence, KV lengths from 0 up, pieces of 1 to many tiles
    lengths = [700, 0, 33, 1000, 1, 257, 64, 0]
    q_lens = [2, 3, 4, 1, 0, 4, 3, 2]
    w = synth.make_batch(lengths, "bf16", kv_dtype, seed=222, name="mtp-ragged", q_lens=q_lens)
    (_, _), _, out = _check_batch(w, rows_per_split=rows, what=f"ragged q rows, rows_per_split={rows} kv={kv_dtype}")
    qo = w.qo_indptr
    o = out.float().cpu().numpy()
    for b in (1, 7):  # no KV rows: zeros
        assert np.all(o[qo[b]:qo[b + 1]] == 0.0)


def test_multi_token_plan_without_host_indptr():
    w = synth.make_batch([100, 7, 900, 64], "fp8", "fp8", seed=333, name="mtp-no-host", q_lens=[2, 2, 1, 2])
    _check_batch(w, use_host_indptr=False, rows_per_split=128, what="q_len <= 2, plan without host indptr")
    _check_batch(w, use_host_indptr=True, rows_per_split=2048, what="q_len <= 2, one split per sequence")


def test_multi_token_rows_equal_single_token_runs():
    # query rows of a sequence do not interact: each row of a two-row run matches
    # a one-row run of the same query on the same KV (within the parity bar)
    lengths = [3000, 17]
    w2 = synth.make_batch(lengths, "bf16", "fp8", seed=444, name="mtp-pair", q_lens=[2, 2])
    b2 = dev.upload(w2)
    out2 = dev.run(dev.plan_for(b2, rows_per_split=512), b2)
    for r in range(2):
        w1 = synth.make_batch(lengths, "bf16", "fp8", seed=444, name="mtp-single", q_lens=[1, 1])
        w1.q = np.ascontiguousarray(w2.q[[r, 2 + r]])
        b1 = dev.upload(w1)
        out1 = dev.run(dev.plan_for(b1, rows_per_split=512), b1)
        torch.cuda.synchronize()
        a = _bf16_out_to_f64(out2)[[r, 2 + r]]
        c = _bf16_out_to_f64(out1)
        _compare(a, c, f"row {r} of q_len 2 vs a one-row run")


# ------------------------------------------------------------- logit soft-cap

@pytest.mark.parametrize("q_dtype,kv_dtype", COMBOS)
def test_soft_cap_all_formats(q_dtype, kv_dtype):
    # scores here are about N(0, 1): a cap of 1 bends most of them
    w = synth.make_batch(EDGE_LENGTHS, q_dtype, kv_dtype, seed=121, name="softcap")
    w.logit_cap = 1.0
    _check_batch(w, what=f"logit_cap 1.0 {q_dtype}/{kv_dtype}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
def test_soft_cap_with_query_rows_and_splits(kv_dtype):
    w = synth.make_batch([700, 0, 33, 1000, 257], "bf16", kv_dtype, seed=131, name="softcap-mtp", q_lens=[2, 1, 2, 0, 2])
    w.logit_cap = 0.5
    _check_batch(w, rows_per_split=96, what=f"logit_cap 0.5, q_len <= 2, rows_per_split=96 kv={kv_dtype}")


def test_soft_cap_saturating_scores():
    # queries scaled by 16 (exact in bf16): scores about N(0, 256), most of them
    # far past the cap of 4, where tanh saturates
    w = synth.make_batch([1000, 64, 4000], "bf16", "fp8", seed=141, name="softcap-sat")
    w.q = synth.bf16_bits(synth.bf16_to_f32(w.q) * 16.0)
    w.logit_cap = 4.0
    _check_batch(w, rows_per_split=256, what="logit_cap 4, saturating scores")


# ------------------------------------------------------------- paged KV (page size 1)

PAGED_COMBOS = COMBOS


def _paged_equals_contiguous(w, pw, rows_per_split=0, what=""):
    """The paged run reads the same CSR rows as the contiguous one, through the
    indices: with the same cut (the paged plan's, whose residency may differ)
    the outputs agree bit for bit."""
    b, pb = dev.upload(w), dev.upload(pw)
    paged_plan = dev.plan_for(pb, rows_per_split=rows_per_split)
    d = mla.mla_decode_plan_describe(paged_plan)
    # the same cut: the base range length (paired ranges split 2R unevenly)
    rows = (d["rows_per_split"] + d["second_rows_per_split"]) // 2 if d["paired_splits"] else d["rows_per_split"]
    plan = dev.plan_for(b, rows_per_split=rows)
    assert mla.mla_decode_plan_describe(plan)["num_splits"] == d["num_splits"]
    o1 = dev.run(plan, b)
    o2 = dev.run(paged_plan, pb)
    torch.cuda.synchronize()
    same = bool(torch.equal(o1.view(torch.int16), o2.view(torch.int16)))
    _say(f"{what}: paged == contiguous bitwise: {same}")
    assert same


@pytest.mark.parametrize("q_dtype,kv_dtype", PAGED_COMBOS)
def test_paged_edge_lengths(q_dtype, kv_dtype):
    w = synth.make_batch(EDGE_LENGTHS, q_dtype, kv_dtype, seed=151, name="paged-edges")
    pw = synth.page_workload(w, seed=152, spare_rows=777)
    _check_batch(pw, what=f"paged {q_dtype}/{kv_dtype}")
    _paged_equals_contiguous(w, pw, what=f"paged {q_dtype}/{kv_dtype}")


@pytest.mark.parametrize("q_dtype,kv_dtype", PAGED_COMBOS)
def test_pages_edge_lengths(q_dtype, kv_dtype):
    # pages of 32 rows (one tile) at the edge lengths, every format pair
    w = synth.make_batch(EDGE_LENGTHS, q_dtype, kv_dtype, seed=153, name="pages-edges")
    pw = synth.page_workload(w, seed=154, spare_rows=777, page_size=32)
    _check_batch(pw, what=f"pages of 32 {q_dtype}/{kv_dtype}")
    _paged_equals_contiguous(w, pw, what=f"pages of 32 {q_dtype}/{kv_dtype}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("rows", [32, 96, 512])
def test_paged_query_rows_cap_and_splits(kv_dtype, rows):
    w = synth.make_batch([700, 0, 33, 1000, 1, 257], "bf16", kv_dtype, seed=161, name="paged-mix",
                         q_lens=[2, 1, 4, 0, 3, 1])
    w.logit_cap = 2.0
    pw = synth.page_workload(w, seed=162, spare_rows=100)
    _check_batch(pw, rows_per_split=rows, what=f"paged, q rows <= 4, cap 2, rows_per_split={rows} kv={kv_dtype}")
    _paged_equals_contiguous(w, pw, rows_per_split=rows, what=f"paged mix rows={rows} kv={kv_dtype}")


@pytest.mark.parametrize("cap", [0.0, 2.5])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
def test_paged_two_query_rows(kv_dtype, cap):
    # at most two query rows per sequence: the two-row paged kernels, with and
    # without the soft-cap, against the oracle and bitwise against contiguous KV
    w = synth.make_batch([700, 0, 33, 1000, 1, 257], "bf16", kv_dtype, seed=181, name="paged-q2",
                         q_lens=[2, 1, 2, 0, 2, 1])
    w.logit_cap = cap
    pw = synth.page_workload(w, seed=182, spare_rows=100)
    (_, _), plan, _ = _check_batch(pw, rows_per_split=96, what=f"paged, q rows <= 2, cap {cap}, kv={kv_dtype}")
    assert mla.mla_decode_plan_describe(plan)["query_tokens"] == 2
    _paged_equals_contiguous(w, pw, rows_per_split=96, what=f"paged q2 cap={cap} kv={kv_dtype}")


@pytest.mark.parametrize("page_size", [2, 16, 64, 256])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "mxfp4"])
def test_pages_of_several_rows(kv_dtype, page_size):
    # pages of page_size rows listed per sequence: query rows 0-4, a cap and
    # forced splits (pieces start inside pages), against the oracle and bitwise
    # against contiguous KV
    w = synth.make_batch([700, 0, 33, 1000, 1, 257], "bf16", kv_dtype, seed=201, name="pages",
                         q_lens=[2, 1, 4, 0, 3, 1])
    w.logit_cap = 2.0
    pw = synth.page_workload(w, seed=202 + page_size, spare_rows=3 * page_size, page_size=page_size)
    (_, _), plan, _ = _check_batch(pw, rows_per_split=96, what=f"pages of {page_size} rows, kv={kv_dtype}")
    _paged_equals_contiguous(w, pw, rows_per_split=96, what=f"pages of {page_size} rows kv={kv_dtype}")


def test_pages_full_size():
    # bs 64, KV 8192 fp8 in pages of 16 rows, in the planner's launch
    # configuration: every sequence against the oracle, the whole output
    # bitwise against the contiguous run
    w = synth.make_workload("bs64_kv8192_fp8")
    pw = synth.page_workload(w, seed=211, spare_rows=w.total_kv // 8, page_size=16)
    _check_batch(pw, poison=False, what="bs64 kv8192 fp8 pages of 16 (every sequence)")
    _paged_equals_contiguous(w, pw, what="bs64 kv8192 fp8 pages of 16")


def test_paged_plan_without_host_indptr():
    w = synth.make_batch([100, 7, 900, 64], "bf16", "fp8", seed=171, name="paged-no-host")
    pw = synth.page_workload(w, seed=172, spare_rows=64)
    _check_batch(pw, use_host_indptr=False, rows_per_split=128, what="paged, plan without host indptr")


def test_paged_mxfp4_ragged_full_size():
    # the ragged MXFP4 batch scattered over a buffer with 1/16 spare rows (every
    # scale-row offset in its 16-byte unit occurs), every sequence against the
    # oracle, the whole output bitwise against the contiguous run
    w = synth.make_workload("bs128_ragged_mxfp4")
    pw = synth.page_workload(w, seed=191, spare_rows=w.total_kv // 16)
    _check_batch(pw, poison=False, what="ragged mxfp4 paged (every sequence)")
    _paged_equals_contiguous(w, pw, what="ragged mxfp4 paged")


def test_paged_full_size():
    # bs 64, KV 8192 fp8 scattered over a buffer with 1/8 spare rows, in the
    # planner's launch configuration: every sequence against the oracle, the
    # whole output bitwise against the contiguous run
    w = synth.make_workload("bs64_kv8192_fp8")
    pw = synth.page_workload(w, seed=181, spare_rows=w.total_kv // 8)
    _check_batch(pw, poison=False, what="bs64 kv8192 fp8 paged (every sequence)")
    _paged_equals_contiguous(w, pw, what="bs64 kv8192 fp8 paged")


def test_runs_are_deterministic():
    w = synth.make_batch([3000, 17, 4000], "bf16", "fp8", seed=707, name="det")
    b = dev.upload(w)
    plan = dev.plan_for(b)
    o1 = dev.run(plan, b).clone()
    o2 = dev.run(plan, b)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_run_on_a_side_stream():
    w = synth.make_batch([500, 600], "bf16", "fp8", seed=808, name="stream")
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=128)
    s = torch.cuda.Stream()
    out = torch.empty((2, 16, 512), dtype=torch.bfloat16, device="cuda")
    ws = dev.workspace_for(plan)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dev.run(plan, b, out, ws, stream=s)
    s.synchronize()
    ref, _ = oracle.decode_workload(w, threads=8)
    _compare(_bf16_out_to_f64(out), ref, "side stream")


def _widened_batch(q_len, seed):
    """Several query rows, a soft-cap and paged KV at once."""
    w = synth.make_batch([900, 64, 3000, 1, 2500], "bf16", "fp8", seed=seed, name="widened",
                         q_lens=[q_len, 1, q_len, 0, q_len])
    w.logit_cap = 3.0
    return synth.page_workload(w, seed=seed + 1, spare_rows=300)


@pytest.mark.parametrize("widened", [False, True])
def test_split_then_merge_equals_run(widened):
    """mla_decode_split (or _split_paged) followed by mla_decode_merge on one
    stream gives the same bits as mla_decode_run (or _run_paged)."""
    if widened:
        w = _widened_batch(4, 1011)
    else:
        w = synth.make_batch([900, 64, 3000, 1, 2500], "bf16", "fp8", seed=1001, name="split+merge")
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=256)
    ws = dev.workspace_for(plan)
    a_out = torch.full((b.total_q, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    b_out = torch.full_like(a_out, float("nan"))
    dev.run(plan, b, a_out, ws)
    dev.run_split(plan, b, b_out, ws)
    dev.run_merge(plan, b, b_out, ws)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16))


@pytest.mark.parametrize("widened", [False, True])
def test_graph_replays_match_eager(widened):
    """mla_decode_run (or _run_paged with several query rows and a soft-cap)
    captured in a HIP graph (no memset nodes: the library records none) and
    replayed several times, with eager work and a synchronisation between
    replays; every replay must equal the eager result bit for bit, and the
    oracle within tolerance."""
    if widened:
        w = _widened_batch(2, 919)
    else:
        w = synth.make_batch([700, 1500, 33, 4096], "bf16", "fp8", seed=909, name="graph")
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=256)
    ws = dev.workspace_for(plan)
    eager = torch.empty((b.total_q, 16, 512), dtype=torch.bfloat16, device="cuda")
    dev.run(plan, b, eager, ws)
    torch.cuda.synchronize()
    out = torch.full_like(eager, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dev.run(plan, b, out, ws, stream=s)  # warm the stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev.run(plan, b, out, ws, stream=torch.cuda.current_stream())
    for rep in range(4):
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda") * 2.0  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs from eager"
        del scratch
    ref, _ = oracle.decode_workload(w, threads=8)
    _compare(_bf16_out_to_f64(out), ref, "graph replay")


# ------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("q_len", [2, 4])
def test_multi_token_full_size(q_len):
    # bs 64, KV 8192 fp8 with q_len query rows per sequence, in the launch
    # configuration the planner picks; every sequence against the oracle
    w = synth.make_batch([8192] * 64, "bf16", "fp8", seed=30 + q_len, name=f"bs64_kv8192_fp8_q{q_len}",
                         q_lens=[q_len] * 64)
    _check_batch(w, poison=False, what=f"bs64 kv8192 fp8 q_len {q_len} (every sequence)")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity_at_full_size(name):
    # the five workloads in the planner's own launch configuration (the one the
    # benchmark times), every sequence against the oracle
    w = synth.make_workload(name)
    (_, _), _, out = _check_batch(w, poison=False, what=f"{name} (every sequence)")
    # and properties that hold for every output: finite, and each output column
    # a convex combination of the value rows (|out| <= max |V| + bf16 rounding)
    o = out.float()
    assert bool(torch.isfinite(o).all())
    if w.kv_dtype == "bf16":
        bound = float(np.abs(synth.bf16_to_f32(w.kv[:, :512])).max())
    elif w.kv_dtype == "fp8":
        bound = 448.0 * float(w.kv_scale)
    else:
        bound = 6.0 * 2.0 ** (int(w.kv_scale.max()) - 127)
    assert float(o.abs().max()) <= bound * 1.01


# ------------------------------------------------------------- staged start

@pytest.mark.parametrize("q_dtype,kv_dtype", [("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8"), ("fp8", "bf16"),
                                             ("bf16", "mxfp4"), ("fp8", "mxfp4")])
@pytest.mark.parametrize("rows", [32, 64, 96, 1024])
@pytest.mark.parametrize("page", [0, 1, 16])
def test_staged_start_equals_searched_start(q_dtype, kv_dtype, rows, page):
    """A plan made with the host offsets starts each stage-1 workgroup from a
    table of first pieces (tile 0, the query row and the rest of the ring
    prologue issued before any other load); a plan without them searches
    kv_indptr.  Same cut, same bits: sequences shorter than the ring, starting
    exactly at a range boundary, empty ones, and KV rows past the last sequence
    (workgroups with no piece at all).  Paged KV (page > 0 rows per page): the
    table gives the first piece, whose index and query loads then go out at
    once."""
    lengths = [1, 31, 32, 33, 64, 0, 200, 1000, 5, 96, 0, 2, 700]
    w = synth.make_batch(lengths, q_dtype, kv_dtype, seed=909 + rows, name="staged")
    if page <= 1:
        # CSR rows no sequence uses (with pages of several rows the CSR space
        # ends with the last sequence)
        extra = synth.make_batch([3 * rows + 17], "bf16", kv_dtype, seed=910, name="tail")
        w.kv = np.concatenate([w.kv, extra.kv])
        if kv_dtype == "mxfp4":
            w.kv_scale = np.concatenate([w.kv_scale, extra.kv_scale])  # and their E8M0 rows
    if page:
        w = synth.page_workload(w, seed=911 + rows, spare_rows=150, page_size=page)
    b = dev.upload(w)
    staged = dev.plan_for(b, rows_per_split=rows, use_host_indptr=True)
    searched = dev.plan_for(b, rows_per_split=rows, use_host_indptr=False)
    assert mla.mla_decode_plan_describe(staged)["first_piece_table"] == 1
    assert mla.mla_decode_plan_describe(searched)["first_piece_table"] == 0
    o1 = dev.run(staged, b)
    o2 = dev.run(searched, b)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ref, _ = oracle.decode_workload(w, threads=_host_threads())
    _compare(_bf16_out_to_f64(o1), ref, f"staged start {q_dtype}/{kv_dtype} rows {rows} page {page}")


@pytest.mark.parametrize("kv_dtype", ["fp8", "mxfp4"])
@pytest.mark.parametrize("groups", [768, 769])
def test_first_piece_table_at_its_limit(kv_dtype, groups):
    """768 stage-1 workgroups carry the first-piece table in the kernel
    arguments, 769 do not: both against the searched start bit for bit and
    against the oracle, with ragged sequences over 32-row ranges."""
    rng = np.random.default_rng(4242 + groups)
    total = groups * 32 - 5
    cuts = np.sort(rng.choice(np.arange(1, total), size=40, replace=False))
    lengths = np.diff(np.concatenate([[0], cuts, [total]])).tolist()
    w = synth.make_batch(lengths, "bf16", kv_dtype, seed=4243 + groups, name="table_limit")
    b = dev.upload(w)
    table = dev.plan_for(b, rows_per_split=32, use_host_indptr=True)
    searched = dev.plan_for(b, rows_per_split=32, use_host_indptr=False)
    d = mla.mla_decode_plan_describe(table)
    assert d["num_splits"] == groups
    assert d["first_piece_table"] == (1 if groups <= 768 else 0)
    o1 = dev.run(table, b)
    o2 = dev.run(searched, b)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ref, _ = oracle.decode_workload(w, threads=_host_threads())
    _compare(_bf16_out_to_f64(o1), ref, f"first-piece table, {groups} workgroups, {kv_dtype}")


def test_ring_read_runs_and_leaves_the_sink():
    """The memory-side reference (stage 1's ring with no arithmetic) streams a
    buffer in every share shape - more workgroups than tiles, uneven shares -
    and writes nothing but, with the practically impossible XOR, its sink."""
    nbytes = 18432 * 1000
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for wgs in (1, 3, 512, 2000):
        mla.mla_debug_stream_ring(buf, nbytes, wgs, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    assert bool((buf == 1).all())


# ------------------------------------------------------------- paired ranges

@pytest.mark.parametrize("skew", [120, 250])
@pytest.mark.parametrize("kv_dtype,q_len,paged", [("fp8", 1, False), ("bf16", 1, False), ("mxfp4", 1, False),
                                                  ("fp8", 2, False), ("fp8", 1, True), ("mxfp4", 2, True)])
def test_paired_ranges(kv_dtype, q_len, paged, skew):
    """Plans whose CUs each take a longer first and a shorter second range
    (planned here for 15 CUs, so 30 ranges over a ragged batch, pieces crossing
    pair boundaries) against the oracle, in every stage-1 variant family."""
    lengths = [700, 1000, 33, 1, 2500, 77, 300, 189]
    w = synth.make_batch(lengths, "bf16", kv_dtype, seed=1212 + skew, name="paired", q_lens=[q_len] * len(lengths))
    if paged:
        w = synth.page_workload(w, seed=1213, spare_rows=200)
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=150, num_cus=15, age_skew=skew)
    d = mla.mla_decode_plan_describe(plan)
    assert d["paired_splits"] == 15 and d["num_splits"] == 30
    out = dev.run(plan, b, workspace=dev.workspace_for(plan, fill=float("nan")))
    torch.cuda.synchronize()
    ref, _ = oracle.decode_workload(w, threads=_host_threads())
    _compare(_bf16_out_to_f64(out), ref, f"paired ranges kv={kv_dtype} q_len={q_len} paged={paged} skew={skew}")


@pytest.mark.parametrize("J", [1, 2, 4])
@pytest.mark.parametrize("kv_dtype,q_len,paged", [("fp8", 1, False), ("bf16", 1, False), ("mxfp4", 1, False),
                                                  ("fp8", 2, True)])
def test_xcd_grouped_pairs(kv_dtype, q_len, paged, J):
    """Paired ranges with J consecutive pairs placed on one XCD's CUs (planned
    for 32 CUs: 64 ranges of a ragged batch, pieces crossing pair boundaries)
    against the oracle; the grouping only moves ranges between workgroups, so
    the output is also bitwise that of the ungrouped plan."""
    lengths = [700, 1000, 33, 1, 2500, 77, 300, 189] * 2 + [640]
    w = synth.make_batch(lengths, "bf16", kv_dtype, seed=1414 + J, name="xcd-grouped", q_lens=[q_len] * len(lengths))
    if paged:
        w = synth.page_workload(w, seed=1415, spare_rows=200)
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=160, num_cus=32, xcd_group=J)
    d = mla.mla_decode_plan_describe(plan)
    assert d["paired_splits"] == 32 and d["num_splits"] == 64 and d["xcd_group"] == J
    out = dev.run(plan, b, workspace=dev.workspace_for(plan, fill=float("nan")))
    flat = dev.run(dev.plan_for(b, rows_per_split=160, num_cus=32, xcd_group=-1), b)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), flat.view(torch.int16))
    ref, _ = oracle.decode_workload(w, threads=_host_threads())
    _compare(_bf16_out_to_f64(out), ref, f"xcd-grouped pairs J={J} kv={kv_dtype} q_len={q_len} paged={paged}")
