"""Seeded input generator: determinism, encoders against torch's casts, and the
shapes of the five decode workloads (no GPU)."""
import numpy as np
import pytest
import torch

import synth


def test_streams_are_deterministic_and_distinct():
    a = synth.normal_bf16(7, 1, 5000, threads=1)
    b = synth.normal_bf16(7, 1, 5000, threads=4)
    c = synth.normal_bf16(7, 2, 5000)
    d = synth.normal_bf16(8, 1, 5000)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    # counter based: a suffix of the stream equals the stream's own elements
    assert np.array_equal(synth.normal_bf16(7, 1, 10), a[:10])


def test_normal_moments():
    x = synth.bf16_to_f32(synth.normal_bf16(3, 1, 400_000)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert abs(np.mean(x ** 4) - 3.0) < 0.05


def test_e4m3fn_encoder_matches_torch_round_to_nearest_even(rng):
    x = np.concatenate([
        rng.standard_normal(20000) * 50,
        rng.standard_normal(5000) * 1e-3,             # subnormal range
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 1.0625, 1.1875, 0.0029296875]),
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    got = synth.encode_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch(rng):
    x = (rng.standard_normal(10000) * 10).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)


def test_mxfp4_encoder_block_rule():
    x = np.zeros((1, 576), dtype=np.float32)
    x[0, :32] = np.linspace(-5, 7, 32)          # amax 7 -> exponent floor(log2 7) - 2 = 0
    x[0, 32:64] = 0.0                            # all-zero block -> scale byte 127
    x[0, 64:96] = 0.3                            # amax 0.3 -> floor(log2 .3) - 2 = -4
    packed, scales = synth.encode_mxfp4(x)
    assert scales[0, 0] == 127 and scales[0, 1] == 127 and scales[0, 2] == 127 - 4
    # 7 saturates to 6 (code 7); -5 ties between 4 and 6 -> even code (4 -> code 6), sign bit set
    assert packed[0, 15] >> 4 == 0x7
    assert packed[0, 0] & 0xF == 0x8 | 0x6
    # 0.3 / 2^-4 = 4.8 -> nearest E2M1 magnitude 4 (code 6)
    assert packed[0, 32] == 0x66


def test_uniform_lengths_range_and_reproducible():
    a = synth.uniform_lengths(5, 3, 20000, 1, 16384)
    assert a.min() >= 1 and a.max() <= 16384
    assert np.array_equal(a, synth.uniform_lengths(5, 3, 20000, 1, 16384))
    assert abs(a.mean() - 8192.5) < 100


@pytest.mark.parametrize("name", ["bs4_kv1024_bf16", "bs32_kv1024_fp8", "bs128_ragged_mxfp4"])
def test_workload_shapes(name):
    w = synth.make_workload(name)
    spec = synth.WORKLOADS[name]
    assert w.batch_size == spec["bs"] and w.total_q == spec["bs"]
    assert w.q.shape == (spec["bs"], 16, 576)
    if w.kv_dtype == "mxfp4":
        assert w.kv.shape == (w.total_kv, 288) and w.kv_scale.shape == (w.total_kv, 18)
    else:
        assert w.kv.shape == (w.total_kv, 576)
    if w.kv_dtype == "fp8":
        codes = w.kv.reshape(-1)
        # per-tensor scale = amax / 448: the extreme element maps to +-448
        assert np.any((codes & 0x7F) == 0x7E)
        assert not np.any((codes & 0x7F) == 0x7F)
    assert w.kv_indptr[-1] == w.total_kv
    if spec["kv_len"] != "ragged":
        assert np.all(np.diff(w.kv_indptr) == spec["kv_len"])


@pytest.mark.parametrize("page_size", [1, 4, 32])
def test_page_layout_is_a_valid_scatter(page_size):
    # every CSR row lands on its own buffer row, in whole pages listed per
    # sequence, and the rows no sequence uses hold other data
    w = synth.make_batch([70, 0, 33, 1, 128], "bf16", "mxfp4", seed=31)
    pw = synth.page_workload(w, seed=32, spare_rows=40, page_size=page_size)
    P = page_size
    assert pw.total_kv == w.total_kv and pw.kv_rows % P == 0
    lens = np.diff(w.kv_indptr.astype(np.int64))
    if P == 1:
        dest = pw.kv_indices.astype(np.int64)
        assert pw.kv_page_indptr is None
    else:
        kpp = pw.kv_page_indptr.astype(np.int64)
        assert np.array_equal(np.diff(kpp), (lens + P - 1) // P) and kpp[0] == 0
        assert len(set(pw.kv_indices.tolist())) == pw.kv_indices.size  # no page shared
        dest = np.concatenate([pw.kv_indices[kpp[b] + np.arange(n) // P].astype(np.int64) * P + np.arange(n) % P
                               for b, n in enumerate(lens)])
    assert dest.min() >= 0 and dest.max() < pw.kv_rows and np.unique(dest).size == dest.size
    assert np.array_equal(pw.kv[dest], w.kv) and np.array_equal(pw.kv_scale[dest], w.kv_scale)
    unused = np.setdiff1d(np.arange(pw.kv_rows), dest)
    assert unused.size >= 40 and np.any(pw.kv[unused] != 0)
