"""The oracle's pins must catch plausible mistakes.

Each case below copies the oracle's C source, plants one mistake (a dropped
term, a wrong sign, index, bias or operand order), compiles the copy with gcc
into a temporary directory and runs a battery of pin checks against it.  The
unmodified oracle must pass every check; every mutant must fail at least one.
Nothing here touches the GPU or the oracle under ``oracle/``.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

H, D, V = 16, 576, 512
SM = 1.0 / 24.0

MUTANTS = {
    "rope_dims_dropped": ("for (int d = 0; d < D; ++d) dot += qrow[d] * kvrows[j * D + d];",
                          "for (int d = 0; d < V; ++d) dot += qrow[d] * kvrows[j * D + d];"),
    "value_columns_offset": ("out[v] += scores[j] * kvrows[j * D + v];",
                             "out[v] += scores[j] * kvrows[j * D + v + (D - V)];"),
    "softmax_sign": ("const double w = exp(scores[j] - m);", "const double w = exp(m - scores[j]);"),
    "sm_scale_dropped": ("scores[j] = p->sm_scale * dot;", "scores[j] = dot;"),
    "e4m3_bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal": ("mag = ldexp((double)m / 8.0, 1 - 7);", "mag = ldexp((double)m / 8.0, 0 - 7);"),
    "nibble_order": ("(c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF)",
                     "(c & 1) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4)"),
    "e2m1_bias": ("ldexp(1.0 + (double)m / 2.0, e - 1)", "ldexp(1.0 + (double)m / 2.0, e)"),
    "mx_block_index": ("scales[r * (dim / 32) + c / 32]", "scales[r * (dim / 32) + c / 64]"),
    "lse_drops_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "fp8_kv_scale_dropped": ("for (int d = 0; d < D; ++d) dst[d] = oracle_e4m3fn_value(row[d]) * s;",
                             "for (int d = 0; d < D; ++d) dst[d] = oracle_e4m3fn_value(row[d]);"),
    "q_head_stride": ("const int64_t base = (t * p->num_heads + h) * (int64_t)D;",
                      "const int64_t base = (t * p->num_heads) * (int64_t)D + h;"),
    "normalisation_dropped": ("for (int v = 0; v < V; ++v) out[v] /= l;", ""),
    "paged_index_ignored": ("else if (sh->kv_indices)\n        row = sh->kv_indices[j0 + j];", ""),
    "page_offset_dropped": ("* sh->page_size + j % sh->page_size;", "* sh->page_size;"),
    "page_list_start_ignored": ("sh->kv_indices[sh->kv_page_indptr[b] + j / sh->page_size]",
                                "sh->kv_indices[j / sh->page_size]"),
    "soft_cap_outer_factor_dropped": ("scores[j] = p->logit_cap * tanh(scores[j] / p->logit_cap);",
                                      "scores[j] = tanh(scores[j] / p->logit_cap);"),
    "soft_cap_before_sm_scale": ("scores[j] = p->sm_scale * dot;\n    if (p->logit_cap > 0.0) scores[j] = p->logit_cap * tanh(scores[j] / p->logit_cap);",
                                 "scores[j] = dot;\n    if (p->logit_cap > 0.0) scores[j] = p->logit_cap * tanh(scores[j] / p->logit_cap);\n    scores[j] *= p->sm_scale;"),
}


def _bf16(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


def _f(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def _torch_ref(qd, kd, qo, kvp):
    out = np.empty((qd.shape[0], H, V))
    for b in range(len(kvp) - 1):
        k = torch.from_numpy(kd[kvp[b]:kvp[b + 1]])
        for t in range(qo[b], qo[b + 1]):
            s = (torch.from_numpy(qd[t]) * SM) @ k.T
            out[t] = (torch.softmax(s, dim=-1) @ k[:, :V]).numpy()
    return out


def pin_battery(lib):
    """Returns the names of the checks that fail for this oracle build."""
    failed = []
    rng = np.random.default_rng(99)

    # decoder tables against torch casts and the OCP definitions
    ref8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ok = all((math.isnan(lib.oracle_e4m3fn_value(c)) and math.isnan(ref8[c])) or lib.oracle_e4m3fn_value(c) == ref8[c]
             for c in range(256))
    if not ok:
        failed.append("e4m3fn_table")
    e2m1 = [0, .5, 1, 1.5, 2, 3, 4, 6]
    if any(lib.oracle_e2m1_value(n) != (-1 if n & 8 else 1) * e2m1[n & 7] for n in range(16)):
        failed.append("e2m1_table")
    packed = np.zeros((1, 288), dtype=np.uint8)
    scales = np.full((1, 18), 127, dtype=np.uint8)
    packed[0, 0], packed[0, 16], scales[0, 1] = 0x21, 0x73, 130
    out = np.empty((1, 576))
    lib.oracle_decode_mxfp4(packed.ctypes.data, scales.ctypes.data, 1, 576, out.ctypes.data)
    if not (out[0, 0] == 0.5 and out[0, 1] == 1.0 and out[0, 32] == 12.0 and out[0, 33] == 48.0):
        failed.append("mxfp4_spot")

    # single row, bf16
    q = _bf16(rng.standard_normal((2, H, D)))
    kv = _bf16(rng.standard_normal((2, D)))
    o, l = oracle.mla_decode(q, kv, [0, 1, 2], [0, 1, 2], lib=lib)
    if not np.array_equal(o[0, 0], _f(kv[0])[:V]):
        failed.append("single_row")
    s = SM * (_f(q)[0] @ _f(kv)[0])
    if not np.allclose(l[0], s, rtol=1e-12):
        failed.append("single_row_lse")

    # independent torch fp64 formulation, bf16 and fp8 (non power-of-two scales)
    lengths = [3, 40, 1]
    kvp = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    qo = np.arange(4, dtype=np.int32)
    qb = _bf16(rng.standard_normal((3, H, D)))
    kb = _bf16(rng.standard_normal((kvp[-1], D)))
    o, _ = oracle.mla_decode(qb, kb, qo, kvp, lib=lib)
    if not np.allclose(o, _torch_ref(_f(qb), _f(kb), qo, kvp), rtol=1e-10, atol=1e-12):
        failed.append("torch_bf16")
    qc = synth.encode_e4m3fn(rng.standard_normal((3, H, D)) * 50)
    kc = synth.encode_e4m3fn(rng.standard_normal((kvp[-1], D)) * 50)
    qs, ks = np.float32(0.031), np.float32(0.027)
    o, _ = oracle.mla_decode(qc, kc, qo, kvp, q_dtype="fp8", kv_dtype="fp8", q_scale=qs, kv_scale=ks, lib=lib)
    t8 = lambda c, sc: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(sc)
    if not np.allclose(o, _torch_ref(t8(qc, qs), t8(kc, ks), qo, kvp), rtol=1e-10, atol=1e-12):
        failed.append("torch_a8w8")

    # mxfp4 folding identity against the decoded values fed as bf16
    pk, sc = synth.encode_mxfp4(rng.standard_normal((20, D)) * 2)
    qq = _bf16(rng.standard_normal((1, H, D)) * 0.2)
    o4, _ = oracle.mla_decode(qq, pk, [0, 1], [0, 20], kv_dtype="mxfp4", kv_scale=sc, lib=lib)
    dec = np.empty((20, D))
    lib.oracle_decode_mxfp4(pk.ctypes.data, sc.ctypes.data, 20, D, dec.ctypes.data)
    # decoded values are checked against an independent decode written from the table
    nib = np.stack([pk & 0xF, pk >> 4], axis=-1).reshape(20, D)
    mag = np.array(e2m1)[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    indep = mag * np.ldexp(1.0, np.repeat(sc.astype(np.int64) - 127, 32, axis=1))
    ob, _ = oracle.mla_decode(qq, _bf16(indep), [0, 1], [0, 20], lib=lib)
    if not (np.array_equal(dec, indep) and np.array_equal(o4, ob)):
        failed.append("mxfp4_folding")

    # soft-cap: two KV rows in closed form (sigmoid of the capped score difference)
    cap = 0.6
    q2 = _bf16(rng.standard_normal((1, H, D)))
    k2 = _bf16(rng.standard_normal((2, D)))
    o, _ = oracle.mla_decode(q2, k2, [0, 1], [0, 2], lib=lib, logit_cap=cap)
    sc2 = SM * (_f(q2)[0] @ _f(k2).T)  # [H, 2]
    c = cap * np.tanh(sc2 / cap)
    w1 = 1.0 / (1.0 + np.exp(c[:, 1] - c[:, 0]))
    want = w1[:, None] * _f(k2)[0, :V] + (1.0 - w1)[:, None] * _f(k2)[1, :V]
    if not np.allclose(o[0], want, rtol=1e-11, atol=1e-13):
        failed.append("soft_cap_two_rows")

    # paged KV: rows scattered through a permutation read back in CSR order
    perm = rng.permutation(int(kvp[-1])).astype(np.int32)
    scattered = np.empty_like(kb)
    scattered[perm] = kb
    o, _ = oracle.mla_decode(qb, scattered, qo, kvp, lib=lib, kv_indices=perm)
    o2, _ = oracle.mla_decode(qb, kb, qo, kvp, lib=lib)
    if not np.array_equal(o, o2):
        failed.append("paged_permutation")

    # pages of 4 rows: each sequence's rows laid page by page into pages drawn
    # from a permutation, read back in CSR order
    P = 4
    lens = np.diff(np.asarray(kvp, dtype=np.int64))
    starts = np.concatenate([[0], np.cumsum((lens + P - 1) // P)]).astype(np.int32)
    npages = int(starts[-1]) + 3
    page_ids = rng.permutation(npages)[: int(starts[-1])].astype(np.int32)
    paged = np.zeros((npages * P,) + kb.shape[1:], dtype=kb.dtype)
    for b in range(lens.shape[0]):
        for i in range(int(lens[b])):
            paged[int(page_ids[starts[b] + i // P]) * P + i % P] = kb[int(kvp[b]) + i]
    o, _ = oracle.mla_decode(qb, paged, qo, kvp, lib=lib, kv_indices=page_ids, kv_page_indptr=starts, page_size=P)
    if not np.array_equal(o, o2):
        failed.append("pages_of_four")

    # split recombination of LSE-weighted pieces
    qr = np.repeat(qb[1:2], 3, axis=0)
    op, lp = oracle.mla_decode(qr, kb, [0, 1, 2, 3], [3, 10, 30, 43], lib=lib)
    full, _ = oracle.mla_decode(qb[1:2], kb, [0, 1], [3, 43], lib=lib)
    m = lp.max(axis=0)
    w = np.exp(lp - m)
    comb = (w[:, :, None] * op).sum(axis=0) / w.sum(axis=0)[:, None]
    if not np.allclose(comb, full[0], rtol=1e-11, atol=1e-13):
        failed.append("split_recombination")
    return failed


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_unmodified_oracle_passes_battery():
    assert pin_battery(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, mutant_dir):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path_c = os.path.join(mutant_dir, f"{name}.c")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    path_so = os.path.join(mutant_dir, f"lib{name}.so")
    oracle.build(force=True, src=path_c, out=path_so)
    failed = pin_battery(oracle.load(path_so))
    assert failed, f"mutant {name} passed every pin"
