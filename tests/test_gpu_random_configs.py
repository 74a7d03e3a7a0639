"""Seeded random decode configurations on the GPU (MI355X only).

Each case draws everything together: batch size, ragged KV lengths with empty
sequences, a (q, KV) format pair, query rows per sequence (up to four, some
sequences with none), a logit soft-cap, paged KV with pages of 1, 16 or 64
rows, and the planner's inputs (host offsets or not, forced range sizes, the
CU count, paired ranges with an age skew and XCD grouping).  The output is
compared element by element with the fp64 oracle, and the workspace starts
poisoned with NaN.  The draws are a fixed list of seeds, so every case is
reproducible and printed before it runs.

A second, wider draw mixes in the shapes the first one rarely reaches: several
hundred short sequences (more than the merge kernel's argument table holds),
and one long sequence among short ones (a sequence split over many ranges next
to sequences that share one).  MLA_RANDOM_SEEDS=a:b and MLA_RANDOM_WIDE_SEEDS=a:b
replace the seed ranges for a longer sweep."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from mla_decode_split_amd import device as dev
import mla_decode_split_amd as mla

from test_gpu_parity import COMBOS, _bf16_out_to_f64, _compare, _host_threads, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _draw(seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5EED]))
    bs = int(rng.integers(1, 41))
    mix = int(rng.integers(0, 3))
    if mix == 0:
        lengths = rng.integers(0, 300, bs)
    elif mix == 1:
        lengths = rng.integers(0, 4000, bs)
    else:
        lengths = np.where(rng.random(bs) < 0.3, 0, rng.integers(1, 9000, bs))
    if lengths.sum() == 0:
        lengths[0] = 1
    q_dtype, kv_dtype = COMBOS[int(rng.integers(len(COMBOS)))]
    max_q = int(rng.choice([1, 1, 2, 3, 4]))
    q_lens = None if max_q == 1 else rng.integers(0, max_q + 1, bs)
    if q_lens is not None:
        # some sequence takes max_q rows (a plan for one row per sequence needs
        # exactly one in each)
        q_lens[int(rng.integers(bs))] = max_q
    cap = float(rng.choice([0.0, 0.0, 1.0, 30.0]))
    page = int(rng.choice([0, 0, 1, 16, 64]))
    host = bool(rng.random() < 0.8)
    total = int(lengths.sum())
    rows = int(rng.choice([0, 0, 32, 64, 160, 512, 2048]))
    opts = dict(rows_per_split=rows, use_host_indptr=host)
    if rows and rng.random() < 0.5:
        # paired ranges: as many CUs as make two workgroups each
        g = -(-total // ((rows + 31) // 32 * 32))
        if g % 2 == 0 and g >= 2:
            cus = g // 2
            opts.update(num_cus=cus, age_skew=int(rng.choice([0, 60, 150, 300])))
            groups = [j for j in (1, 2, 4) if cus % (8 * j) == 0]
            if groups and rng.random() < 0.5:
                opts["xcd_group"] = int(rng.choice(groups))
    return dict(lengths=lengths, q_dtype=q_dtype, kv_dtype=kv_dtype, q_lens=q_lens, cap=cap, page=page, opts=opts)


def _draw_wide(seed):
    c = _draw(seed)
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xA11]))
    kind = int(rng.integers(0, 2))
    if kind == 0:
        # many short sequences, a fifth of them empty
        bs = int(rng.integers(500, 900))
        c["lengths"] = np.where(rng.random(bs) < 0.2, 0, rng.integers(1, 200, bs))
        rows = int(rng.choice([0, 32, 64]))
    else:
        # one long sequence among short ones
        bs = int(rng.integers(2, 20))
        c["lengths"] = rng.integers(0, 50, bs)
        c["lengths"][int(rng.integers(bs))] = int(rng.integers(20000, 60000))
        rows = int(rng.choice([0, 0, 96, 1024]))
    if c["q_lens"] is not None:
        mq = int(c["q_lens"].max())
        c["q_lens"] = rng.integers(0, mq + 1, bs)
        c["q_lens"][0] = mq
    c["opts"] = dict(rows_per_split=rows, use_host_indptr=bool(rng.random() < 0.75))
    return c


def _seeds(var, default):
    v = os.environ.get(var)
    if not v:
        return default
    a, b = (int(x) for x in v.split(":"))
    return range(a, b)


def _run_case(c, seed, label):
    what = (f"{label} #{seed}: bs={len(c['lengths'])} rows={int(c['lengths'].sum())} {c['q_dtype']}/{c['kv_dtype']} "
            f"q_lens={'1' if c['q_lens'] is None else 'up to ' + str(int(c['q_lens'].max()))} cap={c['cap']} "
            f"page={c['page']} plan={c['opts']}")
    _say(what)
    w = synth.make_batch(c["lengths"], c["q_dtype"], c["kv_dtype"], seed=3000 + seed, name=f"{label}-{seed}",
                         q_lens=c["q_lens"])
    w.logit_cap = c["cap"]
    if c["page"]:
        w = synth.page_workload(w, seed=4000 + seed, spare_rows=100, page_size=c["page"])
    b = dev.upload(w)
    plan = dev.plan_for(b, **c["opts"])
    out = torch.full((b.total_q, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    dev.run(plan, b, out, dev.workspace_for(plan, fill=float("nan")))
    torch.cuda.synchronize()
    ref, _ = oracle.decode_workload(w, threads=_host_threads())
    got = _bf16_out_to_f64(out)
    # rows of sequences with no query rows are not written; every other row is compared
    _compare(got, ref, what)
    d = mla.mla_decode_plan_describe(plan)
    _say(f"   plan: {d['num_splits']} ranges of {d['rows_per_split']} rows, paired {d['paired_splits']}, "
         f"xcd group {d['xcd_group']}, stage 2 {d['stage2']}, merge batch {d['merge_batch']}")


@pytest.mark.parametrize("seed", _seeds("MLA_RANDOM_SEEDS", range(200)))
def test_random_config(seed):
    _run_case(_draw(seed), seed, "random")


@pytest.mark.parametrize("seed", _seeds("MLA_RANDOM_WIDE_SEEDS", range(1000, 1040)))
def test_random_config_wide(seed):
    _run_case(_draw_wide(seed), seed, "wide")
