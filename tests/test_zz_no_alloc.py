"""mla_decode_run_noalloc (workspace in the library's static device array)
against mla_decode_run (caller's workspace), through the C ABI, on MI355X:
two calls in a row, the second with a smaller batch, each bitwise equal to
mla_decode_run on the same inputs and within the parity bar of the oracle;
plans larger than the array are refused."""
import numpy as np
import pytest
import torch

import mla_decode_split_amd as mla
import oracle
import synth
from mla_decode_split_amd import device as dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _both(w, rows_per_split=0):
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=rows_per_split)
    ref = dev.run(plan, b)
    got = torch.full_like(ref, float("nan"))
    mla.mla_decode_run_noalloc(plan, b.q, b.q_scale, b.kv, b.kv_scale, b.qo_indptr, b.kv_indptr, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_run_on_two_calls_the_second_smaller():
    cases = [
        (synth.make_workload("bs64_kv8192_fp8"), 0),                                   # 16 MiB of slots
        (synth.make_batch([700, 33, 1000, 1, 257], "bf16", "mxfp4", seed=5, name="small"), 96),
    ]
    for w, rows in cases:
        _say(f"case {w.name}: bs={w.batch_size} total_kv={w.total_kv} rows_per_split={rows}")
        ref, got = _both(w, rows)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), w.name
        exp, _ = oracle.decode_workload(w, threads=8)
        g = got.float().cpu().numpy().astype(np.float64)
        max_abs = float(np.abs(g - exp).max())
        rel = float(np.linalg.norm(g - exp) / np.linalg.norm(exp))
        _say(f"{w.name}: bitwise equal to mla_decode_run; oracle max_abs={max_abs:.3e} rel_l2={rel:.3e}")
        assert max_abs <= 2e-2 and rel <= 1e-2


def test_noalloc_refuses_plans_larger_than_its_array():
    w = synth.make_batch([8192] * 64, "bf16", "fp8", seed=3, name="big-plan")
    b = dev.upload(w)
    plan = dev.plan_for(b, rows_per_split=32)  # 16384 workgroups: 512 MiB of slots
    assert plan.workspace_bytes > 34 << 20
    out = torch.empty((b.total_q, 16, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_run_noalloc(plan, b.q, b.q_scale, b.kv, b.kv_scale, b.qo_indptr, b.kv_indptr, out)
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED
