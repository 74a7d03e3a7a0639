"""Host-side parts of bench.py (no GPU): the one-GPU contract and the check
that ties the recorded HBM traffic to the kernel code it was measured on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _hash_of(text, tmp_path):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.code_sha256(str(p))


def test_code_hash_ignores_comments_and_layout(tmp_path):
    base = 'int f(int x) {  // doubles\n  return 2 * x;  /* two */\n}\nconst char* s = "a // b";\n'
    same = '// a new note\nint f(int x) {\n\n  return 2 * x;\n}\n/* block */ const char* s = "a // b";\n'
    code = 'int f(int x) {  // doubles\n  return 3 * x;\n}\nconst char* s = "a // b";\n'
    literal = 'int f(int x) {  // doubles\n  return 2 * x;\n}\nconst char* s = "a /* b";\n'
    h = _hash_of(base, tmp_path)
    assert _hash_of(same, tmp_path) == h
    assert _hash_of(code, tmp_path) != h
    assert _hash_of(literal, tmp_path) != h  # text inside a string literal is code


def test_recorded_traffic_only_for_the_code_it_was_measured_on(monkeypatch):
    t = dict(bench.TRAFFIC_MEASURED)
    monkeypatch.setattr(bench, "TRAFFIC_MEASURED", dict(t, code_sha256=bench.code_sha256()))
    v = bench._measured_traffic(bench.DEFAULT_WORKLOAD)
    assert v == int(round(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])))
    assert v > 301989888  # more than the KV bytes alone
    assert bench._measured_traffic("bs4_kv1024_bf16") is None  # another workload
    monkeypatch.setattr(bench, "TRAFFIC_MEASURED", dict(t, code_sha256="0" * 64))
    assert bench._measured_traffic(bench.DEFAULT_WORKLOAD) is None  # other code


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_matrix_work_counts_every_kv_row_for_every_query_row():
    class W:
        kv_indptr = [0, 3, 3, 8]   # lengths 3, 0, 5
        qo_indptr = [0, 2, 3, 4]   # query rows 2, 1, 1
    # (3 * 2 + 0 * 1 + 5 * 1) pairs, each QK^T over 576 dims and PV over 512
    # columns for 16 heads at 2 flop per multiply-add
    assert bench.mfma_flop(W) == 11 * 2 * 16 * (576 + 512)
    b = bench.mfma_block(bench.mfma_flop(W), 1.0)
    assert b["unit"] == "TFLOP/s" and b["peak"] == 2500.0
    assert abs(b["frac"] - round(11 * 34816 / 1e-6 / 1e12 / 2500.0, 4)) < 1e-12
