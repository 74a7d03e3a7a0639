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
