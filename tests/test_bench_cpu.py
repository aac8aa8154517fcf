"""Host-side behaviour of bench.py that needs no GPU: one GPU only, and the stored counter record
is used only while it describes the kernel's current sources."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_source_hash_ignores_comments_only():
    b = _bench()
    code = b._CODE_TOKENS
    a = 'int x = 1; // note\n/* block\ncomment */ const char* s = "// kept";\n'
    c = 'int x = 1; // other note\n/* other */ const char* s = "// kept";\n'
    d = 'int x = 2; // note\n/* block\ncomment */ const char* s = "// kept";\n'

    def norm(src):
        return " ".join(code.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src).split())

    assert norm(a) == norm(c)
    assert norm(a) != norm(d)
    assert '"// kept"' in norm(a)


def test_stored_traffic_follows_the_sources(tmp_path, monkeypatch):
    b = _bench()
    rec = {"source_sha256": b.kernel_source_hash(), "hbm_bytes_per_launch": 123}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(b, "TRAFFIC_RECORD", str(path))
    assert b.stored_traffic() == 123
    rec["source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert b.stored_traffic() is None
    monkeypatch.setattr(b, "TRAFFIC_RECORD", str(tmp_path / "missing.json"))
    assert b.stored_traffic() is None
