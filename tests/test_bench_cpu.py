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


def test_record_carries_the_contract_keys():
    import argparse
    import moe_synth as S
    b = _bench()
    cfg = S.CONFIGS["decode35b"]
    rec = b.base_record(argparse.Namespace(warmup=60), cfg, 2750.0, 600 / 2750.0, 600)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config"):
        assert k in rec
    assert rec["n_gpus"] == 1 and rec["higher_is_better"] is True and rec["vs_baseline"] is None
    assert rec["config"]["workload"].startswith("decode35b")
    assert abs(rec["ms_per_step"] - 1e3 / 2750.0) < 1e-3


def test_roofline_and_algorithmic_bytes():
    import moe_synth as S
    b = _bench()
    total, expert_only = b.algorithmic_bytes(S.CONFIGS["decode35b"])
    # 40 layers of 4 experts, 39 heads, the layer-0 router and the float16 in/out vectors of every layer
    assert total == 40 * 4 * 1_769_472 + 39 * 5_790_720 + 256 * 2048 * 2 + 40 * 2 * 2048 * 2 == 510_329_856
    assert expert_only == 40 * (4 * 1_769_472 + 2 * 2048 * 2)
    r = b.roofline("k", total, 362.0, None)
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["achieved"] - total / 362e-6 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
