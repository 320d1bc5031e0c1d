"""Host logic of bench.py, no GPU: whether a committed counter record still
applies to the kernel source it was taken on."""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def fake_tree(tmp_path):
    csrc = tmp_path / "linear_attention_rnn_wkv_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text('#include "a.h"\nint k;\n')
    (csrc / "a.h").write_text('#include "b.h"\nint a;\n')
    (csrc / "b.h").write_text("int b = 1;\n")
    (csrc / "other.h").write_text("int o;\n")
    return csrc


def test_source_hash_covers_included_headers(tmp_path, monkeypatch):
    b = load_bench()
    csrc = fake_tree(tmp_path)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    h0 = b.source_hash("k.hip")
    assert h0 == b.source_hash("k.hip") and len(h0) == 16
    (csrc / "other.h").write_text("int o = 2;\n")  # not included
    assert b.source_hash("k.hip") == h0
    (csrc / "b.h").write_text("int b = 2;\n")  # included through a.h
    h1 = b.source_hash("k.hip")
    assert h1 != h0
    (csrc / "k.hip").write_text('#include "a.h"\nint k = 3;\n')
    assert b.source_hash("k.hip") not in (h0, h1)


def test_measured_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    b = load_bench()
    csrc = fake_tree(tmp_path)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    rec = {"path": {"source_sha256_16": b.source_hash("k.hip"), "bytes_per_launch": 123.0}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert b.measured_traffic("k.hip", "path") == 123.0
    assert b.measured_traffic("k.hip", "no such path") is None
    (csrc / "a.h").write_text('#include "b.h"\nint a = 1;\n')
    assert b.measured_traffic("k.hip", "path") is None


def test_committed_records_match_the_committed_sources():
    # every record of profiles/traffic.json was taken on the sources in the
    # tree (a kernel or header change without new counters fails here)
    b = load_bench()
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    stale = [k for k, r in recs.items()
             if "source" in r and r["source_sha256_16"] != b.source_hash(r["source"])]
    assert not stale, stale
