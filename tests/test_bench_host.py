"""Host-side pieces of bench.py: the comment-blind hash that ties the
committed HBM-traffic counters to the decode sources they were taken on,
and the reading of the counter summary."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_strip_comments_keeps_code_and_literals():
    src = ('int a = 1; // note\n'
           '/* block\n   comment */ int b = 2;   \n'
           '\n'
           'const char* s = "x // y /* z */";\n'
           "char c = '/';  // slash\n")
    assert bench.strip_comments(src) == ('int a = 1;\n int b = 2;\n'
                                         'const char* s = "x // y /* z */";\n'
                                         "char c = '/';")


def _tree(tmp_path, text_by_file):
    for rel, text in text_by_file.items():
        path = tmp_path / rel
        path.parent.mkdir(parents=True, exist_ok=True)
        path.write_text(text)


def test_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    base = {rel: f"int f{i}() {{ return {i}; }}\n" for i, rel in enumerate(bench.DECODE_SOURCES)}
    _tree(tmp_path, base)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.decode_source_hash()
    first = bench.DECODE_SOURCES[0]
    _tree(tmp_path, {first: "// a new comment\n" + base[first] + "/* and another */\n"})
    assert bench.decode_source_hash() == h0
    _tree(tmp_path, {first: base[first].replace("return 0", "return 7")})
    assert bench.decode_source_hash() != h0


def test_traffic_record_is_read_for_its_sources(tmp_path, monkeypatch):
    _tree(tmp_path, {rel: "int x;\n" for rel in bench.DECODE_SOURCES})
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.decode_source_hash()
    rec = tmp_path / "traffic.md"
    rec.write_text('text\ntraffic-json: {"bytes_per_call": 5, "append_call_bytes": 6, '
                   f'"decode_source_hash": "{h}"}}\n')
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic()["append_call_bytes"] == 6
    rec.write_text('traffic-json: {"bytes_per_call": 5, "decode_source_hash": "0000"}\n')
    assert bench.measured_traffic() is None


def test_committed_traffic_record_parses():
    with open(bench.TRAFFIC_FILE) as f:
        lines = [line for line in f if line.startswith("traffic-json:")]
    assert len(lines) == 1
    import json
    rec = json.loads(lines[0].split(":", 1)[1])
    for key in ("bytes_per_call", "append_call_bytes", "main_kernel_bytes",
                "merge_kernel_bytes", "fetch_scale", "write_scale", "decode_source_hash"):
        assert key in rec
    assert rec["append_call_bytes"] >= rec["bytes_per_call"] > 0
