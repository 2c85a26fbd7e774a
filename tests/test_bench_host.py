"""Host logic of bench.py: the kernel-code hash that keys the committed
counter figures, and the lookup that drops them once the code changes."""
import json

import bench

SRC = """// header comment
#include <x.h>
/* block
   comment */
int f(int a) { return a + 1; }   // trailing comment

int g() { return 2; }
"""


def _sha_of(tmp_path, monkeypatch, text, name="k.hip"):
    p = tmp_path / name
    p.write_text(text, encoding="utf-8")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(p))
    return bench.source_sha256()


def test_comment_edits_keep_the_hash(tmp_path, monkeypatch):
    a = _sha_of(tmp_path, monkeypatch, SRC)
    edited = SRC.replace("header comment", "another header").replace("trailing comment", "x") + "\n\n// more\n"
    assert _sha_of(tmp_path, monkeypatch, edited, "k2.hip") == a


def test_code_edits_change_the_hash(tmp_path, monkeypatch):
    a = _sha_of(tmp_path, monkeypatch, SRC)
    assert _sha_of(tmp_path, monkeypatch, SRC.replace("a + 1", "a + 2"), "k2.hip") != a
    assert _sha_of(tmp_path, monkeypatch, SRC.replace("int g() { return 2; }", ""), "k3.hip") != a


def test_traffic_only_for_the_current_code(tmp_path, monkeypatch):
    sha = _sha_of(tmp_path, monkeypatch, SRC)
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps({"kern|wl": {"bytes_per_launch": 123, "source_sha256": sha},
                              "kern|old": {"bytes_per_launch": 456, "source_sha256": "0" * 64}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.traffic_for("kern", "wl") == 123
    assert bench.traffic_for("kern", "old") is None
    assert bench.traffic_for("kern", "missing") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.traffic_for("kern", "wl") is None

