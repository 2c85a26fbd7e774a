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



def test_cpu_threads_follow_affinity_and_share(monkeypatch):
    import os
    n_aff = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    assert bench.cpu_threads() == (n_aff, n_aff)
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.cpu_threads() == (1, n_aff)
    monkeypatch.setenv("OMP_NUM_THREADS", str(n_aff + 100))
    assert bench.cpu_threads() == (n_aff, n_aff)


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_cpu_baseline_reports_single_and_multi_thread(monkeypatch):
    """A tiny workload so the timing loop ends at once: both figures and the
    fields the benchmark line carries are there."""
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    cfg = dict(family="c3", B=4, K=2, V=300)
    r = bench.cpu_baseline(cfg, "sampled", target_seconds=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "rounds/s" and r["value"] > 0
    assert r["cpu_model"] and r["affinity_cpus"] >= 1
    if r["cores"] > 1:
        assert r["single_thread"]["value"] > 0
    g = bench.cpu_baseline(dict(family="c2", B=4, K=2, V=300), "greedy", target_seconds=0.05)
    assert g["value"] > 0
