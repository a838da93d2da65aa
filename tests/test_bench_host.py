"""Host-side pieces of bench.py (no GPU): the code hash that keys the stored
counter ratios, and the ratio lookup."""

import json

import bench


def test_code_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;\n}\n")
    b.write_text("// a comment\nint f(int x) {   \n\n  return x + 1;  // trailing comment\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    hashes = []
    for p in (a, b, c):
        monkeypatch.setattr(bench, "KERNEL_SOURCE", str(p))
        hashes.append(bench.kernel_code_hash())
    assert hashes[0] == hashes[1]
    assert hashes[0] != hashes[2]


def test_stored_ratio_needs_the_same_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f();\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    counters = tmp_path / "traffic.json"
    counters.write_text(json.dumps({"workloads": {"w": {"kernel_code_sha256": bench.kernel_code_hash(),
                                                        "hbm_bytes_per_algorithmic_byte": 1.013}}}))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(counters))
    assert bench.stored_traffic_ratio("w") == 1.013
    assert bench.stored_traffic_ratio("other") is None
    src.write_text("int f();\nint g();\n")
    assert bench.stored_traffic_ratio("w") is None
