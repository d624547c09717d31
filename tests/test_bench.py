"""Host-side logic of bench.py (no GPU): the one-GPU guard, the code hash
that keys the committed counter record, the record lookup, and the flop
count the roofline figures are built on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                           env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def _write_sources(root, body_a, body_b):
    d = os.path.join(root, "joint_attention_non_amd", "csrc")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "a.hip"), "w") as f:
        f.write(body_a)
    with open(os.path.join(d, "b.h"), "w") as f:
        f.write(body_b)


def test_code_hash_ignores_comments_and_blank_space_only(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base_a = "int f(int x) {\n  return x + 1;  // one\n}\n"
    base_b = "#pragma once\n/* header */\nconstexpr int K = 4;\n"
    _write_sources(str(tmp_path), base_a, base_b)
    h0 = bench._source_sha("a.hip", "b.h")
    assert len(h0) == 16
    # comments reworded, blank space changed: same key
    _write_sources(str(tmp_path), "int f(int x) {\n\n    return x + 1;  // add one\n}\n",
                   "#pragma once\n/* the header,\n   reworded */\nconstexpr int K = 4;\n")
    assert bench._source_sha("a.hip", "b.h") == h0
    # any change to the code: a new key
    _write_sources(str(tmp_path), base_a.replace("x + 1", "x + 2"), base_b)
    assert bench._source_sha("a.hip", "b.h") != h0
    _write_sources(str(tmp_path), base_a, base_b.replace("K = 4", "K = 5"))
    assert bench._source_sha("a.hip", "b.h") != h0


def test_traffic_record_is_used_only_for_the_code_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench._traffic("attn_bf16_img2048", "0123456789abcdef") is None   # no record
    with open(tmp_path / "traffic.json", "w") as f:
        json.dump({"attn_bf16_img2048": {"source_sha": "0123456789abcdef", "bytes_per_launch": 12345}}, f)
    assert bench._traffic("attn_bf16_img2048", "0123456789abcdef") == 12345
    assert bench._traffic("attn_bf16_img2048", "fedcba9876543210") is None   # code changed since
    assert bench._traffic("another_kernel", "0123456789abcdef") is None
    with open(tmp_path / "traffic.json", "w") as f:
        f.write("{ not json")
    assert bench._traffic("attn_bf16_img2048", "0123456789abcdef") is None


def test_committed_traffic_record_is_well_formed():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)["attn_bf16_img2048"]
    assert len(rec["source_sha"]) == 16 and int(rec["source_sha"], 16) >= 0
    # fetch and write counts, each scaled by its calibration factor, give the
    # bytes per launch (the factors are stored to five decimals)
    want = (rec["fetch_kib_per_dispatch"] * rec["fetch_factor"] + rec["write_kib_per_dispatch"]
            * rec["write_factor"]) * 1024
    assert abs(rec["bytes_per_launch"] - want) <= 1e-5 * want


def test_dense_flop_count():
    # 4 N^2 D per (b, h): QK^T and PV, two flops per multiply-add
    assert bench._flops_dense(2, 24, 16896, 128) == 4.0 * 2 * 24 * 16896 ** 2 * 128
    assert bench._flops_dense(1, 1, 1, 128) == 512.0
