"""Host logic of bench.py (no GPU): the algorithmic counts the roofline figures divide by, the
source hash that keys the recorded traffic, the traffic records, and the one-GPU rule."""
import os
import pathlib
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_chunk_flops_per_head_token():
    # 2C(3 d_k + 2 d_v) + 6 d_k d_v at C = 64: K K^T, Q K^T, T (beta K), T (beta V) and P Delta
    # over the chunk, W S, Q S and K^T Delta over the state
    assert bench.chunk_flops_per_head_token(128, 128) == 180_224
    assert bench.chunk_flops_per_head_token(64, 64) == 65_536


def test_training_step_drops_the_backward_recompute():
    fwd, bwd = bench.chunk_flops_per_head_token(128, 128), bench.bwd_flops_per_head_token(128, 128)
    recompute = 4 * 64 * 128 + 2 * 64 * 128 + 4 * 128 * 128
    assert bench.train_flops_per_head_token(128, 128) == fwd + bwd - recompute == 540_672


def test_prefill_and_decode_bytes():
    # q, k, v, o in bf16 plus eta and log alpha in fp32: 1 032 B per head-token at d = 128; the
    # mixed workload's prefill adds its 64 final states
    w = wl.WORKLOADS["mixed_b4h16"]
    assert bench.chunk_bytes(w, 2) == 64 * 32768 * 1032 + 64 * 128 * 128 * 4 == 2_168_455_168
    # a decode head-step reads and writes the fp32 state once: 132 104 B
    assert bench.decode_bytes(w, 2) == 64 * 132_104 == 8_454_656
    assert bench.decode_bytes(wl.WORKLOADS["decode_b64h16"], 2) == 135_274_496


def test_sources_hash_ignores_comments_and_spacing(tmp_path, monkeypatch):
    src = pathlib.Path(bench.CSRC)
    for f in bench.PART_SOURCES["decode"]:
        (tmp_path / f).write_text((src / f).read_text())
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    base = bench.sources_sha("decode")
    p = tmp_path / "decode.hip"
    p.write_text("// a new comment line\n" + p.read_text().replace("{", "{  /* note */\n", 1))
    assert bench.sources_sha("decode") == base
    p.write_text(p.read_text() + "\nstatic int extra_symbol;\n")  # a change of code
    assert bench.sources_sha("decode") != base


def test_traffic_records_match_on_workload_part_and_hash(tmp_path, monkeypatch):
    sha = bench.sources_sha("decode")
    rec = tmp_path / "hbm_traffic.txt"
    rec.write_text("header line\n"
                   f"traffic workload=w1 part=decode sources_sha={sha} fetch_bytes=100 write_bytes=23\n"
                   "traffic workload=w2 part=decode sources_sha=0000000000000000 fetch_bytes=1 write_bytes=1\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic("w1", "decode") == 123
    assert bench.recorded_traffic("w2", "decode") is None   # recorded on other code
    assert bench.recorded_traffic("w3", "decode") is None   # never recorded
    assert bench.traffic_key("chunk_bwd", "kda") == "chunk_bwd_kda" and bench.traffic_key("decode", "kla") == "decode"


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       env=env, cwd=str(ROOT), timeout=300)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
