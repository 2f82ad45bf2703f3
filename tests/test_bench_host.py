"""Host logic of bench.py (no GPU): the single-GPU contract, the algorithmic
byte and flop counts the roofline uses, and the committed counter traffic."""
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads

W = workloads.WORKLOADS
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["matrix_game", "lingbot480p", "lingbot720p", "minute"])
def test_append_bytes_per_token_head(name):
    """Inputs read once (2 d bf16 values) plus the written fields: centre
    indices, 2 d/16 code words, the tile parameters spread over the frame's
    tokens, r INT8 coefficients and their fp16 scale."""
    w = W[name]
    d, F, T = w.head_dim, w.frame_tokens, w.group_tokens
    tiles = -(-F // T)
    idx = (1 if w.c_k <= 256 else 2) + (1 if w.c_v <= 256 else 2)
    by_hand = 2 * d * 2 + idx + 2 * (d // 16) * 4 + 2 * (d // 16) * 4 * tiles / F + w.rank + 2
    assert bench.append_bytes_per_token_head(w, None) == pytest.approx(by_hand, rel=1e-12)
    if name == "lingbot480p":
        # 512 B of inputs, 2 B of indices, 64 B of codes, 98 tiles of 64 B over 1,560 tokens, 10 B of PSAC
        assert bench.append_bytes_per_token_head(w, None) == pytest.approx(512 + 2 + 64 + 98 * 64 / 1560 + 10)


@pytest.mark.parametrize("name,blocks", [("matrix_game", 4), ("lingbot480p", 7), ("lingbot720p", 15), ("minute", 7)])
def test_query_blocks(name, blocks):
    assert bench.query_blocks(W[name]) == blocks


def test_attention_flops_count_the_two_products():
    w = W["minute"]
    # Q K^T and P V, 2 flops per multiply-add, PSAC columns not counted
    assert bench.attn_flops(w, w.n_q, w.n_tokens) == 4 * w.heads * w.n_q * w.n_tokens * w.head_dim
    assert bench.attn_flops(w, w.n_q, w.n_tokens) == pytest.approx(11.96163072e12)


def test_committed_traffic_is_tied_to_the_source_hash(tmp_path):
    h = bench.kernel_source_hash()
    for kind in ("attention", "append"):
        for name in ("matrix_game", "lingbot480p", "lingbot720p", "minute"):
            p = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kind, name))
            d = json.load(open(p))
            got = bench.traffic_from_profiles(kind, name, h)
            if d["kernel_source_hash"] == h:
                assert got == d["hbm_bytes_per_launch"] and got > 0
            else:
                assert got is None
    assert bench.traffic_from_profiles("attention", "minute", "0" * 16) is None
    assert bench.traffic_from_profiles("attention", "no_such_workload", h) is None
