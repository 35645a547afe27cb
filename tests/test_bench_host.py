"""bench.py host logic (CPU): the one-GPU contract, the pair count and the algorithmic work
model that the roofline fractions are computed from."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import gen  # noqa: E402
from oracle import oracle as orc  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_pair_count_is_the_sum_of_candidate_counts():
    rng = np.random.default_rng(3)
    for kp in (1, 2, 4):
        docs = [int(x) for x in rng.integers(0, 300, 7)]
        cu = gen.cu_from_lengths(docs)
        T = int(cu[-1])
        _, pos = orc.geometry(cu, T)
        brute = sum(int(orc.candidate_count(int(p), kp)) for p in pos)
        assert bench.pair_count(cu, kp) == brute


def test_workload_pair_counts():
    # 2 x 4096 tokens: 2 * 4096 * 4097 / 2 causal pairs
    inp = {"cu_seqlens": gen.cu_from_lengths([4096, 4096])}
    assert bench.pair_count(inp["cu_seqlens"], 1) == 4096 * 4097
    # one document of 65536 tokens in pools of 4: sum over positions of floor((u+1)/4)
    u = np.arange(65536)
    assert bench.pair_count(gen.cu_from_lengths([65536]), 4) == int(np.sum((u + 1) // 4))


def test_algorithmic_work_model():
    T, H, D, topk = 8192, 64, 128, 512
    inp = {"q": np.zeros((T, H, D), np.uint16), "precision": "fp8", "kpool": 1, "topk": topk, "preprocess": True}
    pairs = 4096 * 4097
    alg = bench.algorithmic(inp, pairs, fused=False)
    assert alg["score_flops"] == 2.0 * H * D * pairs
    # scores read once, indices and scores written, lengths written
    assert alg["topk_bytes"] == pairs * 4 + T * topk * 4 * 2 + T * 4
    # keys: bf16 in, e4m3 out, one scale byte; queries the same per (t, h)
    assert alg["preprocess_bytes"] == T * D * 2 + T * D + T + T * H * D * 2 + T * H * D + T * H
    assert alg["softmax_bytes"] == 2 * T * topk * 4
