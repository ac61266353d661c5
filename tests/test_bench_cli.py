"""The benchmark's host-side contract, without a GPU: the algorithmic byte
counts it divides by the step time (checked against the per-configuration
table derived from the byte formula: logits, x read once, payload with pad
rows, scales, index and weight arrays, gathered rows, y), and its refusal of
runs on more than one GPU."""
import json
import os
import subprocess
import sys

import numpy as np

import oracle
from moe_synth import WORKLOADS, gen_logits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# name -> (dispatch bytes, combine bytes) for the five configurations
TABLE = {
    "tiny": (102_400, 99_328),
    "mixtral_decode": (3_153_920, 3_147_776),
    "dsv3_decode": (9_551_872, 16_523_264),
    "kimi_prefill": (535_298_048, 528_744_448),
    "dsv3_prefill": (1_344_762_368, 2_114_977_792),
}


def _rows(w):
    """Rows of the padded layout at the workload's seed, from the oracle's
    routing: sum over experts of the count rounded up to row_align."""
    idx, _ = oracle.route_topk(gen_logits(w.T, w.E, w.seed, w.zipf_s), w.k)
    c = np.bincount(idx.ravel(), minlength=w.E).astype(np.int64)
    return int(((c + w.row_align - 1) // w.row_align * w.row_align).sum())


def test_algorithmic_bytes_match_the_table():
    for name, want in TABLE.items():
        w = WORKLOADS[name]
        R = _rows(w)
        if w.row_align == 1:
            assert R == w.T * w.k
        got = bench.algorithmic_bytes(w.T, w.H, w.E, w.k, R, w.fp8)
        assert got == want, (name, R, got, want)
    assert _rows(WORKLOADS["dsv3_prefill"]) == 147_584


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                           env=dict(os.environ, **env), capture_output=True, text=True,
                           timeout=120)
        assert r.returncode == 2, r.stderr[-2000:]
        line = json.loads(r.stdout.strip().splitlines()[-1])
        assert "error" in line and "one GPU" in line["error"]
