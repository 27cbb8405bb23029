"""Host logic of bench.py (no GPU): the algorithmic bytes per step that the
HBM fractions divide by, the README's adaptive ratio table as the bench
applies it, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

import bench
from workloads import synthetic as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# per step: 16 B of codes per key and unit; one 128 B record (64 B of 4-bit
# codes + 16 fp32 block weights) per candidate and query head; K and V rows
# of the Top-100 per query head (bf16: 256 B a row, fp32: 512 B)
EXPECTED = {
    #              codes        records      K+V rows
    "tiny4k": (65_536, 65_536, 102_400),
    "llama32k": (4_194_304, 8_388_608, 1_638_400),
    "batched128k": (134_217_728, 134_217_728, 13_107_200),
    "offload1m": (134_217_728, 33_554_432, 1_638_400),
    "drift128k": (16_777_216, 16_777_216, 1_638_400),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes_per_step(name):
    w = S.WORKLOADS[name]
    nb = bench.algorithmic_bytes(w, w.n)
    codes, records, rows = EXPECTED[name]
    assert nb["collide"] == codes
    assert nb["rerank"] == nb["rerank_topk"] == records
    assert nb["attend"] == rows
    # the drift stream also encodes one key per KV head each step: K row in,
    # codes + record + norm out
    assert nb["encode"] == ((256 + 16 + 128 + 4) * w.units if w.append_steps else 0)


def test_byte_counts_follow_the_sizes():
    """The counts scale with keys, units and candidates as their definitions say."""
    w = S.custom("batched128k", n=1000, n_candidates=4096)
    nb = bench.algorithmic_bytes(w, 1000)
    assert nb["collide"] == 16 * 1000 * w.units
    assert nb["rerank"] == 128 * 1000 * w.batch * w.n_q_heads      # n < C: every key is a candidate
    w2 = S.custom("batched128k", n=50, n_candidates=4096)
    assert bench.algorithmic_bytes(w2, 50)["attend"] == 2 * 256 * 50 * w2.batch * w2.n_q_heads   # k > n


def test_adaptive_ratios_follow_the_readme_table():
    table = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_constants.json")))["adaptive_ratios"]["rows"]
    for n in (1, 4999, 5000, 9999, 10000, 29999, 30000, 131072, 1 << 20):
        row = next(r for r in table if r["zone_len_below"] is None or n < r["zone_len_below"])
        beta, rho = bench.zone_ratios_permille(n)
        assert beta == round(1000 * row["candidate_ratio"]) and rho == round(1000 * row["collision_ratio"])
    w = S.WORKLOADS["batched128k_pct"]
    assert bench.candidates_per_call(w, 131072) == 13108          # ceil(0.1 * 131072)
    assert bench.candidates_per_call(S.WORKLOADS["batched128k"], 131072) == 4096


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_secondary_counts_per_step():
    # batched 128K: 16 code-byte lookups per key over 64 units (134 M), and
    # 128 multiply-adds per candidate record over 256 query heads (134 M)
    w = S.WORKLOADS["batched128k"]
    sec = bench.secondary_counts(w, w.n)
    assert sec == {"collision_lut_lookups": 134_217_728, "rerank_macs": 134_217_728}
    # fewer keys than candidates: every key is a candidate
    t = bench.secondary_counts(w, 1000)
    assert t["rerank_macs"] == 128 * 1000 * w.batch * w.n_q_heads
