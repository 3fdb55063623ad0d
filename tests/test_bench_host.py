"""Host-side checks of the benchmark (CPU only): the algorithmic FLOP count of a prefill call
against the values of the per-sequence accounting (2 x parameters per token for the
projections, the causal triangle of each recursion's active tokens for attention, the router
dot products), and the refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ec_counts(cfg):
    ks = oracle.capacity_counts(cfg.cap_num, cfg.cap_den, cfg.seq)
    return np.repeat(np.array(ks)[:, None], cfg.batch, axis=1)


@pytest.mark.parametrize("name,total,per_layer", [("smol360m_bf16", 8.220e12, 9_830_400),
                                                  ("smol135m_bf16", 3.231e12, 3_538_944)])
def test_prefill_flops_at_the_benchmark_shapes(name, total, per_layer):
    cfg = workload.get_config(name)
    assert bench.layer_params(cfg) == per_layer
    fl = bench.flop_counts(cfg, _ec_counts(cfg))
    assert abs(fl["total"] - total) / total < 5e-4
    # projections 2 x P per token on every layer a token runs, and the gate/up share of them
    ks = oracle.capacity_counts(cfg.cap_num, cfg.cap_den, cfg.seq)
    runs = cfg.batch * (2 * cfg.seq + cfg.n_shared * sum(ks))
    assert fl["linear"] == 2 * per_layer * runs
    assert fl["gate_up"] == 2 * cfg.d_model * 2 * cfg.d_ff * runs
    assert fl["gate_up_launches"] == 2 + cfg.n_rec * cfg.n_shared


def test_attention_flops_are_the_causal_triangles():
    """At full capacity every recursion sees all T tokens: attention is (L) causal triangles."""
    cfg = workload.get_config("smol360m_bf16", cap_num=(3, 3, 3))
    fl = bench.flop_counts(cfg, _ec_counts(cfg))
    T = cfg.seq
    pairs = T * (T + 1) // 2
    assert fl["attention"] == 4 * cfg.n_q_heads * cfg.head_dim * pairs * cfg.batch * cfg.n_layers


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in (r.stdout + r.stderr)


def test_memory_kernel_bytes_at_the_360m_shape():
    """Bytes of the memory-bound kernels of one 360M expert-choice call: the recursion-1 router
    reads all 16,384 rows of H (63 MB), the gathers copy and the scatters read twice and write
    once the 16,384 + 10,928 + 5,464 routed rows."""
    cfg = workload.get_config("smol360m_bf16")
    mb = bench.memory_kernel_bytes(cfg, _ec_counts(cfg))
    BT, d = cfg.batch * cfg.seq, cfg.d_model
    M = [16384, 10928, 5464]
    assert mb["router"] == (BT * d * 4 + BT * 4, 1)
    assert mb["gather"] == (8 * d * sum(M), 3)
    assert mb["scatter"] == (12 * d * sum(M), 3)
    assert mb["select"][1] == 3 and mb["select"][0] == 8 * (BT + M[0] + M[1]) + 4 * sum(M)
    rows = 2 * 2 * BT + 2 * cfg.n_shared * sum(M)
    assert mb["rmsnorm"] == (rows * d * 6, 2 * (2 + 3 * cfg.n_shared))
