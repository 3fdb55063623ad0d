"""Helpers of the GPU parity tests: run the HIP library, compare it with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workload


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over token rows of max_i |got - ref| / max_i |ref| (rows of the last axis)."""
    d = ref.shape[-1]
    g = np.asarray(got, np.float64).reshape(-1, d)
    r = np.asarray(ref, np.float64).reshape(-1, d)
    if g.shape[0] == 0:
        return 0.0
    return float(np.max(np.max(np.abs(g - r), axis=1) / np.max(np.abs(r), axis=1)))


def tolerance(cfg) -> float:
    return 1e-4 if cfg.dtype == "f32" else 2e-2


def build_gpu(cfg, weights=None, **kw):
    import adaptive_depth_recursive_amd as mor
    W = workload.make_weights(cfg) if weights is None else weights
    say(f"[gpu] init {cfg.name} dtype={cfg.dtype} B={cfg.batch} T={cfg.seq} d={cfg.d_model} "
        f"L={cfg.n_layers} R={cfg.n_rec} routing={cfg.routing} kv={cfg.kv_mode}")
    return mor.Mor(cfg, W, **kw), W


def run_prefill(model, H0: np.ndarray, debug=True):
    import torch
    h = torch.from_numpy(np.ascontiguousarray(H0, np.float32)).cuda()
    say(f"[gpu] mor_prefill B={H0.shape[0]} T={H0.shape[1]}")
    out = model.prefill_outputs(h, debug=debug)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def gpu_sets(res, cfg, b: int):
    """Active sets of sequence b as a list over r of position arrays."""
    return [res["sel_pos"][r, b, :res["counts"][r, b]] for r in range(cfg.n_rec)]


def check_routing_stagewise(cfg, W, res, H0):
    """Bit-exact routing check: the oracle, given the GPU's own H^r and active set A_{r-1},
    computes the logits in the documented fp32 order and the selection; both must equal the GPU's."""
    B, T, _ = H0.shape
    ks = oracle.capacity_counts(cfg.cap_num, cfg.cap_den, T)
    hist = res["h_per_rec"]
    for b in range(B):
        prev = np.arange(T)
        if cfg.routing == "tc":
            Z = np.stack([oracle.router_logits_fp32(hist[0, b], W["router_w"][j])
                          for j in range(cfg.n_rec)])
            assert np.array_equal(Z.view(np.uint32), res["logits"][:, b].view(np.uint32)), \
                f"TC logits differ (seq {b})"
            depth = np.argmax(Z, axis=0) + 1
            for r in range(1, cfg.n_rec + 1):
                want = np.nonzero(depth >= r)[0]
                assert np.array_equal(gpu_sets(res, cfg, b)[r - 1], want), f"TC set r={r} seq {b}"
            continue
        for r in range(1, cfg.n_rec + 1):
            bias = W["router_b"][r - 1] if cfg.routing == "threshold" else None
            z = oracle.router_logits_fp32(hist[r - 1, b][prev], W["router_w"][r - 1], bias)
            zg = res["logits"][r - 1, b]
            assert np.array_equal(zg[prev].view(np.uint32), z.view(np.uint32)), \
                f"logits differ at r={r} seq {b}: max |dz| {np.max(np.abs(zg[prev] - z))}"
            mask = np.ones(T, bool)
            mask[prev] = False
            assert np.all(np.isnan(zg[mask])), "logit written outside the active set"
            if cfg.routing == "ec":
                want = oracle.select_topk(prev, z, ks[r - 1])
            else:
                want = prev if r == 1 else prev[z > 0]
            got = gpu_sets(res, cfg, b)[r - 1]
            assert np.array_equal(got, want), f"active set differs at r={r} seq {b}"
            assert np.all(res["sel_pos"][r - 1, b, len(got):] == -1)
            prev = got
