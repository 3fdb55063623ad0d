#!/usr/bin/env python3
"""Benchmark of the MoR prefill on one MI355X (the 360M-shape, N_r = 3, bf16 workload).

One step = one mor_prefill call over a batch of 8 sequences of 2048 tokens: first layer,
three expert-choice recursions (capacities 3/3, 2/3, 1/3) over 10 shared layers with
recursion-wise KV caching, last layer. Inputs and weights are seeded synthetic tensors already
resident in HBM when the timed region starts.

Prints one JSON line. Algorithmic FLOPs follow the MoR paper's Appendix D accounting: 2 x
parameters per token for the projections, attention QK^T and PV counted over the causal
triangle only, norms and nonlinearities excluded, each recursion counted over the tokens
actually active there.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15          # dense MFMA bf16, FLOP/s (MI355X)
PEAK_FP32 = 157.3e12
PEAK_HBM = 8.0e12           # B/s
PEAK_CLOCK_GHZ = 2.4        # shader clock the published peaks assume (256 CUs)
KERNEL_SOURCES = {"gate_up": "adaptive_depth_recursive_amd/csrc/k_gemm_bf16.hip",
                  "qkv": "adaptive_depth_recursive_amd/csrc/k_gemm_bf16.hip",
                  "o_proj": "adaptive_depth_recursive_amd/csrc/k_gemm_bf16.hip",
                  "down": "adaptive_depth_recursive_amd/csrc/k_gemm_bf16.hip",
                  "attention": "adaptive_depth_recursive_amd/csrc/k_attn_bf16.hip"}


def layer_params(cfg) -> int:
    d, hd = cfg.d_model, cfg.head_dim
    nq, nkv = cfg.n_q_heads * hd, cfg.n_kv_heads * hd
    return d * (nq + 2 * nkv) + nq * d + 2 * d * cfg.d_ff + cfg.d_ff * d


def flop_counts(cfg, counts, sel_pos=None):
    """Algorithmic FLOPs of one call from the realised active-set sizes counts[r][b]."""
    import numpy as np
    B, T, R, n_s = counts.shape[1], cfg.seq, cfg.n_rec, cfg.n_shared
    d, hd, Hq = cfg.d_model, cfg.head_dim, cfg.n_q_heads
    P = layer_params(cfg)
    P_q_only = P - 2 * d * cfg.n_kv_heads * hd
    tri = lambda n: n * (n + 1) // 2          # causal (query, key) pairs of n tokens
    linear = 2 * P * 2 * B * T
    attn = 2 * 4 * Hq * hd * B * tri(T)
    gate_up = 2 * d * 2 * cfg.d_ff * 2 * B * T
    for r in range(R):
        M = int(counts[r].sum())
        share = cfg.kv_mode == "share" and r >= 1
        linear += n_s * 2 * (P_q_only if share else P) * M
        gate_up += n_s * 2 * d * 2 * cfg.d_ff * M
        if share:
            pairs = 0
            for b in range(B):
                pos = sel_pos[r, b, :counts[r, b]]
                k1 = sel_pos[0, b, :counts[0, b]]
                pairs += int(np.searchsorted(k1, pos, side="right").sum())
            attn += n_s * 4 * Hq * hd * pairs
        else:
            attn += n_s * 4 * Hq * hd * sum(tri(int(c)) for c in counts[r])
    if cfg.routing == "tc":
        router = 2 * d * R * B * T
    else:
        router = 2 * d * (B * T + sum(int(counts[r].sum()) for r in range(R - 1)))
    return {"linear": linear, "attention": attn, "router": router,
            "total": linear + attn + router, "gate_up": gate_up,
            "gate_up_launches": 2 + R * n_s}


def memory_kernel_bytes(cfg, counts):
    """Algorithmic HBM bytes of one call's memory-bound kernels, from the realised counts
    counts[r][b]: the router logits of recursion 1 read every row of H (4 B per element) and
    write one logit per token; the selector reads a logit and a position per token active
    before the recursion and writes the kept positions; the gather reads a row of H and writes
    it to the compacted buffer (8 B per element); the gated scatter reads H and the compacted
    row and writes H (12 B per element); an RMSNorm reads fp32 rows and writes bf16 ones
    (4 + 2 B per element), twice per layer. Returns {kind: (bytes per call, launches per call)}."""
    B, T, R, d = counts.shape[1], cfg.seq, cfg.n_rec, cfg.d_model
    n_s = cfg.n_shared
    es = 2 if cfg.dtype == "bf16" else 4
    BT = B * T
    prev = [BT] + [int(counts[r].sum()) for r in range(R - 1)]
    M = [int(counts[r].sum()) for r in range(R)]
    router_rows = BT * (R if cfg.routing == "tc" else 1)
    rows_normed = 2 * BT * 2 + 2 * n_s * sum(M)
    return {
        "router": (BT * d * 4 + router_rows * 4, 1),
        "select": (sum(8 * p + 4 * m for p, m in zip(prev, M)), R),
        "gather": (sum(8 * m * d for m in M), R),
        "scatter": (sum(12 * m * d for m in M), R),
        "rmsnorm": (rows_normed * d * (4 + es), 2 * (2 + R * n_s)),
    }


def time_kernel_kind(model, kind, h, h_out, steps, launches_per_call):
    """Average launch duration (s) of one kernel kind over `steps` calls, by HIP events on the
    library's stream around every launch of that kind."""
    import torch
    model.timing_enable(kind, launches_per_call * steps)
    torch.cuda.synchronize()
    for _ in range(steps):
        model.prefill(h, h_out)
    torch.cuda.synchronize()
    k_ms, k_n = model.timing_read()
    model.timing_enable("", 0)
    return (k_ms / 1e3) / max(k_n, 1), k_n


def prefill_variant(name, steps, warmup):
    """ms per call, tokens/s and the whole call's share of the bf16 MFMA peak of another prefill
    workload (135M shape; 360M token choice; 360M recursive KV sharing)."""
    import torch
    import adaptive_depth_recursive_amd as mor
    import workload
    cfg = workload.get_config(name)
    W = workload.make_weights(cfg)
    model = mor.Mor(cfg, W)
    h = torch.from_numpy(workload.make_inputs(cfg)).cuda()
    h_out = torch.empty_like(h)
    outs = model.prefill_outputs(h, debug=False)
    torch.cuda.synchronize()
    counts = outs["counts"].cpu().numpy()
    fl = flop_counts(cfg, counts, outs["sel_pos"].cpu().numpy())
    del outs
    for _ in range(warmup):
        model.prefill(h, h_out)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        model.prefill(h, h_out)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    model.close()
    return {"workload": f"{name}: batch {cfg.batch} x seq {cfg.seq}, d {cfg.d_model}, routing "
                        f"{cfg.routing}, {cfg.kv_mode}-wise KV",
            "ms_per_call": ms, "tokens_per_s": cfg.batch * cfg.seq / ms * 1e3,
            "call_flops": fl["total"], "tokens_per_recursion": counts.sum(axis=1).tolist(),
            "mfma_frac": fl["total"] / (ms / 1e3) / PEAK_BF16}


def source_hash(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel: str, workload_name: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current
    kernel source (null otherwise)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_gemm_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


DECODE_SOURCES = ("adaptive_depth_recursive_amd/csrc/k_decode.hip",
                  "adaptive_depth_recursive_amd/csrc/mor_api.hip")


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_profile_record():
    """The committed decode counter summary, if it was taken on the current decode kernels and
    launch sequence (None otherwise)."""
    path = os.path.join(ROOT, "profiles", "decode_smol360m_mor4_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != decode_source_hash():
        return None
    return rec


def decode_traffic_from_profile():
    """HBM-side bytes per decode iteration from the committed counter summary (null when it was
    taken on other sources)."""
    rec = decode_profile_record()
    return rec.get("bytes_per_iteration") if rec else None


def host_threads_and_cpu():
    """BLAS threads the oracle runs with (set to the cores this process may run on), and the
    host CPU model."""
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(limits=threads, user_api="blas")
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [threads])
    except Exception:
        pass
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(threads), model


def cpu_baseline(cfg, weights, H0_np, seq_len: int, n_seq: int = 1):
    """The oracle, as it stands, on the first n_seq sequences of the same workload (host cores)."""
    import numpy as np
    import oracle
    threads, cpu = host_threads_and_cpu()
    x = np.ascontiguousarray(H0_np[:n_seq, :seq_len])
    t0 = time.perf_counter()
    oracle.prefill(cfg.replace(seq=seq_len), weights, x)
    dt = time.perf_counter() - t0
    prec = "float64 with bf16 storage points" if cfg.dtype == "bf16" else "float64"
    return {"value": n_seq * seq_len / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_seq} of {cfg.batch} sequences ({n_seq * seq_len} tokens) of the {cfg.name} "
                      f"prefill, oracle in {prec}; {dt:.1f} s on {cpu}, BLAS threads set to the "
                      f"{len(os.sched_getaffinity(0))} cores available"}


def decode_cpu_baseline(budget_s: float = 10.0):
    """The oracle's token-by-token decode (per-recursion caches), as it stands, on the first
    requests of the same MoR-4 decode workload, in order, until about budget_s seconds of host
    time are spent (the request that crosses the budget is finished)."""
    import numpy as np
    import oracle
    import workload

    threads, cpu = host_threads_and_cpu()
    cfg = workload.get_config("smol360m_mor4_decode")
    W = workload.make_weights(cfg)
    with open(os.path.join(ROOT, "tests", "golden", "decode_router_bias.json")) as f:
        W["router_b"] = np.array(json.load(f)["router_b"], np.float32)
    lens = workload.make_decode_lengths(cfg)
    xs = workload.make_decode_inputs(cfg, lens)
    tok, n, t0 = 0, 0, time.perf_counter()
    while n < min(64, len(lens)) and time.perf_counter() - t0 < budget_s:
        oracle.decode_sequence(cfg, W, xs[n])
        tok += int(lens[n])
        n += 1
    dt = time.perf_counter() - t0
    return {"value": tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {n} of {len(lens)} requests ({tok} tokens) of the same decode "
                      f"workload, one at a time, oracle in float64 with bf16 storage points; "
                      f"{dt:.1f} s on {cpu}"}


def decode_bench(args, kv_mode="recursion"):
    """Depth-wise batched MoR-4 decode of the 360M-shape model (51 slots, 1024 requests with
    Geometric(mean 256) lengths, threshold exit with the calibrated router biases). Timed over
    the steady-state window: iterations while the request queue is not empty (every slot busy).
    kv_mode "share" runs recursive KV sharing (recursions >= 2 read the recursion-1 cache)."""
    import numpy as np
    import torch
    import adaptive_depth_recursive_amd as mor
    import workload

    cfg = workload.get_config("smol360m_mor4_decode", kv_mode=kv_mode)
    W = workload.make_weights(cfg)
    with open(os.path.join(ROOT, "tests", "golden", "decode_router_bias.json")) as f:
        W["router_b"] = np.array(json.load(f)["router_b"], np.float32)
    lens = workload.make_decode_lengths(cfg)
    x = torch.from_numpy(np.concatenate(workload.make_decode_inputs(cfg, lens))).cuda()
    out = torch.empty_like(x)
    dep = torch.zeros(x.shape[0], dtype=torch.int8, device="cuda")
    model = mor.Mor(cfg, W, max_batch=1, max_seq=cfg.max_len, max_slots=cfg.slots,
                    kv_page_tokens=args.kv_page_tokens, max_requests=len(lens))
    model.decode_submit(lens, x, out, dep)
    model.decode_step(args.decode_warmup)          # slots fill on the first iteration
    st0 = model.decode_stats()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms, last, chunks = 0.0, st0, 0
    while last["iterations"] - st0["iterations"] < args.decode_iters:
        ev[0].record()
        model.decode_step(args.decode_chunk)
        ev[1].record()
        st = model.decode_stats()
        if st["admitted"] >= len(lens):          # queue drained during this chunk: window ends
            break
        ms += ev[0].elapsed_time(ev[1])
        last, chunks = st, chunks + 1
    it = last["iterations"] - st0["iterations"]
    tok = last["tokens"] - st0["tokens"]
    byt = sum(last[k] - st0[k] for k in ("weight_bytes", "kv_read_bytes", "kv_write_bytes", "act_bytes"))
    kvr = last["kv_read_bytes"] - st0["kv_read_bytes"]
    s_ = ms / 1e3
    done = dep[dep > 0].cpu().numpy()
    peak_pages = last["kv_pages_peak"]
    model.close()
    return {
        "metric": "MoR-4 decode tokens/sec (360M-shape, 51 slots, depth-wise batching, bf16)",
        "value": tok / s_ if s_ else None, "unit": "tokens/s",
        "ms_per_iteration": ms / max(it, 1), "tokens_per_iteration": tok / max(it, 1),
        "window": f"{it} iterations ({chunks} chunks of {args.decode_chunk}) while the queue of "
                  f"{len(lens)} requests was not empty, after {args.decode_warmup} warmup iterations",
        "roofline": {"bound": "hbm", "achieved": byt / s_ / 1e9 if s_ else None, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": byt / s_ / PEAK_HBM if s_ else None,
                     "traffic": decode_traffic_from_profile() if kv_mode == "recursion" else None,
                     "l2_hit_rate": ((decode_profile_record() or {}).get("l2_hit_rate")
                                     if kv_mode == "recursion" else None),
                     "algorithmic_bytes_per_iteration": byt / max(it, 1),
                     "kv_read_bytes_per_iteration": kvr / max(it, 1)},
        "exit_depth_histogram": np.bincount(done, minlength=cfg.n_rec + 1)[1:].tolist(),
        "kv_cache_peak_bytes": peak_pages * last["page_bytes"],
        "config": {"workload": f"{cfg.name}: d {cfg.d_model}, {cfg.n_q_heads}/{cfg.n_kv_heads} heads x "
                               f"{cfg.head_dim}, FFN {cfg.d_ff}, L {cfg.n_layers} (N_r {cfg.n_rec} x "
                               f"{cfg.n_shared} shared), threshold exit, {cfg.kv_mode}-wise KV, {cfg.slots} slots, "
                               f"{len(lens)} requests, {int(lens.sum())} tokens, "
                               f"{args.kv_page_tokens}-token KV pages"},
    }


def handoff_bench(args):
    """Prefill -> decode hand-over on the 360M MoR-4 model: 51 prompts of 256 tokens prefilled with
    the threshold router, their per-recursion caches handed to the decode engine
    (mor_decode_continue), then the first 51 seeded continuations decoded to the end."""
    import numpy as np
    import torch
    import adaptive_depth_recursive_amd as mor
    import workload

    cfg = workload.get_config("smol360m_mor4_decode")
    W = workload.make_weights(cfg)
    with open(os.path.join(ROOT, "tests", "golden", "decode_router_bias.json")) as f:
        W["router_b"] = np.array(json.load(f)["router_b"], np.float32)
    B, T = cfg.slots, 256
    model = mor.Mor(cfg, W, max_batch=B, max_seq=cfg.max_len, max_slots=B,
                    kv_page_tokens=args.kv_page_tokens, max_requests=B)
    prompts = torch.from_numpy(workload.make_inputs(cfg, batch=B, seq=T)).cuda()
    pout = torch.empty_like(prompts)
    for _ in range(2):
        model.prefill(prompts, pout)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    reps = 5
    for _ in range(reps):
        model.prefill(prompts, pout)
    ev[1].record()
    torch.cuda.synchronize()
    pre_ms = ev[0].elapsed_time(ev[1]) / reps
    counts = torch.empty((cfg.n_rec, B), dtype=torch.int32, device="cuda")
    model.prefill(prompts, pout, counts=counts)
    torch.cuda.synchronize()
    cnt = counts.cpu().numpy()
    lens = np.minimum(workload.make_decode_lengths(cfg)[:B], cfg.max_len - T)
    x = torch.from_numpy(np.concatenate(workload.make_decode_inputs(cfg, lens))).cuda()
    out = torch.empty_like(x)
    dep = torch.zeros(x.shape[0], dtype=torch.int8, device="cuda")
    t0 = time.perf_counter()
    model.decode_continue(lens, x, out, dep)            # synchronises
    hand_s = time.perf_counter() - t0
    kvtok = 2 * cfg.n_kv_heads * cfg.head_dim * 2
    kv_rows = B * T * 2 + cfg.n_shared * int(cnt.sum())  # first, last and every (r, j) stream
    ev[0].record()
    it = model.decode_run(int(lens.sum()), chunk=64)
    ev[1].record()
    torch.cuda.synchronize()
    dec_ms = ev[0].elapsed_time(ev[1])
    model.close()
    return {"prompt": f"{B} x {T} tokens, threshold routing",
            "prefill_ms": pre_ms, "prefill_tokens_per_s": B * T / pre_ms * 1e3,
            "prompt_depth_counts": cnt.sum(axis=1).tolist(),
            "handoff_ms_incl_host": hand_s * 1e3, "handoff_kv_bytes": kv_rows * kvtok,
            "continuation_tokens": int(lens.sum()), "decode_iterations": it,
            "decode_tokens_per_s_all": float(lens.sum()) / dec_ms * 1e3,
            "note": "decode rate over all iterations, including the drain of the longest requests"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="smol360m_bf16")
    ap.add_argument("--roofline-kernel", default="gate_up", choices=sorted(KERNEL_SOURCES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seq", type=int, default=2048, help="tokens of the CPU-baseline sample")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--decode-iters", type=int, default=3000, help="cap of the timed decode window")
    ap.add_argument("--decode-chunk", type=int, default=64)
    ap.add_argument("--decode-warmup", type=int, default=64)
    ap.add_argument("--kv-page-tokens", type=int, default=64)
    ap.add_argument("--handoff-only", action="store_true", help="only the prefill -> decode hand-over leg")
    ap.add_argument("--decode-kv", default="recursion", choices=["recursion", "share"],
                    help="KV mode of --decode-only")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the 135M, token-choice and KV-sharing prefill measurements")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the MoR prefill shards by sequence with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import adaptive_depth_recursive_amd as mor
    import workload

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4}))
        return

    if args.handoff_only:
        print(json.dumps(handoff_bench(args)), flush=True)
        return
    if args.decode_only:
        print(json.dumps(decode_bench(args, args.decode_kv)), flush=True)
        return

    cfg = workload.get_config(args.config)
    W = workload.make_weights(cfg)
    H0 = workload.make_inputs(cfg)
    model = mor.Mor(cfg, W)
    h = torch.from_numpy(H0).cuda()
    h_out = torch.empty_like(h)
    B, T = cfg.batch, cfg.seq

    # realised active sets (static counts for expert choice) for the FLOP accounting
    outs = model.prefill_outputs(h, debug=False)
    torch.cuda.synchronize()
    counts = outs["counts"].cpu().numpy()
    sel_pos = outs["sel_pos"].cpu().numpy()
    del outs
    fl = flop_counts(cfg, counts, sel_pos)

    for _ in range(args.warmup):
        model.prefill(h, h_out)
    torch.cuda.synchronize()

    kind = args.roofline_kernel
    launches_per_call = fl["gate_up_launches"]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # timed region: K whole calls, nothing else on the stream
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        model.prefill(h, h_out)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end)
    # kernel-timing region: the same K calls, with HIP events on the library's stream around
    # every launch of the roofline kernel
    model.timing_enable(kind, launches_per_call * args.steps)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        model.prefill(h, h_out)
    end.record()
    torch.cuda.synchronize()
    ms_ev = start.elapsed_time(end)
    k_ms, k_n = model.timing_read()
    clock_ghz = model.timing_clock()
    model.timing_enable("", 0)

    step_s = ms / 1e3 / args.steps
    tokens_per_s = B * T / step_s
    if kind == "gate_up":
        k_flops_per_launch = fl["gate_up"] / launches_per_call
    else:
        k_flops_per_launch = None
    k_avg_s = (k_ms / 1e3) / max(k_n, 1)
    peak = PEAK_BF16 if cfg.dtype == "bf16" else PEAK_FP32
    achieved = k_flops_per_launch / k_avg_s / 1e12 if k_flops_per_launch else None
    traffic = traffic_from_profile(kind, cfg.name)
    roofline = {"bound": "mfma", "kernel": f"k_gemm_bf16, SwiGLU epilogue ({kind} projection; tile chosen per launch)",
                "achieved": achieved, "peak": peak / 1e12, "unit": "TFLOP/s",
                "frac": (achieved * 1e12 / peak) if achieved else None, "traffic": traffic,
                "avg_launch_us": k_avg_s * 1e6, "launches_timed": k_n,
                "flops_per_launch": k_flops_per_launch,
                "call_achieved": fl["total"] / step_s / 1e12,
                "call_frac": fl["total"] / step_s / peak,
                "clock_ghz": clock_ghz or None,
                "peak_at_clock": (peak / 1e12 * clock_ghz / PEAK_CLOCK_GHZ) if clock_ghz else None,
                "frac_at_clock": (achieved * 1e12 / (peak * clock_ghz / PEAK_CLOCK_GHZ)) if (clock_ghz and achieved) else None,
                "note": "achieved/frac: the dominant kernel per launch; call_achieved/call_frac: the "
                        "whole prefill call (all kernels, algorithmic FLOPs) against the same peak; "
                        "clock_ghz: shader clock during the kernel's timed launches (cycle counter "
                        "against the real-time counter, first workgroup), peak_at_clock/frac_at_clock: "
                        "the peak scaled from its 2.4 GHz to that clock"}

    # memory-bound kernels of the call: algorithmic bytes against HBM
    mem = {}
    for mk, (byts, nl) in memory_kernel_bytes(cfg, counts).items():
        avg_s, n = time_kernel_kind(model, mk, h, h_out, args.steps, nl)
        bpl = byts / nl
        mem[mk] = {"avg_launch_us": avg_s * 1e6, "launches_per_call": nl,
                   "bytes_per_launch": bpl, "GB_per_s": bpl / avg_s / 1e9,
                   "hbm_frac": bpl / avg_s / PEAK_HBM}

    result = {
        "metric": "MoR prefill tokens/sec (360M-shape, N_r=3, bf16) + % of bf16 MFMA peak",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_s * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name} prefill: batch {B} x seq {T}, d {cfg.d_model}, "
                               f"{cfg.n_q_heads}/{cfg.n_kv_heads} heads x {cfg.head_dim}, FFN {cfg.d_ff}, "
                               f"L {cfg.n_layers} (N_r {cfg.n_rec} x {cfg.n_shared} shared), "
                               f"EC capacities {'/'.join(str(c) for c in cfg.cap_num)} of {cfg.cap_den}, "
                               f"{cfg.kv_mode}-wise KV",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "step_flops": fl["total"],
        "step_mfma_frac": fl["total"] / step_s / peak,
        "wall_s_timed": wall,
        "ms_per_step_with_kernel_events": ms_ev / args.steps,
        "roofline": roofline,
        "memory_kernels": mem,
    }
    model.close()
    del h, h_out
    torch.cuda.empty_cache()
    if not args.no_variants:
        result["prefill_variants"] = {
            v: prefill_variant(v, args.steps, args.warmup)
            for v in ("smol135m_bf16", "smol360m_tc_bf16", "smol360m_share_bf16")}
        torch.cuda.empty_cache()
    if not args.no_decode:
        result["decode"] = decode_bench(args, "recursion")
        torch.cuda.empty_cache()
        result["decode_kv_share"] = decode_bench(args, "share")
        torch.cuda.empty_cache()
        result["decode_handoff"] = handoff_bench(args)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, W, H0, args.cpu_seq)
        if cfg.name == "smol360m_bf16":
            others = {}
            for name, nseq in (("tiny_f32", 2), ("smol135m_bf16", 1)):
                c2 = workload.get_config(name)
                others[name] = cpu_baseline(c2, workload.make_weights(c2), workload.make_inputs(c2),
                                            c2.seq, nseq)
            result["cpu_baseline_other_prefills"] = others
        if not args.no_decode:
            result["decode"]["cpu_baseline"] = decode_cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
