"""GPU parity of the depth-wise batched decode engine against the CPU oracle (needs an MI355X).

The engine decodes requests token by token with the static-threshold router, many requests at
different recursion depths sharing every launch. Its results are compared per request with the
oracle's one-shot threshold forward of the whole request (which the oracle's own pins tie to its
token-by-token decode with per-recursion caches):
  - router logits bit-exact given the engine's own hidden states (stage-wise), and each exit
    depth exactly the one those logits decide;
  - fp32 runs free: exit depths equal the oracle's own, hidden states within 1e-4;
  - bf16 is teacher-forced (the oracle adopts the engine's depths), hidden states within 2e-2;
  - per-token results do not depend on the batch: 1, 2 or 5 slots give identical bits.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workload
from tests.gpu_common import rel_err, say, tolerance

pytestmark = pytest.mark.gpu

BIAS_SMALL = np.array([0.0, 0.1, 0.0, -0.1], np.float32)
GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _setup(cfg, slots, bias=BIAS_SMALL, kv_pages=0, page=16, n_req=None, lengths=None):
    import adaptive_depth_recursive_amd as mor
    W = workload.make_weights(cfg)
    W["router_b"] = np.asarray(bias, np.float32)
    lens = workload.make_decode_lengths(cfg, n=n_req) if lengths is None else np.asarray(lengths, np.int32)
    say(f"[gpu] decode init {cfg.name} dtype={cfg.dtype} slots={slots} page={page} "
        f"kv_pages={kv_pages} requests={len(lens)} tokens={int(lens.sum())}")
    model = mor.Mor(cfg, W, max_batch=1, max_seq=cfg.max_len, max_slots=slots,
                    kv_page_tokens=page, kv_pages=kv_pages, max_requests=len(lens))
    return model, W, lens


def _run(model, cfg, lens, inputs, dumps=True):
    import torch
    x = torch.from_numpy(np.concatenate(inputs).astype(np.float32)).cuda()
    n = x.shape[0]
    out = torch.zeros_like(x)
    dep = torch.zeros(n, dtype=torch.int8, device="cuda")
    hd = torch.full((n, cfg.n_rec + 1, cfg.d_model), np.nan, device="cuda") if dumps else None
    zd = torch.empty((n, cfg.n_rec), device="cuda") if dumps else None
    model.decode_submit(lens, x, out, dep, hd, zd)
    say(f"[gpu] decode run {n} tokens")
    iters = model.decode_run(n, chunk=16, max_iters=n * cfg.n_rec + 1000)
    done = model.decode_step(0, sync=True)
    torch.cuda.synchronize()
    assert done[0] == n and done[1] == len(lens), f"unfinished: {done}"
    res = {"out": out.cpu().numpy(), "depth": dep.cpu().numpy().astype(np.int32), "iters": iters}
    if dumps:
        res["h"] = hd.cpu().numpy()
        res["z"] = zd.cpu().numpy()
    return res


def _offsets(lens):
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)


def _check_routing(cfg, W, res, lens):
    """Logits bit-exact given the engine's hidden states; depths exactly what they decide."""
    R = cfg.n_rec
    for i, (o, n) in enumerate(zip(_offsets(lens), lens)):
        for t in range(o, o + n):
            D = res["depth"][t]
            assert 1 <= D <= R
            for r in range(1, min(D + 1, R) + 1):
                z = oracle.router_logits_fp32(res["h"][t, r - 1], W["router_w"][r - 1],
                                              W["router_b"][r - 1])[0]
                assert res["z"][t, r - 1].view(np.uint32) == z.view(np.uint32), (i, t, r)
            for r in range(2, D + 1):
                assert res["z"][t, r - 1] > 0, (t, r)
            if D < R:
                assert not res["z"][t, D] > 0, (t, D)
            assert np.all(np.isnan(res["z"][t, D + 1:])), t


def _compare(cfg, W, res, lens, inputs, teacher, which=None):
    worst = 0.0
    R = cfg.n_rec
    for i, (o, n) in enumerate(zip(_offsets(lens), lens)):
        if which is not None and i not in which:
            continue
        depth = res["depth"][o:o + n]
        forced = [[np.nonzero(depth >= r)[0]] for r in range(1, R + 1)] if teacher else None
        ref = oracle.prefill(cfg.replace(seq=int(n)), W, inputs[i][None], forced_sel=forced)
        p = ref["per_seq"][0]
        own = np.zeros(n, np.int32)
        for r, sel in enumerate(p["own_sel"], start=1):
            own[sel] = r
        if not teacher:
            assert np.array_equal(own, depth), f"request {i}: exit depths differ"
        e = rel_err(res["out"][o:o + n], ref["out"][0])
        for r in range(R + 1):
            rows = np.nonzero(depth >= r)[0] if r else np.arange(n)
            er = rel_err(res["h"][o + rows, r], p["hist"][r][rows])
            assert er <= tolerance(cfg), f"request {i}: H after recursion {r} rel err {er}"
        worst = max(worst, e)
        assert e <= tolerance(cfg), f"request {i}: output rel err {e}"
    return worst


def test_decode_small_f32_free_running():
    cfg = workload.get_config("small_thr_bf16", dtype="f32")
    model, W, lens = _setup(cfg, slots=5)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    worst = _compare(cfg, W, res, lens, inputs, teacher=False)
    say(f"[gpu] decode f32: {len(lens)} requests, {res['iters']} iterations, worst rel err {worst:.2e}, "
        f"depth histogram {np.bincount(res['depth'], minlength=cfg.n_rec + 1)[1:]}")
    model.close()


def test_decode_wide_rows_f32_free_running():
    """d_model 1088 (> 1024 = one float4 per thread of a 256-thread row workgroup): every row
    kernel takes its second chunk; 32-token pages (two pages per 64-key attention tile)."""
    cfg = workload.get_config("small_thr_bf16", dtype="f32", d_model=1088)
    model, W, lens = _setup(cfg, slots=5, page=32)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    worst = _compare(cfg, W, res, lens, inputs, teacher=False)
    say(f"[gpu] decode f32 d 1088: worst rel err {worst:.2e}, "
        f"depth histogram {np.bincount(res['depth'], minlength=cfg.n_rec + 1)[1:]}")
    model.close()


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (8, 2)])
def test_decode_bf16_gqa_ratios(hq, hkv):
    """Decode attention with 1, 2 and 4 query heads per KV head, bf16 teacher-forced."""
    cfg = workload.get_config("small_thr_bf16", n_q_heads=hq, n_kv_heads=hkv)
    model, W, lens = _setup(cfg, slots=5)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    worst = _compare(cfg, W, res, lens, inputs, teacher=True)
    say(f"[gpu] decode bf16 {hq}/{hkv} heads: worst rel err {worst:.2e}")
    model.close()


def test_decode_small_bf16_teacher_forced():
    cfg = workload.get_config("small_thr_bf16")
    model, W, lens = _setup(cfg, slots=5)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    worst = _compare(cfg, W, res, lens, inputs, teacher=True)
    say(f"[gpu] decode bf16: worst rel err {worst:.2e}")
    model.close()


def test_decode_small_bf16_kv_share():
    cfg = workload.get_config("small_thr_bf16", kv_mode="share")
    model, W, lens = _setup(cfg, slots=4)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    _compare(cfg, W, res, lens, inputs, teacher=True)
    model.close()


def test_decode_f32_kv_share_free_running():
    cfg = workload.get_config("small_thr_bf16", dtype="f32", kv_mode="share")
    model, W, lens = _setup(cfg, slots=3, page=32)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    _compare(cfg, W, res, lens, inputs, teacher=False)
    model.close()


def test_decode_results_independent_of_batch():
    """Depth-wise batching changes only which tokens share a launch, never a token's result:
    1, 2 and 5 slots (different admission orders, page sizes and batch mixes) give identical bits."""
    cfg = workload.get_config("small_thr_bf16")
    outs = []
    for slots, page in ((5, 16), (2, 32), (1, 64)):
        model, W, lens = _setup(cfg, slots=slots, page=page)
        inputs = workload.make_decode_inputs(cfg, lens)
        res = _run(model, cfg, lens, inputs, dumps=False)
        outs.append(res)
        model.close()
    for r in outs[1:]:
        assert np.array_equal(r["depth"], outs[0]["depth"])
        assert np.array_equal(r["out"].view(np.uint32), outs[0]["out"].view(np.uint32))


def test_decode_unit_gate_all_depths():
    """Biases that open every recursion: every token runs N_r recursions (the fixed-depth
    recursive model, token by token)."""
    cfg = workload.get_config("small_thr_bf16", dtype="f32", gate_mode="unit")
    model, W, lens = _setup(cfg, slots=4, bias=[0.0, 50.0, 50.0, 50.0], n_req=5)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    assert np.all(res["depth"] == cfg.n_rec)
    _compare(cfg, W, res, lens, inputs, teacher=False)
    model.close()


def test_decode_single_token_requests_and_resubmit():
    """Length-1 requests (admit and leave every few iterations), then a second submission on
    the same handle starts from a clean engine."""
    cfg = workload.get_config("small_thr_bf16", dtype="f32")
    model, W, _ = _setup(cfg, slots=3, lengths=[1] * 7)
    for lens in ([1] * 7, [5, 1, 3]):
        lens = np.array(lens, np.int32)
        inputs = workload.make_decode_inputs(cfg, lens)
        res = _run(model, cfg, lens, inputs)
        _compare(cfg, W, res, lens, inputs, teacher=False)
    model.close()


def test_decode_kv_pool_exhaustion_reported():
    """A pool too small for the batch: the engine stops at the iteration that needs a page it
    cannot get, reports MOR_E_KV_FULL, and every kernel still runs to completion."""
    import torch
    import adaptive_depth_recursive_amd as mor
    cfg = workload.get_config("small_thr_bf16")
    model, W, lens = _setup(cfg, slots=5, kv_pages=12, page=16)
    inputs = workload.make_decode_inputs(cfg, lens)
    x = torch.from_numpy(np.concatenate(inputs)).cuda()
    out = torch.zeros_like(x)
    dep = torch.zeros(x.shape[0], dtype=torch.int8, device="cuda")
    model.decode_submit(lens, x, out, dep)
    with pytest.raises(mor.MorError) as e:
        for _ in range(200):
            model.decode_step(8, sync=True)
    assert e.value.status == mor.MOR_E_KV_FULL
    torch.cuda.synchronize()
    model.close()


def test_decode_full_size_sampled():
    """The 360M-shape MoR-4 decode workload at its launch configuration (51 slots, 64-token
    pages): the first 80 requests of the seeded length distribution, uncapped (up to 1331
    tokens, so the longest requests' attention runs two rounds of 1024 keys per workgroup),
    routing checked stage-wise on every token, the two longest requests and the shortest one
    checked against the oracle (teacher-forced)."""
    cfg = workload.get_config("smol360m_mor4_decode")
    bias = np.array(_gold("decode_router_bias.json")["router_b"], np.float32)
    lens = workload.make_decode_lengths(cfg)[:80]
    model, W, lens = _setup(cfg, slots=cfg.slots, bias=bias, page=64, lengths=lens)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    order = np.argsort(lens, kind="stable")
    which = [int(order[-1]), int(order[-2]), int(order[0])]
    assert lens[which[0]] > 1024
    say(f"[cpu] oracle on requests {which} (lengths {lens[which].tolist()})")
    worst = _compare(cfg, W, res, lens, inputs, teacher=True, which=set(which))
    say(f"[gpu] full-size decode: {int(lens.sum())} tokens, {res['iters']} iterations, "
        f"depths {np.bincount(res['depth'], minlength=cfg.n_rec + 1)[1:]}, worst rel err {worst:.2e}")
    model.close()


def test_decode_long_context_bf16():
    """A request of 1300 tokens next to short ones: the bf16 decode attention (16 waves of
    64-key tiles, 1024 keys per round) takes two rounds from position 1024 on, and every
    wave's next tile overwrites its LDS V tile after the current one was read. Teacher-forced
    against the oracle at 2e-2, routing stage-wise bit-exact."""
    cfg = workload.get_config("small_thr_bf16", max_len=1600)
    model, W, lens = _setup(cfg, slots=3, lengths=[1300, 40, 211])
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    worst = _compare(cfg, W, res, lens, inputs, teacher=True)
    say(f"[gpu] decode bf16 long context: {res['iters']} iterations, worst rel err {worst:.2e}, "
        f"depth histogram {np.bincount(res['depth'], minlength=cfg.n_rec + 1)[1:]}")
    model.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_128_token_pages(dtype):
    """Pages of 128 tokens (larger than a 64-key attention tile: a tile reads half a page) with a
    request that fills several pages; bf16 teacher-forced, fp32 free-running."""
    cfg = workload.get_config("small_thr_bf16", dtype=dtype, max_len=512)
    model, W, lens = _setup(cfg, slots=3, page=128, lengths=[300, 129, 17])
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    worst = _compare(cfg, W, res, lens, inputs, teacher=dtype == "bf16")
    say(f"[gpu] decode {dtype} 128-token pages: worst rel err {worst:.2e}")
    model.close()


def test_decode_full_size_kv_share_sampled():
    """The 360M MoR-4 workload with recursive KV sharing at its launch configuration (51 slots,
    64-token pages): the first 60 requests, routing stage-wise on every token, the longest and
    the shortest request against the oracle (teacher-forced)."""
    cfg = workload.get_config("smol360m_mor4_decode", kv_mode="share")
    bias = np.array(_gold("decode_router_bias.json")["router_b"], np.float32)
    lens = workload.make_decode_lengths(cfg)[:60]
    model, W, lens = _setup(cfg, slots=cfg.slots, bias=bias, page=64, lengths=lens)
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    order = np.argsort(lens, kind="stable")
    which = [int(order[-1]), int(order[0])]
    say(f"[cpu] oracle on requests {which} (lengths {lens[which].tolist()})")
    worst = _compare(cfg, W, res, lens, inputs, teacher=True, which=set(which))
    say(f"[gpu] full-size KV-sharing decode: {int(lens.sum())} tokens, worst rel err {worst:.2e}")
    model.close()


def test_decode_long_context_f32_free_running():
    """fp32 decode attention runs 8 waves (512 keys per round): a 700-token request crosses into
    the second round in the first and last layers and in the recursion-1 layers. Free-running:
    exit depths equal the oracle's own, hidden states within 1e-4."""
    cfg = workload.get_config("small_thr_bf16", dtype="f32", max_len=800)
    model, W, lens = _setup(cfg, slots=3, page=32, lengths=[700, 23, 5])
    inputs = workload.make_decode_inputs(cfg, lens)
    res = _run(model, cfg, lens, inputs)
    _check_routing(cfg, W, res, lens)
    worst = _compare(cfg, W, res, lens, inputs, teacher=False)
    say(f"[gpu] decode f32 long context: {res['iters']} iterations, worst rel err {worst:.2e}")
    model.close()


def test_decode_graph_replay_matches_eager():
    """Iterations replayed from the captured graph (steps of 16) give the same bits as eager
    launches (steps of 4, below the graph size), across many replays with host syncs between."""
    import torch
    cfg = workload.get_config("small_thr_bf16")
    model, W, lens = _setup(cfg, slots=5)
    inputs = workload.make_decode_inputs(cfg, lens)
    x = torch.from_numpy(np.concatenate(inputs)).cuda()
    res = []
    for chunk in (4, 16):
        out = torch.zeros_like(x)
        dep = torch.zeros(x.shape[0], dtype=torch.int8, device="cuda")
        model.decode_submit(lens, x, out, dep)
        model.decode_run(x.shape[0], chunk=chunk, max_iters=x.shape[0] * cfg.n_rec + 1000)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), dep.cpu().numpy()))
    assert np.array_equal(res[0][1], res[1][1])
    assert np.array_equal(res[0][0].view(np.uint32), res[1][0].view(np.uint32))
    model.close()


@pytest.mark.parametrize("dtype,kv_mode,T,lens", [
    ("f32", "recursion", 40, (5, 17, 9)), ("bf16", "recursion", 40, (5, 17, 9)),
    ("f32", "share", 40, (5, 17, 9)), ("bf16", "recursion", 1000, (30, 12)),
    ("f32", "share", 1000, (9, 21))])
def test_decode_continues_prefill(dtype, kv_mode, T, lens):
    """Prefill -> decode hand-over: prompts of T tokens are prefilled with threshold routing,
    then decoded further from the prefill's per-recursion caches (prompts of 1000 tokens put
    the continuation's attention past one round of keys per workgroup in every layer stream
    that recursion 1 feeds). With threshold routing (causal) the result must equal the oracle's
    forward of each whole sequence: fp32 free-running (exact depths), bf16 teacher-forced."""
    import torch
    import adaptive_depth_recursive_amd as mor
    cfg = workload.get_config("small_thr_bf16", dtype=dtype, kv_mode=kv_mode)
    W = workload.make_weights(cfg)
    W["router_b"] = BIAS_SMALL
    lens = np.array(lens, np.int32)
    B = len(lens)
    max_seq = -(-(T + int(lens.max())) // 64) * 64
    say(f"[gpu] decode hand-over {dtype} {kv_mode}: prefill {B} x {T}, continue {lens.tolist()}")
    model = mor.Mor(cfg, W, max_batch=B, max_seq=max_seq, max_slots=B, kv_page_tokens=16,
                    max_requests=B)
    prompt = workload.make_inputs(cfg, batch=B, seq=T)
    pre = model.prefill_outputs(torch.from_numpy(prompt).cuda(), debug=False)
    torch.cuda.synchronize()
    sel = pre["sel_pos"].cpu().numpy()
    cnt = pre["counts"].cpu().numpy()
    cont = workload.make_decode_inputs(cfg, lens)
    x = torch.from_numpy(np.concatenate(cont)).cuda()
    out = torch.zeros_like(x)
    dep = torch.zeros(x.shape[0], dtype=torch.int8, device="cuda")
    hd = torch.full((x.shape[0], cfg.n_rec + 1, cfg.d_model), np.nan, device="cuda")
    zd = torch.empty((x.shape[0], cfg.n_rec), device="cuda")
    model.decode_continue(lens, x, out, dep, hd, zd)
    model.decode_run(x.shape[0], chunk=16, max_iters=4000)
    done = model.decode_step(0, sync=True)
    torch.cuda.synchronize()
    assert done[0] == x.shape[0] and done[1] == B
    res = {"out": out.cpu().numpy(), "depth": dep.cpu().numpy().astype(np.int32),
           "h": hd.cpu().numpy(), "z": zd.cpu().numpy()}
    _check_routing(cfg, W, res, lens)
    offs = _offsets(lens)
    for b in range(B):
        n = int(lens[b])
        full = np.concatenate([prompt[b], cont[b]])[None]
        depth_c = res["depth"][offs[b]:offs[b] + n]
        forced = None
        if dtype == "bf16":
            forced = []
            for r in range(cfg.n_rec):
                ps = sel[r, b, :cnt[r, b]]
                forced.append([np.concatenate([ps, T + np.nonzero(depth_c >= r + 1)[0]])])
        ref = oracle.prefill(cfg.replace(seq=T + n), W, full, forced_sel=forced)
        p = ref["per_seq"][0]
        if dtype == "f32":
            own = np.zeros(T + n, np.int32)
            for r, s_ in enumerate(p["own_sel"], start=1):
                own[s_] = r
            assert np.array_equal(own[T:], depth_c), f"seq {b}: continuation depths differ"
            for r in range(cfg.n_rec):
                assert np.array_equal(p["own_sel"][r][p["own_sel"][r] < T], sel[r, b, :cnt[r, b]])
        e = rel_err(res["out"][offs[b]:offs[b] + n], ref["out"][0][T:])
        say(f"[gpu] hand-over seq {b}: rel err {e:.2e}")
        assert e <= tolerance(cfg), f"seq {b}: continuation output rel err {e}"
    model.close()
