"""mor_route_noalloc (scratch in a static device array, no workspace) against mor_route."""
import numpy as np
import pytest

import workload
from tests.gpu_common import build_gpu, say

pytestmark = pytest.mark.gpu


def _sets(rng, B, T, n):
    act = np.full((B, T), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        p = np.sort(rng.choice(T, size=min(n, T), replace=False)).astype(np.int32)
        act[b, :len(p)] = p
        cnt[b] = len(p)
    return act, cnt


def _same(a, b):
    a, b = a.cpu().numpy(), b.cpu().numpy()
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return np.array_equal(a, b)


@pytest.mark.parametrize("name", ["small_bf16", "small_thr_bf16"])
def test_route_noalloc_equals_route(name):
    """Two calls in a row through the C ABI, the second with a smaller batch and sequence and a
    sparser active set: every output bitwise equal to mor_route's on the same inputs."""
    import torch
    cfg = workload.get_config(name)
    W = workload.make_weights(cfg)
    if cfg.routing == "threshold":
        W["router_b"] = np.array([0.0, 0.1, 0.0, -0.1], np.float32)
    model, W = build_gpu(cfg, W, max_batch=3, max_seq=333)
    rng = np.random.default_rng(5)
    for B, T, n, r in ((3, 333, 333, 1), (3, 333, 250, 2), (2, 101, 40, 3)):
        H = torch.from_numpy(rng.standard_normal((B, T, cfg.d_model)).astype(np.float32)).cuda()
        act, cnt = _sets(rng, B, T, n)
        act_d, cnt_d = torch.from_numpy(act).cuda(), torch.from_numpy(cnt).cuda()
        say(f"[gpu] {name}: mor_route / mor_route_noalloc B={B} T={T} active={n} r={r}")
        want = model.route(H, act_d, cnt_d, r)
        # outputs prefilled with garbage, so stale values would show
        out = (torch.full((B, T), 77, dtype=torch.int32, device="cuda"),
               torch.full((B,), 77, dtype=torch.int32, device="cuda"),
               torch.full((B, T), 3.0, device="cuda"))
        got = model.route_noalloc(H, act_d, cnt_d, r, out=out)
        torch.cuda.synchronize()
        for g, w, what in zip(got, want, ("active_out", "counts_out", "z")):
            assert _same(g, w), (B, T, r, what)
    model.close()


def test_route_noalloc_rejects_beyond_scratch():
    """B*T beyond the static scratch: MOR_E_SHAPE before anything is launched."""
    import torch
    import adaptive_depth_recursive_amd as mor
    cfg = workload.get_config("tiny_f32")
    model, _ = build_gpu(cfg, max_batch=9, max_seq=8192)
    B, T = 9, 8000
    H = torch.zeros((B, T, cfg.d_model), device="cuda")
    act = torch.arange(T, dtype=torch.int32, device="cuda").repeat(B, 1)
    cnt = torch.full((B,), T, dtype=torch.int32, device="cuda")
    with pytest.raises(mor.MorError) as e:
        model.route_noalloc(H, act, cnt, 1)
    assert e.value.status == mor.MOR_E_SHAPE
    assert "static scratch" in str(e.value)
    model.close()
