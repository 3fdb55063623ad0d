"""Test-time recursion scaling (host side and oracle; no GPU): the trained shared blocks unrolled
for more recursions than they were trained with ([Notes] section 'Test-time scaling': depth is a
runtime parameter)."""
import numpy as np
import pytest

import oracle
import workload
from tests.hf_reference import llama_stack


def _mor():
    import adaptive_depth_recursive_amd as mor
    return mor


def test_extend_shapes_and_defaults():
    mor = _mor()
    cfg = workload.get_config("small_f32")                      # N_r 3, L 8, n_s 2, caps 3/2/1 of 3
    W = workload.make_weights(cfg)
    cfg2, W2 = mor.extend_recursions(cfg, W, extra=2)
    assert (cfg2.n_rec, cfg2.n_layers, cfg2.n_shared) == (5, 12, 2)
    assert cfg2.cap_num == (3, 2, 1, 1, 1) and cfg2.cap_den == 3
    assert W2["router_w"].shape == (5, cfg.d_model)
    assert np.array_equal(W2["router_w"][:3], W["router_w"])
    assert np.array_equal(W2["router_w"][3], W["router_w"][2])
    assert W2["shared"] is W["shared"] and W2["first"] is W["first"]
    assert np.array_equal(W2["router_b"], np.zeros(5, np.float32))
    cfg3, W3 = mor.extend_recursions(cfg, W, extra=1, cap_num=(0,), router_w=np.ones(cfg.d_model),
                                     router_b=[0.5])
    assert cfg3.cap_num == (3, 2, 1, 0) and W3["router_b"][3] == np.float32(0.5)
    assert np.array_equal(W3["router_w"][3], np.ones(cfg.d_model, np.float32))


@pytest.mark.parametrize("kw", [dict(extra=0), dict(extra=6), dict(extra=1, cap_num=(1, 1))])
def test_extend_rejects_bad_arguments(kw):
    mor = _mor()
    cfg = workload.get_config("small_f32")
    with pytest.raises(ValueError):
        mor.extend_recursions(cfg, workload.make_weights(cfg), **kw)


@pytest.mark.parametrize("scheme,L", [("sequence", 9), ("middle_sequence", 8)])
def test_extend_rejects_sequence_type_sharing(scheme, L):
    """Under the sequence schemes a deeper unrolling would move blocks to other layers."""
    mor = _mor()
    cfg = workload.get_config("small_f32", sharing=scheme, n_layers=L)
    with pytest.raises(ValueError):
        mor.extend_recursions(cfg, workload.make_weights(cfg))


def test_extended_model_keeps_the_trained_recursions():
    """With the same weights, routers and capacities, the first N_r recursions of the extended
    model are exactly those of the trained depth (expert choice looks only at earlier states);
    the extra recursion then refines a subset of the last set."""
    mor = _mor()
    cfg = workload.get_config("small_f32", batch=2, seq=61)
    W = workload.make_weights(cfg)
    H0 = workload.make_inputs(cfg)
    base = oracle.prefill(cfg, W, H0)
    cfg2, W2 = mor.extend_recursions(cfg, W)
    ext = oracle.prefill(cfg2, W2, H0)
    for pb, pe in zip(base["per_seq"], ext["per_seq"]):
        for r in range(cfg.n_rec):
            assert np.array_equal(pb["sel"][r], pe["sel"][r])
        for r in range(cfg.n_rec + 1):
            assert np.array_equal(pb["hist"][r], pe["hist"][r])
        assert set(pe["sel"][cfg.n_rec]) <= set(pe["sel"][cfg.n_rec - 1])
        assert len(pe["sel"][cfg.n_rec]) == len(pe["sel"][cfg.n_rec - 1])   # cap repeated
    assert not np.allclose(base["out"], ext["out"])


def test_extended_full_capacity_is_the_deeper_unrolled_stack():
    """Full capacity and unit gating: N_r + 1 recursions of the trained pool equal the plain Llama
    stack of the deeper Middle-Cycle unrolling (transformers, float64)."""
    mor = _mor()
    cfg = workload.get_config("small_f32", gate_mode="unit", cap_num=(3, 3, 3), batch=1, seq=23)
    W = workload.make_weights(cfg)
    cfg2, W2 = mor.extend_recursions(cfg, W)
    H0 = workload.make_inputs(cfg2)
    res = oracle.prefill(cfg2, W2, H0)
    layers = [W["first"]] + W["shared"] + [W["last"]]
    ref = llama_stack(cfg2, layers, oracle.layer_map(cfg2.n_layers, cfg2.n_rec), H0)
    assert np.allclose(res["out"], ref, rtol=1e-6, atol=1e-7)
