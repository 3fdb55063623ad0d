"""Seeded synthetic workloads for the Mixture-of-Recursions (MoR) forward pass.

This module only draws numbers and names shapes. It holds none of the
method's arithmetic (no capacities, no routing, no layer maps): the oracle
under ``oracle/`` and the HIP library each compute those on their own. Both
sides receive the same arrays from here.

Shapes follow the SmolLM-based Llama configurations the MoR paper trains on
(MoR paper, Appendix B "Model architecture details": vocabulary 49K, max
length 2K) and the Middle-Cycle depth padding of Appendix D ("135M model with
30 layers ... results in a total of 32 layers"). Trained weights and the
FineWeb-Edu corpus are not available, so every tensor is drawn from a seeded
NumPy PCG64 generator:

  seed 0  weights ~ N(0, 0.02^2); RMSNorm gains = 1; EC routers ~ N(0, 0.02^2);
          token-choice routers ~ N(0, (2/sqrt(d))^2) so logits have std ~2
  seed 1  prefill inputs H0 ~ N(0, 1), [B, T, d]
  seed 2  decode request lengths ~ Geometric(p = 1/256) (mean 256), capped at 2048
  seed 3  decode per-position input hidden states ~ N(0, 1)
  seed 4  calibration batch (decode router biases)

Draw order within seed 0: first layer, shared layers 1..n_s, last layer; inside
a layer Wq, Wk, Wv, Wo, Wg, Wu, Wd; then the router. Every weight matrix is
stored [out][in] (so y = x @ W.T). bf16 configurations round every drawn
weight and input to bfloat16 (round to nearest even); routers stay fp32.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

WEIGHT_STD = 0.02
SEED_WEIGHTS, SEED_INPUTS, SEED_LENGTHS, SEED_DECODE_INPUTS, SEED_CALIB = 0, 1, 2, 3, 4
LAYER_TENSORS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


@dataclass(frozen=True)
class MorConfig:
    name: str
    dtype: str                 # "f32" or "bf16"
    batch: int
    seq: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    n_layers: int              # L, unrolled depth including the two unique layers
    n_rec: int                 # N_r
    cap_num: Tuple[int, ...]   # capacity of recursion r is cap_num[r-1] / cap_den
    cap_den: int
    routing: str = "ec"        # "ec" | "tc" | "threshold"
    kv_mode: str = "recursion" # "recursion" | "share"
    gate_mode: str = "router"  # "router" | "unit"
    sharing: str = "middle_cycle"  # "middle_cycle" | "middle_sequence" | "cycle" | "sequence"
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    # decode-only fields
    slots: int = 0
    n_requests: int = 0
    mean_len: int = 0
    max_len: int = 0

    def replace(self, **kw) -> "MorConfig":
        return dataclasses.replace(self, **kw)

    @property
    def middle(self) -> bool:
        """Middle-* sharing: unique first and last layers around the recursions."""
        return self.sharing.startswith("middle")

    @property
    def n_shared(self) -> int:
        """Layers per recursion (= size of the shared block pool)."""
        return ((self.n_layers - 2) if self.middle else self.n_layers) // self.n_rec


def _c(name, **kw) -> MorConfig:
    return MorConfig(name=name, **kw)


_SMOL360 = dict(d_model=960, n_q_heads=15, n_kv_heads=5, head_dim=64, d_ff=2560)
_SMOL135 = dict(d_model=576, n_q_heads=9, n_kv_heads=3, head_dim=64, d_ff=1536)

CONFIGS: Dict[str, MorConfig] = {
    # Tiny fp32 prefill: 2 x 128, d 64, 4 MHA heads of 16, FFN 256, L = 5 (1 shared layer x 3).
    "tiny_f32": _c("tiny_f32", dtype="f32", batch=2, seq=128, d_model=64, n_q_heads=4,
                   n_kv_heads=4, head_dim=16, d_ff=256, n_layers=5, n_rec=3,
                   cap_num=(3, 2, 1), cap_den=3),
    # 135M-shape bf16 prefill: 8 x 2048, 32 layers (10 shared x 3 + 2).
    "smol135m_bf16": _c("smol135m_bf16", dtype="bf16", batch=8, seq=2048, n_layers=32, n_rec=3,
                        cap_num=(3, 2, 1), cap_den=3, **_SMOL135),
    # 360M-shape bf16 prefill: the headline workload.
    "smol360m_bf16": _c("smol360m_bf16", dtype="bf16", batch=8, seq=2048, n_layers=32, n_rec=3,
                        cap_num=(3, 2, 1), cap_den=3, **_SMOL360),
    # 360M-shape variants: token-choice routing, and recursive KV sharing.
    "smol360m_tc_bf16": _c("smol360m_tc_bf16", dtype="bf16", batch=8, seq=2048, n_layers=32,
                           n_rec=3, cap_num=(3, 2, 1), cap_den=3, routing="tc", **_SMOL360),
    "smol360m_share_bf16": _c("smol360m_share_bf16", dtype="bf16", batch=8, seq=2048,
                              n_layers=32, n_rec=3, cap_num=(3, 2, 1), cap_den=3,
                              kv_mode="share", **_SMOL360),
    # 360M-shape MoR-4 decode: 7 shared layers x 4 + 2 = 30, threshold exit, 51 slots.
    "smol360m_mor4_decode": _c("smol360m_mor4_decode", dtype="bf16", batch=51, seq=2048,
                               n_layers=30, n_rec=4, cap_num=(4, 3, 2, 1), cap_den=4,
                               routing="threshold", slots=51, n_requests=1024, mean_len=256,
                               max_len=2048, **_SMOL360),
    # Small parity configurations: several GEMM/attention tiles and ragged tails, seconds on CPU.
    "small_f32": _c("small_f32", dtype="f32", batch=3, seq=157, d_model=128, n_q_heads=4,
                    n_kv_heads=2, head_dim=32, d_ff=192, n_layers=8, n_rec=3,
                    cap_num=(3, 2, 1), cap_den=3),
    "small_bf16": _c("small_bf16", dtype="bf16", batch=3, seq=333, d_model=192, n_q_heads=6,
                     n_kv_heads=2, head_dim=64, d_ff=512, n_layers=8, n_rec=3,
                     cap_num=(3, 2, 1), cap_den=3),
    "small_tc_bf16": _c("small_tc_bf16", dtype="bf16", batch=3, seq=333, d_model=192,
                        n_q_heads=6, n_kv_heads=2, head_dim=64, d_ff=512, n_layers=8, n_rec=3,
                        cap_num=(3, 2, 1), cap_den=3, routing="tc"),
    "small_share_bf16": _c("small_share_bf16", dtype="bf16", batch=3, seq=333, d_model=192,
                           n_q_heads=6, n_kv_heads=2, head_dim=64, d_ff=512, n_layers=8,
                           n_rec=3, cap_num=(3, 2, 1), cap_den=3, kv_mode="share"),
    "small_thr_bf16": _c("small_thr_bf16", dtype="bf16", batch=3, seq=200, d_model=192,
                         n_q_heads=6, n_kv_heads=2, head_dim=64, d_ff=512, n_layers=10,
                         n_rec=4, cap_num=(4, 3, 2, 1), cap_den=4, routing="threshold",
                         slots=5, n_requests=12, mean_len=24, max_len=64),
}


def get_config(name: str, **overrides) -> MorConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


# ----------------------------------------------------------------------------- drawing
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Used only to quantise freshly drawn inputs; inputs are finite by construction.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x = x64.astype(np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def layer_shapes(cfg: MorConfig) -> Dict[str, Tuple[int, int]]:
    d, hd = cfg.d_model, cfg.head_dim
    return {
        "wq": (cfg.n_q_heads * hd, d),
        "wk": (cfg.n_kv_heads * hd, d),
        "wv": (cfg.n_kv_heads * hd, d),
        "wo": (d, cfg.n_q_heads * hd),
        "wg": (cfg.d_ff, d),
        "wu": (cfg.d_ff, d),
        "wd": (d, cfg.d_ff),
    }


def make_weights(cfg: MorConfig, seed: int = SEED_WEIGHTS) -> Dict[str, object]:
    """Draw all weights. Returns {"first": layer, "shared": [layer]*n_s, "last": layer,
    "router_w": [N_r][d] float32, "router_b": [N_r] float32}; a layer is a dict of
    [out][in] float32 arrays plus "g_attn"/"g_ffn" gains (ones). Under Cycle and Sequence
    sharing there are no unique layers: "first" and "last" are None and are not drawn."""
    span = cfg.n_layers - 2 if cfg.middle else cfg.n_layers
    if cfg.sharing not in ("middle_cycle", "middle_sequence", "cycle", "sequence"):
        raise ValueError(cfg.sharing)
    if span % cfg.n_rec != 0 or span < cfg.n_rec:
        raise ValueError("the shared span of layers must be a positive multiple of n_rec")
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = layer_shapes(cfg)

    def draw_layer():
        lay = {k: _store(rng.standard_normal(shapes[k]) * WEIGHT_STD, cfg.dtype)
               for k in LAYER_TENSORS}
        lay["g_attn"] = np.ones(cfg.d_model, np.float32)
        lay["g_ffn"] = np.ones(cfg.d_model, np.float32)
        return lay

    first = draw_layer() if cfg.middle else None
    shared = [draw_layer() for _ in range(cfg.n_shared)]
    last = draw_layer() if cfg.middle else None
    if cfg.routing == "tc":
        std = 2.0 / np.sqrt(cfg.d_model)
    else:
        std = WEIGHT_STD
    router_w = (rng.standard_normal((cfg.n_rec, cfg.d_model)) * std).astype(np.float32)
    router_b = np.zeros(cfg.n_rec, np.float32)
    return {"first": first, "shared": shared, "last": last,
            "router_w": router_w, "router_b": router_b}


def make_inputs(cfg: MorConfig, seed: int = SEED_INPUTS, batch: Optional[int] = None,
                seq: Optional[int] = None) -> np.ndarray:
    """Prefill input hidden states H0 ~ N(0,1), float32 [B, T, d] (bf16 values for bf16)."""
    B = cfg.batch if batch is None else batch
    T = cfg.seq if seq is None else seq
    rng = np.random.Generator(np.random.PCG64(seed))
    return _store(rng.standard_normal((B, T, cfg.d_model)), cfg.dtype)


def make_decode_lengths(cfg: MorConfig, seed: int = SEED_LENGTHS,
                        n: Optional[int] = None) -> np.ndarray:
    """Generated lengths ~ Geometric(p = 1/mean_len) (support >= 1), capped at max_len."""
    n = cfg.n_requests if n is None else n
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.geometric(1.0 / cfg.mean_len, size=n)
    return np.minimum(lens, cfg.max_len).astype(np.int32)


def make_decode_inputs(cfg: MorConfig, lengths: np.ndarray,
                       seed: int = SEED_DECODE_INPUTS) -> List[np.ndarray]:
    """Per-request input hidden states ~ N(0,1): list of float32 [len_i, d], drawn in request order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [_store(rng.standard_normal((int(n), cfg.d_model)), cfg.dtype) for n in lengths]


def make_calibration_inputs(cfg: MorConfig, batch: int, seq: int,
                            seed: int = SEED_CALIB) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return _store(rng.standard_normal((batch, seq, cfg.d_model)), cfg.dtype)
