"""Plain CPU oracle of the Mixture-of-Recursions (MoR) forward pass.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP library under ``adaptive_depth_recursive_amd/``.

Sources (cited by page title and section):
  [MoR]   "Mixture-of-Recursions: Learning Dynamic Recursive Depths for Adaptive
          Token-Level Computation", Appendices A.1-A.3, B, D.
  [Notes] "Mixture-of-Recursions: Adaptive Token Depth" reading notes,
          sections 1 (parameter sharing), 2.1 (expert-choice), 2.2 (token-choice),
          3.1 (recursion-wise caching), 3.2 (recursive KV sharing), 4 (serving).
  [Kun]   Mixture-of-Recursions reading notes (latent-reasoning series 02/03),
          paragraph on routing and caching ("路由选择深度，缓存定义可见上下文").

Arithmetic: float64 everywhere. For a bf16 configuration, values are rounded to
bfloat16 (nearest, ties to even) exactly where the library stores them in bf16:
the normalised GEMM inputs, Q/K/V after RoPE, the unnormalised softmax
probabilities before the PV product, the attention output, and the SwiGLU output.
The residual stream is kept in float64 here (the library keeps it in fp32).
Router logits are decisions, so they are computed in fp32 in the one fixed order
documented at ``router_logits_fp32`` (the same order the library uses).

Parity status (pins in tests/test_oracle_pins.py):
  bf16_round: bitwise against torch's float32 -> bfloat16 conversion (random values,
  exact ties on even and odd kept bits, subnormals, the largest finite values,
  infinities, NaN payloads).
  layer_map, capacity_counts, select_topk, attention, block, prefill (expert-choice,
  token-choice, recursion-wise and shared KV, every sharing scheme), threshold_forward,
  decode_sequence, sigmoid: pinned.
  The expert-choice gated update at real gates in (0, 1) and the token-choice update at
  the chosen depth are pinned to a transformers Llama stack run on the routed tokens and
  combined by the update formula as read here (H + g (F(H) - H), F the n_s-layer block,
  one gate per token per recursion). These pins fix the oracle to that reading; the
  reading itself (the pages print g f(H) + H, and the token-choice formula is garbled)
  is a choice, listed with the other readings where the design is documented.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

WAVE = 64  # lanes in the fixed-order router reduction

__all__ = [
    "bf16_round", "layer_map", "recursion_of_layer", "capacity_counts", "rmsnorm",
    "rope", "attention", "block", "router_logits_fp32", "sigmoid", "select_topk",
    "prefill", "threshold_forward", "decode_sequence", "kv_entries", "to_f64_weights",
    "calibrate_threshold_bias", "shared_schedule",
]


# ----------------------------------------------------------------------------- precision
def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value of ``x`` (ties to even), returned as float64.

    The value is first taken to float32, then its low 16 bits are rounded away: adding
    0x7FFF plus the lowest kept bit and truncating rounds to nearest with ties to the even
    neighbour, also for subnormals, and carries into the exponent (the largest finite
    values round up to infinity). A NaN stays a NaN (the carry would turn some NaN
    payloads into an infinity or a zero).
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    with np.errstate(invalid="ignore"):                # signalling-NaN payloads
        r = u.astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    r[nan] = np.nan
    return r


def _store(x: np.ndarray, bf16: bool) -> np.ndarray:
    return bf16_round(x) if bf16 else x


# ----------------------------------------------------------------------------- structure
def layer_map(n_layers: int, n_rec: int, scheme: str = "middle_cycle") -> List[int]:
    """Parameter block used by each unrolled layer l = 0..L-1.

    [Notes] section 1 and [MoR] Appendix A.1:
      cycle:            Phi'_{l mod (L/N_r)}
      sequence:         Phi'_{floor(l / N_r)}
      middle_cycle:     Phi_0 first, Phi'_{((l-1) mod ((L-2)/N_r)) + 1} for l = 1..L-2,
                        a unique last block (index n_s + 1)
      middle_sequence:  Phi_0 first, Phi'_{floor((l-1)/N_r) + 1}, unique last block
    """
    L, R = n_layers, n_rec
    if scheme == "cycle":
        if L % R:
            raise ValueError("cycle sharing needs L divisible by N_r")
        return [l % (L // R) for l in range(L)]
    if scheme == "sequence":
        if L % R:
            raise ValueError("sequence sharing needs L divisible by N_r")
        return [l // R for l in range(L)]
    if (L - 2) % R:
        raise ValueError("middle sharing needs L - 2 divisible by N_r")
    n_s = (L - 2) // R
    if scheme == "middle_cycle":
        mid = [((l - 1) % n_s) + 1 for l in range(1, L - 1)]
    elif scheme == "middle_sequence":
        mid = [((l - 1) // R) + 1 for l in range(1, L - 1)]
    else:
        raise ValueError(scheme)
    return [0] + mid + [n_s + 1]


def recursion_of_layer(n_layers: int, n_rec: int) -> List[int]:
    """Recursion step (1..N_r) of each middle layer under Middle-Cycle; 0 for the unique layers."""
    n_s = (n_layers - 2) // n_rec
    return [0] + [(l - 1) // n_s + 1 for l in range(1, n_layers - 1)] + [0]


def capacity_counts(cap_num: Sequence[int], cap_den: int, T: int) -> List[int]:
    """Tokens kept at each recursion: ceil(cap_r * T), cap_r = cap_num[r]/cap_den.

    [Kun]: at N_r = 3 the recursions process 3/3, 2/3, 1/3 of the original
    sequence; [MoR] Appendix D computes FLOPs from these per-depth lengths.
    Integer ceiling, so no float rounding enters the count.
    """
    return [(int(c) * T + cap_den - 1) // cap_den for c in cap_num]


# ----------------------------------------------------------------------------- block
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Llama RMSNorm ([MoR] Appendix B: Llama-based architecture): x / sqrt(mean(x^2)+eps) * g."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, Llama rotate-half convention, on x [n, heads, hd] at positions pos [n].

    Pair (i, i + hd/2) is rotated by angle pos * theta^(-2i/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, qpos: np.ndarray,
              kpos: np.ndarray, bf16: bool) -> np.ndarray:
    """Causal softmax attention by original position: query t sees key s iff kpos[s] <= qpos[t].

    q [nq, Hq, hd], k/v [nk, Hkv, hd]; query head h reads kv head h // (Hq/Hkv); scale 1/sqrt(hd).
    For bf16 the unnormalised probabilities exp(s - max) are rounded to bf16 before the
    product with V; the normaliser sums the unrounded ones.
    Returns [nq, Hq*hd].
    """
    nq, Hq, hd = q.shape
    if nq == 0:
        return np.zeros((0, Hq * hd))
    Hkv = k.shape[1]
    G = Hq // Hkv
    allowed = np.asarray(kpos)[None, :] <= np.asarray(qpos)[:, None]
    out = np.empty((nq, Hq, hd))
    for h in range(Hq):
        kh = h // G
        s = (q[:, h, :] @ k[:, kh, :].T) / math.sqrt(hd)
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        denom = p.sum(axis=1, keepdims=True)
        out[:, h, :] = (_store(p, bf16) @ v[:, kh, :]) / denom
    return out.reshape(nq, Hq * hd)


def _silu(x):
    return x / (1.0 + np.exp(-x))


def block(W: Dict[str, np.ndarray], X: np.ndarray, pos: np.ndarray, cfg,
          kv_prefix: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None,
          kv_src: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None):
    """One Llama pre-norm decoder layer f(X; Phi) ([Notes] section 1; [MoR] Appendix B).

    X [n, d] float64 (rows ordered by position), pos [n] original positions.
    kv_prefix: cached (k, v, pos) placed before this call's own keys (decode).
    kv_src: attend to these keys instead of computing K/V (recursive KV sharing,
    [Notes] section 3.2). Returns (X_new, (k, v, kpos) of this call's own K/V or None).
    """
    bf = cfg.dtype == "bf16"
    n = X.shape[0]
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    a = _store(rmsnorm(X, W["g_attn"], cfg.rms_eps), bf)
    q = _store(rope((a @ W["wq"].T).reshape(n, Hq, hd), pos, cfg.rope_theta), bf)
    own = None
    if kv_src is None:
        k = _store(rope((a @ W["wk"].T).reshape(n, Hkv, hd), pos, cfg.rope_theta), bf)
        v = _store((a @ W["wv"].T).reshape(n, Hkv, hd), bf)
        own = (k, v, np.asarray(pos))
        if kv_prefix is not None and len(kv_prefix[2]):
            k = np.concatenate([kv_prefix[0], k])
            v = np.concatenate([kv_prefix[1], v])
            kpos = np.concatenate([kv_prefix[2], pos])
        else:
            kpos = np.asarray(pos)
    else:
        k, v, kpos = kv_src
    o = _store(attention(q, k, v, pos, kpos, bf), bf)
    X = X + o @ W["wo"].T
    b = _store(rmsnorm(X, W["g_ffn"], cfg.rms_eps), bf)
    h = _store(_silu(b @ W["wg"].T) * (b @ W["wu"].T), bf)
    X = X + h @ W["wd"].T
    return X, own


# ----------------------------------------------------------------------------- routing
def router_logits_fp32(H: np.ndarray, w: np.ndarray, bias: Optional[float] = None) -> np.ndarray:
    """Router logit z_t = w . H_t in fp32, in one fixed order ([Notes] 2.1: g = G(theta_r^T H)).

    Order: H_t is taken to fp32. Lane l of a 64-lane group keeps p_l = 0 and, for the
    d-indices i = l, l+64, l+128, ... ascending, sets p_l = fl(p_l + fl(H_t[i] * w[i]))
    (product and sum rounded separately). The 64 partials are then folded pairwise:
    for o = 32, 16, 8, 4, 2, 1: p_l = fl(p_l + p_{l+o}) for l < o. z = p_0, then
    z = fl(z + bias) when a bias is given. -0.0 is returned as +0.0.
    """
    x = np.asarray(H, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    w32 = np.asarray(w, dtype=np.float32)
    n, d = x.shape
    dp = -(-d // WAVE) * WAVE
    xp = np.zeros((n, dp), np.float32)
    xp[:, :d] = x
    wp = np.zeros(dp, np.float32)
    wp[:d] = w32
    p = np.zeros((n, WAVE), np.float32)
    for m in range(dp // WAVE):
        p = p + xp[:, m * WAVE:(m + 1) * WAVE] * wp[m * WAVE:(m + 1) * WAVE]
    o = WAVE // 2
    while o:
        p = p[:, :o] + p[:, o:2 * o]
        o //= 2
    z = p[:, 0].copy()
    if bias is not None:
        z = z + np.float32(bias)
    z[z == 0] = np.float32(0.0)
    return z


def sigmoid(z) -> np.ndarray:
    """Router gate G = sigmoid ([Notes] 2.1), in float64."""
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def select_topk(active_pos: np.ndarray, z: np.ndarray, k: int) -> np.ndarray:
    """Expert-choice top-k over the active set ([Notes] 2.1; hierarchical filtering).

    Ranks tokens by logit descending, equal logits by lower position first, keeps the
    first k and returns their positions in ascending order.
    """
    active_pos = np.asarray(active_pos)
    zz = np.asarray(z, np.float64)
    if np.isnan(zz).any():
        raise ValueError("NaN router logit")
    order = np.lexsort((active_pos, -zz))
    return np.sort(active_pos[order[:k]])


# ----------------------------------------------------------------------------- forward
def to_f64_weights(weights: dict) -> dict:
    def lay(L):
        return None if L is None else {k: np.asarray(v, np.float64) for k, v in L.items()}
    return {"first": lay(weights.get("first")), "shared": [lay(s) for s in weights["shared"]],
            "last": lay(weights.get("last")),
            "router_w": np.asarray(weights["router_w"], np.float32),
            "router_b": np.asarray(weights.get("router_b", np.zeros(len(weights["router_w"]))),
                                   np.float32)}


def _softmax(z):
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def shared_schedule(cfg) -> List[List[int]]:
    """Index into the shared pool of the layer at (recursion r, position j), as [r-1][j-1].

    The routed recursions are consecutive spans of n_s unrolled layers (after the unique
    first layer under Middle-* sharing); the layer-to-block map of the sharing scheme
    ([Notes] section 1, [MoR] Appendix A.1, see layer_map) decides which block each
    unrolled layer of a span uses. Under Cycle and Middle-Cycle position j always uses
    block j; under Sequence and Middle-Sequence consecutive layers repeat a block N_r times.
    """
    scheme = getattr(cfg, "sharing", "middle_cycle")
    R, L = cfg.n_rec, cfg.n_layers
    lm = layer_map(L, R, scheme)
    middle = scheme.startswith("middle")
    mid = lm[1:-1] if middle else lm
    n_s = len(mid) // R
    base = 1 if middle else 0                       # layer_map numbers the pool from 1 under Middle-*
    return [[mid[(r - 1) * n_s + (j - 1)] - base for j in range(1, n_s + 1)]
            for r in range(1, R + 1)]


def _prefill_one(cfg, W, h0, ks, forced, gate_mode, update):
    T = h0.shape[0]
    pos_all = np.arange(T)
    sched = shared_schedule(cfg)
    R, n_s = cfg.n_rec, len(sched[0])
    middle = getattr(cfg, "sharing", "middle_cycle").startswith("middle")
    if middle:
        H, kv_first = block(W["first"], h0, pos_all, cfg)
    else:                                           # Cycle / Sequence: no unique entry layer
        H, kv_first = np.array(h0, np.float64), None
    hist = [H.copy()]
    kv = {"first": kv_first}
    rec1 = {}
    active = pos_all
    sel_list, own_list, z_list, g_list = [], [], [], []
    if cfg.routing == "tc":
        # [Notes] 2.2: g_t = softmax(Theta^T H^1_t) once, depth i = argmax_j g_jt.
        Z = np.stack([router_logits_fp32(H, W["router_w"][j]) for j in range(R)], axis=1)
        depth = np.argmax(Z, axis=1) + 1            # argmax returns the lowest index on ties
        probs = _softmax(Z.astype(np.float64))
        z_list = [Z]
        own_depth = depth.copy()
        if forced is not None:                      # teacher forcing: depth = last set holding t
            depth = np.zeros(T, np.int64)
            for r in range(1, R + 1):
                depth[np.asarray(forced[r - 1], np.int64)] = r
    for r in range(1, R + 1):
        if cfg.routing == "ec":
            z = router_logits_fp32(H[active], W["router_w"][r - 1])
            own = select_topk(active, z, ks[r - 1])
            sel = own if forced is None else np.asarray(forced[r - 1])
            g = sigmoid(z[np.searchsorted(active, sel)])
            z_list.append((active.copy(), z))
            own_list.append(own)
        elif cfg.routing == "threshold":
            z = router_logits_fp32(H[active], W["router_w"][r - 1], W["router_b"][r - 1])
            keep = np.ones(len(active), bool) if r == 1 else (z > 0)
            own = active[keep]
            sel = own if forced is None else np.asarray(forced[r - 1])
            g = sigmoid(z[np.searchsorted(active, sel)])
            z_list.append((active.copy(), z))
            own_list.append(own)
        elif cfg.routing == "tc":
            own_list.append(pos_all[own_depth >= r])
            sel = pos_all[depth >= r]
            g = np.where(depth[sel] == r, probs[sel, r - 1], 1.0)
        else:
            raise ValueError(cfg.routing)
        X = H[sel]
        for j in range(1, n_s + 1):
            Wj = W["shared"][sched[r - 1][j - 1]]
            if cfg.kv_mode == "share" and r >= 2:
                # recursive KV sharing reuses the recursion-1 keys of the same position j
                X, _ = block(Wj, X, sel, cfg, kv_src=rec1[j])
            else:
                X, kvj = block(Wj, X, sel, cfg)
                kv[(r, j)] = kvj
                if r == 1:
                    rec1[j] = kvj
        Hs = H[sel]
        if gate_mode == "unit":
            H[sel] = X
        elif cfg.routing == "tc":
            # Reading of the token-choice update: plain recursion before the chosen
            # depth, gated delta at the chosen depth (pinned to a Llama stack combined
            # by this rule; the rule itself is the reading).
            last = depth[sel] == r
            Hn = X.copy()
            Hn[last] = Hs[last] + g[last, None] * (X[last] - Hs[last])
            H[sel] = Hn
        elif update == "delta":
            # Reading of the gated update ([Notes] 2.1): H + g * (f(H) - H), f the n_s-layer block.
            H[sel] = Hs + g[:, None] * (X - Hs)
        elif update == "literal":
            H[sel] = g[:, None] * X + Hs
        else:
            raise ValueError(update)
        hist.append(H.copy())
        sel_list.append(np.asarray(sel))
        g_list.append(g)
        active = np.asarray(sel)
    if middle:
        out, kv_last = block(W["last"], H, pos_all, cfg)
    else:                                           # Cycle / Sequence: no unique exit layer
        out, kv_last = H.copy(), None
    kv["last"] = kv_last
    res = {"out": out, "sel": sel_list, "own_sel": own_list, "z": z_list, "gate": g_list,
           "hist": hist, "kv": kv}
    if cfg.routing == "tc":
        res["depth"] = depth
        res["own_depth"] = own_depth
    return res


def prefill(cfg, weights, H0: np.ndarray, forced_sel=None, gate_mode: Optional[str] = None,
            update: str = "delta", keep_kv: bool = False) -> dict:
    """MoR prefill over a batch, one sequence at a time (sequences are independent).

    [Notes] sections 1 and 2.1, [MoR] Appendix A: the configured sharing scheme's unrolling
    (Middle-Cycle by default; see shared_schedule); at recursion r
    the router scores the tokens active at r-1, keeps ceil(cap_r * T) of them (expert
    choice), runs the n_s shared layers on them with attention restricted to tokens
    active at r (recursion-wise caching, [Notes] 3.1) or to the recursion-1 keys
    (recursive KV sharing, [Notes] 3.2), and merges the result with the gate.

    forced_sel: optional [N_r][B] position arrays to use instead of the oracle's own
    selection (teacher forcing, any routing mode); the oracle's own choice is still
    returned in "own_sel" ("own_depth" for token choice).
    Returns a dict of per-sequence lists plus "out" [B, T, d].
    """
    W = to_f64_weights(weights)
    B, T, _ = H0.shape
    ks = capacity_counts(cfg.cap_num, cfg.cap_den, T)
    gm = gate_mode or cfg.gate_mode
    per = []
    for b in range(B):
        fb = None if forced_sel is None else [forced_sel[r][b] for r in range(cfg.n_rec)]
        rb = _prefill_one(cfg, W, np.asarray(H0[b], np.float64), ks, fb, gm, update)
        if not keep_kv:
            rb.pop("kv")
        per.append(rb)
    out = np.stack([p["out"] for p in per])
    return {"out": out, "per_seq": per, "counts": ks}


def threshold_forward(cfg, weights, h0: np.ndarray, gate_mode: Optional[str] = None) -> dict:
    """One-shot forward of one sequence with the static-threshold router ([Notes] 2.1).

    Recursion 1 runs every token; at r >= 2 a token continues iff
    z^r = theta_r . H^r + b_r > 0 (equivalently sigmoid > 0.5).
    """
    assert cfg.routing == "threshold"
    W = to_f64_weights(weights)
    res = _prefill_one(cfg, W, np.asarray(h0, np.float64), None, None,
                       gate_mode or cfg.gate_mode, "delta")
    depth = np.zeros(h0.shape[0], np.int32)
    for r, sel in enumerate(res["sel"], start=1):
        depth[sel] = r
    res["depth"] = depth
    return res


def decode_sequence(cfg, weights, inputs: np.ndarray, gate_mode: Optional[str] = None) -> dict:
    """Token-by-token decode of one sequence with per-recursion KV caches.

    [Notes] 3.1 (recursion-wise caching) and 4 (depth-wise serving): token p runs the
    first layer against the first-layer cache, recursion 1, then recursion r >= 2 only
    while theta_r . H + b_r > 0, each recursion-r layer attending to the cache of that
    (r, layer) (or to the recursion-1 cache under KV sharing), then the last layer.
    Returns outputs [n, d] and exit depths [n].
    """
    if getattr(cfg, "sharing", "middle_cycle") != "middle_cycle":
        raise ValueError("depth-wise decode is defined for Middle-Cycle sharing")
    W = to_f64_weights(weights)
    gm = gate_mode or cfg.gate_mode
    R, d = cfg.n_rec, cfg.d_model
    n_s = len(shared_schedule(cfg)[0])
    Hkv, hd = cfg.n_kv_heads, cfg.head_dim

    def empty():
        return (np.zeros((0, Hkv, hd)), np.zeros((0, Hkv, hd)), np.zeros(0, np.int64))

    def append(c, kv):
        return (np.concatenate([c[0], kv[0]]), np.concatenate([c[1], kv[1]]),
                np.concatenate([c[2], kv[2]]))

    cache = {"first": empty(), "last": empty()}
    for r in range(1, R + 1):
        for j in range(1, n_s + 1):
            cache[(r, j)] = empty()
    n = inputs.shape[0]
    outs = np.empty((n, d))
    depth = np.zeros(n, np.int32)
    for p in range(n):
        pos = np.array([p])
        x, kv = block(W["first"], np.asarray(inputs[p:p + 1], np.float64), pos, cfg,
                      kv_prefix=cache["first"])
        cache["first"] = append(cache["first"], kv)
        for r in range(1, R + 1):
            z = router_logits_fp32(x, W["router_w"][r - 1], W["router_b"][r - 1])[0]
            if r >= 2 and not z > 0:
                break
            g = float(sigmoid(z))
            X = x
            for j in range(1, n_s + 1):
                if cfg.kv_mode == "share" and r >= 2:
                    X, _ = block(W["shared"][j - 1], X, pos, cfg, kv_src=cache[(1, j)])
                else:
                    X, kv = block(W["shared"][j - 1], X, pos, cfg, kv_prefix=cache[(r, j)])
                    cache[(r, j)] = append(cache[(r, j)], kv)
            x = X if gm == "unit" else x + g * (X - x)
            depth[p] = r
        o, kv = block(W["last"], x, pos, cfg, kv_prefix=cache["last"])
        cache["last"] = append(cache["last"], kv)
        outs[p] = o[0]
    return {"out": outs, "depth": depth, "cache": cache}


def calibrate_threshold_bias(cfg, weights, H: np.ndarray) -> np.ndarray:
    """Router biases b_r under which the static-threshold router keeps the configured capacities.

    The pages' inference router continues a token to recursion r iff sigmoid(theta_r . H + b_r)
    exceeds 0.5 ([Notes] 2.1), with a router trained so that the kept fractions follow the
    capacities (3/3, 2/3, 1/3 of the sequence at N_r = 3; [Kun]). Without trained weights the
    bias stands in for that training: b_1 = 0 (recursion 1 runs every token), and for r >= 2,
    with b_2..b_{r-1} already fixed, b_r is minus the (1 - cap_r/cap_{r-1}) quantile of the
    unbiased logits theta_r . H^{r-1} over the tokens active at r-1 of the calibration batch
    H [B, T, d], so that a fraction cap_r/cap_{r-1} of them continue.
    Returns float32 [N_r].
    """
    assert cfg.routing == "threshold"
    R = cfg.n_rec
    b = np.zeros(R, np.float32)
    for r in range(2, R + 1):
        trial = dict(weights)
        bb = b.copy()
        bb[r - 1:] = np.float32(1e30)          # keep every token open from recursion r on
        trial["router_b"] = bb
        res = prefill(cfg.replace(seq=H.shape[1]), trial, H)
        zs = []
        for p in res["per_seq"]:
            active = p["sel"][r - 2]
            zs.append(router_logits_fp32(p["hist"][r - 1][active], weights["router_w"][r - 1]))
        z = np.concatenate(zs).astype(np.float64)
        q = cfg.cap_num[r - 1] / cfg.cap_num[r - 2]
        b[r - 1] = np.float32(-np.quantile(z, 1.0 - q))
    return b


def kv_entries(kv: dict, n_shared: int) -> Tuple[int, int]:
    """(entries in the shared-layer caches, entries in the unique-layer caches), per sequence."""
    shared = sum(len(v[2]) for k, v in kv.items() if isinstance(k, tuple))
    unique = sum(len(kv[k][2]) for k in ("first", "last") if k in kv)
    return shared, unique
