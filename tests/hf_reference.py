"""An independent Llama stack from the `transformers` library, used to pin the oracle's block.

The stack is transformers' own LlamaModel (eager attention, float64, CPU) with its final
norm removed; each unrolled layer is loaded with the weights of the parameter block the
given layer map assigns to it. Nothing here is shared with the oracle or the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch


def llama_stack(cfg, layers, block_ids, H0: np.ndarray, position_ids=None) -> np.ndarray:
    """Run H0 [B, n, d] through the stack. position_ids [n] (optional, ascending) gives the rows'
    rotary positions; attention stays causal over the row order, which for ascending positions
    is causal by position restricted to the given rows."""
    from transformers import LlamaConfig, LlamaModel

    hf = LlamaConfig(hidden_size=cfg.d_model, intermediate_size=cfg.d_ff,
                     num_attention_heads=cfg.n_q_heads, num_key_value_heads=cfg.n_kv_heads,
                     head_dim=cfg.head_dim, rms_norm_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
                     num_hidden_layers=len(block_ids), vocab_size=8,
                     max_position_embeddings=max(4096, H0.shape[1] + 1 + (0 if position_ids is None else int(np.max(position_ids)))),
                     attention_bias=False, mlp_bias=False)
    hf._attn_implementation = "eager"
    model = LlamaModel(hf).double().eval()
    model.norm = torch.nn.Identity()
    names = {"wq": "self_attn.q_proj.weight", "wk": "self_attn.k_proj.weight",
             "wv": "self_attn.v_proj.weight", "wo": "self_attn.o_proj.weight",
             "wg": "mlp.gate_proj.weight", "wu": "mlp.up_proj.weight",
             "wd": "mlp.down_proj.weight", "g_attn": "input_layernorm.weight",
             "g_ffn": "post_attention_layernorm.weight"}
    with torch.no_grad():
        for li, bid in enumerate(block_ids):
            params = dict(model.layers[li].named_parameters())
            for k, n in names.items():
                params[n].copy_(torch.from_numpy(np.asarray(layers[bid][k], np.float64)))
        x = torch.from_numpy(np.asarray(H0, np.float64))
        pid, mask = None, None
        if position_ids is not None:
            pid = torch.as_tensor(np.asarray(position_ids, np.int64))[None].expand(x.shape[0], -1)
            # an explicit causal mask: gaps in position_ids would otherwise be taken as the
            # boundaries of packed sequences
            n = x.shape[1]
            keep = torch.tril(torch.ones(n, n, dtype=torch.bool))
            mask = torch.zeros(n, n, dtype=torch.float64).masked_fill(~keep, float("-inf"))
            mask = mask[None, None].expand(x.shape[0], 1, n, n)
        out = model(inputs_embeds=x, position_ids=pid, attention_mask=mask,
                    use_cache=False).last_hidden_state
    return out.numpy()
