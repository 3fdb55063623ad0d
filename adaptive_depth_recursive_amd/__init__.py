"""Python binding of libmor.so, the MI355X Mixture-of-Recursions library (include/mor.h).

Argument marshalling only: every step of the forward pass runs in the HIP kernels behind the
C ABI. PyTorch provides device memory and the stream. Importing this module does not load the
library; the first call does, and fails loudly if it has not been built
(``python -m adaptive_depth_recursive_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmor.so")

MOR_MAX_REC = 8
MOR_OK, MOR_E_INVALID, MOR_E_SHAPE, MOR_E_WORKSPACE = 0, -1, -2, -3
MOR_E_KV_FULL, MOR_E_HIP, MOR_E_STATE = -4, -5, -6
MOR_F32, MOR_BF16 = 0, 1
ROUTING = {"ec": 0, "tc": 1, "threshold": 2}
KV_MODE = {"recursion": 0, "share": 1}
GATE_MODE = {"router": 0, "unit": 1}
SHARING = {"middle_cycle": 0, "middle_sequence": 1, "cycle": 2, "sequence": 3}
DTYPE = {"f32": MOR_F32, "bf16": MOR_BF16}


class MorError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mor status {status}: {msg}")
        self.status = status


class mor_config(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("n_layers", ctypes.c_int32), ("n_rec", ctypes.c_int32),
        ("cap_num", ctypes.c_int32 * MOR_MAX_REC), ("cap_den", ctypes.c_int32),
        ("routing", ctypes.c_int32), ("kv_mode", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("max_batch", ctypes.c_int32), ("max_seq", ctypes.c_int32),
        ("max_slots", ctypes.c_int32), ("kv_page_tokens", ctypes.c_int32),
        ("kv_pages", ctypes.c_int32), ("max_requests", ctypes.c_int32),
        ("sharing", ctypes.c_int32),
    ]


class mor_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")]


class mor_weights(ctypes.Structure):
    _fields_ = [("first", mor_block_weights), ("last", mor_block_weights),
                ("shared", ctypes.POINTER(mor_block_weights)),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmor.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m adaptive_depth_recursive_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.mor_abi_version.restype = i32
        L.mor_last_error.restype = ctypes.c_char_p
        L.mor_workspace_bytes.restype = sz
        L.mor_workspace_bytes.argtypes = [ctypes.POINTER(mor_config)]
        L.mor_init.restype = i32
        L.mor_init.argtypes = [ctypes.POINTER(mor_config), ctypes.POINTER(mor_weights), vp, sz,
                               vp, ctypes.POINTER(vp)]
        L.mor_prefill.restype = i32
        L.mor_prefill.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]
        L.mor_route.restype = i32
        L.mor_route.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
        L.mor_route_noalloc.restype = i32
        L.mor_route_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
        L.mor_kv_view.restype = i32
        L.mor_kv_view.argtypes = [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                  ctypes.POINTER(i32)]
        L.mor_get_error_flags.restype = i32
        L.mor_get_error_flags.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.mor_timing_enable.restype = i32
        L.mor_timing_enable.argtypes = [vp, i32, i32]
        L.mor_timing_read.restype = i32
        L.mor_timing_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
        L.mor_timing_clock.restype = i32
        L.mor_timing_clock.argtypes = [vp, ctypes.POINTER(ctypes.c_double)]
        L.mor_decode_submit.restype = i32
        L.mor_decode_submit.argtypes = [vp, i32, ctypes.POINTER(i32), vp, vp, vp, vp, vp, vp]
        L.mor_decode_continue.restype = i32
        L.mor_decode_continue.argtypes = [vp, i32, ctypes.POINTER(i32), vp, vp, vp, vp, vp, vp]
        L.mor_decode_step.restype = i32
        L.mor_decode_step.argtypes = [vp, i32, vp, ctypes.POINTER(i32)]
        L.mor_decode_stats.restype = i32
        L.mor_decode_stats.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int64)]
        L.mor_destroy.restype = None
        L.mor_destroy.argtypes = [vp]
        _lib = L
    return _lib


EXPORTED = ("mor_abi_version", "mor_last_error", "mor_workspace_bytes", "mor_init",
            "mor_prefill", "mor_route", "mor_route_noalloc", "mor_kv_view", "mor_get_error_flags", "mor_timing_enable",
            "mor_timing_read", "mor_timing_clock", "mor_decode_submit", "mor_decode_continue", "mor_decode_step", "mor_decode_stats",
            "mor_destroy")
KERNEL_KINDS = {"qkv": 1, "attention": 2, "o_proj": 3, "gate_up": 4, "down": 5, "router": 6,
                "select": 7, "gather": 8, "scatter": 9, "rmsnorm": 10}


def _check(status: int):
    if status != MOR_OK:
        raise MorError(status, lib().mor_last_error().decode())


def make_config(cfg, max_batch: Optional[int] = None, max_seq: Optional[int] = None,
                max_slots: int = 0, kv_page_tokens: int = 64, kv_pages: int = 0,
                max_requests: int = 1) -> mor_config:
    """A mor_config from any object with the workload configuration's attribute names.
    max_slots > 0 plans the depth-wise batched decode engine (threshold routing only)."""
    c = mor_config()
    c.d_model, c.n_q_heads, c.n_kv_heads = cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads
    c.head_dim, c.d_ff, c.n_layers, c.n_rec = cfg.head_dim, cfg.d_ff, cfg.n_layers, cfg.n_rec
    for i, v in enumerate(cfg.cap_num):
        c.cap_num[i] = int(v)
    c.cap_den = cfg.cap_den
    c.routing, c.kv_mode = ROUTING[cfg.routing], KV_MODE[cfg.kv_mode]
    c.gate_mode, c.dtype = GATE_MODE[cfg.gate_mode], DTYPE[cfg.dtype]
    c.rms_eps, c.rope_theta = cfg.rms_eps, cfg.rope_theta
    c.max_batch = cfg.batch if max_batch is None else max_batch
    c.max_seq = cfg.seq if max_seq is None else max_seq
    c.max_slots, c.kv_page_tokens = max_slots, kv_page_tokens
    c.kv_pages, c.max_requests = kv_pages, max_requests
    c.sharing = SHARING[getattr(cfg, "sharing", "middle_cycle")]
    return c


def extend_recursions(cfg, weights: Dict, extra: int = 1, cap_num=None, router_w=None,
                      router_b=None):
    """Test-time recursion scaling (MoR's depth is a runtime parameter: the same shared blocks can
    be unrolled further at inference, without retraining).

    Returns (cfg', weights') that run N_r + extra recursions over the same pool of n_s shared
    blocks: n_rec and n_layers grow by `extra` spans of n_s layers. Only the cycle-type schemes
    (middle_cycle, cycle) keep every block's place when the depth grows, so only they are
    accepted. The extra steps' capacities (numerators over cap_den) default to the last trained
    capacity; their router rows and biases default to the last trained ones.
    cfg must be a dataclass with the workload configuration's fields.
    """
    import dataclasses

    import numpy as np
    if extra < 1:
        raise ValueError("extra must be >= 1")
    sharing = getattr(cfg, "sharing", "middle_cycle")
    if sharing not in ("middle_cycle", "cycle"):
        raise ValueError("test-time recursion scaling needs cycle-type sharing")
    R = cfg.n_rec + extra
    if R > MOR_MAX_REC:
        raise ValueError(f"at most {MOR_MAX_REC} recursions")
    n_s = cfg.n_shared
    caps = tuple(cfg.cap_num[:cfg.n_rec]) + (
        tuple(cap_num) if cap_num is not None else (cfg.cap_num[cfg.n_rec - 1],) * extra)
    if len(caps) != R:
        raise ValueError("cap_num must give one capacity per extra recursion")
    L = R * n_s + (2 if sharing == "middle_cycle" else 0)
    cfg2 = dataclasses.replace(cfg, n_rec=R, n_layers=L, cap_num=caps)
    rw = np.asarray(weights["router_w"], np.float32)
    add_w = (np.repeat(rw[-1:], extra, axis=0) if router_w is None
             else np.asarray(router_w, np.float32).reshape(extra, -1))
    w2 = dict(weights)
    w2["router_w"] = np.concatenate([rw, add_w])
    rb = weights.get("router_b")
    if rb is not None or router_b is not None:
        rb = np.zeros(cfg.n_rec, np.float32) if rb is None else np.asarray(rb, np.float32)
        add_b = (np.repeat(rb[-1:], extra) if router_b is None
                 else np.asarray(router_b, np.float32).reshape(extra))
        w2["router_b"] = np.concatenate([rb, add_b])
    return cfg2, w2


def workspace_bytes(c: mor_config) -> int:
    n = lib().mor_workspace_bytes(ctypes.byref(c))
    if n == 0:
        raise MorError(MOR_E_INVALID, lib().mor_last_error().decode())
    return n


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Mor:
    """One initialised library handle with its device weights and workspace (torch tensors).

    weights: {"first": layer, "shared": [layer], "last": layer, "router_w": [N_r][d],
              "router_b": [N_r]} with [out][in] matrices (numpy or torch) and fp32 gains;
              "first"/"last" are None (or absent) under cycle / sequence sharing.
    """

    LAYER_KEYS = (("wq", "wq"), ("wk", "wk"), ("wv", "wv"), ("wo", "wo"), ("w_gate", "wg"),
                  ("w_up", "wu"), ("w_down", "wd"), ("g_attn", "g_attn"), ("g_ffn", "g_ffn"))

    def __init__(self, cfg, weights: Dict, device="cuda", max_batch=None, max_seq=None,
                 stream=None, max_slots=0, kv_page_tokens=64, kv_pages=0, max_requests=1):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.c = make_config(cfg, max_batch, max_seq, max_slots, kv_page_tokens, kv_pages,
                             max_requests)
        wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self._keep: List = []

        def dev(x, dt):
            t = torch.as_tensor(x).to(device=self.device, dtype=dt).contiguous()
            self._keep.append(t)
            return t

        def block(layer):
            bw = mor_block_weights()
            for cname, key in self.LAYER_KEYS:
                dt = torch.float32 if key.startswith("g_") else wdt
                setattr(bw, cname, dev(layer[key], dt).data_ptr())
            return bw

        w = mor_weights()
        if weights.get("first") is not None:        # absent under cycle / sequence sharing
            w.first = block(weights["first"])
        if weights.get("last") is not None:
            w.last = block(weights["last"])
        shared = (mor_block_weights * max(1, len(weights["shared"])))()
        for i, layer in enumerate(weights["shared"]):
            shared[i] = block(layer)
        w.shared = shared
        w.router_w = dev(weights["router_w"], torch.float32).data_ptr()
        rb = weights.get("router_b")
        w.router_b = None if rb is None else dev(rb, torch.float32).data_ptr()
        self.ws_bytes = workspace_bytes(self.c)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(lib().mor_init(ctypes.byref(self.c), ctypes.byref(w), self.workspace.data_ptr(),
                              self.ws_bytes, _stream(stream), ctypes.byref(h)))
        self.handle = h
        self._keep.clear()          # the library copied what it needs into the workspace

    def close(self):
        if getattr(self, "handle", None):
            lib().mor_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls -------------------------------------------------------------------------
    def prefill(self, h_in, h_out=None, sel_pos=None, counts=None, logits=None, h_per_rec=None,
                stream=None):
        """mor_prefill on device tensors; h_in is fp32 [B, T, d]. Returns h_out."""
        import torch
        B, T, d = h_in.shape
        if h_out is None:
            h_out = torch.empty_like(h_in)
        _check(lib().mor_prefill(self.handle, h_in.data_ptr(), B, T, h_out.data_ptr(),
                                 _ptr(sel_pos), _ptr(counts), _ptr(logits), _ptr(h_per_rec),
                                 _stream(stream)))
        return h_out

    def prefill_outputs(self, h_in, debug=True, stream=None):
        """Prefill with every optional output allocated; returns a dict of device tensors."""
        import torch
        B, T, d = h_in.shape
        R = self.cfg.n_rec
        dev = h_in.device
        out = {
            "out": torch.empty_like(h_in),
            "sel_pos": torch.empty((R, B, T), dtype=torch.int32, device=dev),
            "counts": torch.empty((R, B), dtype=torch.int32, device=dev),
            "logits": torch.empty((R, B, T), dtype=torch.float32, device=dev),
            "h_per_rec": torch.empty((R + 1, B, T, d), dtype=torch.float32, device=dev) if debug else None,
        }
        self.prefill(h_in, out["out"], out["sel_pos"], out["counts"], out["logits"],
                     out["h_per_rec"], stream)
        return out

    def route(self, H, active_in, counts_in, r, stream=None):
        """mor_route: returns (active_out [B, T], counts_out [B], z [B, T])."""
        import torch
        B, T, _ = H.shape
        act = torch.empty((B, T), dtype=torch.int32, device=H.device)
        cnt = torch.empty((B,), dtype=torch.int32, device=H.device)
        z = torch.empty((B, T), dtype=torch.float32, device=H.device)
        _check(lib().mor_route(self.handle, H.data_ptr(), active_in.data_ptr(),
                               counts_in.data_ptr(), r, B, T, act.data_ptr(), cnt.data_ptr(),
                               z.data_ptr(), _stream(stream)))
        return act, cnt, z

    def route_noalloc(self, H, active_in, counts_in, r, out=None, stream=None):
        """mor_route_noalloc (scratch in the library's static device array): returns
        (active_out [B, T], counts_out [B], z [B, T]); out may pass those three tensors."""
        import torch
        B, T, _ = H.shape
        if out is None:
            out = (torch.empty((B, T), dtype=torch.int32, device=H.device),
                   torch.empty((B,), dtype=torch.int32, device=H.device),
                   torch.empty((B, T), dtype=torch.float32, device=H.device))
        act, cnt, z = out
        _check(lib().mor_route_noalloc(self.handle, H.data_ptr(), active_in.data_ptr(),
                                       counts_in.data_ptr(), r, B, T, act.data_ptr(),
                                       cnt.data_ptr(), z.data_ptr(), _stream(stream)))
        return act, cnt, z

    def kv_view(self, stream_index: int):
        """(K device pointer, V^T device pointer, kpad) of one layer's cache."""
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        kpad = ctypes.c_int32()
        _check(lib().mor_kv_view(self.handle, stream_index, ctypes.byref(k), ctypes.byref(v),
                                 ctypes.byref(kpad)))
        return k.value, v.value, kpad.value

    def kv_tensors(self, stream_index: int, B: int):
        """K [B, kpad, Hkv, hd] and V^T [B, Hkv, hd, kpad] as views into the workspace."""
        import torch
        k, v, kpad = self.kv_view(stream_index)
        es = 2 if self.cfg.dtype == "bf16" else 4
        dt = torch.bfloat16 if es == 2 else torch.float32
        Hkv, hd = self.cfg.n_kv_heads, self.cfg.head_dim
        base = self.workspace.data_ptr()
        n = B * kpad * Hkv * hd
        kt = self.workspace[k - base:k - base + n * es].view(dt).view(B, kpad, Hkv, hd)
        vt = self.workspace[v - base:v - base + n * es].view(dt).view(B, Hkv, hd, kpad)
        return kt, vt

    # -- depth-wise batched decode ----------------------------------------------------
    def decode_submit(self, lengths, inputs, outputs, exit_depth, h_dump=None, z_dump=None,
                      stream=None):
        """mor_decode_submit: lengths is a host int sequence; inputs/outputs fp32 [tokens, d],
        exit_depth int8 [tokens], optional h_dump [tokens, N_r+1, d] and z_dump [tokens, N_r]
        device tensors (kept alive by this object until the next submit)."""
        import numpy as np
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
        self._dec_keep = (inputs, outputs, exit_depth, h_dump, z_dump)
        _check(lib().mor_decode_submit(
            self.handle, int(lens.size), lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            inputs.data_ptr(), outputs.data_ptr(), exit_depth.data_ptr(), _ptr(h_dump),
            _ptr(z_dump), _stream(stream)))

    def decode_continue(self, lengths, inputs, outputs, exit_depth, h_dump=None, z_dump=None,
                        stream=None):
        """mor_decode_continue: request b continues sequence b of the last prefill."""
        import numpy as np
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
        self._dec_keep = (inputs, outputs, exit_depth, h_dump, z_dump)
        _check(lib().mor_decode_continue(
            self.handle, int(lens.size), lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            inputs.data_ptr(), outputs.data_ptr(), exit_depth.data_ptr(), _ptr(h_dump),
            _ptr(z_dump), _stream(stream)))

    def decode_step(self, n_iters: int, sync: bool = False, stream=None):
        """mor_decode_step: enqueue n_iters iterations; with sync=True returns
        (tokens finished, requests finished, iterations run)."""
        if not sync:
            _check(lib().mor_decode_step(self.handle, n_iters, _stream(stream), None))
            return None
        prog = (ctypes.c_int32 * 3)()
        _check(lib().mor_decode_step(self.handle, n_iters, _stream(stream), prog))
        return prog[0], prog[1], prog[2]

    def decode_stats(self, stream=None) -> Dict[str, int]:
        """mor_decode_stats as a dict (synchronises)."""
        out = (ctypes.c_int64 * 10)()
        _check(lib().mor_decode_stats(self.handle, _stream(stream), out))
        keys = ("tokens", "requests", "admitted", "iterations", "weight_bytes", "kv_read_bytes",
                "kv_write_bytes", "act_bytes", "kv_pages_peak", "page_bytes")
        return dict(zip(keys, (int(v) for v in out)))

    def decode_run(self, total_tokens: int, chunk: int = 32, max_iters: int = 1 << 22, stream=None):
        """Steps until every submitted token is finished; returns the iterations run."""
        it = 0
        while True:
            done, _, iters = self.decode_step(chunk, sync=True, stream=stream)
            it = iters
            if done >= total_tokens or it >= max_iters:
                return it

    def timing_enable(self, kind: str, max_launches: int):
        _check(lib().mor_timing_enable(self.handle, KERNEL_KINDS[kind] if kind else 0, max_launches))

    def timing_read(self):
        """(summed kernel milliseconds, launches) recorded since timing_enable / the last read."""
        ms, n = ctypes.c_double(), ctypes.c_int32()
        _check(lib().mor_timing_read(self.handle, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def timing_clock(self) -> float:
        """Shader clock in GHz over the projection launches recorded since timing_enable (0.0 if
        none were sampled)."""
        ghz = ctypes.c_double()
        _check(lib().mor_timing_clock(self.handle, ctypes.byref(ghz)))
        return ghz.value

    def error_flags(self, stream=None) -> int:
        f = ctypes.c_uint32()
        _check(lib().mor_get_error_flags(self.handle, _stream(stream), ctypes.byref(f)))
        return f.value
