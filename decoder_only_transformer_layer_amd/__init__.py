"""Python binding of libgptfwd (nanochat GPT forward + next-token loss on MI355X / gfx950).

Argument marshalling only: every step of the forward pass runs in the HIP kernels of
``libgptfwd.so`` behind the C ABI of ``include/gptfwd.h`` and ``include/gptfwd_ops.h``.  The
functions below carry the C names and take either integers (device addresses) or torch
tensors, whose ``data_ptr()`` is passed through.  PyTorch supplies device memory and the
stream (``torch.cuda.current_stream()`` unless one is given); nothing is computed in Python.

If the shared library is missing, every entry point raises ``RuntimeError``: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Any, Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptfwd.so")

GPT_OK, GPT_E_INVALID_ARG, GPT_E_UNSUPPORTED, GPT_E_WORKSPACE, GPT_E_HIP, GPT_E_DEVICE_INPUT = 0, -1, -2, -3, -4, -5
GPT_F32, GPT_BF16 = 0, 1
GPT_NOALLOC_MAX_BYTES = 64 << 20  # the fixed workspace array of gpt_fwd_loss_noalloc
(GPT_KERNEL_QKV, GPT_KERNEL_ATTENTION, GPT_KERNEL_ATTN_OUT, GPT_KERNEL_MLP_UP, GPT_KERNEL_MLP_DOWN,
 GPT_KERNEL_LM_HEAD) = 1, 2, 3, 4, 5, 6

EXPORTED = [
    "gpt_validate", "gpt_workspace_bytes", "gpt_fwd_loss", "gpt_fwd_loss_timed", "gpt_fwd_loss_nested",
    "gpt_device_status", "gpt_status_string", "gpt_fwd_loss_noalloc",
    "gpt_kv_cache_bytes", "gpt_decode_workspace_bytes", "gpt_decode_step", "gpt_sample",
    "gpt_prefill_workspace_bytes", "gpt_prefill",
    "gpt_op_embed_norm", "gpt_op_mix_norm", "gpt_op_rope_table", "gpt_op_qk_rope_norm",
    "gpt_op_linear", "gpt_op_qkv", "gpt_op_attention", "gpt_op_lm_head_ce_workspace",
    "gpt_op_lm_head_ce",
]


class gpt_cfg(ctypes.Structure):
    _fields_ = [
        ("n_layer", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_head", ctypes.c_int32),
        ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("mlp_dim", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("window", ctypes.POINTER(ctypes.c_int32)),
        ("softcap", ctypes.c_float), ("rope_base", ctypes.c_float), ("attn_scale", ctypes.c_float),
        ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("has_ve", ctypes.POINTER(ctypes.c_uint8)), ("looped", ctypes.c_int32),
        ("nested_c1", ctypes.c_int32),
    ]


class gpt_weights(ctypes.Structure):
    _fields_ = [
        ("wte", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
        ("resid_lambda", ctypes.c_void_p), ("x0_lambda", ctypes.c_void_p),
        ("wq", ctypes.POINTER(ctypes.c_void_p)), ("wk", ctypes.POINTER(ctypes.c_void_p)),
        ("wv", ctypes.POINTER(ctypes.c_void_p)), ("wo", ctypes.POINTER(ctypes.c_void_p)),
        ("w1", ctypes.POINTER(ctypes.c_void_p)), ("w2", ctypes.POINTER(ctypes.c_void_p)),
        ("ve", ctypes.POINTER(ctypes.c_void_p)), ("ve_gate", ctypes.POINTER(ctypes.c_void_p)),
        ("pass_emb", ctypes.c_void_p), ("gate_logit", ctypes.c_void_p),
    ]


class gpt_launch_timing(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("capacity", ctypes.c_int32),
        ("begin", ctypes.POINTER(ctypes.c_void_p)), ("end", ctypes.POINTER(ctypes.c_void_p)),
        ("recorded", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libgptfwd.so not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sig = {
        "gpt_validate": (I, [ctypes.POINTER(gpt_cfg)]),
        "gpt_workspace_bytes": (S, [ctypes.POINTER(gpt_cfg)]),
        "gpt_fwd_loss": (I, [ctypes.POINTER(gpt_cfg), ctypes.POINTER(gpt_weights), P, P, P, P, P, P, S, P]),
        "gpt_fwd_loss_timed": (I, [ctypes.POINTER(gpt_cfg), ctypes.POINTER(gpt_weights), P, P, P, P, P, P, S, P,
                                   ctypes.POINTER(gpt_launch_timing)]),
        "gpt_fwd_loss_nested": (I, [ctypes.POINTER(gpt_cfg), ctypes.POINTER(gpt_weights), P, P, P, P, P, P, P, P,
                                    P, S, P, ctypes.POINTER(gpt_launch_timing)]),
        "gpt_device_status": (I, [P, P]),
        "gpt_fwd_loss_noalloc": (I, [ctypes.POINTER(gpt_cfg), ctypes.POINTER(gpt_weights), P, P, P, P, P, P]),
        "gpt_kv_cache_bytes": (S, [ctypes.POINTER(gpt_cfg)]),
        "gpt_decode_workspace_bytes": (S, [ctypes.POINTER(gpt_cfg)]),
        "gpt_decode_step": (I, [ctypes.POINTER(gpt_cfg), ctypes.POINTER(gpt_weights), P, P, P, P, P, S, P]),
        "gpt_sample": (I, [P, I, I, I, F, P, P, P]),
        "gpt_prefill_workspace_bytes": (S, [ctypes.POINTER(gpt_cfg)]),
        "gpt_prefill": (I, [ctypes.POINTER(gpt_cfg), ctypes.POINTER(gpt_weights), P, I, P, P, P, P, S, P]),
        "gpt_status_string": (ctypes.c_char_p, [I]),
        "gpt_op_embed_norm": (I, [I, P, P, P, P, P, P, P, I, I, I, F, P, P]),
        "gpt_op_mix_norm": (I, [I, P, P, P, P, I, I, P, I, I, F, P]),
        "gpt_op_rope_table": (I, [P, I, I, F, P]),
        "gpt_op_qk_rope_norm": (I, [I, P, I, P, I, I, I, I, F, P]),
        "gpt_op_linear": (I, [I, I, P, P, I, I, I, P, P]),
        "gpt_op_qkv": (I, [P, P, P, P, I, I, I, I, I, I, P, F, P, P, P]),
        "gpt_op_attention": (I, [I, P, P, P, I, I, I, I, I, I, F, P]),
        "gpt_op_lm_head_ce_workspace": (S, [I, I, I]),
        "gpt_op_lm_head_ce": (I, [I, P, P, P, P, I, I, I, F, P, P, P, P, S, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(x: Any) -> Optional[int]:
    """Device address of a torch tensor, or an int / None passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _require(t: Any, name: str, dtype: str, numel: int, optional: bool = True) -> None:
    """Marshalling check of a tensor handed to the library by the DeviceModel / Decoder methods:
    a torch tensor on a GPU with the given dtype ("int32" or "float32"), contiguous, holding
    `numel` elements (the C functions read or write exactly that many).  None passes when
    `optional`; an int is taken as a raw device address and passes unchecked."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: required")
    if isinstance(t, int):
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor or a device address, got {type(t).__name__}")
    if t.dtype != getattr(torch, dtype):
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")


def _stream(stream: Any) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class GptError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gpt_status_string(status)} ({status})")


def _check(status: int, where: str) -> int:
    if status != GPT_OK:
        raise GptError(status, where)
    return status


# ----------------------------------------------------------------------------- configuration

def layer_windows(pattern: str, short_window: int, seq_len: int, n_layer: int) -> List[int]:
    """Per-layer window sizes: the short/long pattern tiled over the layers ("S" = short
    window, "L" = seq_len), the last layer forced long ("The Mathematics of Karpathy's
    nanochat", section "Sliding Window Pattern")."""
    sizes = {"S": short_window, "L": seq_len}
    w = [sizes[pattern[l % len(pattern)]] for l in range(n_layer)]
    w[-1] = seq_len
    return w


def ve_layers(n_layer: int) -> List[int]:
    """Layers that mix a value embedding into v: every other layer, the last one always
    ("The Mathematics of Karpathy's nanochat", section "Value Embeddings (ResFormer)")."""
    return [1 if l % 2 == (n_layer - 1) % 2 else 0 for l in range(n_layer)]


def make_cfg(p: Any, batch: Optional[int] = None, windows: Optional[Sequence[int]] = None) -> gpt_cfg:
    """gpt_cfg from any object with the preset attribute names (n_layer, d_model, ...); a
    true ``value_embeds`` attribute selects value embeddings on the ve_layers() layers.

    The window and has_ve arrays are kept alive on the returned structure."""
    if windows is None:
        windows = layer_windows(p.window_pattern, p.short_window, p.seq_len, p.n_layer)
    win = (ctypes.c_int32 * p.n_layer)(*[int(w) for w in windows])
    ve = (ctypes.c_uint8 * p.n_layer)(*ve_layers(p.n_layer)) if getattr(p, "value_embeds", False) else None
    c = gpt_cfg(p.n_layer, p.d_model, p.n_head, p.n_kv_head, p.head_dim, p.mlp_dim, p.vocab,
                p.seq_len, p.batch if batch is None else batch,
                ctypes.cast(win, ctypes.POINTER(ctypes.c_int32)),
                p.softcap, p.rope_base, p.attn_scale, p.norm_eps,
                GPT_BF16 if p.dtype == "bf16" else GPT_F32,
                None if ve is None else ctypes.cast(ve, ctypes.POINTER(ctypes.c_uint8)),
                1 if getattr(p, "looped", False) else 0, int(getattr(p, "nested_c1", 0) or 0))
    c._win, c._ve = win, ve
    return c


# ----------------------------------------------------------------------------- C entry points

def gpt_status_string(status: int) -> str:
    return _load().gpt_status_string(status).decode()


def gpt_validate(cfg: gpt_cfg) -> int:
    return _load().gpt_validate(ctypes.byref(cfg))


def gpt_workspace_bytes(cfg: gpt_cfg) -> int:
    return _load().gpt_workspace_bytes(ctypes.byref(cfg))


def gpt_fwd_loss(cfg: gpt_cfg, weights: gpt_weights, tokens, targets, loss, mean_loss, logits,
                 workspace, workspace_bytes: int, stream=None) -> int:
    return _load().gpt_fwd_loss(ctypes.byref(cfg), ctypes.byref(weights), _ptr(tokens), _ptr(targets),
                                _ptr(loss), _ptr(mean_loss), _ptr(logits), _ptr(workspace),
                                workspace_bytes, _stream(stream))


def gpt_fwd_loss_timed(cfg: gpt_cfg, weights: gpt_weights, tokens, targets, loss, mean_loss, logits,
                       workspace, workspace_bytes: int, stream, timing: Optional[gpt_launch_timing]) -> int:
    return _load().gpt_fwd_loss_timed(ctypes.byref(cfg), ctypes.byref(weights), _ptr(tokens), _ptr(targets),
                                      _ptr(loss), _ptr(mean_loss), _ptr(logits), _ptr(workspace),
                                      workspace_bytes, _stream(stream),
                                      None if timing is None else ctypes.byref(timing))


def gpt_fwd_loss_nested(cfg: gpt_cfg, weights: gpt_weights, tokens, targets, loss, mean_loss, logits,
                        loss_k1, mean_k1, logits_k1, workspace, workspace_bytes: int, stream=None,
                        timing: Optional[gpt_launch_timing] = None) -> int:
    return _load().gpt_fwd_loss_nested(ctypes.byref(cfg), ctypes.byref(weights), _ptr(tokens), _ptr(targets),
                                       _ptr(loss), _ptr(mean_loss), _ptr(logits), _ptr(loss_k1),
                                       _ptr(mean_k1), _ptr(logits_k1), _ptr(workspace), workspace_bytes,
                                       _stream(stream), None if timing is None else ctypes.byref(timing))


def gpt_fwd_loss_noalloc(cfg: gpt_cfg, weights: gpt_weights, tokens, targets, loss, mean_loss, logits,
                         stream=None) -> int:
    return _load().gpt_fwd_loss_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _ptr(tokens), _ptr(targets),
                                        _ptr(loss), _ptr(mean_loss), _ptr(logits), _stream(stream))


def launch_timing(kind: int, begin_events, end_events) -> gpt_launch_timing:
    """A gpt_launch_timing over torch.cuda.Event pairs (each recorded once beforehand, so that the
    underlying hipEvent_t exists)."""
    n = len(begin_events)
    b = (ctypes.c_void_p * n)(*[e.cuda_event for e in begin_events])
    e = (ctypes.c_void_p * n)(*[e.cuda_event for e in end_events])
    t = gpt_launch_timing(kind, n, ctypes.cast(b, ctypes.POINTER(ctypes.c_void_p)),
                          ctypes.cast(e, ctypes.POINTER(ctypes.c_void_p)), 0)
    t._keep = (b, e)  # the arrays must outlive the call
    return t


def gpt_kv_cache_bytes(cfg: gpt_cfg) -> int:
    return _load().gpt_kv_cache_bytes(ctypes.byref(cfg))


def gpt_decode_workspace_bytes(cfg: gpt_cfg) -> int:
    return _load().gpt_decode_workspace_bytes(ctypes.byref(cfg))


def gpt_decode_step(cfg: gpt_cfg, weights: gpt_weights, tokens, pos, kv_cache, logits, workspace,
                    workspace_bytes: int, stream=None) -> int:
    return _load().gpt_decode_step(ctypes.byref(cfg), ctypes.byref(weights), _ptr(tokens), _ptr(pos),
                                   _ptr(kv_cache), _ptr(logits), _ptr(workspace), workspace_bytes,
                                   _stream(stream))


def gpt_prefill_workspace_bytes(cfg: gpt_cfg) -> int:
    return _load().gpt_prefill_workspace_bytes(ctypes.byref(cfg))


def gpt_prefill(cfg: gpt_cfg, weights: gpt_weights, tokens, prompt_len: int, lens, kv_cache, logits,
                workspace, workspace_bytes: int, stream=None) -> int:
    return _load().gpt_prefill(ctypes.byref(cfg), ctypes.byref(weights), _ptr(tokens), prompt_len, _ptr(lens),
                               _ptr(kv_cache), _ptr(logits), _ptr(workspace), workspace_bytes, _stream(stream))


def gpt_sample(logits, batch: int, vocab: int, top_k: int, temperature: float, u, out, stream=None) -> int:
    return _load().gpt_sample(_ptr(logits), batch, vocab, top_k, temperature, _ptr(u), _ptr(out),
                              _stream(stream))


def gpt_device_status(workspace, stream=None) -> int:
    return _load().gpt_device_status(_ptr(workspace), _stream(stream))


def gpt_op_embed_norm(dtype, tokens, wte, lam, mu, x0, x, xn, M, C, V, eps, flags, stream=None) -> int:
    return _load().gpt_op_embed_norm(dtype, _ptr(tokens), _ptr(wte), _ptr(lam), _ptr(mu), _ptr(x0),
                                     _ptr(x), _ptr(xn), M, C, V, eps, _ptr(flags), _stream(stream))


def gpt_op_mix_norm(dtype, x, x0, lam, mu, layer, mix, xn, M, C, eps, stream=None) -> int:
    return _load().gpt_op_mix_norm(dtype, _ptr(x), _ptr(x0), _ptr(lam), _ptr(mu), layer, int(mix),
                                   _ptr(xn), M, C, eps, _stream(stream))


def gpt_op_rope_table(cs, T, D, base, stream=None) -> int:
    return _load().gpt_op_rope_table(_ptr(cs), T, D, base, _stream(stream))


def gpt_op_qk_rope_norm(dtype, qk, ld, cs, M, T, nheads, D, eps, stream=None) -> int:
    return _load().gpt_op_qk_rope_norm(dtype, _ptr(qk), ld, _ptr(cs), M, T, nheads, D, eps, _stream(stream))


def gpt_op_linear(dtype, epi, a, w, M, N, K, out, stream=None) -> int:
    return _load().gpt_op_linear(dtype, epi, _ptr(a), _ptr(w), M, N, K, _ptr(out), _stream(stream))


def gpt_op_qkv(xn, wq, wk, wv, B, T, C, H, Hkv, D, cs, eps, qk, vt, stream=None) -> int:
    return _load().gpt_op_qkv(_ptr(xn), _ptr(wq), _ptr(wk), _ptr(wv), B, T, C, H, Hkv, D, _ptr(cs), eps,
                              _ptr(qk), _ptr(vt), _stream(stream))


def gpt_op_attention(dtype, qk, vt, o, B, T, H, Hkv, D, window, scale, stream=None) -> int:
    return _load().gpt_op_attention(dtype, _ptr(qk), _ptr(vt), _ptr(o), B, T, H, Hkv, D, window, scale,
                                    _stream(stream))


def gpt_op_lm_head_ce_workspace(dtype, M, V) -> int:
    return _load().gpt_op_lm_head_ce_workspace(dtype, M, V)


def gpt_op_lm_head_ce(dtype, xf, wu, targets, tokens, M, C, V, cap, loss, mean, logits, workspace,
                      workspace_bytes, stream=None) -> int:
    return _load().gpt_op_lm_head_ce(dtype, _ptr(xf), _ptr(wu), _ptr(targets), _ptr(tokens), M, C, V, cap,
                                     _ptr(loss), _ptr(mean), _ptr(logits), _ptr(workspace),
                                     workspace_bytes, _stream(stream))


# ----------------------------------------------------------------------------- device model

def to_device(a: np.ndarray, dtype: str, device: str = "cuda"):
    """Upload a host array: bf16 given as uint16 bit patterns, or float32."""
    import torch
    if dtype == "bf16":
        a = np.ascontiguousarray(a, dtype=np.uint16)
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class DeviceModel:
    """Device-resident weights of one configuration plus the structures gpt_fwd_loss needs.

    ``weights`` is any object with attributes wte, lm_head, resid_lambda, x0_lambda and
    per-layer lists wq, wk, wv, wo, w1, w2 (numpy arrays: uint16 bf16 bits or float32), plus
    per-layer ve and ve_gate lists when the configuration has value embeddings, and
    pass_emb ([2, C]) and gate_logit ([L] float32) for the looped trunk.  For a nested
    configuration each per-layer linear is its two row blocks [block1, block2]; they are
    uploaded back to back into one buffer, the storage gpt_weights documents.
    """

    def __init__(self, p: Any, weights: Any, batch: Optional[int] = None, device: str = "cuda",
                 windows: Optional[Sequence[int]] = None):
        import torch
        self.p = p
        self.batch = p.batch if batch is None else batch
        self.cfg = make_cfg(p, self.batch, windows)
        st = gpt_validate(self.cfg)
        _check(st, "gpt_validate")
        dt = p.dtype
        self.t: Dict[str, Any] = {
            "wte": to_device(weights.wte, dt, device),
            "lm_head": to_device(weights.lm_head, dt, device),
            "resid_lambda": torch.from_numpy(np.asarray(weights.resid_lambda, np.float32)).to(device),
            "x0_lambda": torch.from_numpy(np.asarray(weights.x0_lambda, np.float32)).to(device),
        }
        arrs = {}
        nested = bool(getattr(p, "nested_c1", 0))
        for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
            mats = getattr(weights, n)
            if nested:
                mats = [np.concatenate([np.ravel(b) for b in blocks]) for blocks in mats]
            self.t[n] = [to_device(m, dt, device) for m in mats]
            arrs[n] = (ctypes.c_void_p * p.n_layer)(*[m.data_ptr() for m in self.t[n]])
        ve_ptr = gate_ptr = None
        if getattr(p, "value_embeds", False):
            sel = ve_layers(p.n_layer)   # upload only the tables the selected layers read
            self.t["ve"] = [to_device(m, dt, device) if s else None for m, s in zip(weights.ve, sel)]
            self.t["ve_gate"] = [to_device(m, dt, device) if s else None for m, s in zip(weights.ve_gate, sel)]
            for n in ("ve", "ve_gate"):
                arrs[n] = (ctypes.c_void_p * p.n_layer)(*[m.data_ptr() if m is not None else None
                                                         for m in self.t[n]])
            ve_ptr = ctypes.cast(arrs["ve"], ctypes.POINTER(ctypes.c_void_p))
            gate_ptr = ctypes.cast(arrs["ve_gate"], ctypes.POINTER(ctypes.c_void_p))
        pe_ptr = gl_ptr = None
        if getattr(p, "looped", False):
            self.t["pass_emb"] = to_device(weights.pass_emb, dt, device)
            self.t["gate_logit"] = torch.from_numpy(np.asarray(weights.gate_logit, np.float32)).to(device)
            pe_ptr, gl_ptr = self.t["pass_emb"].data_ptr(), self.t["gate_logit"].data_ptr()
        self._arrs = arrs
        self.w = gpt_weights(self.t["wte"].data_ptr(), self.t["lm_head"].data_ptr(),
                             self.t["resid_lambda"].data_ptr(), self.t["x0_lambda"].data_ptr(),
                             *[ctypes.cast(arrs[n], ctypes.POINTER(ctypes.c_void_p))
                               for n in ("wq", "wk", "wv", "wo", "w1", "w2")], ve_ptr, gate_ptr,
                             pe_ptr, gl_ptr)
        self.ws_bytes = gpt_workspace_bytes(self.cfg)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        off = (-self.ws.data_ptr()) % 256
        self.ws_ptr = self.ws.data_ptr() + off

    def forward(self, tokens, targets=None, loss=None, mean=None, logits=None, stream=None,
                timing: Optional[gpt_launch_timing] = None) -> int:
        """Enqueue gpt_fwd_loss (gpt_fwd_loss_timed if `timing` is given) on device tensors
        (outputs preallocated by the caller): tokens, targets int32 [B, T]; loss fp32 [B, T];
        mean fp32 [1]; logits fp32 [B, T, V]."""
        self._check_io(tokens, targets, loss, mean, logits)
        if timing is not None:
            return gpt_fwd_loss_timed(self.cfg, self.w, tokens, targets, loss, mean, logits,
                                      self.ws_ptr, self.ws_bytes, stream, timing)
        return gpt_fwd_loss(self.cfg, self.w, tokens, targets, loss, mean, logits, self.ws_ptr,
                            self.ws_bytes, stream)

    def forward_noalloc(self, tokens, targets=None, loss=None, mean=None, logits=None, stream=None) -> int:
        """gpt_fwd_loss_noalloc on device tensors (as forward): the library's fixed workspace
        array instead of this model's."""
        self._check_io(tokens, targets, loss, mean, logits)
        return gpt_fwd_loss_noalloc(self.cfg, self.w, tokens, targets, loss, mean, logits, stream)

    def forward_nested(self, tokens, targets=None, loss=None, mean=None, logits=None, loss_k1=None,
                       mean_k1=None, logits_k1=None, stream=None,
                       timing: Optional[gpt_launch_timing] = None) -> int:
        """Enqueue gpt_fwd_loss_nested (full model and kfront=1 outputs from one pass); the _k1
        outputs have the shapes of their full-model counterparts."""
        self._check_io(tokens, targets, loss, mean, logits)
        self._check_io(tokens, targets, loss_k1, mean_k1, logits_k1)
        return gpt_fwd_loss_nested(self.cfg, self.w, tokens, targets, loss, mean, logits, loss_k1,
                                   mean_k1, logits_k1, self.ws_ptr, self.ws_bytes, stream, timing)

    def _check_io(self, tokens, targets, loss, mean, logits) -> None:
        n = self.batch * self.p.seq_len
        _require(tokens, "tokens", "int32", n, optional=False)
        _require(targets, "targets", "int32", n)
        _require(loss, "loss", "float32", n)
        _require(mean, "mean", "float32", 1)
        _require(logits, "logits", "float32", n * self.p.vocab)

    def call_nested(self, tokens, targets=None, want_logits: bool = False):
        """Allocate outputs, run gpt_fwd_loss_nested, and return a dict with loss, mean, logits
        and loss_k1, mean_k1, logits_k1 (None where not computed)."""
        import torch
        B, T, V = self.batch, self.p.seq_len, self.p.vocab
        dev = tokens.device
        out = {}
        for sfx in ("", "_k1"):
            out["loss" + sfx] = torch.empty((B, T), dtype=torch.float32, device=dev) if targets is not None else None
            out["mean" + sfx] = torch.empty(1, dtype=torch.float32, device=dev) if targets is not None else None
            out["logits" + sfx] = torch.empty((B, T, V), dtype=torch.float32, device=dev) if want_logits else None
        _check(self.forward_nested(tokens, targets, out["loss"], out["mean"], out["logits"], out["loss_k1"],
                                   out["mean_k1"], out["logits_k1"]), "gpt_fwd_loss_nested")
        return out

    def __call__(self, tokens, targets=None, want_logits: bool = False):
        """Allocate outputs, run, and return (loss [B,T], mean [1], logits or None)."""
        import torch
        B, T, V = self.batch, self.p.seq_len, self.p.vocab
        dev = tokens.device
        loss = torch.empty((B, T), dtype=torch.float32, device=dev) if targets is not None else None
        mean = torch.empty(1, dtype=torch.float32, device=dev) if targets is not None else None
        logits = torch.empty((B, T, V), dtype=torch.float32, device=dev) if want_logits else None
        _check(self.forward(tokens, targets, loss, mean, logits), "gpt_fwd_loss")
        return loss, mean, logits

    def device_status(self) -> int:
        return gpt_device_status(self.ws_ptr)


class Decoder:
    """Decode-step state over the weights of a DeviceModel: a KV cache for `batch` rows of up to
    the preset's seq_len positions and the step's workspace (both device buffers owned here).
    Every call only enqueues work on the current (or given) stream."""

    def __init__(self, model: DeviceModel):
        import torch
        self.m = model
        self.cfg = model.cfg
        _check(gpt_validate(self.cfg), "gpt_validate")
        self.cache_bytes = gpt_kv_cache_bytes(self.cfg)
        self.ws_bytes = gpt_decode_workspace_bytes(self.cfg)
        if self.cache_bytes == 0 or self.ws_bytes == 0:
            raise GptError(GPT_E_UNSUPPORTED, "decode configuration")
        dev = model.ws.device
        self.cache = torch.empty(self.cache_bytes + 256, dtype=torch.uint8, device=dev)
        self.cache_ptr = self.cache.data_ptr() + (-self.cache.data_ptr()) % 256
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=dev)
        self.ws_ptr = self.ws.data_ptr() + (-self.ws.data_ptr()) % 256

    def step(self, tokens, pos, logits, stream=None) -> int:
        """Enqueue gpt_decode_step: tokens, pos device int32 [B]; logits device fp32 [B, V]."""
        B = self.m.batch
        _require(tokens, "tokens", "int32", B, optional=False)
        _require(pos, "pos", "int32", B, optional=False)
        _require(logits, "logits", "float32", B * self.m.p.vocab, optional=False)
        return gpt_decode_step(self.cfg, self.m.w, tokens, pos, self.cache_ptr, logits, self.ws_ptr,
                               self.ws_bytes, stream)

    def prefill(self, tokens, prompt_len: int, logits, lens=None, stream=None) -> int:
        """Enqueue gpt_prefill on tokens [B, prompt_len] (device int32, contiguous); the forward
        uses the DeviceModel's workspace."""
        B = self.m.batch
        _require(tokens, "tokens", "int32", B * prompt_len, optional=False)
        _require(logits, "logits", "float32", B * self.m.p.vocab, optional=False)
        _require(lens, "lens", "int32", B)
        need = gpt_prefill_workspace_bytes(self.cfg)
        if self.m.ws_bytes < need:
            raise GptError(GPT_E_WORKSPACE, "prefill workspace")
        return gpt_prefill(self.cfg, self.m.w, tokens, prompt_len, lens, self.cache_ptr, logits,
                           self.m.ws_ptr, self.m.ws_bytes, stream)

    def device_status(self) -> int:
        return gpt_device_status(self.ws_ptr)
