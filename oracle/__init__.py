"""Reference oracle for the nanochat GPT forward pass with next-token loss.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct CPU
implementation of what the forward+loss path computes, written from the pages'
equations in NumPy, in float64 by default.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library never calls it and shares no code with it; both
sides only consume the seeded inputs of ``gptdata``.

Sources (cited by page title and section):
  [M]  "The Mathematics of Karpathy's nanochat" -- sections "High-Level Forward
       Pass", "RMS Normalization", "Rotary Position Embeddings (RoPE)",
       "Causal Self-Attention", "QK-Norm with Sharpening", "Scaled Dot-Product
       Attention with Sliding Window", "Feed-Forward Network (MLP)", "Residual
       Stream with Learnable Scalars", "Value Embeddings (ResFormer)", "Logit
       Softcap", "Cross-Entropy Loss", "Pseudocode: One Training Step".
  [R]  "Reading nanochat Source: From Configuration to a Training Step" --
       sections 2 (shifted targets), 5.2-5.4 (attention order, block, LM head).
  [S]  "nanochat depth sweep" -- section "Architecture" (SSSL windows, last
       block full context, x0 re-injection, +-15 softcap).
  [L]  "looped-nanochat-d24" -- section "What is the routing loop?" (two-pass
       trunk, attention-logit prior from pass 1, softplus gate, pass
       embeddings).
  [F]  "Fully Nested Transformers" -- the StairFormer description: block lower
       triangular weights, PrefixRMSNorm, per-block heads, kfront submodel
       forward, prefix cross-entropy.
  [M]  also section "Inference: Generating Text" (the autoregressive loop) and
       its "Sampling Controls" (temperature, top-k filtering, greedy at 0).

Readings where the pages are silent or disagree (each frozen as a config field
so the oracle and the GPU path cannot silently diverge):
  * attention logit = attn_scale * <q_hat, k_hat> with q_hat = RMSNorm(RoPE(q));
    attn_scale defaults to 1/sqrt(head_dim).  [M] instead multiplies q and k
    by 1.15 with no 1/sqrt(d) ("QK-Norm with Sharpening"); that reading is
    attn_scale = 1.15**2 and needs no code change.
  * RMSNorm(u) = u / sqrt(mean(u^2) + eps) with eps = cfg.norm_eps (1e-6):
    [M] "RMS Normalization" defines it without eps and remarks that the
    library call adds 1e-6.  Every norm (embedding, pre-attention, pre-MLP,
    QK-norm, final) uses the same eps.
  * window w counts visible keys including the query itself: key j is visible
    from query i iff j <= i and i - j < w; w >= T is plain causal attention.
  * SSSL pattern: layer l (0-based) takes pattern[l mod len(pattern)], and the
    last layer is always long (w = T).  Short window = cfg.short_window.
  * RoPE positions are 0..T-1 within each packed row; no document masking.
  * GQA head map: query head h reads KV head floor(h * Hkv / H).
  * ignored targets (-1) contribute a per-token loss of 0 and are excluded
    from the mean; with no valid target the mean is NaN.
  * looped two-pass trunk (when cfg.looped): pass p (0, 1) starts from
    RMSNorm(W_E[t] + pass_emb[p]); pass-2 layer l takes the prior of pass-1
    layer l (identity routing), shares that layer's window mask and scale,
    and the loss comes from pass 2 only.
  * nested model (cfg.nested_c1 > 0, two blocks): the residual splits into
    dims [0, c1) and [c1, C); every other dimension (q/k/v heads, MLP hidden)
    splits in the same proportion; every per-layer linear is block lower
    triangular, stored as its row blocks [out_1, in_1] and [out_2, in_1+in_2];
    every RMSNorm is the PrefixRMSNorm (block-1 coordinates over the RMS of
    dims [0, c1), block-2 coordinates over the RMS of all dims); the lm_head is
    shared, kfront=1 reading input columns [0, c1).  No value embeddings.
  * sampling: the logits sampled from are the softcapped ones (the page's
    worked example samples "logits (after softcapping)"); top-k keeps every
    token whose logit is >= the k-th largest (ties at the threshold stay, as
    the page's masking of values below the k-th one does); a draw with
    temperature > 0 is the inverse CDF of the kept tokens' softmax(z / tau)
    in vocabulary order at a uniform u in [0, 1) supplied by the caller (the
    page's multinomial draw with its random number made an input); temperature
    0 is the argmax, the first index among equal maxima.
  * value embeddings (when cfg.value_embeds): the gate reads the first 12
    channels of the attention block's normalised input x_tilde (the input of
    the Q/K/V projections), and the mixed value v + g * e is what attention
    averages; layers follow the pages' selection rule (has_ve).

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` to something other than itself (worked examples
printed on the pages, closed forms, invariants, library routines or brute
force); none is parity unpinned.
"""
from __future__ import annotations

import math
from typing import Any, Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "rms_norm", "rope_angles", "apply_rope", "layer_windows", "visible_mask",
    "attention", "linear", "relu_squared", "softcap", "token_losses",
    "mean_loss", "has_ve", "value_embed_mix", "softplus", "attention_with_prior", "block",
    "forward_row", "forward", "prefix_rms_norm", "blocktri_linear", "forward_nested_row",
    "forward_nested", "top_k_keep", "sample_next", "generate",
]


# ----------------------------------------------------------------------------- RMSNorm

def rms_norm(u: np.ndarray, eps: float = 0.0) -> np.ndarray:
    """RMSNorm over the last axis, no gain and no bias.

    [M] "RMS Normalization", Definition: divide by the root of the mean square
    of the vector's entries (eps added inside the root, see module readings).
    """
    ms = np.mean(u * u, axis=-1, keepdims=True)
    return u / np.sqrt(ms + eps)


# ----------------------------------------------------------------------------- RoPE

def rope_angles(T: int, head_dim: int, base: float, dtype=np.float64):
    """cos/sin tables of shape [T, head_dim/2].

    [M] "Rotary Position Embeddings (RoPE)", Frequency Construction:
    omega_j = base^(-2j/d_h) for j < d_h/2 and angle phi_{t,j} = t * omega_j
    for positions t = 0..T-1.  Computed in float64.
    """
    j = np.arange(head_dim // 2, dtype=np.float64)
    omega = 1.0 / (float(base) ** (2.0 * j / head_dim))
    t = np.arange(T, dtype=np.float64)
    phi = np.outer(t, omega)
    return np.cos(phi).astype(dtype), np.sin(phi).astype(dtype)


def apply_rope(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate u[..., T, heads, d] (positions along axis -3) by the half-split rule.

    [M] "Rotary Position Embeddings (RoPE)", Rotation Application: with
    u = [u1 | u2] split into halves, the result is
    [u1 cos + u2 sin | -u1 sin + u2 cos] elementwise at the row's position.
    ``cos``/``sin`` are [T, d/2]; they broadcast over the head axis.
    """
    d2 = u.shape[-1] // 2
    u1, u2 = u[..., :d2], u[..., d2:]
    c = cos[:, None, :]
    s = sin[:, None, :]
    return np.concatenate([u1 * c + u2 * s, -u1 * s + u2 * c], axis=-1)


# ----------------------------------------------------------------------------- windows

def layer_windows(pattern: str, short_window: int, seq_len: int, n_layer: int) -> List[int]:
    """Per-layer window sizes for a tiled short/long pattern.

    [M] "Sliding Window Pattern": the pattern string is tiled across the
    layers, "L" means full context (w = T), "S" the short window, and the last
    layer always gets full context.  [S] "Architecture" states the same for
    the SSSL pattern.  The short window size follows the workload presets
    (T/2), not the T/3 rounding of [M] (module readings).
    """
    out = []
    for l in range(n_layer):
        ch = pattern[l % len(pattern)]
        if ch == "L":
            out.append(seq_len)
        elif ch == "S":
            out.append(short_window)
        else:
            raise ValueError(f"unknown window character {ch!r}")
    out[-1] = seq_len
    return out


def visible_mask(T: int, window: int) -> np.ndarray:
    """Boolean [T, T]: key j visible from query i iff j <= i and i - j < window.

    [M] "Scaled Dot-Product Attention with Sliding Window": the logit is kept
    for j <= i and i - j < w, and is -inf otherwise.
    """
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= i) & (i - j < window)


# ----------------------------------------------------------------------------- attention

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int, scale: float) -> np.ndarray:
    """Windowed causal softmax attention for one row.

    q: [T, H, D]; k: [T, Hkv, D]; v: [T, Hkv, Dv] with H a multiple of Hkv.  Returns
    [T, H, Dv].
    [M] "Scaled Dot-Product Attention with Sliding Window": o_{h,i} is the
    softmax-weighted sum of v_{h,j} over visible keys j.  Computed as an
    explicit masked T x T matrix per head.  Query head h reads KV head
    floor(h * Hkv / H) ([M] "Causal Self-Attention" allows Hkv < H without
    fixing the map; contiguous groups are the reading used here).
    """
    T, H, D = q.shape
    Hkv = k.shape[1]
    mask = visible_mask(T, window)
    out = np.empty((T, H, v.shape[-1]), dtype=np.result_type(q, v))
    for h in range(H):
        g = (h * Hkv) // H
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        s = np.where(mask, s, -np.inf)
        m = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - m)
        a = e / np.sum(e, axis=-1, keepdims=True)
        out[:, h, :] = a @ v[:, g, :]
    return out


def softplus(z):
    """log(1 + exp(z)), the routing gate of [L] "What is the routing loop?" (g = softplus of
    the per-layer gate logit); written as max(z, 0) + log1p(exp(-|z|)) to stay finite."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def attention_with_prior(q: np.ndarray, k: np.ndarray, v: np.ndarray, q1: np.ndarray,
                         k1: np.ndarray, g: float, window: int, scale: float) -> np.ndarray:
    """Windowed causal attention whose logits carry the pass-1 prior.

    [L] "What is the routing loop?": attn_logits = q2 k2^T / sqrt(D) + g q1 k1^T / sqrt(D)
    (here with the configured scale in place of 1/sqrt(D)), then the usual masked softmax over
    the visible keys and the weighted sum of v.  q, q1: [T, H, D]; k, k1, v: [T, Hkv, D].
    Explicit T x T logits per head, as written on the page.
    """
    T, H, D = q.shape
    Hkv = k.shape[1]
    mask = visible_mask(T, window)
    out = np.empty((T, H, v.shape[-1]), dtype=np.result_type(q, v))
    for h in range(H):
        gh = (h * Hkv) // H
        s = scale * (q[:, h, :] @ k[:, gh, :].T) + g * scale * (q1[:, h, :] @ k1[:, gh, :].T)
        s = np.where(mask, s, -np.inf)
        m = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - m)
        out[:, h, :] = (e / np.sum(e, axis=-1, keepdims=True)) @ v[:, gh, :]
    return out


# ----------------------------------------------------------------------------- MLP, head

def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x @ w^T for a row-major [out, in] weight with no bias ([M] "Causal
    Self-Attention", Projections; "Feed-Forward Network (MLP)")."""
    return x @ w.T


def relu_squared(z: np.ndarray) -> np.ndarray:
    """max(0, z)^2 ([M] "Feed-Forward Network (MLP)")."""
    r = np.maximum(z, 0.0)
    return r * r


def softcap(z: np.ndarray, cap: float = 15.0) -> np.ndarray:
    """cap * tanh(z / cap) ([M] "Logit Softcap"; [R] 5.4)."""
    return cap * np.tanh(z / cap)


def token_losses(zhat: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Per-token cross-entropy log(sum_v exp(zhat_v)) - zhat_y, 0 where y = -1.

    [M] "Cross-Entropy Loss": negative log-softmax at the target, with targets
    equal to -1 excluded.  logsumexp uses the row maximum as shift.
    """
    zhat = np.asarray(zhat)
    m = np.max(zhat, axis=-1)
    lse = m + np.log(np.sum(np.exp(zhat - m[..., None]), axis=-1))
    valid = targets >= 0
    idx = np.where(valid, targets, 0)
    picked = np.take_along_axis(zhat, idx[..., None].astype(np.int64), axis=-1)[..., 0]
    return np.where(valid, lse - picked, 0.0)


def mean_loss(losses: np.ndarray, targets: np.ndarray) -> float:
    """Mean over tokens with target != -1; NaN when there are none ([M]
    "Cross-Entropy Loss", the set of kept positions)."""
    valid = targets >= 0
    n = int(np.count_nonzero(valid))
    if n == 0:
        return float("nan")
    return float(np.sum(np.where(valid, losses, 0.0)) / n)


# ----------------------------------------------------------------------------- value embeddings

def has_ve(l: int, n_layer: int) -> bool:
    """[M] "Value Embeddings (ResFormer)", layer selection: layer l (0-based) takes a value
    embedding iff l mod 2 equals (L - 1) mod 2 -- every other layer, the last one always."""
    return l % 2 == (n_layer - 1) % 2


def value_embed_mix(v: np.ndarray, e: np.ndarray, x_gate: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """Gated value-embedding mix for one row.

    [M] "Value Embeddings (ResFormer)": the gate is 3 * sigmoid of a linear map of the input's
    first channels, one scalar per KV head and position, broadcast over the head dimension,
    and v_h <- v_h + g_h * e_h.  v, e: [T, Hkv, D]; x_gate: [T, n] (the first n channels);
    w_gate: [Hkv, n].
    """
    logit = x_gate @ w_gate.T
    g = 3.0 / (1.0 + np.exp(-logit))
    return v + g[:, :, None] * e


# ----------------------------------------------------------------------------- forward

def _get(params: Any, name: str, layer: Optional[int] = None):
    a = params[name]
    return a if layer is None else a[layer]


def block(x: np.ndarray, x0: np.ndarray, l: int, cfg: Any, params: Any, window: int,
          cos: np.ndarray, sin: np.ndarray, dt, internals: Optional[Dict] = None,
          tokens: Optional[np.ndarray] = None, prior: Optional[tuple] = None) -> np.ndarray:
    """One transformer layer on one row x [T, C].

    [M] "Residual Stream with Learnable Scalars" and "High-Level Forward Pass"
    step 3: rescale x <- lambda_l x + mu_l x0, then x += Attn(RMSNorm(x)) and
    x += MLP(RMSNorm(x)).  Inside attention ([M] "Causal Self-Attention",
    "QK-Norm with Sharpening"; [R] 5.2): project q, k, v with no bias, RoPE on
    q and k, per-head RMSNorm of q and k, windowed attention, merge heads,
    output projection.  With value embeddings on a selected layer ([M] "Value Embeddings
    (ResFormer)"), v is mixed with the gated table rows of ``tokens`` before attention.
    ``prior`` = (q1, k1, g) adds the pass-1 logit prior of the looped trunk ([L]).
    """
    T, C = x.shape
    H, Hkv, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    eps = cfg.norm_eps
    lam = float(np.asarray(_get(params, "resid_lambda"))[l])
    mu = float(np.asarray(_get(params, "x0_lambda"))[l])
    x = lam * x + mu * x0
    xin = x
    xn = rms_norm(x, eps)
    q = linear(xn, np.asarray(_get(params, "wq", l), dtype=dt)).reshape(T, H, D)
    k = linear(xn, np.asarray(_get(params, "wk", l), dtype=dt)).reshape(T, Hkv, D)
    v = linear(xn, np.asarray(_get(params, "wv", l), dtype=dt)).reshape(T, Hkv, D)
    if getattr(cfg, "value_embeds", False) and has_ve(l, cfg.n_layer):
        e = np.asarray(_get(params, "ve", l)[tokens], dtype=dt).reshape(T, Hkv, D)
        wg = np.asarray(_get(params, "ve_gate", l), dtype=dt)
        v = value_embed_mix(v, e, xn[:, :wg.shape[1]], wg)
    q = rms_norm(apply_rope(q, cos, sin), eps)
    k = rms_norm(apply_rope(k, cos, sin), eps)
    if prior is None:
        o = attention(q, k, v, window, cfg.attn_scale)
    else:
        o = attention_with_prior(q, k, v, prior[0], prior[1], prior[2], window, cfg.attn_scale)
    x = x + linear(o.reshape(T, H * D), np.asarray(_get(params, "wo", l), dtype=dt))
    xa = x
    xm = rms_norm(x, eps)
    h = relu_squared(linear(xm, np.asarray(_get(params, "w1", l), dtype=dt)))
    x = x + linear(h, np.asarray(_get(params, "w2", l), dtype=dt))
    if internals is not None:
        internals.update(xin=xin, xn=xn, q=q, k=k, v=v, o=o, x_attn=xa, xm=xm, h=h, x_out=x)
    return x


def forward_row(cfg: Any, params: Any, tokens: np.ndarray, targets: Optional[np.ndarray],
                dtype=np.float64, want_logits: bool = False, want_internals: bool = False,
                windows: Optional[Sequence[int]] = None) -> Dict[str, Any]:
    """Forward pass of one packed row (tokens [T]) and its next-token loss.

    [M] "High-Level Forward Pass" steps 1-6 and "Pseudocode: One Training
    Step" steps 1-11: embed and RMSNorm, keep x0, L blocks, final RMSNorm,
    untied lm_head, softcap, cross-entropy.  Rows of a batch never interact,
    so a batch is this function applied row by row.
    """
    dt = np.dtype(dtype)
    T = tokens.shape[0]
    eps = cfg.norm_eps
    if windows is None:
        windows = layer_windows(cfg.window_pattern, cfg.short_window, cfg.seq_len, cfg.n_layer)
    cos, sin = rope_angles(T, cfg.head_dim, cfg.rope_base, dtype=dt)
    wte = np.asarray(_get(params, "wte"))
    res: Dict[str, Any] = {}
    layers = []
    priors = None
    if getattr(cfg, "looped", False):
        # [L] "What is the routing loop?": pass 1 runs the ordinary trunk and keeps every
        # layer's normalised, rotated q and k; pass 2 starts again from the embeddings.
        pe = np.asarray(_get(params, "pass_emb"), dtype=dt)
        gates = softplus(np.asarray(_get(params, "gate_logit"), dtype=np.float64))
        x = rms_norm(np.asarray(wte[tokens], dtype=dt) + pe[0], eps)
        x0 = x
        priors = []
        for l in range(cfg.n_layer):
            cap: Dict[str, Any] = {}
            x = block(x, x0, l, cfg, params, windows[l], cos, sin, dt, cap, tokens=tokens)
            priors.append((cap["q"], cap["k"], float(gates[l])))
        x = rms_norm(np.asarray(wte[tokens], dtype=dt) + pe[1], eps)
    else:
        x = rms_norm(np.asarray(wte[tokens], dtype=dt), eps)
    x0 = x
    for l in range(cfg.n_layer):
        internals = {} if want_internals else None
        x = block(x, x0, l, cfg, params, windows[l], cos, sin, dt, internals, tokens=tokens,
                  prior=None if priors is None else priors[l])
        if want_internals:
            layers.append(internals)
    xf = rms_norm(x, eps)
    wu = np.asarray(_get(params, "lm_head"), dtype=dt)
    if targets is not None:
        # chunk over positions to bound the [T, V] logits held at once
        losses = np.zeros(T, dtype=dt)
        step = max(1, (1 << 24) // max(1, wu.shape[0]))
        logits_parts = []
        for a in range(0, T, step):
            zh = softcap(linear(xf[a:a + step], wu), cfg.softcap)
            losses[a:a + step] = token_losses(zh, targets[a:a + step])
            if want_logits:
                logits_parts.append(zh)
        res["losses"] = losses
        if want_logits:
            res["logits"] = np.concatenate(logits_parts, axis=0)
    elif want_logits:
        res["logits"] = softcap(linear(xf, wu), cfg.softcap)
    if want_internals:
        res["x0"] = x0
        res["layers"] = layers
        res["xf"] = xf
    return res


# ----------------------------------------------------------------------------- nested model

def prefix_rms_norm(u: np.ndarray, c1: int, eps: float = 0.0) -> np.ndarray:
    """PrefixRMSNorm with two blocks ([F] and the nested configuration): coordinates [0, c1)
    are divided by the RMS of dims [0, c1), coordinates [c1, C) by the RMS of all dims, so the
    first block never sees the second.  Block 1 is exactly RMSNorm of the prefix."""
    first = rms_norm(np.ascontiguousarray(u[..., :c1]), eps)
    if c1 == u.shape[-1]:
        return first
    return np.concatenate([first, rms_norm(u, eps)[..., c1:]], axis=-1)


def blocktri_linear(x: np.ndarray, blocks: Sequence[np.ndarray], in1: int) -> np.ndarray:
    """x W^T for a block lower triangular W given as its row blocks ([F]: the upper block is
    zero and only the live blocks are stored): rows of block 1 read inputs [0, in1), rows of
    block 2 read all inputs.  Block 1 is computed on the contiguous input prefix, exactly as a
    standalone model of that width would."""
    w1, w2 = blocks
    y1 = linear(np.ascontiguousarray(x[..., :in1]), w1)
    if w2.shape[0] == 0:
        return y1
    return np.concatenate([y1, linear(x, w2)], axis=-1)


def forward_nested_row(cfg: Any, params: Any, tokens: np.ndarray, targets: Optional[np.ndarray],
                       dtype=np.float64, want_logits: bool = False,
                       windows: Optional[Sequence[int]] = None) -> Dict[str, Any]:
    """Nested (two-block StairFormer) forward of one row and both prefix losses.

    [F]: the nanochat forward with every linear block lower triangular and every norm a
    PrefixRMSNorm, so the first block of the residual stream evolves as a standalone model of
    width c1 would; one pass gives the kfront=1 logits (input columns [0, c1) of the final
    normalised stream against the same columns of the shared lm_head) and the full logits.
    Returns ``losses`` (full model), ``losses_k1`` (kfront=1) and optionally both logits.
    """
    dt = np.dtype(dtype)
    T = tokens.shape[0]
    eps, c1, C = cfg.norm_eps, cfg.nested_c1, cfg.d_model
    H, Hkv, D, F = cfg.n_head, cfg.n_kv_head, cfg.head_dim, cfg.mlp_dim
    h1d, f1 = H * c1 // C * D, F * c1 // C   # inner widths of the head and hidden dims
    if windows is None:
        windows = layer_windows(cfg.window_pattern, cfg.short_window, cfg.seq_len, cfg.n_layer)
    cos, sin = rope_angles(T, D, cfg.rope_base, dtype=dt)
    blk = lambda n, l: [np.asarray(b, dtype=dt) for b in _get(params, n, l)]
    wte = np.asarray(_get(params, "wte"))
    x = prefix_rms_norm(np.asarray(wte[tokens], dtype=dt), c1, eps)
    x0 = x
    lam_all = np.asarray(_get(params, "resid_lambda"))
    mu_all = np.asarray(_get(params, "x0_lambda"))
    for l in range(cfg.n_layer):
        x = float(lam_all[l]) * x + float(mu_all[l]) * x0
        xn = prefix_rms_norm(x, c1, eps)
        q = blocktri_linear(xn, blk("wq", l), c1).reshape(T, H, D)
        k = blocktri_linear(xn, blk("wk", l), c1).reshape(T, Hkv, D)
        v = blocktri_linear(xn, blk("wv", l), c1).reshape(T, Hkv, D)
        q = rms_norm(apply_rope(q, cos, sin), eps)
        k = rms_norm(apply_rope(k, cos, sin), eps)
        o = attention(q, k, v, windows[l], cfg.attn_scale)
        x = x + blocktri_linear(o.reshape(T, H * D), blk("wo", l), h1d)
        xm = prefix_rms_norm(x, c1, eps)
        h = relu_squared(blocktri_linear(xm, blk("w1", l), c1))
        x = x + blocktri_linear(h, blk("w2", l), f1)
    xf = prefix_rms_norm(x, c1, eps)
    wu = np.asarray(_get(params, "lm_head"), dtype=dt)
    wu1 = np.ascontiguousarray(wu[:, :c1])
    xf1 = np.ascontiguousarray(xf[:, :c1])
    res: Dict[str, Any] = {}
    step = max(1, (1 << 24) // max(1, wu.shape[0]))
    for key, xs, w in (("", xf, wu), ("_k1", xf1, wu1)):
        losses = np.zeros(T, dtype=dt)
        parts = []
        for a in range(0, T, step):
            zh = softcap(linear(xs[a:a + step], w), cfg.softcap)
            if targets is not None:
                losses[a:a + step] = token_losses(zh, targets[a:a + step])
            if want_logits:
                parts.append(zh)
        if targets is not None:
            res["losses" + key] = losses
        if want_logits:
            res["logits" + key] = np.concatenate(parts, axis=0)
    return res


def forward_nested(cfg: Any, params: Any, tokens: np.ndarray, targets: Optional[np.ndarray] = None,
                   dtype=np.float64, want_logits: bool = False, rows: Optional[Sequence[int]] = None,
                   windows: Optional[Sequence[int]] = None) -> Dict[str, Any]:
    """Batched nested forward: ``losses``/``mean`` (full model) and ``losses_k1``/``mean_k1``
    (kfront=1), plus ``logits``/``logits_k1`` when asked."""
    rows = list(range(tokens.shape[0])) if rows is None else list(rows)
    acc: Dict[str, list] = {}
    for b in rows:
        r = forward_nested_row(cfg, params, tokens[b], None if targets is None else targets[b],
                               dtype=dtype, want_logits=want_logits, windows=windows)
        for k, v in r.items():
            acc.setdefault(k, []).append(v)
    res: Dict[str, Any] = {k: np.stack(v) for k, v in acc.items()}
    if targets is not None:
        res["mean"] = mean_loss(res["losses"], targets[rows])
        res["mean_k1"] = mean_loss(res["losses_k1"], targets[rows])
    return res


def forward(cfg: Any, params: Any, tokens: np.ndarray, targets: Optional[np.ndarray] = None,
            dtype=np.float64, want_logits: bool = False, rows: Optional[Sequence[int]] = None,
            windows: Optional[Sequence[int]] = None) -> Dict[str, Any]:
    """Batched forward+loss on tokens [B, T] (optionally only ``rows``).

    Returns ``losses`` [b, T] (when targets are given), ``mean`` over the
    evaluated rows' valid targets, and ``logits`` [b, T, V] when asked.

    ``params`` maps ``wte``, ``lm_head``, ``resid_lambda``, ``x0_lambda`` to
    arrays and ``wq``, ``wk``, ``wv``, ``wo``, ``w1``, ``w2`` to per-layer
    sequences of row-major [out, in] arrays (any float dtype; converted to
    ``dtype`` one layer at a time); with ``cfg.value_embeds`` also ``ve``
    (per layer [V, Hkv*D]) and ``ve_gate`` (per layer [Hkv, 12]); with
    ``cfg.looped`` also ``pass_emb`` ([2, C]) and ``gate_logit`` ([L]).
    """
    if getattr(cfg, "nested_c1", 0):
        return forward_nested(cfg, params, tokens, targets, dtype, want_logits, rows, windows)
    rows = list(range(tokens.shape[0])) if rows is None else list(rows)
    out_l, out_z = [], []
    for b in rows:
        r = forward_row(cfg, params, tokens[b], None if targets is None else targets[b],
                        dtype=dtype, want_logits=want_logits, windows=windows)
        if targets is not None:
            out_l.append(r["losses"])
        if want_logits:
            out_z.append(r["logits"])
    res: Dict[str, Any] = {}
    if targets is not None:
        L = np.stack(out_l)
        res["losses"] = L
        res["mean"] = mean_loss(L, targets[rows])
    if want_logits:
        res["logits"] = np.stack(out_z)
    return res


# ----------------------------------------------------------------------------- generation

def top_k_keep(z: np.ndarray, k: Optional[int]) -> np.ndarray:
    """[M] "Sampling Controls", top-k filtering: the tokens kept for sampling -- every v with
    z_v >= the k-th largest logit (all of them when k is None or k >= V)."""
    z = np.asarray(z)
    if k is None or k >= z.shape[-1]:
        return np.ones(z.shape, dtype=bool)
    if k < 1:
        raise ValueError("top_k must be >= 1")
    kth = np.sort(z)[::-1][k - 1]
    return z >= kth


def sample_next(zhat: np.ndarray, top_k: Optional[int], temperature: float, u: float) -> int:
    """One draw of the next token from the softcapped logits of one position ([M] "Sampling
    Controls"): temperature 0 is the argmax (first index on ties); otherwise
    P(v) = exp(z_v / tau) / sum_{kept v'} exp(z_v' / tau) over the top-k kept tokens, and the
    token is the first v in vocabulary order whose cumulative probability exceeds u."""
    z = np.asarray(zhat, dtype=np.float64)
    if temperature == 0.0:
        return int(np.argmax(z))
    if not temperature > 0.0:
        raise ValueError("temperature must be >= 0")
    keep = top_k_keep(z, top_k)
    s = np.where(keep, z / temperature, -np.inf)
    e = np.exp(s - np.max(s))
    cdf = np.cumsum(e / np.sum(e))
    idx = int(np.searchsorted(cdf, u, side="right"))   # first index with cdf > u
    idx = min(idx, z.shape[-1] - 1)
    while not keep[idx]:          # u within rounding of 1: the last kept token
        idx -= 1
    return idx


def generate(cfg: Any, params: Any, prompt: np.ndarray, n_new: int, top_k: Optional[int],
             temperature: float, u: np.ndarray, windows: Optional[Sequence[int]] = None
             ) -> Dict[str, Any]:
    """[M] "Inference: Generating Text": from a prompt [B, P], n_new times run the full
    forward on the sequence so far, take the softcapped logits at the last position and
    append one sampled token per row (u [n_new, B] are the draws).  The forward's windows
    are those of a sequence of cfg.seq_len tokens (the model's configuration), applied to the
    sequence so far.  Returns the tokens [B, P + n_new] and the logits each step sampled from
    [n_new, B, V]."""
    seq = np.array(prompt, dtype=np.int64)
    if windows is None:
        windows = layer_windows(cfg.window_pattern, cfg.short_window, cfg.seq_len, cfg.n_layer)
    steps = []
    for i in range(n_new):
        z = forward(cfg, params, seq, want_logits=True, windows=windows)["logits"][:, -1, :]
        nxt = [sample_next(z[b], top_k, temperature, float(u[i][b])) for b in range(seq.shape[0])]
        seq = np.concatenate([seq, np.array(nxt, dtype=np.int64)[:, None]], axis=1)
        steps.append(z)
    return {"tokens": seq, "logits": np.stack(steps)}
