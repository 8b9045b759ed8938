"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This module holds workload *shapes* and *random draws* only: configuration
presets, Gaussian weight tensors, uniform token rows, and the fp32 -> bf16
round-to-nearest-even used to store weights in bf16.  It computes none of the
model's arithmetic (no norm, attention, projection or loss lives here), so the
oracle and the GPU path can both consume what it produces without sharing any
of the method.

Workload stand-in: the pages train nanochat on packed 2,048-token rows of
tokenised web text (32,768-entry BPE vocabulary).  That text is not available,
so uniform random token ids of the same shape and vocabulary stand in for it;
weights are Gaussian N(0, 1/fan_in) rather than trained values.

Draw order for one preset (seeded ``numpy.random.default_rng(seed)``):
  1. token embedding table W_E [V, C]
  2. per layer: W_Q, W_K, W_V, W_O, W_1, W_2
  3. lm_head W_U [V, C]
  4. per-layer residual scalars lambda[L] then x0 scalars mu[L]
  5. (value-embedding presets only) per layer: value-embedding table [V, Hkv*D] ~ N(0, 1)
     and gate weights [Hkv, 12] ~ N(0, 1/12), drawn for every layer (the model uses the
     layers its selection rule picks)
  6. (looped presets only) pass embeddings [2, C] ~ N(0, 1/C), then per-layer routing gate
     logits [L] = ln(exp(0.05) - 1) + 0.1 N(0, 1) (float32), i.e. gates near 0.05
  7. token rows [B, T+1]

Nested presets (nested_c1 > 0, two blocks): every per-layer linear is block lower triangular
and drawn as its two row blocks, in order: row block 1 [out_1, in_1] ~ N(0, 1/in_1), then row
block 2 [out_2, in_1 + in_2] ~ N(0, 1/(in_1 + in_2)); each dimension splits in the proportion
nested_c1 : d_model (q/k/v by heads, the MLP hidden proportionally).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Preset", "PRESETS", "preset", "Weights", "make_weights", "make_tokens",
    "bf16_round_bits", "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Preset:
    """Shape and draw recipe of one workload (sizes only, no arithmetic)."""
    name: str
    n_layer: int
    d_model: int
    n_head: int
    n_kv_head: int
    head_dim: int
    mlp_dim: int
    vocab: int
    seq_len: int
    batch: int
    dtype: str                    # "f32" or "bf16": storage type of weights and activations
    window_pattern: str = "SSSL"  # tiled over layers; the last layer is always long
    short_window: int = 1024
    softcap: float = 15.0
    rope_base: float = 100000.0
    norm_eps: float = 1e-6
    lambda_range: tuple = (1.0, 1.0)   # resid scalar lambda: constant if lo == hi, else U[lo, hi]
    mu_range: tuple = (0.1, 0.1)       # x0 scalar mu: constant if lo == hi, else U[lo, hi]
    seed: int = 0
    qk_scale: Optional[float] = None   # attention logit scale; None means 1/sqrt(head_dim)
    value_embeds: bool = False         # per-layer value-embedding tables and gates are drawn
    ve_gate_channels: int = 12         # input channels the value-embedding gate reads
    looped: bool = False               # two-pass trunk: pass embeddings and routing gate logits
    nested_c1: int = 0                 # > 0: two nested blocks, the inner one nested_c1 wide

    @property
    def attn_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim) if self.qk_scale is None else float(self.qk_scale)

    @property
    def tokens_per_batch(self) -> int:
        return self.batch * self.seq_len

    def with_(self, **kw) -> "Preset":
        return dataclasses.replace(self, **kw)


PRESETS: Dict[str, Preset] = {
    # depth 2, width 128, one head of 128, V=4096, T=256, B=2, fp32, short window 128
    "tiny": Preset("tiny", 2, 128, 1, 1, 128, 512, 4096, 256, 2, "f32", short_window=128),
    # nanochat d12: width 768, 6 heads of 128, V=32768, T=2048, B=4, bf16
    "d12": Preset("d12", 12, 768, 6, 6, 128, 3072, 32768, 2048, 4, "bf16", short_window=1024),
    # nanochat d24: width 1536, 12 heads of 128, V=32768, T=2048, B=8, bf16, seeded lambda/mu
    "d24": Preset("d24", 24, 1536, 12, 12, 128, 6144, 32768, 2048, 8, "bf16", short_window=1024,
                  lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2)),
    # StairFormer nested d24: 24 heads of 64 in blocks of 6 + 18 (inner width 384), B=4
    "d24nest": Preset("d24nest", 24, 1536, 24, 24, 64, 6144, 32768, 2048, 4, "bf16", short_window=1024,
                      lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), nested_c1=384),
    # looped two-pass d24 (B=4)
    "d24loop": Preset("d24loop", 24, 1536, 12, 12, 128, 6144, 32768, 2048, 4, "bf16", short_window=1024,
                      lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), looped=True),
    # d24 with grouped-query attention (4 KV heads) and value embeddings
    "d24gve": Preset("d24gve", 24, 1536, 12, 4, 128, 6144, 32768, 2048, 8, "bf16", short_window=1024,
                     lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), value_embeds=True),
}


def preset(name: str, **overrides) -> Preset:
    p = PRESETS[name]
    return p.with_(**overrides) if overrides else p


# ----------------------------------------------------------------------------- bf16 storage

def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN; finite values round by adding 0x7fff plus
    the lowest kept bit before truncating the low 16 bits.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly representable fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- weights

@dataclasses.dataclass
class Weights:
    """One preset's parameters.

    For bf16 presets every matrix is held as uint16 bf16 bit patterns; for f32
    presets as float32.  ``value(a)`` returns the float32 values either way.
    Matrices are row-major [out_features, in_features].  In nested presets each per-layer
    linear is a list of its row blocks ([out_1, in_1], [out_2, in_1 + in_2]).
    """
    dtype: str
    wte: np.ndarray                 # [V, C]
    wq: List[np.ndarray]            # L x [H*D, C]
    wk: List[np.ndarray]            # L x [Hkv*D, C]
    wv: List[np.ndarray]            # L x [Hkv*D, C]
    wo: List[np.ndarray]            # L x [C, H*D]
    w1: List[np.ndarray]            # L x [F, C]
    w2: List[np.ndarray]            # L x [C, F]
    lm_head: np.ndarray             # [V, C]
    resid_lambda: np.ndarray        # [L] float32
    x0_lambda: np.ndarray           # [L] float32
    ve: Optional[List[np.ndarray]] = None       # L x [V, Hkv*D] value-embedding tables
    ve_gate: Optional[List[np.ndarray]] = None  # L x [Hkv, ve_gate_channels] gate weights
    pass_emb: Optional[np.ndarray] = None       # [2, C] per-pass embeddings (looped)
    gate_logit: Optional[np.ndarray] = None     # [L] float32 routing gate logits (looped)

    def value(self, a):
        if isinstance(a, list):
            return [self.value(b) for b in a]
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a

    def matrices(self):
        yield "wte", self.wte
        for i in range(len(self.wq)):
            for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
                yield f"{n}{i}", getattr(self, n)[i]
        yield "lm_head", self.lm_head


def _gauss(rng: np.random.Generator, shape, fan_in: int, dtype: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(1.0 / math.sqrt(fan_in))
    return bf16_round_bits(a) if dtype == "bf16" else a


def _scalars(rng: np.random.Generator, rng_lohi: tuple, n: int) -> np.ndarray:
    lo, hi = rng_lohi
    if lo == hi:
        return np.full(n, lo, dtype=np.float32)
    return rng.uniform(lo, hi, n).astype(np.float32)


def make_weights(p: Preset, rng: Optional[np.random.Generator] = None) -> Weights:
    """Draw one preset's weights in the fixed order documented above.

    Pass ``rng`` to continue an existing stream (``make_tokens`` then draws from
    the same generator); otherwise a fresh ``default_rng(p.seed)`` is used.
    """
    if rng is None:
        rng = np.random.default_rng(p.seed)
    C, H, Hkv, D, F, V, L = p.d_model, p.n_head, p.n_kv_head, p.head_dim, p.mlp_dim, p.vocab, p.n_layer
    wte = _gauss(rng, (V, C), C, p.dtype)
    wq, wk, wv, wo, w1, w2 = [], [], [], [], [], []
    if p.nested_c1:
        c1 = p.nested_c1
        part = lambda n: n * c1 // C  # inner share of a dimension

        def blocks(out, inp):
            o1, i1 = part(out), part(inp)
            return [_gauss(rng, (o1, i1), i1, p.dtype), _gauss(rng, (out - o1, inp), inp, p.dtype)]
    for _ in range(L):
        if p.nested_c1:
            wq.append(blocks(H * D, C))
            wk.append(blocks(Hkv * D, C))
            wv.append(blocks(Hkv * D, C))
            wo.append(blocks(C, H * D))
            w1.append(blocks(F, C))
            w2.append(blocks(C, F))
            continue
        wq.append(_gauss(rng, (H * D, C), C, p.dtype))
        wk.append(_gauss(rng, (Hkv * D, C), C, p.dtype))
        wv.append(_gauss(rng, (Hkv * D, C), C, p.dtype))
        wo.append(_gauss(rng, (C, H * D), H * D, p.dtype))
        w1.append(_gauss(rng, (F, C), C, p.dtype))
        w2.append(_gauss(rng, (C, F), F, p.dtype))
    lm_head = _gauss(rng, (V, C), C, p.dtype)
    lam = _scalars(rng, p.lambda_range, L)
    mu = _scalars(rng, p.mu_range, L)
    ve = ve_gate = None
    if p.value_embeds:
        ve, ve_gate = [], []
        for _ in range(L):
            ve.append(_gauss(rng, (V, Hkv * D), 1, p.dtype))
            ve_gate.append(_gauss(rng, (Hkv, p.ve_gate_channels), p.ve_gate_channels, p.dtype))
    pass_emb = gate_logit = None
    if p.looped:
        pass_emb = _gauss(rng, (2, C), C, p.dtype)
        gate_logit = (np.float32(math.log(math.expm1(0.05)))
                      + np.float32(0.1) * rng.standard_normal(L, dtype=np.float32)).astype(np.float32)
    return Weights(p.dtype, wte, wq, wk, wv, wo, w1, w2, lm_head, lam, mu, ve, ve_gate,
                   pass_emb, gate_logit)


def make_tokens(p: Preset, rng: np.random.Generator, batch: Optional[int] = None,
                ignore_frac: float = 0.0):
    """Uniform token rows [B, T+1] split into (tokens, targets), both int32 [B, T].

    ``ignore_frac`` > 0 marks that fraction of targets (chosen uniformly, drawn
    after the rows) as -1, the ignore index.
    """
    B = p.batch if batch is None else batch
    rows = rng.integers(0, p.vocab, size=(B, p.seq_len + 1), dtype=np.int64).astype(np.int32)
    tokens = np.ascontiguousarray(rows[:, :-1])
    targets = np.ascontiguousarray(rows[:, 1:])
    if ignore_frac > 0.0:
        mask = rng.random(targets.shape) < ignore_frac
        targets = np.where(mask, np.int32(-1), targets).astype(np.int32)
    return tokens, targets


def make_inputs(p: Preset, batch: Optional[int] = None, ignore_frac: float = 0.0):
    """Weights then tokens from one ``default_rng(p.seed)`` stream."""
    rng = np.random.default_rng(p.seed)
    w = make_weights(p, rng)
    tokens, targets = make_tokens(p, rng, batch=batch, ignore_frac=ignore_frac)
    return w, tokens, targets
