"""Shared test helpers: adapters between gptdata's seeded inputs and the oracle."""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

import gptdata

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


class _LazyLayers:
    """Per-layer float32 view of a list of stored matrices (bf16 bits or f32)."""

    def __init__(self, w: gptdata.Weights, mats):
        self._w, self._m = w, mats

    def __getitem__(self, i):
        return self._w.value(self._m[i])

    def __len__(self):
        return len(self._m)


def oracle_params(w: gptdata.Weights) -> dict:
    """Map gptdata weights to the oracle's parameter names (float32 values)."""
    return {
        "wte": w.value(w.wte),
        "lm_head": w.value(w.lm_head),
        "resid_lambda": w.resid_lambda,
        "x0_lambda": w.x0_lambda,
        "wq": _LazyLayers(w, w.wq), "wk": _LazyLayers(w, w.wk), "wv": _LazyLayers(w, w.wv),
        "wo": _LazyLayers(w, w.wo), "w1": _LazyLayers(w, w.w1), "w2": _LazyLayers(w, w.w2),
        **({"ve": _LazyLayers(w, w.ve), "ve_gate": _LazyLayers(w, w.ve_gate)} if w.ve is not None else {}),
        **({"pass_emb": w.value(w.pass_emb), "gate_logit": w.gate_logit} if w.pass_emb is not None else {}),
    }


def dense_params(p: gptdata.Preset, seed: int = 0) -> dict:
    """Materialised float64 parameters of a small f32 preset (editable lists)."""
    w = gptdata.make_weights(p.with_(dtype="f32", seed=seed))
    d = {
        "wte": w.wte.astype(np.float64), "lm_head": w.lm_head.astype(np.float64),
        "resid_lambda": w.resid_lambda.astype(np.float64).copy(),
        "x0_lambda": w.x0_lambda.astype(np.float64).copy(),
    }
    for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
        d[n] = [[b.astype(np.float64) for b in m] if isinstance(m, list) else m.astype(np.float64)
                for m in getattr(w, n)]
    if w.ve is not None:
        d["ve"] = [m.astype(np.float64) for m in w.ve]
        d["ve_gate"] = [m.astype(np.float64) for m in w.ve_gate]
    if w.pass_emb is not None:
        d["pass_emb"] = w.pass_emb.astype(np.float64)
        d["gate_logit"] = w.gate_logit.astype(np.float64).copy()
    return d


def small_preset(**kw) -> gptdata.Preset:
    """A few-layer float config the oracle runs in milliseconds."""
    base = dict(name="small", n_layer=2, d_model=16, n_head=2, n_kv_head=2, head_dim=8,
                mlp_dim=64, vocab=50, seq_len=12, batch=2, dtype="f32",
                short_window=4, norm_eps=0.0)
    base.update(kw)
    return gptdata.Preset(**base)
