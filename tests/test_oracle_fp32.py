"""The float32 form of the oracle (used for the full-size GPU comparisons, where float64 would
take minutes per row) against its float64 form: the same arithmetic in a shorter type, so the
per-token losses may differ only by float32 rounding (~1e-6 here), far inside the 2e-2 bf16 bar.
Covers the plain model with windows, value embeddings, the looped trunk and the nested model."""
import numpy as np
import pytest

import gptdata
import oracle
from helpers import dense_params


def _presets():
    base = dict(n_layer=3, d_model=64, n_head=4, n_kv_head=2, head_dim=16, mlp_dim=256, vocab=300,
                seq_len=96, batch=2, dtype="f32", short_window=32,
                lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2))
    return {
        "plain": gptdata.Preset(name="p32", **base),
        "ve": gptdata.Preset(name="v32", value_embeds=True, **base),
        "looped": gptdata.Preset(name="l32", looped=True, **base),
        "nested": gptdata.Preset(name="n32", nested_c1=16, **{**base, "n_kv_head": 4}),
    }


@pytest.mark.parametrize("kind", ["plain", "ve", "looped", "nested"])
def test_fp32_oracle_matches_fp64(kind):
    p = _presets()[kind]
    prm = dense_params(p, seed=3)
    tok, tgt = gptdata.make_tokens(p, np.random.default_rng(7))
    r64 = oracle.forward(p, prm, tok, tgt, dtype=np.float64)
    r32 = oracle.forward(p, prm, tok, tgt, dtype=np.float32)
    for sfx in (("", "_k1") if p.nested_c1 else ("",)):
        d = np.max(np.abs(r32["losses" + sfx].astype(np.float64) - r64["losses" + sfx]))
        assert r32["losses" + sfx].dtype == np.float32
        assert d <= 1e-4, (kind, sfx, d)
        assert abs(r32["mean" + sfx] - r64["mean" + sfx]) <= 1e-5
