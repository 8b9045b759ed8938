"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

Each mutation replaces one oracle function with a wrong variant through
monkeypatch; the listed pins must then raise.  This shows the pins constrain
every step of the forward pass, not only that the oracle agrees with itself.
"""
import numpy as np
import pytest

import oracle
import oracle_pins as P

_orig = {n: getattr(oracle, n) for n in ("apply_rope", "visible_mask", "relu_squared", "softcap",
                                          "token_losses", "rms_norm", "attention", "block", "linear",
                                          "has_ve", "value_embed_mix", "softplus",
                                          "attention_with_prior", "prefix_rms_norm",
                                          "blocktri_linear", "top_k_keep", "sample_next")}


def _rope_sign(u, cos, sin):
    d2 = u.shape[-1] // 2
    u1, u2 = u[..., :d2], u[..., d2:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([u1 * c - u2 * s, u1 * s + u2 * c], axis=-1)


def _rope_interleaved(u, cos, sin):
    u1, u2 = u[..., 0::2], u[..., 1::2]
    c, s = cos[:, None, :], sin[:, None, :]
    y = np.empty_like(u)
    y[..., 0::2] = u1 * c + u2 * s
    y[..., 1::2] = -u1 * s + u2 * c
    return y


def _mask_off_by_one(T, w):
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    return (j <= i) & (i - j <= w)


def _mask_not_causal(T, w):
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    return np.abs(i - j) < w


def _relu(z):
    return np.maximum(z, 0.0)


def _no_softcap(z, cap=15.0):
    return z


def _ce_off_index(zhat, targets):
    return _orig["token_losses"](zhat, np.where(targets >= 0, (targets + 1) % zhat.shape[-1], targets))


def _attention_no_scale(q, k, v, window, scale):
    return _orig["attention"](q, k, v, window, 1.0)


def _attention_mod_map(q, k, v, window, scale):
    H, Hkv = q.shape[1], k.shape[1]
    rep = np.arange(H) % Hkv
    return _orig["attention"](q, k[:, rep], v[:, rep], window, scale)


def _linear_square_transposed(x, w):
    return x @ (w if w.shape[0] == w.shape[1] else w.T)


def _block_patched(kind):
    """Wrap block() with a mistake in the residual-scalar or norm handling."""
    import oracle as o

    def blk(x, x0, l, cfg, params, window, cos, sin, dt, internals=None, **kw):
        if kind == "no_mix":
            prm = dict(params)
            prm["resid_lambda"] = np.ones_like(np.asarray(params["resid_lambda"]))
            prm["x0_lambda"] = np.zeros_like(np.asarray(params["x0_lambda"]))
            return _orig["block"](x, x0, l, cfg, prm, window, cos, sin, dt, internals, **kw)
        if kind == "swap_mix":
            prm = dict(params)
            prm["resid_lambda"], prm["x0_lambda"] = params["x0_lambda"], params["resid_lambda"]
            return _orig["block"](x, x0, l, cfg, prm, window, cos, sin, dt, internals, **kw)
        raise AssertionError(kind)
    return blk


def _forward_row_no_final_norm(monkeypatch):
    calls = {"n": 0}
    real = _orig["rms_norm"]

    # The final norm is the last rms_norm call of forward_row on the full [T, C]
    # stream; drop it by making rms_norm the identity right after the last block.
    real_block = _orig["block"]

    def blk(*a, **k):
        out = real_block(*a, **k)
        calls["n"] += 1
        return out

    def norm(u, eps=0.0):
        if calls.get("armed"):
            calls["armed"] = False
            return u
        return real(u, eps)

    def blk_arm(x, x0, l, cfg, *rest, **kw):
        out = blk(x, x0, l, cfg, *rest, **kw)
        if l == cfg.n_layer - 1:
            calls["armed"] = True
        return out

    monkeypatch.setattr(oracle, "block", blk_arm)
    monkeypatch.setattr(oracle, "rms_norm", norm)


def _qk_no_norm(monkeypatch):
    real = _orig["rms_norm"]

    def norm(u, eps=0.0):
        if u.ndim == 3:           # per-head [T, H, D] tensors are only q and k
            return u
        return real(u, eps)
    monkeypatch.setattr(oracle, "rms_norm", norm)


def _no_pre_norm(monkeypatch):
    real = _orig["rms_norm"]
    real_block = _orig["block"]
    state = {"in_block": False, "count": 0}

    def norm(u, eps=0.0):
        if state["in_block"] and u.ndim == 2:
            state["count"] += 1
            if state["count"] == 1:    # the pre-attention norm of each block
                return u
        return real(u, eps)

    def blk(*a, **k):
        state["in_block"], state["count"] = True, 0
        try:
            return real_block(*a, **k)
        finally:
            state["in_block"] = False
    monkeypatch.setattr(oracle, "rms_norm", norm)
    monkeypatch.setattr(oracle, "block", blk)


def _ve_no_factor3(v, e, x_gate, w_gate):
    g = 1.0 / (1.0 + np.exp(-(x_gate @ w_gate.T)))
    return v + g[:, :, None] * e


def _ve_even_layers(l, n_layer):
    return l % 2 == 0


def _ve_gate_unnormed(monkeypatch):
    """Gate fed from the un-normalised residual stream instead of the block's normed input."""
    real_block = _orig["block"]
    real_mix = _orig["value_embed_mix"]
    state = {}

    def blk(x, x0, l, cfg, params, *a, **k):
        lam = float(np.asarray(params["resid_lambda"])[l])
        mu = float(np.asarray(params["x0_lambda"])[l])
        state["x"] = lam * x + mu * x0
        return real_block(x, x0, l, cfg, params, *a, **k)

    def mix(v, e, x_gate, w_gate):
        return real_mix(v, e, state["x"][:, :x_gate.shape[1]], w_gate)
    monkeypatch.setattr(oracle, "block", blk)
    monkeypatch.setattr(oracle, "value_embed_mix", mix)


def _prior_from_pass_two(q, k, v, q1, k1, g, window, scale):
    return _orig["attention_with_prior"](q, k, v, q, k, g, window, scale)


def _routing_reversed(monkeypatch):
    """Pass-2 layer l takes the prior of pass-1 layer L-1-l."""
    real_block = _orig["block"]
    caps = []

    def blk(x, x0, l, cfg, params, window, cos, sin, dt, internals=None, tokens=None, prior=None):
        if prior is None and getattr(cfg, "looped", False) and internals is not None and "q" not in internals:
            out = real_block(x, x0, l, cfg, params, window, cos, sin, dt, internals, tokens=tokens)
            caps.append((internals["q"], internals["k"]))
            return out
        if prior is not None:
            n = cfg.n_layer
            q1, k1 = caps[-n:][n - 1 - l]
            prior = (q1, k1, prior[2])
        return real_block(x, x0, l, cfg, params, window, cos, sin, dt, internals, tokens=tokens, prior=prior)
    monkeypatch.setattr(oracle, "block", blk)


def _prefix_norm_own_rms(u, c1, eps=0.0):
    first = _orig["rms_norm"](np.ascontiguousarray(u[..., :c1]), eps)
    if c1 == u.shape[-1]:
        return first
    return np.concatenate([first, _orig["rms_norm"](np.ascontiguousarray(u[..., c1:]), eps)], axis=-1)


def _top_k_drops_ties(z, k):
    """Exactly k tokens kept (a stable sort decides among equal logits)."""
    z = np.asarray(z)
    if k is None or k >= z.shape[-1]:
        return np.ones(z.shape, dtype=bool)
    keep = np.zeros(z.shape, dtype=bool)
    keep[np.argsort(-z, kind="stable")[:k]] = True
    return keep


def _sampler(temperature_op="div", greedy_last=False, strict=True):
    """A sampler with one planted mistake selected by the arguments."""
    def sample(zhat, top_k, temperature, u):
        z = np.asarray(zhat, dtype=np.float64)
        if temperature == 0.0:
            return int(len(z) - 1 - np.argmax(z[::-1])) if greedy_last else int(np.argmax(z))
        keep = oracle.top_k_keep(z, top_k)
        zs = z * temperature if temperature_op == "mul" else z / temperature
        s = np.where(keep, zs, -np.inf)
        e = np.exp(s - np.max(s))
        cdf = np.cumsum(e / np.sum(e))
        idx = int(np.searchsorted(cdf, u, side="right" if strict else "left"))
        return min(idx, z.shape[-1] - 1)
    return sample


def _blocktri_no_lower_block(x, blocks, in1):
    w1, w2 = blocks
    y1 = np.ascontiguousarray(x[..., :in1]) @ w1.T
    if w2.shape[0] == 0:
        return y1
    return np.concatenate([y1, x[..., in1:] @ w2[:, in1:].T], axis=-1)


MUTATIONS = {
    "rope_sign": (lambda mp: mp.setattr(oracle, "apply_rope", _rope_sign), [P.pin_rope_worked_example]),
    "rope_interleaved": (lambda mp: mp.setattr(oracle, "apply_rope", _rope_interleaved),
                         [P.pin_rope_is_complex_rotation]),
    "window_off_by_one": (lambda mp: mp.setattr(oracle, "visible_mask", _mask_off_by_one),
                          [P.pin_attention_identical_keys, P.pin_visible_mask_bruteforce]),
    "not_causal": (lambda mp: mp.setattr(oracle, "visible_mask", _mask_not_causal),
                   [P.pin_attention_locality, P.pin_causality_and_rows]),
    "relu_not_squared": (lambda mp: mp.setattr(oracle, "relu_squared", _relu),
                         [P.pin_relu_squared_worked_example, P.pin_relu_squared_homogeneity]),
    "no_softcap": (lambda mp: mp.setattr(oracle, "softcap", _no_softcap),
                   [P.pin_softcap_table, P.pin_logits_bounded]),
    "ce_wrong_target": (lambda mp: mp.setattr(oracle, "token_losses", _ce_off_index), [P.pin_cross_entropy]),
    "attention_no_scale": (lambda mp: mp.setattr(oracle, "attention", _attention_no_scale),
                           [P.pin_attention_bruteforce]),
    "gqa_modulo_map": (lambda mp: mp.setattr(oracle, "attention", _attention_mod_map),
                       [P.pin_attention_gqa_duplication]),
    "square_weight_transposed": (lambda mp: mp.setattr(oracle, "linear", _linear_square_transposed),
                                 [P.pin_head_permutation]),
    "no_x0_mix": (lambda mp: mp.setattr(oracle, "block", _block_patched("no_mix")), [P.pin_x0_reset]),
    "swapped_mix": (lambda mp: mp.setattr(oracle, "block", _block_patched("swap_mix")), [P.pin_x0_reset]),
    "no_final_norm": (_forward_row_no_final_norm, [P.pin_identity_blocks_closed_form]),
    "no_qk_norm": (_qk_no_norm, [P.pin_qk_scale_invariance, P.pin_internal_norms]),
    "no_pre_attn_norm": (_no_pre_norm, [P.pin_internal_norms]),
    "ve_gate_without_factor_3": (lambda mp: mp.setattr(oracle, "value_embed_mix", _ve_no_factor3),
                                 [P.pin_value_embedding_worked_example, P.pin_value_embedding_zero_gate]),
    "ve_on_even_layers": (lambda mp: mp.setattr(oracle, "has_ve", _ve_even_layers), [P.pin_ve_layer_rule]),
    "ve_gate_from_unnormed_stream": (_ve_gate_unnormed, [P.pin_value_embedding_gate_scale_invariance]),
    "gate_without_softplus": (lambda mp: mp.setattr(oracle, "softplus", lambda z: np.asarray(z, dtype=np.float64)),
                              [P.pin_softplus_library, P.pin_looped_equal_passes_closed_form]),
    "prior_from_pass_two": (lambda mp: mp.setattr(oracle, "attention_with_prior", _prior_from_pass_two),
                            [P.pin_looped_prior_comes_from_pass_one, P.pin_looped_augmented_width]),
    "routing_reversed": (_routing_reversed, [P.pin_looped_equal_passes_closed_form]),
    "prefix_norm_block2_own_rms": (lambda mp: mp.setattr(oracle, "prefix_rms_norm", _prefix_norm_own_rms),
                                   [P.pin_prefix_rms_norm]),
    "blocktri_without_lower_block": (lambda mp: mp.setattr(oracle, "blocktri_linear", _blocktri_no_lower_block),
                                     [P.pin_blocktri_zero_padded_dense]),
    "top_k_drops_ties": (lambda mp: mp.setattr(oracle, "top_k_keep", _top_k_drops_ties), [P.pin_top_k_keeps_ties]),
    "temperature_multiplies": (lambda mp: mp.setattr(oracle, "sample_next", _sampler(temperature_op="mul")),
                               [P.pin_sampling_closed_form_probabilities]),
    "greedy_last_index": (lambda mp: mp.setattr(oracle, "sample_next", _sampler(greedy_last=True)),
                          [P.pin_greedy_first_index_on_ties]),
    "cdf_not_strict": (lambda mp: mp.setattr(oracle, "sample_next", _sampler(strict=False)),
                       [P.pin_inverse_cdf_strict_boundary]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_caught(name, monkeypatch):
    apply, catchers = MUTATIONS[name]
    apply(monkeypatch)
    failed = []
    for pin in catchers:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} was not caught by {[p.__name__ for p in catchers]}"
