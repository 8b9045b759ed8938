"""Pins of the oracle against facts that do not come from the oracle itself.

Each pin is a function that raises AssertionError when the oracle disagrees
with a worked example printed on the pages (fixtures in tests/golden/), a
closed form, an invariant the pages state, a library routine, or a brute-force
computation on tiny inputs.  ``test_oracle_pins.py`` runs them all;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle and checks
that some pin catches each one.

Page citations: [M] = "The Mathematics of Karpathy's nanochat" (section named
per pin), [S] = "nanochat depth sweep", section "Architecture".
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special

import gptdata
import oracle
from helpers import dense_params, golden, small_preset

EX = golden("worked_examples.json")


def _round_eq(got, expected, decimals):
    got = np.round(np.asarray(got, dtype=np.float64), decimals)
    assert np.array_equal(got, np.round(np.asarray(expected, dtype=np.float64), decimals)), (got, expected)


# ----------------------------------------------------------------------------- RMSNorm

def pin_rmsnorm_worked_example():
    """[M] "RMS Normalization" worked example, to the printed 3 decimals."""
    e = EX["rmsnorm"]
    _round_eq(oracle.rms_norm(np.array(e["x"]), 0.0), e["expected"], e["decimals"])


def pin_rmsnorm_unit_rms():
    """[M] "RMS Normalization": the output has unit RMS (eps = 0), any scale."""
    rng = np.random.default_rng(1)
    for d in (1, 3, 128, 1536):
        u = rng.standard_normal((5, d)) * rng.uniform(0.01, 100, (5, 1))
        y = oracle.rms_norm(u, 0.0)
        assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-12)
        assert np.allclose(oracle.rms_norm(7.5 * u, 0.0), y, rtol=1e-13, atol=1e-13)


def pin_rmsnorm_eps_small_input():
    """With eps > 0, a tiny vector maps to u/sqrt(eps) scale, not unit RMS."""
    u = np.full(4, 1e-6)
    y = oracle.rms_norm(u, 1e-6)
    assert np.allclose(y, u / math.sqrt(1e-12 + 1e-6), rtol=1e-14)


# ----------------------------------------------------------------------------- RoPE

def pin_rope_worked_example():
    """[M] "Rotary Position Embeddings (RoPE)" worked example, d_h=4, base 1e5, t=5."""
    e = EX["rope"]
    T = e["position"] + 1
    cos, sin = oracle.rope_angles(T, e["head_dim"], e["base"])
    u = np.zeros((T, 1, e["head_dim"]))
    u[e["position"], 0] = e["q"]
    y = oracle.apply_rope(u, cos, sin)[e["position"], 0]
    _round_eq(y, e["expected"], e["decimals"])


def pin_rope_is_complex_rotation():
    """RoPE on the half-split pairs equals multiplying z_j = u_j + i u_{j+d/2} by
    exp(-i t omega_j), omega_j = base^(-2j/d) (complex arithmetic in NumPy)."""
    rng = np.random.default_rng(2)
    T, H, D, base = 9, 3, 16, 1e5
    u = rng.standard_normal((T, H, D))
    cos, sin = oracle.rope_angles(T, D, base)
    y = oracle.apply_rope(u, cos, sin)
    j = np.arange(D // 2)
    omega = base ** (-2.0 * j / D)
    ph = np.exp(-1j * np.arange(T)[:, None] * omega[None, :])[:, None, :]
    z = (u[..., :D // 2] + 1j * u[..., D // 2:]) * ph
    assert np.allclose(y[..., :D // 2], z.real, atol=1e-12)
    assert np.allclose(y[..., D // 2:], z.imag, atol=1e-12)


def pin_rope_relative_position():
    """[M] RoPE Proposition: <RoPE(q,m), RoPE(k,n)> depends on m - n only, and
    equals the proposition's sum over pairs with angle phi_{m-n}."""
    rng = np.random.default_rng(3)
    D, base = 8, 1e5
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    T = 40
    cos, sin = oracle.rope_angles(T, D, base)

    def rot(v, t):
        u = np.zeros((T, 1, D))
        u[t, 0] = v
        return oracle.apply_rope(u, cos, sin)[t, 0]

    for m, n, s in ((7, 3, 11), (20, 20, 5), (2, 9, 30)):
        a = rot(q, m) @ rot(k, n)
        b = rot(q, m + s) @ rot(k, n + s)
        assert abs(a - b) < 1e-12
        d2 = D // 2
        omega = base ** (-2.0 * np.arange(d2) / D)
        ph = (m - n) * omega
        q1, q2, k1, k2 = q[:d2], q[d2:], k[:d2], k[d2:]
        ref = np.sum((q1 * k1 + q2 * k2) * np.cos(ph) + (q2 * k1 - q1 * k2) * np.sin(ph))
        assert abs(a - ref) < 1e-12


def pin_rope_position_zero_and_norm():
    """Position 0 is the identity; RoPE preserves each head's norm, so it
    commutes with per-head RMSNorm."""
    rng = np.random.default_rng(4)
    T, H, D = 6, 2, 8
    u = rng.standard_normal((T, H, D))
    cos, sin = oracle.rope_angles(T, D, 1e5)
    y = oracle.apply_rope(u, cos, sin)
    assert np.array_equal(y[0], u[0])
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(u, axis=-1), atol=1e-12)
    assert np.allclose(oracle.rms_norm(y, 0.0), oracle.apply_rope(oracle.rms_norm(u, 0.0), cos, sin),
                       atol=1e-12)


def pin_qknorm_worked_example():
    """[M] "QK-Norm with Sharpening" worked example: RMSNorm of q1."""
    e = EX["qknorm"]
    _round_eq(oracle.rms_norm(np.array(e["q"]), 0.0), e["expected"], e["decimals"])


# ----------------------------------------------------------------------------- windows

def pin_layer_windows():
    """[M] "Sliding Window Pattern" and [S] "Architecture": SSSL tiled, last
    layer full.  d24: 18 short + 6 long; d12: 9 + 3; tiny: [128, 256]."""
    for name, n_short, n_long in (("d24", 18, 6), ("d12", 9, 3), ("tiny", 1, 1)):
        p = gptdata.preset(name)
        w = oracle.layer_windows(p.window_pattern, p.short_window, p.seq_len, p.n_layer)
        assert len(w) == p.n_layer and w[-1] == p.seq_len
        assert w.count(p.short_window) == n_short and w.count(p.seq_len) == n_long, (name, w)
        for l in range(p.n_layer - 1):
            assert w[l] == (p.seq_len if l % 4 == 3 else p.short_window)
    assert oracle.layer_windows("SSSL", 128, 256, 2) == [128, 256]


def pin_visible_mask_bruteforce():
    """Window rule by explicit loops: j <= i and i - j < w."""
    for T, w in ((7, 1), (7, 3), (9, 9), (5, 50)):
        m = oracle.visible_mask(T, w)
        for i in range(T):
            for j in range(T):
                assert m[i, j] == (j <= i and i - j < w)


# ----------------------------------------------------------------------------- attention

def _bruteforce_attention(q, k, v, window, scale):
    T, H, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros_like(q)
    for h in range(H):
        g = h * Hkv // H
        for i in range(T):
            js = [j for j in range(T) if j <= i and i - j < window]
            s = [scale * sum(q[i, h, d] * k[j, g, d] for d in range(D)) for j in js]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for d in range(D):
                out[i, h, d] = sum(e[n] * v[js[n], g, d] for n in range(len(js))) / z
    return out


def pin_attention_bruteforce():
    """Masked softmax attention against per-query Python loops (tiny T, GQA)."""
    rng = np.random.default_rng(5)
    for T, H, Hkv, D, w, sc in ((6, 2, 2, 4, 3, 0.5), (7, 4, 2, 3, 7, 1.3225), (5, 3, 1, 2, 1, 0.7)):
        q, k, v = rng.standard_normal((T, H, D)), rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
        assert np.allclose(oracle.attention(q, k, v, w, sc), _bruteforce_attention(q, k, v, w, sc), atol=1e-12)


def pin_attention_identical_keys():
    """Closed form: with every key equal, the softmax is uniform over the
    visible keys, so o_i is the mean of v_j over j in [max(0, i-w+1), i]."""
    rng = np.random.default_rng(6)
    T, D = 20, 4
    k = np.tile(rng.standard_normal((1, 1, D)), (T, 1, 1))
    q = rng.standard_normal((T, 1, D))
    v = rng.standard_normal((T, 1, D))
    for w in (1, 2, 5, 19, 20, 64):
        o = oracle.attention(q, k, v, w, 0.9)
        for i in range(T):
            lo = max(0, i - w + 1)
            assert np.allclose(o[i, 0], v[lo:i + 1, 0].mean(axis=0), atol=1e-12), (w, i)


def pin_attention_locality():
    """[M] window definition: perturbing keys/values outside query i's window
    (j > i or i - j >= w) leaves o_i bitwise unchanged; w = 1 gives o_i = v_i."""
    rng = np.random.default_rng(7)
    T, H, D, w = 16, 2, 4, 5
    q, k, v = (rng.standard_normal((T, H, D)) for _ in range(3))
    o = oracle.attention(q, k, v, w, 0.5)
    for i in (0, 4, 9, 15):
        k2, v2 = k.copy(), v.copy()
        for j in range(T):
            if j > i or i - j >= w:
                k2[j] += rng.standard_normal((H, D))
                v2[j] += rng.standard_normal((H, D))
        o2 = oracle.attention(q, k2, v2, w, 0.5)
        assert np.array_equal(o2[i], o[i])
    assert np.allclose(oracle.attention(q, k, v, 1, 0.5), v, atol=1e-15)
    assert np.array_equal(oracle.attention(q, k, v, T, 0.5), oracle.attention(q, k, v, 10 * T, 0.5))


def pin_attention_gqa_duplication():
    """GQA with Hkv heads equals MHA whose KV heads repeat each KV head for its
    contiguous group of H/Hkv query heads."""
    rng = np.random.default_rng(8)
    T, H, Hkv, D = 9, 6, 2, 4
    q = rng.standard_normal((T, H, D))
    k, v = rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    rep = np.repeat(np.arange(Hkv), H // Hkv)
    assert np.allclose(oracle.attention(q, k, v, 4, 0.6),
                       oracle.attention(q, k[:, rep], v[:, rep], 4, 0.6), atol=1e-14)


# ----------------------------------------------------------------------------- MLP, head

def pin_relu_squared_worked_example():
    """[M] "Feed-Forward Network (MLP)" worked example."""
    e = EX["relu_squared"]
    _round_eq(oracle.relu_squared(np.array(e["h"])), e["expected"], e["decimals"])


def pin_softcap_table():
    """[M] "Logit Softcap" worked example (rows printed correctly) and bounds."""
    e = EX["softcap"]
    _round_eq(oracle.softcap(np.array(e["z"]), e["cap"]), e["expected"], e["decimals"])
    z = np.linspace(-1e4, 1e4, 2001)
    y = oracle.softcap(z, 15.0)
    assert np.all(np.abs(y) <= 15.0) and np.all(np.diff(y) >= 0)
    assert np.allclose(oracle.softcap(-z, 15.0), -y)
    assert abs(oracle.softcap(np.array(1e-6), 15.0) - 1e-6) < 1e-15


def pin_cross_entropy():
    """Cross-entropy against scipy.special.logsumexp; zero logits give ln V;
    ignored targets give 0 and drop out of the mean; no valid target -> NaN."""
    rng = np.random.default_rng(9)
    z = rng.standard_normal((7, 33)) * 4
    y = rng.integers(0, 33, 7)
    y[2] = -1
    got = oracle.token_losses(z, y)
    for t in range(7):
        ref = 0.0 if y[t] < 0 else scipy.special.logsumexp(z[t]) - z[t, y[t]]
        assert abs(got[t] - ref) < 1e-12
    assert abs(oracle.mean_loss(got, y) - np.sum(got) / 6) < 1e-12
    V = EX["initial_loss"]["vocab"]
    l0 = oracle.token_losses(np.zeros((1, V)), np.array([17]))
    assert abs(l0[0] - math.log(V)) < 1e-12
    _round_eq(l0[0], EX["initial_loss"]["expected"], EX["initial_loss"]["decimals"])
    assert math.isnan(oracle.mean_loss(np.zeros(3), np.array([-1, -1, -1])))


# ----------------------------------------------------------------------------- whole model

def _fwd(p, params, tokens, targets=None, **kw):
    return oracle.forward(p, params, tokens, targets, **kw)


def _tokens(p, seed=11):
    rng = np.random.default_rng(seed)
    return rng.integers(0, p.vocab, (p.batch, p.seq_len + 1)).astype(np.int32)


def pin_identity_blocks_closed_form():
    """[M] end-to-end trace: with W_O = W_2 = 0 every block is the identity, so
    x stays a positive multiple of x0 and the logits are
    softcap(RMSNorm(W_E[t]) W_U^T) (RMSNorm computed here directly)."""
    p = small_preset(n_layer=3)
    prm = dense_params(p)
    prm["wo"] = [np.zeros_like(a) for a in prm["wo"]]
    prm["w2"] = [np.zeros_like(a) for a in prm["w2"]]
    prm["lm_head"] = prm["lm_head"] * 9.0   # push logits into the non-linear softcap range
    rows = _tokens(p)
    r = _fwd(p, prm, rows[:, :-1], want_logits=True)
    e = prm["wte"][rows[:, :-1]]
    xf = e / np.sqrt(np.mean(e * e, axis=-1, keepdims=True))
    z = xf @ prm["lm_head"].T
    assert np.allclose(r["logits"], 15.0 * np.tanh(z / 15.0), atol=1e-10)


def pin_zero_head_loss_is_ln_v():
    """W_U = 0 gives uniform logits, so every token's loss is ln V exactly."""
    p = small_preset(vocab=97)
    prm = dense_params(p)
    prm["lm_head"] = np.zeros_like(prm["lm_head"])
    rows = _tokens(p)
    r = _fwd(p, prm, rows[:, :-1], rows[:, 1:])
    assert np.allclose(r["losses"], math.log(97), atol=1e-12)
    assert abs(r["mean"] - math.log(97)) < 1e-12


def pin_logits_bounded():
    """[M] "Logit Softcap": every logit lies in (-15, 15)."""
    p = small_preset()
    prm = dense_params(p)
    prm["lm_head"] = prm["lm_head"] * 1e3
    rows = _tokens(p)
    z = _fwd(p, prm, rows[:, :-1], want_logits=True)["logits"]
    assert np.all(np.abs(z) <= 15.0) and np.max(np.abs(z)) > 14.0


def pin_causality_and_rows():
    """Outputs at position t do not depend on tokens after t; rows of a batch
    do not interact."""
    p = small_preset(n_layer=2, seq_len=10)
    prm = dense_params(p)
    rows = _tokens(p)
    tok = rows[:, :-1]
    z = _fwd(p, prm, tok, want_logits=True)["logits"]
    tok2 = tok.copy()
    tok2[0, 6:] = (tok2[0, 6:] + 5) % p.vocab
    z2 = _fwd(p, prm, tok2, want_logits=True)["logits"]
    assert np.array_equal(z2[0, :6], z[0, :6]) and np.array_equal(z2[1], z[1])
    assert not np.allclose(z2[0, 6:], z[0, 6:])


def pin_window_end_to_end():
    """One layer, MLP off (W_2 = 0): the logits at position i depend on token j
    iff j == i or j < i <= j + w - 1 (the window, [M] window definition)."""
    w = 3
    p = small_preset(n_layer=1, seq_len=10, short_window=w, window_pattern="S")
    prm = dense_params(p)
    prm["w2"] = [np.zeros_like(prm["w2"][0])]
    tok = _tokens(p)[:, :-1]
    win = [w]
    z = _fwd(p, prm, tok, want_logits=True, windows=win)["logits"]
    for j in (0, 4, 8):
        t2 = tok.copy()
        t2[0, j] = (t2[0, j] + 1) % p.vocab
        z2 = _fwd(p, prm, t2, want_logits=True, windows=win)["logits"]
        for i in range(p.seq_len):
            changed = not np.array_equal(z2[0, i], z[0, i])
            assert changed == (j <= i <= j + w - 1), (j, i)


def pin_head_permutation():
    """Permuting heads consistently (rows of W_Q/W_K/W_V by head, the matching
    input columns of W_O) leaves the model unchanged."""
    p = small_preset(n_head=3, n_kv_head=3, d_model=24, head_dim=8)
    prm = dense_params(p)
    rows = _tokens(p)
    z = _fwd(p, prm, rows[:, :-1], want_logits=True)["logits"]
    perm = np.array([2, 0, 1])
    idx = (perm[:, None] * p.head_dim + np.arange(p.head_dim)[None, :]).reshape(-1)
    for n in ("wq", "wk", "wv"):
        prm[n] = [a[idx] for a in prm[n]]
    prm["wo"] = [a[:, idx] for a in prm["wo"]]
    z2 = _fwd(p, prm, rows[:, :-1], want_logits=True)["logits"]
    assert np.allclose(z, z2, atol=1e-11)


def pin_relu_squared_homogeneity():
    """relu(c z)^2 = c^2 relu(z)^2: scaling W_1 by c and W_2 by 1/c^2 leaves the
    model unchanged (pins the square in the MLP)."""
    p = small_preset()
    prm = dense_params(p)
    rows = _tokens(p)
    z = _fwd(p, prm, rows[:, :-1], want_logits=True)["logits"]
    c = 3.0
    prm["w1"] = [a * c for a in prm["w1"]]
    prm["w2"] = [a / (c * c) for a in prm["w2"]]
    z2 = _fwd(p, prm, rows[:, :-1], want_logits=True)["logits"]
    assert np.allclose(z, z2, atol=1e-11)


def pin_qk_scale_invariance():
    """QK-norm makes the model invariant to positive scaling of W_Q and W_K
    (eps = 0), and the embedding norm to scaling of W_E."""
    p = small_preset()
    prm = dense_params(p)
    rows = _tokens(p)
    z = _fwd(p, prm, rows[:, :-1], want_logits=True)["logits"]
    prm["wq"] = [a * 5.0 for a in prm["wq"]]
    prm["wk"] = [a * 0.2 for a in prm["wk"]]
    prm["wte"] = prm["wte"] * 3.0
    z2 = _fwd(p, prm, rows[:, :-1], want_logits=True)["logits"]
    assert np.allclose(z, z2, atol=1e-11)


def pin_x0_reset():
    """[M] "Residual Stream with Learnable Scalars": lambda_l = 0, mu_l = 1 resets
    the stream to x0 at layer l, so the model equals the model made of layers
    l..L-1 alone; and lambda scales the incoming stream (checked with
    lambda_l = 0, mu_l = 2 against lambda_l = 0, mu_l = 1 on a no-op stack)."""
    p = small_preset(n_layer=3)
    prm = dense_params(p)
    rows = _tokens(p)
    tok = rows[:, :-1]
    prm["resid_lambda"][1] = 0.0
    prm["x0_lambda"][1] = 1.0
    full_w = oracle.layer_windows(p.window_pattern, p.short_window, p.seq_len, p.n_layer)
    z = _fwd(p, prm, tok, want_logits=True, windows=full_w)["logits"]
    sub = {k: (v[1:] if isinstance(v, list) else v) for k, v in prm.items()}
    sub["resid_lambda"] = prm["resid_lambda"][1:]
    sub["x0_lambda"] = prm["x0_lambda"][1:]
    ps = p.with_(n_layer=2)
    z2 = _fwd(ps, sub, tok, want_logits=True, windows=full_w[1:])["logits"]
    assert np.allclose(z, z2, atol=1e-11)
    # lambda weights the incoming stream: with no-op blocks the final norm hides
    # any positive scale, so instead compare lambda=1,mu=0 (pure residual) with
    # lambda=0,mu=1 after one real block: they must differ.
    prm2 = dense_params(p.with_(n_layer=2))
    prm2["resid_lambda"][1], prm2["x0_lambda"][1] = 1.0, 0.0
    za = _fwd(p.with_(n_layer=2), prm2, tok, want_logits=True)["logits"]
    prm2["resid_lambda"][1], prm2["x0_lambda"][1] = 0.0, 1.0
    zb = _fwd(p.with_(n_layer=2), prm2, tok, want_logits=True)["logits"]
    assert not np.allclose(za, zb)


def pin_internal_norms():
    """Every normalised tensor the pages name has unit RMS (eps = 0): the
    embedding x0, the pre-attention and pre-MLP inputs, per-head q and k after
    QK-norm, and the final norm."""
    p = small_preset(n_layer=2)
    prm = dense_params(p)
    tok = _tokens(p)[0, :-1]
    r = oracle.forward_row(p, prm, tok, None, want_internals=True)

    def unit(a):
        return np.allclose(np.mean(a * a, axis=-1), 1.0, atol=1e-12)

    assert unit(r["x0"]) and unit(r["xf"])
    for li in r["layers"]:
        assert unit(li["xn"]) and unit(li["xm"]) and unit(li["q"]) and unit(li["k"])
        assert not unit(li["v"])


# ----------------------------------------------------------------------------- value embeddings

def pin_value_embedding_worked_example():
    """[M] "Value Embeddings (ResFormer)" worked example: one KV head, d_h = 3, gate logit 1.2
    (a one-channel gate input of 1 and weight 1.2 give that logit).  The page rounds
    sigmoid(1.2) to 3 decimals before scaling, so the gate is checked through the sigmoid to
    the printed decimals and the gate and mixed value within what that rounding implies
    (3 * 0.0005 on the gate, that times |e| plus the printed half-unit on the value)."""
    e = EX["value_embedding"]
    v = np.array(e["v"]).reshape(1, 1, 3)
    ev = np.array(e["e"]).reshape(1, 1, 3)
    out = oracle.value_embed_mix(v, ev, np.ones((1, 1)), np.array([[e["gate_logit"]]]))
    g = (out[0, 0, 0] - e["v"][0]) / e["e"][0]
    _round_eq(g / 3.0, e["expected_sigmoid"], e["sigmoid_decimals"])
    tol_g = 3 * 0.5 * 10.0 ** -e["sigmoid_decimals"]
    assert abs(g - e["expected_gate"]) <= tol_g + 1e-12
    tol_v = tol_g * np.abs(np.array(e["e"])) + 0.5 * 10.0 ** -e["decimals"]
    assert np.all(np.abs(out.reshape(3) - np.array(e["expected"])) <= tol_v + 1e-12), out


def pin_value_embedding_zero_gate():
    """A zero gate weight gives g = 3 * sigmoid(0) = 1.5 exactly, whatever the input."""
    rng = np.random.default_rng(3)
    v, e = rng.standard_normal((5, 2, 4)), rng.standard_normal((5, 2, 4))
    out = oracle.value_embed_mix(v, e, rng.standard_normal((5, 12)), np.zeros((2, 12)))
    assert np.allclose(out, v + 1.5 * e, rtol=0, atol=1e-15)


def pin_ve_layer_rule():
    """[M] "Value Embeddings (ResFormer)": alternating layers with the last one always
    included -- L = 24 selects the odd layers, L = 5 the even ones."""
    assert [l for l in range(24) if oracle.has_ve(l, 24)] == list(range(1, 24, 2))
    assert [l for l in range(5) if oracle.has_ve(l, 5)] == [0, 2, 4]
    for L in range(1, 9):
        assert oracle.has_ve(L - 1, L)
        assert all(oracle.has_ve(l, L) != oracle.has_ve(l + 1, L) for l in range(L - 1))


def _ve_preset(**kw):
    base = dict(n_layer=3, n_head=4, n_kv_head=2, head_dim=4, d_model=16, value_embeds=True)
    base.update(kw)
    return small_preset(**base)


def pin_value_embedding_zero_tables():
    """All-zero value-embedding tables leave the forward pass exactly as without them."""
    p = _ve_preset()
    prm = dense_params(p)
    prm["ve"] = [np.zeros_like(a) for a in prm["ve"]]
    rows = _tokens(p)
    a = _fwd(p, prm, rows[:, :-1], rows[:, 1:], want_logits=True)
    b = _fwd(p.with_(value_embeds=False), prm, rows[:, :-1], rows[:, 1:], want_logits=True)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["losses"], b["losses"])
    c = _fwd(p, dense_params(p), rows[:, :-1], rows[:, 1:])   # non-zero tables do change it
    assert not np.allclose(c["losses"], a["losses"])


def pin_value_embedding_gate_scale_invariance():
    """The gate reads the block's normalised input, so scaling the residual stream entering
    a block (x and x0 together) leaves the mixed values unchanged; the last layer (which
    always has a value embedding) is checked."""
    p = _ve_preset(n_layer=2)
    prm = dense_params(p)
    rng = np.random.default_rng(5)
    T, C = p.seq_len, p.d_model
    x, x0 = rng.standard_normal((T, C)), rng.standard_normal((T, C))
    tok = rng.integers(0, p.vocab, T)
    cos, sin = oracle.rope_angles(T, p.head_dim, p.rope_base)
    l = p.n_layer - 1
    ia, ib = {}, {}
    oracle.block(x, x0, l, p, prm, T, cos, sin, np.float64, ia, tokens=tok)
    oracle.block(37.0 * x, 37.0 * x0, l, p, prm, T, cos, sin, np.float64, ib, tokens=tok)
    assert np.allclose(ia["v"], ib["v"], rtol=1e-12, atol=1e-12)
    base = {}
    oracle.block(x, x0, l, p.with_(value_embeds=False), prm, T, cos, sin, np.float64, base, tokens=tok)
    assert not np.allclose(ia["v"], base["v"])


# ----------------------------------------------------------------------------- looped trunk

def pin_softplus_library():
    """The routing gate's softplus against numpy's log(exp(0) + exp(z)), from -1000 to 1000."""
    z = np.concatenate([np.linspace(-60, 60, 241), [-1000.0, -745.0, 0.0, 745.0, 1000.0]])
    assert np.allclose(oracle.softplus(z), np.logaddexp(0.0, z), rtol=1e-15, atol=0)
    assert oracle.softplus(0.0) == math.log(2.0)


def pin_looped_augmented_width():
    """[L] "What is the routing loop?": the prior q2 k2^T + g q1 k1^T equals ordinary attention
    over the augmented-width Q = [q2, sqrt(g) q1], K = [k2, sqrt(g) k1] (GQA 4:2, two windows)."""
    rng = np.random.default_rng(8)
    T, H, Hkv, D = 9, 4, 2, 5
    q, q1 = rng.standard_normal((T, H, D)), rng.standard_normal((T, H, D))
    k, k1, v = (rng.standard_normal((T, Hkv, D)) for _ in range(3))
    for g, w in ((0.37, 4), (2.5, 9)):
        r = math.sqrt(g)
        aug = oracle.attention(np.concatenate([q, r * q1], -1), np.concatenate([k, r * k1], -1), v, w, 0.6)
        got = oracle.attention_with_prior(q, k, v, q1, k1, g, w, 0.6)
        assert np.allclose(got, aug, rtol=1e-12, atol=1e-12)


def _loop_preset(**kw):
    base = dict(n_layer=2, n_head=2, n_kv_head=2, head_dim=8, d_model=16, looped=True)
    base.update(kw)
    return small_preset(**base)


def pin_looped_zero_gate_is_plain_with_pass_embedding():
    """Gate logits of -1000 make g = 0, so pass 1 has no effect and the result is the plain
    model whose embedding rows are W_E[t] + pass_emb[1] (bitwise)."""
    p = _loop_preset(n_layer=3)
    prm = dense_params(p)
    prm["gate_logit"] = np.full(p.n_layer, -1000.0)
    rows = _tokens(p)
    a = _fwd(p, prm, rows[:, :-1], rows[:, 1:], want_logits=True)
    plain = dict(prm)
    plain["wte"] = prm["wte"] + prm["pass_emb"][1]
    b = _fwd(p.with_(looped=False), plain, rows[:, :-1], rows[:, 1:], want_logits=True)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["losses"], b["losses"])


def pin_looped_equal_passes_closed_form():
    """With equal pass embeddings, pass 1's layer-0 q and k are pass 2's own, so (gate of
    layer 1 off) layer 0's logits become (1 + g_0) times the plain ones: the looped model
    equals plain blocks with attention scale s(1 + softplus(logit_0)) on layer 0."""
    p = _loop_preset()
    prm = dense_params(p)
    prm["pass_emb"] = np.stack([prm["pass_emb"][0], prm["pass_emb"][0]])
    prm["gate_logit"] = np.array([0.8, -1000.0])
    rows = _tokens(p)
    tok, tgt = rows[0, :-1], rows[0, 1:]
    got = _fwd(p, prm, tok[None], tgt[None], want_logits=True)
    T = p.seq_len
    cos, sin = oracle.rope_angles(T, p.head_dim, p.rope_base)
    win = oracle.layer_windows(p.window_pattern, p.short_window, T, p.n_layer)
    g0 = math.log1p(math.exp(0.8))
    x = oracle.rms_norm(prm["wte"][tok] + prm["pass_emb"][0], p.norm_eps)
    x0 = x
    base = p.with_(looped=False)
    x = oracle.block(x, x0, 0, base.with_(qk_scale=p.attn_scale * (1.0 + g0)), prm, win[0], cos, sin, np.float64)
    x = oracle.block(x, x0, 1, base, prm, win[1], cos, sin, np.float64)
    z = oracle.softcap(oracle.rms_norm(x, p.norm_eps) @ prm["lm_head"].T, p.softcap)
    assert np.allclose(got["logits"][0], z, rtol=1e-10, atol=1e-10)


def pin_looped_prior_comes_from_pass_one():
    """Different pass embeddings give pass 1 different q, k than pass 2 has, so the single
    layer's result departs from the equal-passes closed form (which it meets when they match)."""
    p = _loop_preset(n_layer=1)
    prm = dense_params(p)
    rows = _tokens(p)
    tok, tgt = rows[:, :-1], rows[:, 1:]
    g0 = float(oracle.softplus(prm["gate_logit"][0]))
    plain = dict(prm)
    plain["wte"] = prm["wte"] + prm["pass_emb"][1]
    ref = _fwd(p.with_(looped=False, qk_scale=p.attn_scale * (1.0 + g0)), plain, tok, tgt)
    got = _fwd(p, prm, tok, tgt)
    assert not np.allclose(got["losses"], ref["losses"], rtol=1e-6, atol=1e-6)
    same = dict(prm)
    same["pass_emb"] = np.stack([prm["pass_emb"][1], prm["pass_emb"][1]])
    assert np.allclose(_fwd(p, same, tok, tgt)["losses"], ref["losses"], rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------------------- nested model

def _nest_preset(**kw):
    base = dict(n_layer=2, n_head=4, n_kv_head=4, head_dim=8, d_model=32, mlp_dim=128,
                nested_c1=8, seq_len=12, vocab=50)
    base.update(kw)
    return small_preset(**base)


def _inner_params(prm, c1):
    inner = {"wte": np.ascontiguousarray(prm["wte"][:, :c1]),
             "lm_head": np.ascontiguousarray(prm["lm_head"][:, :c1]),
             "resid_lambda": prm["resid_lambda"], "x0_lambda": prm["x0_lambda"]}
    for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
        inner[n] = [blocks[0] for blocks in prm[n]]
    return inner


def pin_nested_inner_equals_standalone():
    """[F]: the top-left corner of the nested network is the smaller model -- the kfront=1
    losses and logits of one pass of the full model equal, bitwise, those of the standalone
    inner model (width c1, the first heads, the inner MLP width, W_E and W_U restricted to
    the first c1 columns, the diagonal blocks of every linear)."""
    p = _nest_preset()
    prm = dense_params(p)
    rows = _tokens(p)
    tok, tgt = rows[:, :-1], rows[:, 1:]
    got = _fwd(p, prm, tok, tgt, want_logits=True)
    c1 = p.nested_c1
    inner = p.with_(nested_c1=0, d_model=c1, n_head=p.n_head * c1 // p.d_model,
                    n_kv_head=p.n_kv_head * c1 // p.d_model, mlp_dim=p.mlp_dim * c1 // p.d_model)
    ref = _fwd(inner, _inner_params(prm, c1), tok, tgt, want_logits=True)
    assert np.array_equal(got["logits_k1"], ref["logits"])
    assert np.array_equal(got["losses_k1"], ref["losses"]) and got["mean_k1"] == ref["mean"]
    assert not np.allclose(got["losses"], got["losses_k1"])


def pin_nested_one_block_is_plain():
    """With a single block (c1 = C) the nested forward is the plain model, bitwise."""
    p = _nest_preset(nested_c1=32)
    prm = dense_params(p)
    rows = _tokens(p)
    tok, tgt = rows[:, :-1], rows[:, 1:]
    got = _fwd(p, prm, tok, tgt, want_logits=True)
    plain = dict(prm)
    for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
        plain[n] = [blocks[0] for blocks in prm[n]]
    ref = _fwd(p.with_(nested_c1=0), plain, tok, tgt, want_logits=True)
    assert np.array_equal(got["logits"], ref["logits"]) and np.array_equal(got["losses"], ref["losses"])


def pin_blocktri_zero_padded_dense():
    """[F]: a block lower triangular linear is the dense product with the upper block zero."""
    rng = np.random.default_rng(12)
    o1, o2, i1, i2 = 3, 5, 4, 6
    w1, w2 = rng.standard_normal((o1, i1)), rng.standard_normal((o2, i1 + i2))
    dense = np.zeros((o1 + o2, i1 + i2))
    dense[:o1, :i1], dense[o1:, :] = w1, w2
    x = rng.standard_normal((7, i1 + i2))
    assert np.allclose(oracle.blocktri_linear(x, [w1, w2], i1), x @ dense.T, rtol=1e-13, atol=1e-13)


def pin_prefix_rms_norm():
    """PrefixRMSNorm: the first block is RMSNorm of the prefix (unit RMS, blind to the rest:
    changing the second block leaves it bitwise unchanged); with a zero prefix the second
    block is x2 / RMS(x) over all C dims, whose RMS over its own C - c1 dims is sqrt(C/(C-c1))."""
    rng = np.random.default_rng(13)
    C, c1 = 12, 4
    x = rng.standard_normal((6, C)) * rng.uniform(0.1, 10, (6, 1))
    y = oracle.prefix_rms_norm(x, c1, 0.0)
    assert np.allclose(np.mean(y[:, :c1] ** 2, axis=-1), 1.0, rtol=0, atol=1e-12)
    x2 = x.copy()
    x2[:, c1:] *= 7.0
    assert np.array_equal(oracle.prefix_rms_norm(x2, c1, 0.0)[:, :c1], y[:, :c1])
    z = x.copy()
    z[:, :c1] = 0.0
    yz = oracle.prefix_rms_norm(z, c1, 1e-30)   # tiny eps: the zero prefix itself stays finite
    assert np.allclose(np.sqrt(np.mean(yz[:, c1:] ** 2, axis=-1)), math.sqrt(C / (C - c1)), rtol=1e-12)


def pin_nested_filtration():
    """Changing only weights that act on or produce the second block (row block 2 of every
    linear, the lm_head's later columns) leaves the kfront=1 losses bitwise unchanged."""
    p = _nest_preset()
    prm = dense_params(p)
    rows = _tokens(p)
    tok, tgt = rows[:, :-1], rows[:, 1:]
    a = _fwd(p, prm, tok, tgt)
    prm2 = dict(prm)
    for n in ("wq", "wk", "wv", "wo", "w1", "w2"):
        prm2[n] = [[b0, 3.0 * b1] for b0, b1 in prm[n]]
    prm2["lm_head"] = prm["lm_head"].copy()
    prm2["lm_head"][:, p.nested_c1:] *= -2.0
    b = _fwd(p, prm2, tok, tgt)
    assert np.array_equal(a["losses_k1"], b["losses_k1"])
    assert not np.allclose(a["losses"], b["losses"])


# ----------------------------------------------------------------------------- generation

def pin_sampling_worked_example_greedy():
    """[M] "Inference: Generating Text" worked example: at temperature 0 the draw is the
    largest logit ("announced"), whatever u and top-k are."""
    e = EX["sampling"]
    z = np.array(e["logits"])
    for u in (0.0, 0.3, 0.999):
        for k in (None, 1, 3):
            assert oracle.sample_next(z, k, 0.0, u) == e["greedy"]


def pin_greedy_first_index_on_ties():
    """Temperature 0 is the argmax; among equal maxima the first index (brute force)."""
    rng = np.random.default_rng(21)
    for _ in range(50):
        z = rng.integers(-3, 4, size=9).astype(np.float64)
        best = 0
        for i in range(9):
            if z[i] > z[best]:
                best = i
        assert oracle.sample_next(z, None, 0.0, 0.5) == best


def pin_sampling_closed_form_probabilities():
    """[M] "Sampling Controls": with logits tau*ln(1, 2, 4) (+ any shift) the temperature
    softmax is (1/7, 2/7, 4/7) exactly, so midpoints of a uniform grid of 7000 draws split
    1000 / 2000 / 4000 (the inverse CDF in vocabulary order)."""
    tau = 0.8
    z = tau * np.log(np.array([1.0, 2.0, 4.0])) + 3.25
    n = 7000
    counts = np.zeros(3, dtype=int)
    for i in range(n):
        counts[oracle.sample_next(z, None, tau, (i + 0.5) / n)] += 1
    assert counts.tolist() == [1000, 2000, 4000], counts


def pin_sampling_temperature_scale_invariance():
    """Only z / tau matters: scaling logits and temperature together leaves every draw."""
    rng = np.random.default_rng(22)
    z = rng.standard_normal(40) * 3
    for u in rng.random(200):
        assert oracle.sample_next(z, 7, 0.7, u) == oracle.sample_next(2.5 * z, 7, 1.75, u)


def pin_top_k_keeps_ties():
    """[M] "Sampling Controls" top-k: tokens below the k-th largest logit are removed, so logits
    equal to it stay; with two equal maxima and k = 1 both are drawn, each for half of u."""
    z = np.array([1.0, 3.0, 3.0, 2.0])
    assert oracle.top_k_keep(z, 1).tolist() == [False, True, True, False]
    assert oracle.top_k_keep(z, 3).tolist() == [False, True, True, True]
    assert oracle.top_k_keep(z, None).all() and oracle.top_k_keep(z, 4).all()
    for tau in (0.3, 1.0, 5.0):
        assert oracle.sample_next(z, 1, tau, 0.25) == 1 and oracle.sample_next(z, 1, tau, 0.75) == 2


def pin_top_k_one_is_greedy():
    """Top-1 sampling at any temperature and u is the argmax (distinct logits)."""
    rng = np.random.default_rng(23)
    for _ in range(100):
        z = rng.standard_normal(30)
        assert oracle.sample_next(z, 1, float(rng.uniform(0.1, 3)), float(rng.random())) == int(np.argmax(z))


def pin_inverse_cdf_strict_boundary():
    """Two equal logits: the cumulative probability of token 0 is exactly 1/2, and the draw is
    the first token whose cumulative probability exceeds u, so u = 1/2 draws token 1."""
    z = np.array([0.5, 0.5])
    assert oracle.sample_next(z, None, 1.0, 0.4999) == 0
    assert oracle.sample_next(z, None, 1.0, 0.5) == 1


def pin_generation_logits_are_one_forward():
    """Causality: the logits that each generation step samples from equal the logits at the
    same positions of one forward pass over the final sequence."""
    p = small_preset(n_layer=2, seq_len=16, vocab=40, short_window=5)
    prm = dense_params(p)
    rng = np.random.default_rng(24)
    prompt = rng.integers(0, p.vocab, size=(2, 5))
    u = rng.random((6, 2))
    g = oracle.generate(p, prm, prompt, 6, top_k=10, temperature=0.9, u=u)
    full = oracle.forward(p, prm, g["tokens"][:, :-1], want_logits=True,
                          windows=oracle.layer_windows(p.window_pattern, p.short_window, p.seq_len, p.n_layer))
    for i in range(6):
        assert np.allclose(g["logits"][i], full["logits"][:, 4 + i, :], rtol=1e-10, atol=1e-12)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
