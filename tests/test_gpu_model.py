"""End-to-end parity of gpt_fwd_loss (through the C ABI) against the oracle.

Bars (fixed for this path): fp32 path -- relative error of the mean loss <= 1e-4 and logits
within 1e-3 of the largest |logit|; bf16 path -- per-token loss |error| <= 2e-2 and mean-loss
|error| <= 5e-3, logits |error| RMS <= 6e-3 and max <= 3e-2.

At the full sizes of the workload presets (d12, d24, d24gve, d24loop, d24nest) every row of the
batch is compared: the GPU runs the whole batch once, in the launch configuration the benchmark
times, and the oracle (in float32, which differs from its float64 form by ~1e-6 in the loss)
evaluates one row per test (rows never interact, so a row's losses are exactly the oracle's
forward of that row); a last test per preset checks the mean over all B*T tokens.
"""
import dataclasses
import math
import os

import numpy as np
import pytest

import decoder_only_transformer_layer_amd as gf
import gptdata
import oracle
from gpu_helpers import params_of, torch_mod

pytestmark = pytest.mark.gpu


def _run(p, w, tok, tgt, want_logits=False, windows=None):
    torch = torch_mod()
    m = gf.DeviceModel(p, w, batch=tok.shape[0], windows=windows)
    t_tok = torch.from_numpy(tok).cuda()
    t_tgt = torch.from_numpy(tgt).cuda() if tgt is not None else None
    loss, mean, logits = m(t_tok, t_tgt, want_logits=want_logits)
    torch.cuda.synchronize()
    out = {
        "losses": None if loss is None else loss.cpu().numpy().astype(np.float64),
        "mean": None if mean is None else float(mean.item()),
        "logits": None if logits is None else logits.cpu().numpy().astype(np.float64),
        "status": m.device_status(),
    }
    return m, out


def _check_bf16(got, ref, rows=None):
    lg = got["losses"] if rows is None else got["losses"][rows]
    err = np.abs(lg - ref["losses"])
    print(f"  per-token |err| max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2, err.max()
    if rows is None:
        assert abs(got["mean"] - ref["mean"]) <= 5e-3
    else:
        valid = ref["losses"] != 0
        assert abs(lg[valid].mean() - ref["losses"][valid].mean()) <= 5e-3


def _check_logits_bf16(got, ref):
    """bf16 logits: every operand of the last product is a bf16-rounded activation (unit
    roundoff 2^-9), so each logit carries an error of a few 1e-3 (RMS); the bar is on that RMS
    and on the maximum over all B*T*V logits, which for ~1e6 samples lies about 5 RMS out."""
    d = got - ref
    rms, mx = float(np.sqrt(np.mean(d * d))), float(np.max(np.abs(d)))
    print(f"  logits |err| rms {rms:.3e} max {mx:.3e}")
    assert rms <= 6e-3 and mx <= 3e-2
    assert np.all(np.abs(got) <= 15.0)


def test_tiny_fp32():
    """Tiny fp32 config: depth 2, width 128, one head of 128, V=4096, T=256, B=2."""
    p = gptdata.preset("tiny")
    w, tok, tgt = gptdata.make_inputs(p)
    _, got = _run(p, w, tok, tgt, want_logits=True)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True)
    assert got["status"] == gf.GPT_OK
    rel = abs(got["mean"] - ref["mean"]) / abs(ref["mean"])
    zerr = np.max(np.abs(got["logits"] - ref["logits"])) / np.max(np.abs(ref["logits"]))
    print(f"  tiny fp32: mean rel err {rel:.2e}, logits err/max {zerr:.2e}")
    assert rel <= 1e-4
    assert zerr <= 1e-3
    assert np.max(np.abs(got["losses"] - ref["losses"])) <= 1e-3


def _ragged_preset(**kw):
    base = dict(name="ragged", n_layer=3, d_model=256, n_head=4, n_kv_head=2, head_dim=128,
                mlp_dim=1024, vocab=1000, seq_len=320, batch=2, dtype="bf16", short_window=100,
                lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=5)
    base.update(kw)
    return gptdata.Preset(**base)


def test_ragged_bf16_gqa_with_ignores_and_logits():
    """Tails everywhere: B*T = 640 rows (not a multiple of 256), T = 320 (2.5 query tiles),
    V = 1000 (not a multiple of 128), GQA 4:2, windows 100/64/full, 10% ignored targets."""
    p = _ragged_preset()
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.1)
    windows = [100, 64, 320]
    _, got = _run(p, w, tok, tgt, want_logits=True, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True, windows=windows)
    _check_bf16(got, ref)
    assert np.all(got["losses"][tgt == -1] == 0.0)
    _check_logits_bf16(got["logits"], ref["logits"])


def test_qkv_384_tiles_bf16_ragged():
    """q, k and v each a multiple of three 128-wide heads (6 query heads, 3 KV heads): the q/k/v
    projection runs as one launch of 256x384 tiles in RoPE-pair column order, here with the
    input row scale of layers >= 1 and B*T = 576 rows (the last row block partial)."""
    p = _ragged_preset(d_model=512, n_head=6, n_kv_head=3, mlp_dim=1024, seq_len=192, batch=3,
                       seed=19)
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.05)
    windows = [100, 64, 192]
    _, got = _run(p, w, tok, tgt, want_logits=True, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True, windows=windows)
    _check_bf16(got, ref)
    _check_logits_bf16(got["logits"], ref["logits"])


def test_head_dim_64_bf16():
    p = _ragged_preset(n_head=4, n_kv_head=2, head_dim=64, seq_len=256, vocab=777, seed=9)
    w, tok, tgt = gptdata.make_inputs(p)
    _, got = _run(p, w, tok, tgt)
    _check_bf16(got, oracle.forward(p, params_of(w), tok, tgt))


def test_single_row_bf16():
    """One row of 64 tokens (the shortest bf16 sequence): B*T = 64 rows, a quarter of one
    256-row GEMM tile and a single query tile; V = 333; windows 24 / full; 10% ignored targets;
    the logits as well."""
    p = _ragged_preset(n_layer=2, seq_len=64, batch=1, vocab=333, seed=13)
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.1)
    windows = [24, 64]
    _, got = _run(p, w, tok, tgt, want_logits=True, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True, windows=windows)
    assert got["status"] == gf.GPT_OK
    _check_bf16(got, ref)
    assert np.all(got["losses"][tgt == -1] == 0.0)
    _check_logits_bf16(got["logits"], ref["logits"])


def test_edge_cases_bf16():
    """Window 1 everywhere; an out-of-range token; all targets ignored; minimal T."""
    p = _ragged_preset(n_layer=2, seq_len=64, batch=3, vocab=300, seed=11)
    w, tok, tgt = gptdata.make_inputs(p)
    # window 1: attention returns each position's own value
    _, got = _run(p, w, tok, tgt, windows=[1, 1])
    _check_bf16(got, oracle.forward(p, params_of(w), tok, tgt, windows=[1, 1]))
    # out-of-range token: its loss is NaN and the device status reports it
    bad = tok.copy()
    bad[1, 5] = p.vocab + 3
    _, got = _run(p, w, bad, tgt)
    assert got["status"] == gf.GPT_E_DEVICE_INPUT
    assert math.isnan(got["losses"][1, 5])
    # out-of-range target
    badt = tgt.copy()
    badt[0, 0] = p.vocab
    _, got = _run(p, w, tok, badt)
    assert got["status"] == gf.GPT_E_DEVICE_INPUT and math.isnan(got["losses"][0, 0])
    # no valid target: mean is NaN
    _, got = _run(p, w, tok, np.full_like(tgt, -1))
    assert got["status"] == gf.GPT_OK and math.isnan(got["mean"])
    # logits only (no targets)
    _, got = _run(p, w, tok, None, want_logits=True)
    ref = oracle.forward(p, params_of(w), tok, None, want_logits=True)
    _check_logits_bf16(got["logits"], ref["logits"])


def test_deterministic_bf16():
    p = _ragged_preset(seed=13)
    w, tok, tgt = gptdata.make_inputs(p)
    torch = torch_mod()
    m = gf.DeviceModel(p, w)
    t_tok, t_tgt = torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()
    a, am, _ = m(t_tok, t_tgt)
    b, bm, _ = m(t_tok, t_tgt)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(am, bm)


# ----------------------------------------------------------------------------- full sizes

FULL_ROWS = {"d12": 4, "d24": 8, "d24gve": 8, "d24loop": 4, "d24nest": 4}
_INPUTS = {}
_FULL = {}


def _inputs(name):
    """Seeded inputs of a workload preset (generated once per session)."""
    if name not in _INPUTS:
        p = gptdata.preset(name)
        w, tok, tgt = gptdata.make_inputs(p)
        _INPUTS[name] = (p, w, tok, tgt)
    return _INPUTS[name]


def _full(name):
    """The GPU's outputs for the whole batch of preset `name` (one call, computed once) and the
    oracle's rows, filled in as the row tests run."""
    if name not in _FULL:
        p, w, tok, tgt = _inputs(name)
        got = (_run_nested if p.nested_c1 else _run)(p, w, tok, tgt)[1]
        assert got["status"] == gf.GPT_OK
        _FULL[name] = {"p": p, "tok": tok, "tgt": tgt, "got": got, "prm": params_of(w), "rows": {}}
    return _FULL[name]


def _oracle_row(f, b):
    if b not in f["rows"]:
        f["rows"][b] = oracle.forward(f["p"], f["prm"], f["tok"], f["tgt"], rows=[b], dtype=np.float32)
    return f["rows"][b]


def _suffixes(f):
    return ("", "_k1") if f["p"].nested_c1 else ("",)


def _check_row(name, b):
    f = _full(name)
    ref = _oracle_row(f, b)
    for sfx in _suffixes(f):
        err = np.abs(f["got"]["losses" + sfx][b] - ref["losses" + sfx][0])
        print(f"  {name}{sfx} row {b}: per-token |err| max {err.max():.3e} mean {err.mean():.3e}", flush=True)
        assert err.max() <= 2e-2, (name, sfx, b, err.max())


def _check_mean(name):
    """Every row against the oracle (rows not yet evaluated are evaluated here), then the mean
    over all B*T tokens; the preset's buffers are released afterwards."""
    f = _full(name)
    try:
        for sfx in _suffixes(f):
            ref = np.concatenate([_oracle_row(f, b)["losses" + sfx] for b in range(f["p"].batch)])
            got = f["got"]["losses" + sfx]
            err = np.abs(got - ref)
            ref_mean = oracle.mean_loss(ref, f["tgt"])
            merr = abs(f["got"]["mean" + sfx] - ref_mean)
            print(f"  {name}{sfx} all {got.size} tokens: per-token |err| max {err.max():.3e} "
                  f"mean {err.mean():.3e}; mean loss gpu {f['got']['mean' + sfx]:.6f} oracle "
                  f"{ref_mean:.6f} |err| {merr:.3e}", flush=True)
            assert err.max() <= 2e-2 and merr <= 5e-3
    finally:
        _FULL.pop(name, None)


@pytest.mark.parametrize("b", range(FULL_ROWS["d12"]))
def test_d12_row(b):
    """nanochat d12 at its full size (B=4, T=2048), row b against the oracle."""
    _check_row("d12", b)


def test_d12_all_tokens():
    _check_mean("d12")


@pytest.mark.parametrize("b", range(FULL_ROWS["d24"]))
def test_d24_row(b):
    """nanochat d24 at the benchmarked size and launch (B=8, T=2048), row b against the oracle."""
    _check_row("d24", b)


def test_d24_all_tokens():
    _check_mean("d24")


@pytest.fixture(scope="module")
def d24():
    return _inputs("d24")


def test_d24_bf16_past_32bit_offsets(d24):
    """B=176 at the d24 shape: 360,448 rows, so the MLP activations hold more than 2^31 elements
    and the fp32 residual stream more than 2^31 bytes (14.6 GB of workspace).  Every loss must be
    finite, and the oracle's 512-token prefixes of the first and the last row (the latter past
    both 32-bit boundaries) must match."""
    p0, w, _, _ = d24
    p = p0.with_(batch=176)
    tok, tgt = gptdata.make_tokens(p, np.random.default_rng(p.seed + 1))
    _, got = _run(p, w, tok, tgt)
    assert got["status"] == gf.GPT_OK
    assert np.all(np.isfinite(got["losses"])) and math.isfinite(got["mean"])
    prm = params_of(w)
    pre = p0.with_(seq_len=512, batch=1)
    wins = oracle.layer_windows(p0.window_pattern, p0.short_window, p0.seq_len, p0.n_layer)
    for b in (0, p.batch - 1):
        ref = oracle.forward(pre, prm, tok[b:b + 1, :512], tgt[b:b + 1, :512], windows=wins)
        err = np.abs(got["losses"][b, :512] - ref["losses"][0])
        print(f"  row {b} prefix: max |err| {err.max():.3e}")
        assert err.max() <= 2e-2


def test_launch_timing_hook_bf16():
    """gpt_fwd_loss_timed stamps one event pair per launch of the chosen kind and leaves the
    results bit-identical to gpt_fwd_loss."""
    torch = torch_mod()
    p = _ragged_preset(seed=17)
    w, tok, tgt = gptdata.make_inputs(p)
    m = gf.DeviceModel(p, w)
    t_tok, t_tgt = torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()
    ref, ref_mean, _ = m(t_tok, t_tgt)
    per_step = {gf.GPT_KERNEL_QKV: p.n_layer, gf.GPT_KERNEL_ATTENTION: p.n_layer,
                gf.GPT_KERNEL_ATTN_OUT: p.n_layer, gf.GPT_KERNEL_MLP_UP: p.n_layer,
                gf.GPT_KERNEL_MLP_DOWN: p.n_layer, gf.GPT_KERNEL_LM_HEAD: 1}
    for kind, n in per_step.items():
        evb = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        eve = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        for e in evb + eve:
            e.record()
        t = gf.launch_timing(kind, evb, eve)
        loss = torch.empty_like(ref)
        mean = torch.empty_like(ref_mean)
        assert m.forward(t_tok, t_tgt, loss, mean, None, None, timing=t) == gf.GPT_OK
        torch.cuda.synchronize()
        assert t.recorded == n
        us = [b.elapsed_time(e) * 1e3 for b, e in zip(evb[:n], eve[:n])]
        assert all(0.0 < u < 1e6 for u in us), us
        assert torch.equal(loss, ref) and torch.equal(mean, ref_mean)


# ----------------------------------------------------------------------------- value embeddings

def test_gqa_value_embeddings_fp32():
    """fp32 path with GQA 4:2 and value embeddings on alternating layers (last included)."""
    p = gptdata.Preset(name="ve32", n_layer=3, d_model=128, n_head=4, n_kv_head=2, head_dim=64,
                       mlp_dim=512, vocab=1000, seq_len=128, batch=2, dtype="f32", short_window=64,
                       value_embeds=True, seed=21)
    w, tok, tgt = gptdata.make_inputs(p)
    _, got = _run(p, w, tok, tgt, want_logits=True)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True)
    rel = abs(got["mean"] - ref["mean"]) / abs(ref["mean"])
    zerr = np.max(np.abs(got["logits"] - ref["logits"])) / np.max(np.abs(ref["logits"]))
    print(f"  ve fp32: mean rel err {rel:.2e}, logits err/max {zerr:.2e}")
    assert rel <= 1e-4 and zerr <= 1e-3
    # the value embeddings change the result (the tables are not silently skipped)
    ref0 = oracle.forward(p.with_(value_embeds=False), params_of(w), tok, tgt)
    assert abs(ref0["mean"] - got["mean"]) > 1e-3


def test_gqa_value_embeddings_bf16_ragged():
    """bf16 fused QKV epilogue with value embeddings: GQA 4:2, B*T = 640 rows (ragged tile
    tail), V = 1000, 10% ignored targets, windows 100 / 64 / full."""
    p = _ragged_preset(value_embeds=True, seed=23)
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.1)
    windows = [100, 64, 320]
    _, got = _run(p, w, tok, tgt, want_logits=True, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True, windows=windows)
    _check_bf16(got, ref)
    ref0 = oracle.forward(p.with_(value_embeds=False), params_of(w), tok, tgt, windows=windows)
    assert np.max(np.abs(ref0["losses"] - ref["losses"])) > 0.1


@pytest.mark.parametrize("b", range(FULL_ROWS["d24gve"]))
def test_d24gve_row(b):
    """d24 with 4 KV heads and value embeddings at the benchmarked size (B=8, T=2048), row b."""
    _check_row("d24gve", b)


def test_d24gve_all_tokens():
    _check_mean("d24gve")


# ----------------------------------------------------------------------------- looped trunk

def test_looped_fp32():
    """fp32 looped two-pass trunk (GQA 2:1, head_dim 64): pass-1 prior on every pass-2 layer."""
    p = gptdata.Preset(name="loop32", n_layer=3, d_model=128, n_head=2, n_kv_head=1, head_dim=64,
                       mlp_dim=512, vocab=800, seq_len=128, batch=2, dtype="f32", short_window=64,
                       looped=True, seed=31)
    w, tok, tgt = gptdata.make_inputs(p)
    w.gate_logit[:] = np.array([0.5, -1.0, 1.5], np.float32)   # gates well away from 0
    _, got = _run(p, w, tok, tgt, want_logits=True)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True)
    rel = abs(got["mean"] - ref["mean"]) / abs(ref["mean"])
    zerr = np.max(np.abs(got["logits"] - ref["logits"])) / np.max(np.abs(ref["logits"]))
    print(f"  looped fp32: mean rel err {rel:.2e}, logits err/max {zerr:.2e}")
    assert rel <= 1e-4 and zerr <= 1e-3


def test_looped_bf16_ragged():
    """bf16 looped trunk: GQA 4:2, B*T = 640 rows (ragged), windows 100 / 64 / full, ignores."""
    p = _ragged_preset(looped=True, seed=33)
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.1)
    w.gate_logit[:] = np.array([1.0, 0.2, 2.0], np.float32)
    windows = [100, 64, 320]
    _, got = _run(p, w, tok, tgt, want_logits=True, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True, windows=windows)
    _check_bf16(got, ref)
    # the prior matters at these gates
    ref0 = oracle.forward(p.with_(looped=False), params_of(w), tok, tgt, windows=windows)
    assert np.max(np.abs(ref0["losses"] - ref["losses"])) > 0.05


@pytest.mark.parametrize("b", range(FULL_ROWS["d24loop"]))
def test_d24loop_row(b):
    """Looped two-pass d24 at its configured size (B=4, T=2048), row b."""
    _check_row("d24loop", b)


def test_d24loop_all_tokens():
    _check_mean("d24loop")


# ----------------------------------------------------------------------------- nested model

def _run_nested(p, w, tok, tgt, want_logits=False, windows=None):
    torch = torch_mod()
    m = gf.DeviceModel(p, w, batch=tok.shape[0], windows=windows)
    t_tok = torch.from_numpy(tok).cuda()
    t_tgt = torch.from_numpy(tgt).cuda() if tgt is not None else None
    r = m.call_nested(t_tok, t_tgt, want_logits=want_logits)
    torch.cuda.synchronize()
    out = {"status": m.device_status()}
    for k, v in r.items():
        if v is None:
            out[k] = None
        elif k.startswith("mean"):
            out[k] = float(v.item())
        else:
            out[k] = v.cpu().numpy().astype(np.float64)
    out["losses"], out["losses_k1"] = out.pop("loss"), out.pop("loss_k1")
    return m, out


def _inner_model(p, w):
    """The standalone inner model of a nested preset: width c1, the first heads and hidden
    units, W_E and W_U restricted to their first c1 columns, the diagonal blocks."""
    c1 = p.nested_c1
    q = p.with_(nested_c1=0, d_model=c1, n_head=p.n_head * c1 // p.d_model,
                n_kv_head=p.n_kv_head * c1 // p.d_model, mlp_dim=p.mlp_dim * c1 // p.d_model)
    wi = dataclasses.replace(
        w, wte=np.ascontiguousarray(w.wte[:, :c1]), lm_head=np.ascontiguousarray(w.lm_head[:, :c1]),
        **{n: [blocks[0] for blocks in getattr(w, n)] for n in ("wq", "wk", "wv", "wo", "w1", "w2")})
    return q, wi


def _nest32():
    return gptdata.Preset(name="nest32", n_layer=3, d_model=256, n_head=4, n_kv_head=4, head_dim=64,
                          mlp_dim=1024, vocab=800, seq_len=128, batch=2, dtype="f32", short_window=64,
                          lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), nested_c1=64, seed=41)


def test_nested_fp32():
    """fp32 nested model (blocks 64 + 192, one inner head of 64): full and kfront=1 outputs from
    one pass against the oracle."""
    p = _nest32()
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.1)
    _, got = _run_nested(p, w, tok, tgt, want_logits=True)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True)
    assert got["status"] == gf.GPT_OK
    for sfx in ("", "_k1"):
        rel = abs(got["mean" + sfx] - ref["mean" + sfx]) / abs(ref["mean" + sfx])
        zerr = np.max(np.abs(got["logits" + sfx] - ref["logits" + sfx])) / np.max(np.abs(ref["logits" + sfx]))
        print(f"  nested fp32{sfx}: mean rel err {rel:.2e}, logits err/max {zerr:.2e}")
        assert rel <= 1e-4 and zerr <= 1e-3
        assert np.all(got["losses" + sfx][tgt == -1] == 0.0)
    assert not np.allclose(got["losses"], got["losses_k1"])


def test_nested_fp32_inner_is_standalone_bitwise():
    """The top-left corner is the smaller model: on the fp32 path the kfront=1 losses and
    logits of the nested pass equal, bit for bit, those of the standalone inner model run
    through gpt_fwd_loss (the inner GEMMs, norms and attention heads accumulate in the same
    order)."""
    p = _nest32()
    w, tok, tgt = gptdata.make_inputs(p)
    _, got = _run_nested(p, w, tok, tgt, want_logits=True)
    q, wi = _inner_model(p, w)
    _, ref = _run(q, wi, tok, tgt, want_logits=True)
    assert np.array_equal(got["logits_k1"], ref["logits"])
    assert np.array_equal(got["losses_k1"], ref["losses"]) and got["mean_k1"] == ref["mean"]


def _nest_bf16(**kw):
    base = dict(name="nestbf", n_layer=3, d_model=512, n_head=4, n_kv_head=4, head_dim=128,
                mlp_dim=2048, vocab=1000, seq_len=320, batch=2, dtype="bf16", short_window=100,
                lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), nested_c1=128, seed=43)
    base.update(kw)
    return gptdata.Preset(**base)


def test_nested_bf16_fused_ragged():
    """bf16 nested, head_dim 128 (the fused q/k/v epilogue placing both row blocks' heads):
    blocks 128 + 384, B*T = 640 rows, V = 1000, windows 100 / 64 / full, ignored targets,
    both logits."""
    p = _nest_bf16()
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.1)
    windows = [100, 64, 320]
    _, got = _run_nested(p, w, tok, tgt, want_logits=True, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, tgt, want_logits=True, windows=windows)
    _check_bf16(got, ref)
    k1 = {"losses": got["losses_k1"], "mean": got["mean_k1"]}
    _check_bf16(k1, {"losses": ref["losses_k1"], "mean": ref["mean_k1"]})
    for sfx in ("", "_k1"):
        _check_logits_bf16(got["logits" + sfx], ref["logits" + sfx])


def test_nested_bf16_gqa_d64():
    """bf16 nested with head_dim 64 and GQA 8:4 (blocks 256 + 256: 4 + 4 query heads, 2 + 2 KV
    heads), B = 3; the inner outputs also match the standalone inner model run on the GPU."""
    p = _nest_bf16(n_head=8, n_kv_head=4, head_dim=64, nested_c1=256, seq_len=256, batch=3,
                   vocab=777, seed=45)
    w, tok, tgt = gptdata.make_inputs(p)
    _, got = _run_nested(p, w, tok, tgt)
    ref = oracle.forward(p, params_of(w), tok, tgt)
    _check_bf16(got, ref)
    _check_bf16({"losses": got["losses_k1"], "mean": got["mean_k1"]},
                {"losses": ref["losses_k1"], "mean": ref["mean_k1"]})
    q, wi = _inner_model(p, w)
    _, alone = _run(q, wi, tok, tgt)
    err = np.max(np.abs(got["losses_k1"] - alone["losses"]))
    print(f"  kfront=1 vs standalone inner model: max |err| {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("b", range(FULL_ROWS["d24nest"]))
def test_d24nest_row(b):
    """StairFormer d24 at its configured size (24 heads of 64 in blocks 6 + 18, B=4, T=2048):
    both losses (full model and kfront=1) of row b."""
    _check_row("d24nest", b)


def test_d24nest_all_tokens():
    _check_mean("d24nest")
