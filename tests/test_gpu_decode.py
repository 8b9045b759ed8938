"""Decoding through the C ABI (gpt_decode_step, gpt_sample) against the oracle.

A decode step at position t must give the logits that the oracle's full forward gives at
position t of the same sequence ("The Mathematics of Karpathy's nanochat", section "Inference:
Generating Text": the next token comes from the logits at the last position; attention is causal,
so the cached keys and values of earlier positions are all a step needs).  Bars as for the
forward: fp32 logits within 1e-3 of the largest |logit|; bf16 logits |error| RMS <= 6e-3 and max
<= 3e-2.  The sampler is compared token by token with oracle.sample_next on the same logits and
draws; where they differ, the GPU's token must still be a valid draw: kept by top-k, with u within
rounding (1e-5) of its cumulative-probability interval.
"""
import math

import numpy as np
import pytest

import decoder_only_transformer_layer_amd as gf
import gptdata
import oracle
from gpu_helpers import params_of, torch_mod

pytestmark = pytest.mark.gpu


def _decode_all(p, w, tok, lag=None, windows=None):
    """Feed tok [B, T] through T decode steps; row b's position at step s is s - lag[b] (rows
    that have not started repeat position 0).  Returns the logits [B, T, V] by position."""
    torch = torch_mod()
    B, T = tok.shape
    m = gf.DeviceModel(p, w, batch=B, windows=windows)
    d = gf.Decoder(m)
    lag = np.zeros(B, dtype=np.int64) if lag is None else np.asarray(lag)
    t_tok = torch.from_numpy(tok.astype(np.int32)).cuda()
    logits = torch.empty((B, p.vocab), dtype=torch.float32, device="cuda")
    out = np.zeros((B, T, p.vocab))
    steps = T + int(lag.max())
    for s in range(steps):
        pos = np.clip(s - lag, 0, T - 1).astype(np.int32)
        t_pos = torch.from_numpy(pos).cuda()
        cur = t_tok[torch.arange(B, device="cuda"), t_pos.long()].contiguous()
        assert d.step(cur, t_pos, logits) == gf.GPT_OK
        z = logits.cpu().numpy().astype(np.float64)
        for b in range(B):
            if s - lag[b] >= 0 and s - lag[b] < T:
                out[b, s - lag[b]] = z[b]
    torch.cuda.synchronize()
    assert d.device_status() == gf.GPT_OK
    return out


def test_decode_matches_forward_fp32():
    """fp32, GQA 2:1, head_dim 64, windows 16 / full; row 1 runs two positions behind row 0."""
    p = gptdata.Preset(name="dec32", n_layer=2, d_model=128, n_head=2, n_kv_head=1, head_dim=64,
                       mlp_dim=512, vocab=500, seq_len=48, batch=2, dtype="f32", short_window=16,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=51)
    w, tok, _ = gptdata.make_inputs(p)
    got = _decode_all(p, w, tok, lag=[0, 2])
    ref = oracle.forward(p, params_of(w), tok, want_logits=True)["logits"]
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    print(f"  decode fp32: logits err/max {err:.2e}")
    assert err <= 1e-3


def test_decode_single_row_fp32():
    """fp32 with one row, d_model 192 (three K steps of 64), a query group of 3 (3 heads of 64 on
    one KV head), a 333-entry vocabulary, 40 positions (not a multiple of 64), window 16 / full."""
    p = gptdata.Preset(name="dec1f", n_layer=2, d_model=192, n_head=3, n_kv_head=1, head_dim=64,
                       mlp_dim=768, vocab=333, seq_len=40, batch=1, dtype="f32", short_window=16,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=69)
    w, tok, _ = gptdata.make_inputs(p)
    got = _decode_all(p, w, tok)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True)["logits"]
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    print(f"  decode fp32: logits err/max {err:.2e}")
    assert err <= 1e-3


def _check_bf16_logits(got, ref):
    d = got - ref
    rms, mx = float(np.sqrt(np.mean(d * d))), float(np.max(np.abs(d)))
    print(f"  logits |err| rms {rms:.3e} max {mx:.3e}")
    assert rms <= 6e-3 and mx <= 3e-2


def test_decode_matches_forward_bf16():
    """bf16, GQA 4:2, head_dim 128, windows 32 / 64 / full over 128 positions, 3 rows."""
    p = gptdata.Preset(name="dec16", n_layer=3, d_model=256, n_head=4, n_kv_head=2, head_dim=128,
                       mlp_dim=1024, vocab=1000, seq_len=128, batch=3, dtype="bf16", short_window=32,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=53)
    w, tok, _ = gptdata.make_inputs(p)
    windows = [32, 64, 128]
    got = _decode_all(p, w, tok, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True, windows=windows)["logits"]
    _check_bf16_logits(got, ref)


def test_decode_matches_forward_bf16_d64():
    """bf16 at head_dim 64 (the 64-wide RoPE/QK-norm, the chunk kernel's 8 x 32 output layout),
    MHA with 6 heads, windows 40 / full over 192 positions (two 128-key chunks), 2 rows, row 1
    one position behind row 0."""
    p = gptdata.Preset(name="dec64", n_layer=2, d_model=384, n_head=6, n_kv_head=6, head_dim=64,
                       mlp_dim=1536, vocab=900, seq_len=192, batch=2, dtype="bf16", short_window=40,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=61)
    w, tok, _ = gptdata.make_inputs(p)
    windows = [40, 192]
    got = _decode_all(p, w, tok, lag=[0, 1], windows=windows)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True, windows=windows)["logits"]
    _check_bf16_logits(got, ref)


def test_decode_group8_multichunk_bf16():
    """bf16 at the largest query group the decode attention takes (8 query heads on one KV
    head, head_dim 128), 320 cache positions so that windows of 200 and full span up to three
    128-key chunks; row 1 runs three positions behind row 0."""
    p = gptdata.Preset(name="dec8g", n_layer=2, d_model=256, n_head=8, n_kv_head=1, head_dim=128,
                       mlp_dim=1024, vocab=700, seq_len=320, batch=2, dtype="bf16", short_window=200,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=57)
    w, tok, _ = gptdata.make_inputs(p)
    windows = [200, 320]
    got = _decode_all(p, w, tok, lag=[0, 3], windows=windows)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True, windows=windows)["logits"]
    _check_bf16_logits(got, ref)


def test_decode_32_rows_bf16():
    """bf16 with the most rows a decode step takes (32: every lane of the products' batch operand
    live, the row scales of rows 8-31 summed by the later wavefronts), GQA 2:1, rows staggered
    by up to three positions."""
    p = gptdata.Preset(name="dec32r", n_layer=2, d_model=256, n_head=4, n_kv_head=2, head_dim=64,
                       mlp_dim=1024, vocab=600, seq_len=64, batch=32, dtype="bf16", short_window=24,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=63)
    w, tok, _ = gptdata.make_inputs(p)
    got = _decode_all(p, w, tok, lag=np.arange(32) % 4)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True)["logits"]
    _check_bf16_logits(got, ref)


def test_decode_single_row_bf16():
    """bf16 with one row (one live lane of the products' batch operand), d_model 640 (ten K steps
    of 64: the products' two-deep tile loop with a ragged last round), a query group of 5 (10
    heads of 64 on 2 KV heads), MLP down left unsplit, a 333-entry vocabulary (a ragged last
    lm_head row block), windows 40 / full over 64 positions."""
    p = gptdata.Preset(name="dec1r", n_layer=2, d_model=640, n_head=10, n_kv_head=2, head_dim=64,
                       mlp_dim=1280, vocab=333, seq_len=64, batch=1, dtype="bf16", short_window=40,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=65)
    w, tok, _ = gptdata.make_inputs(p)
    windows = [40, 64]
    got = _decode_all(p, w, tok, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True, windows=windows)["logits"]
    _check_bf16_logits(got, ref)


def test_decode_widest_bf16():
    """bf16 at the widest model decoding takes (d_model 4096: the out-projection leaves 128
    per-block row sums, the most a product's row scale takes), one layer, 2 rows over 64
    positions, row 1 one position behind row 0."""
    p = gptdata.Preset(name="decwide", n_layer=1, d_model=4096, n_head=32, n_kv_head=32, head_dim=128,
                       mlp_dim=4096, vocab=512, seq_len=64, batch=2, dtype="bf16", short_window=64,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=59)
    w, tok, _ = gptdata.make_inputs(p)
    got = _decode_all(p, w, tok, lag=[0, 1])
    ref = oracle.forward(p, params_of(w), tok, want_logits=True)["logits"]
    _check_bf16_logits(got, ref)


def test_decode_d24_positions():
    """d24 weights, 2 rows, the whole 2048-token cache: logits at positions 0, 511, 1023, 1024,
    1500 and 2047 of row 0 against one oracle forward of that row."""
    p = gptdata.preset("d24").with_(batch=2)
    w, tok, _ = gptdata.make_inputs(p)
    torch = torch_mod()
    m = gf.DeviceModel(p, w, batch=2)
    d = gf.Decoder(m)
    t_tok = torch.from_numpy(tok).cuda()
    logits = torch.empty((2, p.vocab), dtype=torch.float32, device="cuda")
    check = [0, 511, 1023, 1024, 1500, 2047]
    got = {}
    for s in range(p.seq_len):
        t_pos = torch.full((2,), s, dtype=torch.int32, device="cuda")
        assert d.step(t_tok[:, s].contiguous(), t_pos, logits) == gf.GPT_OK
        if s in check:
            got[s] = logits[0].cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert d.device_status() == gf.GPT_OK
    ref = oracle.forward(p, params_of(w), tok[:1], want_logits=True)["logits"][0]
    _check_bf16_logits(np.stack([got[s] for s in check]), ref[check])


def test_decode_bad_inputs():
    """An out-of-range token or position gives NaN logits for that row only and a device error;
    the other rows are unaffected."""
    p = gptdata.Preset(name="decbad", n_layer=2, d_model=128, n_head=2, n_kv_head=2, head_dim=64,
                       mlp_dim=256, vocab=300, seq_len=64, batch=3, dtype="bf16", short_window=32,
                       seed=55)
    w, tok, _ = gptdata.make_inputs(p)
    torch = torch_mod()
    m = gf.DeviceModel(p, w, batch=3)
    d = gf.Decoder(m)
    logits = torch.empty((3, p.vocab), dtype=torch.float32, device="cuda")
    cur = torch.tensor([tok[0, 0], p.vocab + 5, tok[2, 0]], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0, 0, 0], dtype=torch.int32, device="cuda")
    assert d.step(cur, pos, logits) == gf.GPT_OK
    z = logits.cpu().numpy()
    assert np.all(np.isnan(z[1])) and np.all(np.isfinite(z[[0, 2]]))
    assert d.device_status() == gf.GPT_E_DEVICE_INPUT
    cur = torch.from_numpy(tok[:, 0].copy()).cuda()
    pos = torch.tensor([0, p.seq_len, -1], dtype=torch.int32, device="cuda")
    assert d.step(cur, pos, logits) == gf.GPT_OK
    z = logits.cpu().numpy()
    assert np.all(np.isfinite(z[0])) and np.all(np.isnan(z[1:]))
    assert d.device_status() == gf.GPT_E_DEVICE_INPUT
    ref = oracle.forward(p, params_of(w), tok[:1, :1], want_logits=True)["logits"][0, 0]
    assert np.max(np.abs(z[0] - ref)) <= 3e-2


def _valid_draw(z, k, tau, u, tok):
    """The GPU's token is a valid draw at u: kept by top-k and u within 1e-5 of its interval of
    the (fp64) cumulative distribution in vocabulary order."""
    keep = oracle.top_k_keep(z, k if k and k > 0 else None)
    if not keep[tok]:
        return False
    s = np.where(keep, z / tau, -np.inf)
    e = np.exp(s - np.max(s))
    cdf = np.cumsum(e / e.sum())
    lo = cdf[tok - 1] if tok > 0 else 0.0
    return lo - 1e-5 <= u <= cdf[tok] + 1e-5


@pytest.mark.parametrize("V", [100, 5003, 32768])
def test_sampler_matches_oracle(V):
    """Greedy with planted ties, top-k = 1, 7, 50, all (0 and V), temperatures 0.5 / 1 / 2."""
    torch = torch_mod()
    rng = np.random.default_rng(V)
    B = 6
    z = (rng.standard_normal((B, V)) * 2.5).astype(np.float32)
    z[0, [3, V - 1]] = z[0].max() + 1.0     # equal maxima: greedy takes the first
    z[1, 10:14] = 4.0                         # ties at a top-k threshold
    z[1, 14:] = np.minimum(z[1, 14:], 3.0)
    z[1, :10] = np.minimum(z[1, :10], 3.0)
    t_z = torch.from_numpy(z).cuda()
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    mism = 0
    for k in (0, 1, 2, 7, 50, V):
        for tau in (0.0, 0.5, 1.0, 2.0):
            for trial in range(3):
                u = rng.random(B).astype(np.float32)
                t_u = torch.from_numpy(u).cuda()
                assert gf.gpt_sample(t_z, B, V, k, tau, t_u, out) == gf.GPT_OK
                got = out.cpu().numpy()
                for b in range(B):
                    zb = z[b].astype(np.float64)
                    ref = oracle.sample_next(zb, k if k > 0 else None, tau, float(u[b]))
                    if got[b] != ref:
                        mism += 1
                        assert tau > 0 and _valid_draw(zb, k, tau, float(u[b]), int(got[b])), (k, tau, b)
    print(f"  V={V}: {mism} boundary-rounding differences")
    assert mism <= 2


def test_greedy_generation_matches_oracle():
    """fp32 model: decode + greedy sampling for 12 new tokens after a 6-token prompt, against the
    oracle's generate (full forward per step)."""
    torch = torch_mod()
    p = gptdata.Preset(name="gen32", n_layer=2, d_model=128, n_head=2, n_kv_head=2, head_dim=64,
                       mlp_dim=512, vocab=200, seq_len=32, batch=2, dtype="f32", short_window=8,
                       seed=57)
    w, tok, _ = gptdata.make_inputs(p)
    prompt, n_new = tok[:, :6], 12
    ref = oracle.generate(p, params_of(w), prompt, n_new, top_k=None, temperature=0.0,
                          u=np.zeros((n_new, 2)))
    m = gf.DeviceModel(p, w, batch=2)
    d = gf.Decoder(m)
    logits = torch.empty((2, p.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    u = torch.zeros(2, dtype=torch.float32, device="cuda")
    seq = [torch.from_numpy(prompt[:, i].astype(np.int32)).cuda() for i in range(prompt.shape[1])]
    for s in range(prompt.shape[1] + n_new - 1):
        pos = torch.full((2,), s, dtype=torch.int32, device="cuda")
        assert d.step(seq[s], pos, logits) == gf.GPT_OK
        if s >= prompt.shape[1] - 1:
            assert gf.gpt_sample(logits, 2, p.vocab, 0, 0.0, u, nxt) == gf.GPT_OK
            seq.append(nxt.clone())
    got = torch.stack(seq, dim=1).cpu().numpy()
    assert np.array_equal(got, ref["tokens"]), (got, ref["tokens"])


def test_decode_step_graph_replay():
    """A decode step captured once in a HIP graph and replayed for successive positions (new
    token and position values written between replays, with eager work in between) gives, at
    every replay, the logits of the same steps run eagerly."""
    torch = torch_mod()
    p = gptdata.Preset(name="decgraph", n_layer=2, d_model=256, n_head=2, n_kv_head=2, head_dim=128,
                       mlp_dim=1024, vocab=700, seq_len=64, batch=2, dtype="bf16", short_window=16,
                       seed=59)
    w, tok, _ = gptdata.make_inputs(p)
    n = 12
    eager = []
    m = gf.DeviceModel(p, w, batch=2)
    d = gf.Decoder(m)
    logits = torch.empty((2, p.vocab), dtype=torch.float32, device="cuda")
    for s in range(n):
        t_pos = torch.full((2,), s, dtype=torch.int32, device="cuda")
        assert d.step(torch.from_numpy(tok[:, s].copy()).cuda(), t_pos, logits) == gf.GPT_OK
        eager.append(logits.cpu().numpy().copy())
    d2 = gf.Decoder(m)   # fresh cache
    cur = torch.zeros(2, dtype=torch.int32, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = torch.empty((2, p.vocab), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # warm-up launch outside the capture
        assert d2.step(cur, pos, out) == gf.GPT_OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert d2.step(cur, pos, out) == gf.GPT_OK
    for s in range(n):
        cur.copy_(torch.from_numpy(tok[:, s].copy()))
        pos.fill_(s)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1000, device="cuda").sum()   # eager work between replays
        assert np.array_equal(out.cpu().numpy(), eager[s]), s
        del junk
    assert d2.device_status() == gf.GPT_OK


def _prefill_then_decode(p, w, tok, P, lens, n_steps, windows=None):
    """Prefill positions [0, P) of every row (row b's prompt is its first lens[b] tokens), then
    decode n_steps more tokens per row from position lens[b].  Returns the prefill logits [B, V]
    and the decode logits [n_steps, B, V]."""
    torch = torch_mod()
    B = tok.shape[0]
    m = gf.DeviceModel(p, w, batch=B, windows=windows)
    d = gf.Decoder(m)
    t_tok = torch.from_numpy(tok.astype(np.int32)).cuda()
    t_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, p.vocab), dtype=torch.float32, device="cuda")
    assert d.prefill(t_tok[:, :P].contiguous(), P, logits, lens=t_lens) == gf.GPT_OK
    first = logits.cpu().numpy().astype(np.float64)
    assert m.device_status() == gf.GPT_OK
    steps = []
    for s in range(n_steps):
        pos = t_lens + s
        cur = t_tok[torch.arange(B, device="cuda"), pos.long()].contiguous()
        assert d.step(cur, pos.contiguous(), logits) == gf.GPT_OK
        steps.append(logits.cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    assert d.device_status() == gf.GPT_OK
    return first, np.stack(steps)


def test_prefill_then_decode_fp32():
    """fp32: prompts of 20 and 13 tokens in one padded batch of 20, then 10 decode steps each;
    every logit vector against the oracle's forward of that row's sequence."""
    p = gptdata.Preset(name="pre32", n_layer=2, d_model=128, n_head=2, n_kv_head=1, head_dim=64,
                       mlp_dim=512, vocab=500, seq_len=48, batch=2, dtype="f32", short_window=16,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=61)
    w, tok, _ = gptdata.make_inputs(p)
    lens = [20, 13]
    first, steps = _prefill_then_decode(p, w, tok, 20, lens, 10)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True)["logits"]   # causal: all positions
    scale = np.max(np.abs(ref))
    for b, n in enumerate(lens):
        assert np.max(np.abs(first[b] - ref[b, n - 1])) / scale <= 1e-3
        for s in range(10):
            assert np.max(np.abs(steps[s, b] - ref[b, n + s])) / scale <= 1e-3


def test_prefill_then_decode_bf16():
    """bf16, GQA 4:2, head_dim 128, windows 32 / 64 / full: a padded batch of 64 with prompts of
    64, 50 and 33 tokens, then 20 decode steps per row."""
    p = gptdata.Preset(name="pre16", n_layer=3, d_model=256, n_head=4, n_kv_head=2, head_dim=128,
                       mlp_dim=1024, vocab=1000, seq_len=128, batch=3, dtype="bf16", short_window=32,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=63)
    w, tok, _ = gptdata.make_inputs(p)
    windows = [32, 64, 128]
    lens = [64, 50, 33]
    first, steps = _prefill_then_decode(p, w, tok, 64, lens, 20, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True, windows=windows)["logits"]
    got = np.concatenate([first[None]] + [steps[s][None] for s in range(20)])
    want = np.stack([np.stack([ref[b, lens[b] - 1 + s] for b in range(3)]) for s in range(21)])
    _check_bf16_logits(got, want)


def test_prefill_then_decode_single_row_bf16():
    """bf16, one row (a 64-row forward for the prefill), GQA 2:1 at head_dim 64, a 333-entry
    vocabulary: a prompt of 37 tokens padded to 64, then 32 decode steps (positions 37 to 68: the
    first 27 overwrite the cache slots the prefill filled past the prompt, the last 5 go past the
    padded length)."""
    p = gptdata.Preset(name="pre1r", n_layer=2, d_model=256, n_head=4, n_kv_head=2, head_dim=64,
                       mlp_dim=1024, vocab=333, seq_len=128, batch=1, dtype="bf16", short_window=48,
                       lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2), seed=67)
    w, tok, _ = gptdata.make_inputs(p)
    windows = [48, 128]
    lens = [37]
    first, steps = _prefill_then_decode(p, w, tok, 64, lens, 32, windows=windows)
    ref = oracle.forward(p, params_of(w), tok, want_logits=True, windows=windows)["logits"]
    got = np.concatenate([first[None]] + [steps[s][None] for s in range(32)])
    want = np.stack([ref[0, lens[0] - 1 + s][None] for s in range(33)])
    _check_bf16_logits(got, want)
