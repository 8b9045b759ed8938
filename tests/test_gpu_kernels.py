"""Per-kernel parity on the GPU: each component entry point of libgptfwd against the oracle's
function for the same step, element by element, on the same seeded inputs.

Tolerances follow from the arithmetic: fp32 accumulation is exact to ~1e-6 relative at these
sizes, so outputs stored in bf16 (8 significant bits, RNE) may differ from the fp64 oracle by
one bf16 rounding (2^-9 relative) plus that; fp32 outputs must agree to ~1e-5.
"""
import math

import numpy as np
import pytest

import decoder_only_transformer_layer_amd as gf
import oracle
from gpu_helpers import bf16_dev, empty, f32_dev, to_host, torch_mod

pytestmark = pytest.mark.gpu

BF, F32 = gf.GPT_BF16, gf.GPT_F32


def _sync():
    torch_mod().cuda.synchronize()


def _ok(st, what):
    assert st == gf.GPT_OK, f"{what}: {gf.gpt_status_string(st)}"


def _bf16_close(got, ref, rel=2 ** -8, atol=1e-5):
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + atol
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} mismatches, worst {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"


# ----------------------------------------------------------------------------- GEMM

# (16384, 1536): 256x384 tiles (one round); (8192, 768) and (1000, 576): 256x192 tiles, the
# latter with ragged rows; (8192, 4352): 17 column blocks of 256 over 32 row blocks, split into
# 16 blocks of 256x256 (two whole rounds) and a 256x128 column tail (the shifted output, and
# residual, pointers of the tail); (16384, 4608, ...) via QKV below.
@pytest.mark.parametrize("M,N,K", [(300, 384, 192), (512, 1000, 128), (8192, 8192, 64), (64, 128, 6144),
                                   (16384, 1536, 64), (8192, 768, 128), (1000, 576, 64), (8192, 4352, 64)])
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_linear_bf16(M, N, K, epi):
    rng = np.random.default_rng(100 + M + N + K + epi)
    a, a64 = bf16_dev(rng.standard_normal((M, K), dtype=np.float32))
    w, w64 = bf16_dev(rng.standard_normal((N, K), dtype=np.float32) / np.float32(math.sqrt(K)))
    ref = oracle.linear(a64, w64)
    if epi == 2:
        out, x64 = f32_dev(rng.standard_normal((M, N), dtype=np.float32))
        ref = x64 + ref
    else:
        out = empty((M, N), "bf16")
        if epi == 1:
            ref = oracle.relu_squared(ref)
    _ok(gf.gpt_op_linear(BF, epi, a, w, M, N, K, out), "linear")
    _sync()
    got = to_host(out)
    if epi == 2:
        assert np.max(np.abs(got - ref)) < 1e-4
    else:
        _bf16_close(got, ref, atol=1e-5 * (1 + np.abs(ref).max()))


@pytest.mark.parametrize("epi", [0, 1, 2])
def test_linear_f32(epi):
    rng = np.random.default_rng(7)
    M, N, K = 130, 200, 70
    a, a64 = f32_dev(rng.standard_normal((M, K), dtype=np.float32))
    w, w64 = f32_dev(rng.standard_normal((N, K), dtype=np.float32))
    ref = oracle.linear(a64, w64)
    if epi == 2:
        out, x64 = f32_dev(rng.standard_normal((M, N), dtype=np.float32))
        ref = ref + x64
    else:
        out = empty((M, N), "f32")
        if epi == 1:
            ref = oracle.relu_squared(ref)
    _ok(gf.gpt_op_linear(F32, epi, a, w, M, N, K, out), "linear f32")
    _sync()
    got = to_host(out)
    assert np.max(np.abs(got - ref) / (1 + np.abs(ref))) < 1e-5


# ----------------------------------------------------------------------------- rows

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [128, 1536, 768])
def test_embed_and_mix_norm(dtype, C):
    torch = torch_mod()
    rng = np.random.default_rng(C)
    M, V, eps = 333, 517, 1e-6
    tab = rng.standard_normal((V, C), dtype=np.float32) * np.float32(0.3)
    if dtype == "bf16":
        wte, wte64 = bf16_dev(tab)
    else:
        wte, wte64 = f32_dev(tab)
    tok = rng.integers(0, V, M).astype(np.int32)
    lam, mu = np.float32(0.93), np.float32(0.17)
    t_tok = torch.from_numpy(tok).cuda()
    t_lam = torch.tensor([lam, 1.05], dtype=torch.float32).cuda()
    t_mu = torch.tensor([mu, 0.07], dtype=torch.float32).cuda()
    x0, x = empty((M, C), "f32"), empty((M, C), "f32")
    xn = empty((M, C), dtype)
    flags = torch.zeros(4, dtype=torch.int32).cuda()
    _ok(gf.gpt_op_embed_norm(BF if dtype == "bf16" else F32, t_tok, wte, t_lam, t_mu, x0, x, xn, M, C, V,
                             eps, flags), "embed")
    _sync()
    rx0 = oracle.rms_norm(wte64[tok], eps)
    rx = float(lam) * rx0 + float(mu) * rx0
    rxn = oracle.rms_norm(rx, eps)
    assert np.max(np.abs(to_host(x0) - rx0)) < 1e-5
    assert np.max(np.abs(to_host(x) - rx)) < 1e-5
    if dtype == "bf16":
        _bf16_close(to_host(xn), rxn, atol=1e-6)
    else:
        assert np.max(np.abs(to_host(xn) - rxn)) < 1e-5
    assert int(flags[0].item()) == 0
    # mix with layer 1's scalars, then the plain norm
    xin = rng.standard_normal((M, C), dtype=np.float32) * np.float32(3.0)
    x.copy_(torch.from_numpy(xin).cuda())
    _ok(gf.gpt_op_mix_norm(BF if dtype == "bf16" else F32, x, x0, t_lam, t_mu, 1, 1, xn, M, C, eps), "mix")
    _sync()
    rmix = 1.05 * xin.astype(np.float64) + 0.07 * to_host(x0)
    assert np.max(np.abs(to_host(x) - rmix)) < 1e-5
    tol = 2 ** -8 if dtype == "bf16" else 1e-6
    assert np.all(np.abs(to_host(xn) - oracle.rms_norm(rmix, eps)) <= tol * np.abs(oracle.rms_norm(rmix, eps)) + 1e-6)
    _ok(gf.gpt_op_mix_norm(BF if dtype == "bf16" else F32, x, x0, t_lam, t_mu, 0, 0, xn, M, C, eps), "norm")
    _sync()
    assert np.max(np.abs(to_host(x) - rmix)) < 1e-5       # unchanged without mix
    assert np.all(np.abs(to_host(xn) - oracle.rms_norm(rmix, eps)) <= tol * np.abs(oracle.rms_norm(rmix, eps)) + 1e-6)


def test_embed_flags_bad_token():
    torch = torch_mod()
    M, C, V = 8, 128, 50
    wte, _ = bf16_dev(np.ones((V, C), np.float32))
    tok = torch.tensor([0, 1, 2, 50, 3, -1, 4, 5], dtype=torch.int32).cuda()
    lam = torch.ones(1).cuda()
    x0, x, xn = empty((M, C), "f32"), empty((M, C), "f32"), empty((M, C), "bf16")
    flags = torch.zeros(4, dtype=torch.int32).cuda()
    _ok(gf.gpt_op_embed_norm(BF, tok, wte, lam, lam, x0, x, xn, M, C, V, 1e-6, flags), "embed")
    _sync()
    assert int(flags[0].item()) & 1


# ----------------------------------------------------------------------------- RoPE, QKV

def test_rope_table():
    torch = torch_mod()
    T, D = 2048, 128
    cs = torch.empty((T, D // 2, 2), dtype=torch.float32).cuda()
    _ok(gf.gpt_op_rope_table(cs, T, D, 1e5), "rope table")
    _sync()
    c, s = oracle.rope_angles(T, D, 1e5)
    got = cs.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got[..., 0] - c)) < 1e-7 and np.max(np.abs(got[..., 1] - s)) < 1e-7


@pytest.mark.parametrize("H,Hkv,D,B,T", [(2, 2, 128, 2, 192), (4, 2, 128, 2, 192), (2, 2, 64, 2, 192),
                                         (8, 4, 64, 2, 256), (3, 1, 128, 2, 192), (6, 6, 64, 2, 256),
                                         (12, 4, 128, 8, 2048), (12, 12, 128, 8, 2048),
                                         (3, 3, 128, 2, 192), (6, 3, 128, 3, 224)])
def test_qkv_rope_norm_bf16(H, Hkv, D, B, T):
    """(2, 2, 64), (3, 1, 128) and (6, 6, 64) put a q/k or k/v boundary inside a 256-wide
    tile (at 128 or 384 columns, the nested model's 384-wide head blocks), which the tile loads
    from two weight matrices.  (12, 4, 128): the GQA projection over 16384 rows (2.5 rounds of
    256x256 tiles: two rounds and a tail of 256x128 tiles).  (12, 12, 128): the d24 projection
    shape.  It and (3, 3, 128), (6, 3, 128) (q, k and v each a multiple of three 128-wide heads;
    384 and 672 rows, so the last row block is partial) run the fused form as one launch of
    256x384 tiles whose q|k tiles hold their columns in RoPE-pair order, with the middle head of
    each tile split over two wavefronts."""
    torch = torch_mod()
    rng = np.random.default_rng(H * 10 + Hkv + D)
    C, eps = 256, 1e-6
    M = B * T
    xn, xn64 = bf16_dev(oracle.rms_norm(rng.standard_normal((M, C)), 0).astype(np.float32))
    wq, wq64 = bf16_dev(rng.standard_normal((H * D, C), dtype=np.float32) / np.float32(16))
    wk, wk64 = bf16_dev(rng.standard_normal((Hkv * D, C), dtype=np.float32) / np.float32(16))
    wv, wv64 = bf16_dev(rng.standard_normal((Hkv * D, C), dtype=np.float32) / np.float32(16))
    qk = empty((M, (H + Hkv) * D), "bf16")
    vt = empty((B, Hkv, D, T), "bf16")
    _ok(gf.gpt_op_qkv(xn, wq, wk, wv, B, T, C, H, Hkv, D, None, eps, qk, vt), "qkv")
    cs = torch.empty((T, D // 2, 2), dtype=torch.float32).cuda()
    _ok(gf.gpt_op_rope_table(cs, T, D, 1e5), "rope table")
    _sync()
    raw = to_host(qk)
    # projections before the in-place RoPE + norm
    _bf16_close(raw[:, :H * D], oracle.linear(xn64, wq64), atol=1e-4)
    _bf16_close(raw[:, H * D:], oracle.linear(xn64, wk64), atol=1e-4)
    v = oracle.linear(xn64, wv64).reshape(B, T, Hkv, D)
    _bf16_close(to_host(vt), v.transpose(0, 2, 3, 1), atol=1e-4)
    _ok(gf.gpt_op_qk_rope_norm(BF, qk, (H + Hkv) * D, cs, M, T, H + Hkv, D, eps), "rope norm")
    _sync()
    got = to_host(qk).reshape(B, T, H + Hkv, D)
    c, s = oracle.rope_angles(T, D, 1e5)
    for b in range(B):
        u = raw.reshape(B, T, H + Hkv, D)[b]           # the bf16 projections the kernel read
        ref = oracle.rms_norm(oracle.apply_rope(u, c, s), eps)
        assert np.max(np.abs(got[b] - ref)) < 2e-2
        assert np.mean(np.abs(got[b] - ref)) < 2e-3
    if True:
        # fused form: RoPE + norm on the fp32 projection inside the GEMM epilogue (a wavefront
        # owns one 128-wide head or two 64-wide ones)
        qk2 = empty((M, (H + Hkv) * D), "bf16")
        vt2 = empty((B, Hkv, D, T), "bf16")
        _ok(gf.gpt_op_qkv(xn, wq, wk, wv, B, T, C, H, Hkv, D, cs, eps, qk2, vt2), "qkv fused")
        _sync()
        assert torch.equal(vt2, vt)
        got2 = to_host(qk2).reshape(B, T, H + Hkv, D)
        u64 = np.concatenate([oracle.linear(xn64, wq64), oracle.linear(xn64, wk64)], axis=1).reshape(B, T, H + Hkv, D)
        for b in range(B):
            ref = oracle.rms_norm(oracle.apply_rope(u64[b], c, s), eps)
            _bf16_close(got2[b], ref, rel=2 ** -8, atol=2e-5)


# ----------------------------------------------------------------------------- attention

def _attn_inputs(rng, B, T, H, Hkv, D):
    q = oracle.rms_norm(rng.standard_normal((B, T, H, D)), 0)
    k = oracle.rms_norm(rng.standard_normal((B, T, Hkv, D)), 0)
    v = rng.standard_normal((B, T, Hkv, D))
    return q, k, v


@pytest.mark.parametrize("H,Hkv,D", [(2, 2, 128), (4, 2, 128), (3, 1, 64)])
@pytest.mark.parametrize("window", [1, 7, 64, 100, 130, 320, 5000])
def test_attention_bf16(H, Hkv, D, window):
    torch = torch_mod()
    rng = np.random.default_rng(window * 7 + H + D)
    B, T = 2, 320
    q, k, v = _attn_inputs(rng, B, T, H, Hkv, D)
    qk, qk64 = bf16_dev(np.concatenate([q, k], axis=2).reshape(B * T, (H + Hkv) * D).astype(np.float32))
    vt, vt64 = bf16_dev(np.ascontiguousarray(v.transpose(0, 2, 3, 1)).astype(np.float32))
    o = empty((B * T, H * D), "bf16")
    scale = 1.0 / math.sqrt(D)
    _ok(gf.gpt_op_attention(BF, qk, vt, o, B, T, H, Hkv, D, window, scale), "attention")
    _sync()
    got = to_host(o).reshape(B, T, H, D)
    q64 = qk64.reshape(B, T, H + Hkv, D)[:, :, :H]
    k64 = qk64.reshape(B, T, H + Hkv, D)[:, :, H:]
    v64 = vt64.transpose(0, 3, 1, 2)
    for b in range(B):
        ref = oracle.attention(q64[b], k64[b], v64[b], window, scale)
        err = np.abs(got[b] - ref)
        assert err.max() < 2.5e-2, (b, err.max())
        assert err.mean() < 3e-3, (b, err.mean())


@pytest.mark.parametrize("B,H,Hkv,window", [(2, 16, 16, 256), (4, 12, 4, 5000), (2, 16, 2, 300)])
def test_attention_bf16_many_heads(B, H, Hkv, window):
    """Grids of many (batch, head) pairs: 32 pairs with a 256-key window (every query block
    spans a window edge), 48 pairs with GQA (3 query heads per KV head) and full windows, and
    32 pairs with 8 query heads per KV head and a 300-key window.  Every head against the
    oracle."""
    torch = torch_mod()
    rng = np.random.default_rng(B * 100 + H)
    T, D = 512, 64
    q, k, v = _attn_inputs(rng, B, T, H, Hkv, D)
    qk, qk64 = bf16_dev(np.concatenate([q, k], axis=2).reshape(B * T, (H + Hkv) * D).astype(np.float32))
    vt, vt64 = bf16_dev(np.ascontiguousarray(v.transpose(0, 2, 3, 1)).astype(np.float32))
    o = empty((B * T, H * D), "bf16")
    scale = 1.0 / math.sqrt(D)
    _ok(gf.gpt_op_attention(BF, qk, vt, o, B, T, H, Hkv, D, window, scale), "attention")
    _sync()
    got = to_host(o).reshape(B, T, H, D)
    x = qk64.reshape(B, T, H + Hkv, D)
    v64 = vt64.transpose(0, 3, 1, 2)
    for b in range(B):
        ref = oracle.attention(x[b, :, :H], x[b, :, H:], v64[b], window, scale)
        err = np.abs(got[b] - ref)
        assert err.max() < 2.5e-2, (b, err.max())
        assert err.mean() < 3e-3, (b, err.mean())


def test_attention_sharp_scale_and_f32():
    """Page 5's reading of the logit scale (1.15^2, no 1/sqrt(d)) and the fp32 kernel."""
    torch = torch_mod()
    rng = np.random.default_rng(3)
    B, T, H, Hkv, D = 1, 256, 2, 1, 128
    q, k, v = _attn_inputs(rng, B, T, H, Hkv, D)
    # bf16 with the sharp scale
    qk, qk64 = bf16_dev(np.concatenate([q, k], axis=2).reshape(B * T, -1).astype(np.float32))
    vt, vt64 = bf16_dev(np.ascontiguousarray(v.transpose(0, 2, 3, 1)).astype(np.float32))
    o = empty((B * T, H * D), "bf16")
    _ok(gf.gpt_op_attention(BF, qk, vt, o, B, T, H, Hkv, D, 100, 1.3225), "attention")
    _sync()
    x = qk64.reshape(B, T, H + Hkv, D)
    ref = oracle.attention(x[0, :, :H], x[0, :, H:], vt64.transpose(0, 3, 1, 2)[0], 100, 1.3225)
    assert np.max(np.abs(to_host(o).reshape(T, H, D) - ref)) < 5e-2
    # fp32 kernel: q, k, v side by side
    qkv, qkv64 = f32_dev(np.concatenate([q, k, v], axis=2).reshape(B * T, -1))
    of = empty((B * T, H * D), "f32")
    _ok(gf.gpt_op_attention(F32, qkv, None, of, B, T, H, Hkv, D, 37, 0.2), "attention f32")
    _sync()
    y = qkv64.reshape(T, H + 2 * Hkv, D)
    ref = oracle.attention(y[:, :H], y[:, H:H + Hkv], y[:, H + Hkv:], 37, 0.2)
    assert np.max(np.abs(to_host(of).reshape(T, H, D) - ref)) < 1e-5


# ----------------------------------------------------------------------------- lm_head + CE

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,C,V", [(300, 256, 1000), (256, 128, 4096), (257, 192, 1003)])
def test_lm_head_ce(dtype, M, C, V):
    """(257, 192, 1003): ragged rows, and a vocabulary that is neither a multiple of the
    384-wide column blocks nor of 4 (the logits' row pitch takes the element-wise stores)."""
    torch = torch_mod()
    rng = np.random.default_rng(M + V)
    xf_h = oracle.rms_norm(rng.standard_normal((M, C)), 0).astype(np.float32)
    wu_h = rng.standard_normal((V, C), dtype=np.float32) * np.float32(4.0 / math.sqrt(C))
    up = bf16_dev if dtype == "bf16" else f32_dev
    xf, xf64 = up(xf_h)
    wu, wu64 = up(wu_h)
    tgt = rng.integers(0, V, M).astype(np.int32)
    tgt[::7] = -1
    tok = rng.integers(0, V, M).astype(np.int32)
    t_tgt, t_tok = torch.from_numpy(tgt).cuda(), torch.from_numpy(tok).cuda()
    loss = empty((M,), "f32")
    mean = empty((1,), "f32")
    logits = empty((M, V), "f32")
    dt = BF if dtype == "bf16" else F32
    need = gf.gpt_op_lm_head_ce_workspace(dt, M, V)
    ws = torch.empty(need + 256, dtype=torch.uint8).cuda()
    wsp = ws.data_ptr() + (-ws.data_ptr()) % 256
    _ok(gf.gpt_op_lm_head_ce(dt, xf, wu, t_tgt, t_tok, M, C, V, 15.0, loss, mean, logits, wsp, need), "ce")
    _sync()
    zh = oracle.softcap(oracle.linear(xf64, wu64), 15.0)
    ref = oracle.token_losses(zh, tgt)
    assert np.max(np.abs(to_host(logits) - zh)) < 2e-4
    assert np.max(np.abs(to_host(loss) - ref)) < 2e-4
    assert abs(float(mean.item()) - oracle.mean_loss(ref, tgt)) < 1e-4
    # all targets ignored -> mean NaN, losses 0
    t_tgt.fill_(-1)
    _ok(gf.gpt_op_lm_head_ce(dt, xf, wu, t_tgt, t_tok, M, C, V, 15.0, loss, mean, None, wsp, need), "ce")
    _sync()
    assert math.isnan(float(mean.item())) and float(loss.abs().max().item()) == 0.0
