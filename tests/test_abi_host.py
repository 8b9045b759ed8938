"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before touching any device (these run without a GPU)."""
import ctypes
import os
import re

import pytest

import decoder_only_transformer_layer_amd as gf
import gptdata

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("gptfwd.h", "gptfwd_ops.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(gpt_\w+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gf.LIB_PATH):
        pytest.skip("libgptfwd.so not built")
    return gf._load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(gf.EXPORTED) == names


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert gf.gpt_status_string(s) not in ("", "unknown status")
    assert gf.gpt_status_string(7) == "unknown status"


def _cfg(**kw):
    p = gptdata.preset("d24")
    c = gf.make_cfg(p)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_validate_presets(lib):
    for name in ("tiny", "d12", "d24", "d24gve", "d24loop", "d24nest"):
        c = gf.make_cfg(gptdata.preset(name))
        assert gf.gpt_validate(c) == gf.GPT_OK, name
        assert gf.gpt_workspace_bytes(c) > 0


@pytest.mark.parametrize("field,value,status", [
    ("n_layer", 0, gf.GPT_E_INVALID_ARG),
    ("batch", 0, gf.GPT_E_INVALID_ARG),             # empty inputs are rejected, not skipped
    ("seq_len", 0, gf.GPT_E_INVALID_ARG),
    ("vocab", 1, gf.GPT_E_INVALID_ARG),
    ("n_kv_head", 5, gf.GPT_E_INVALID_ARG),        # 12 % 5 != 0
    ("softcap", 0.0, gf.GPT_E_INVALID_ARG),
    ("attn_scale", -1.0, gf.GPT_E_INVALID_ARG),
    ("norm_eps", -1e-6, gf.GPT_E_INVALID_ARG),
    ("dtype", 7, gf.GPT_E_INVALID_ARG),
    ("head_dim", 96, gf.GPT_E_UNSUPPORTED),
    ("d_model", 1000, gf.GPT_E_UNSUPPORTED),
    ("mlp_dim", 6100, gf.GPT_E_UNSUPPORTED),
    ("seq_len", 2000, gf.GPT_E_UNSUPPORTED),        # bf16 needs T % 64 == 0
    ("seq_len", 1 << 19, gf.GPT_E_UNSUPPORTED),     # one row's q/k: 2^19 * 24 * 128 * 2 B > 2^31
])
def test_validate_rejects(lib, field, value, status):
    c = _cfg(**{field: value})
    assert gf.gpt_validate(c) == status
    assert gf.gpt_workspace_bytes(c) == 0


def test_validate_rejects_bad_window(lib):
    c = _cfg()
    c._win[3] = 0
    assert gf.gpt_validate(c) == gf.GPT_E_INVALID_ARG
    c.window = None
    assert gf.gpt_validate(c) == gf.GPT_E_INVALID_ARG
    assert lib.gpt_validate(None) == gf.GPT_E_INVALID_ARG


def _weights(L, fake=0x100000):
    arr = (ctypes.c_void_p * L)(*[fake + 256 * i for i in range(L)])
    ptr = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    w = gf.gpt_weights(fake, fake, fake, fake, ptr, ptr, ptr, ptr, ptr, ptr)
    w._keep = arr
    return w


def test_fwd_loss_argument_errors_return_before_launch(lib):
    """Every host-detectable error returns before any HIP call: fake device addresses are
    never dereferenced."""
    c = _cfg()
    L = c.n_layer
    w = _weights(L)
    need = gf.gpt_workspace_bytes(c)
    F = 0x200000
    call = lambda **kw: lib.gpt_fwd_loss(
        ctypes.byref(kw.get("cfg", c)), ctypes.byref(kw.get("w", w)) if kw.get("w", w) is not None else None,
        kw.get("tokens", F), kw.get("targets", F), kw.get("loss", F), kw.get("mean", F),
        kw.get("logits", None), kw.get("ws", 0x10000000), kw.get("wsb", need), None)
    assert call(tokens=None) == gf.GPT_E_INVALID_ARG
    assert call(w=None) == gf.GPT_E_INVALID_ARG
    assert call(loss=None) == gf.GPT_E_INVALID_ARG          # targets given, loss missing
    assert call(targets=None, logits=None) == gf.GPT_E_INVALID_ARG  # nothing to compute
    assert call(ws=None) == gf.GPT_E_WORKSPACE
    assert call(wsb=need - 1) == gf.GPT_E_WORKSPACE
    assert call(ws=0x10000000 + 8) == gf.GPT_E_WORKSPACE   # not 256-aligned
    w2 = _weights(L)
    w2._keep[5] = None
    assert call(w=w2) == gf.GPT_E_INVALID_ARG
    w3 = _weights(L)
    w3._keep[2] = 0x100008                                  # not 16-byte aligned
    assert call(w=w3) == gf.GPT_E_INVALID_ARG
    bad = _cfg(head_dim=96)
    assert call(cfg=bad) == gf.GPT_E_UNSUPPORTED


def test_value_embedding_validation(lib):
    """has_ve needs head_dim 128 on the bf16 path (fp32 takes any) and the tables/gates of
    every selected layer; the selection follows the alternating rule, last layer included."""
    assert gf.ve_layers(24) == [l % 2 for l in range(24)]
    assert gf.ve_layers(5) == [1, 0, 1, 0, 1]
    p = gptdata.preset("d24gve")
    c = gf.make_cfg(p.with_(head_dim=64, n_head=24, n_kv_head=8))
    assert gf.gpt_validate(c) == gf.GPT_E_UNSUPPORTED
    c32 = gf.make_cfg(p.with_(head_dim=64, n_head=24, n_kv_head=8, dtype="f32"))
    assert gf.gpt_validate(c32) == gf.GPT_OK
    c = gf.make_cfg(p)
    assert gf.gpt_validate(c) == gf.GPT_OK
    L, F = c.n_layer, 0x200000
    need = gf.gpt_workspace_bytes(c)
    w = _weights(L)                       # no ve / ve_gate arrays
    call = lambda w: lib.gpt_fwd_loss(ctypes.byref(c), ctypes.byref(w), F, F, F, F, None,
                                      0x10000000, need, None)
    assert call(w) == gf.GPT_E_INVALID_ARG
    arr = (ctypes.c_void_p * L)(*[0x300000 + 256 * i for i in range(L)])
    w.ve = w.ve_gate = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    arr[1] = None                         # layer 1 is selected (L = 24: odd layers)
    assert call(w) == gf.GPT_E_INVALID_ARG


def test_looped_validation(lib):
    """The looped trunk needs head_dim 128 on bf16, a 0/1 flag, and its pass embeddings and
    gate logits."""
    p = gptdata.preset("d24loop")
    c = gf.make_cfg(p)
    assert gf.gpt_validate(c) == gf.GPT_OK
    assert gf.gpt_workspace_bytes(c) > gf.gpt_workspace_bytes(gf.make_cfg(p.with_(looped=False)))
    assert gf.gpt_validate(gf.make_cfg(p.with_(head_dim=64, n_head=24, n_kv_head=24))) == gf.GPT_E_UNSUPPORTED
    bad = gf.make_cfg(p)
    bad.looped = 2
    assert gf.gpt_validate(bad) == gf.GPT_E_INVALID_ARG
    w = _weights(c.n_layer)               # no pass embeddings / gate logits
    need = gf.gpt_workspace_bytes(c)
    F = 0x200000
    assert lib.gpt_fwd_loss(ctypes.byref(c), ctypes.byref(w), F, F, F, F, None, 0x10000000, need,
                            None) == gf.GPT_E_INVALID_ARG


def test_nested_validation(lib):
    """Nested models: exact proportional splits, a 64-multiple inner width, 128-column inner
    q/k/v segments on bf16, no value embeddings or looped trunk; the nested entry point
    rejects a plain model and inconsistent kfront=1 outputs before any launch."""
    p = gptdata.preset("d24nest")
    assert gf.gpt_validate(gf.make_cfg(p)) == gf.GPT_OK
    assert gf.gpt_validate(gf.make_cfg(p.with_(nested_c1=p.d_model))) == gf.GPT_OK    # one block
    assert gf.gpt_validate(gf.make_cfg(p.with_(nested_c1=-64))) == gf.GPT_E_INVALID_ARG
    assert gf.gpt_validate(gf.make_cfg(p.with_(nested_c1=2 * p.d_model))) == gf.GPT_E_INVALID_ARG
    assert gf.gpt_validate(gf.make_cfg(p.with_(nested_c1=352))) == gf.GPT_E_INVALID_ARG  # 24*352 % 1536
    # exact splits, but an inner width of 32 columns
    odd = p.with_(d_model=960, n_head=30, n_kv_head=30, mlp_dim=3840, nested_c1=32, dtype="f32")
    assert gf.gpt_validate(gf.make_cfg(odd)) == gf.GPT_E_UNSUPPORTED
    assert gf.gpt_validate(gf.make_cfg(odd.with_(nested_c1=64))) == gf.GPT_OK
    # bf16: 2 inner heads of 64 = 128 columns is fine, 1 inner KV head of 64 is not
    q = p.with_(n_head=24, n_kv_head=12, nested_c1=128)
    assert gf.gpt_validate(gf.make_cfg(q)) == gf.GPT_E_UNSUPPORTED
    assert gf.gpt_validate(gf.make_cfg(q.with_(dtype="f32"))) == gf.GPT_OK
    assert gf.gpt_validate(gf.make_cfg(p.with_(value_embeds=True))) == gf.GPT_E_UNSUPPORTED
    assert gf.gpt_validate(gf.make_cfg(p.with_(looped=True, head_dim=128, n_head=12, n_kv_head=12))) \
        == gf.GPT_E_UNSUPPORTED
    c = gf.make_cfg(p)
    w = _weights(c.n_layer)
    need = gf.gpt_workspace_bytes(c)
    F = 0x200000

    def call(cfg=c, loss1=F, mean1=F, logits1=None, targets=F):
        return lib.gpt_fwd_loss_nested(ctypes.byref(cfg), ctypes.byref(w), F, targets, F, F, None,
                                       loss1, mean1, logits1, 0x10000000, need, None, None)
    plain = gf.make_cfg(gptdata.preset("d24"))
    assert call(cfg=plain) == gf.GPT_E_INVALID_ARG
    assert call(mean1=None) == gf.GPT_E_INVALID_ARG          # loss_k1 without mean_k1
    assert call(loss1=None) == gf.GPT_E_INVALID_ARG
    assert call(loss1=F + 2) == gf.GPT_E_INVALID_ARG         # misaligned
    assert lib.gpt_fwd_loss_nested(ctypes.byref(c), ctypes.byref(w), F, None, None, None, F, F, F, None,
                                   0x10000000, need, None, None) == gf.GPT_E_INVALID_ARG  # k1 loss, no targets
    assert lib.gpt_fwd_loss_nested(ctypes.byref(c), ctypes.byref(w), F, F, F, F, None, F, F, None,
                                   None, need, None, None) == gf.GPT_E_WORKSPACE


def test_decode_validation_and_argument_errors(lib):
    """Decoding: base models with 1..32 rows and a cache of <= 8192 positions; every
    host-detectable error returns before any launch (fake device addresses are never touched)."""
    p = gptdata.preset("d24")
    c = gf.make_cfg(p)
    assert gf.gpt_kv_cache_bytes(c) == 24 * 2 * 8 * 12 * 2048 * 128 * 2
    assert gf.gpt_decode_workspace_bytes(c) > 0
    # bf16 d_model beyond 4096 (the widest the decode products' row scales and the decode tests
    # cover): refused before any launch (the forward itself takes it)
    wide = p.with_(d_model=8192, n_head=64, n_kv_head=64, mlp_dim=4 * 8192, n_layer=2)
    assert gf.gpt_validate(gf.make_cfg(wide)) == gf.GPT_OK
    for bad in (p.with_(batch=33), p.with_(seq_len=16384), gptdata.preset("d24gve"),
                gptdata.preset("d24loop"), gptdata.preset("d24nest"), wide):
        assert gf.gpt_kv_cache_bytes(gf.make_cfg(bad)) == 0
        assert gf.gpt_decode_workspace_bytes(gf.make_cfg(bad)) == 0
    w = _weights(c.n_layer)
    need = gf.gpt_decode_workspace_bytes(c)
    F, CACHE, WS = 0x200000, 0x40000000, 0x10000000

    def call(cfg=c, tokens=F, pos=F, cache=CACHE, logits=F, ws=WS, wsb=need):
        return lib.gpt_decode_step(ctypes.byref(cfg), ctypes.byref(w), tokens, pos, cache, logits, ws,
                                   wsb, None)
    assert call(tokens=None) == gf.GPT_E_INVALID_ARG
    assert call(pos=None) == gf.GPT_E_INVALID_ARG
    assert call(pos=F + 2) == gf.GPT_E_INVALID_ARG
    assert call(logits=None) == gf.GPT_E_INVALID_ARG
    assert call(cache=None) == gf.GPT_E_INVALID_ARG
    assert call(cache=CACHE + 16) == gf.GPT_E_INVALID_ARG       # not 256-aligned
    assert call(ws=None) == gf.GPT_E_WORKSPACE
    assert call(wsb=need - 1) == gf.GPT_E_WORKSPACE
    assert call(cfg=gf.make_cfg(p.with_(batch=33))) == gf.GPT_E_UNSUPPORTED
    assert call(cfg=gf.make_cfg(gptdata.preset("d24gve"))) == gf.GPT_E_UNSUPPORTED
    assert call(cfg=gf.make_cfg(wide)) == gf.GPT_E_UNSUPPORTED
    pw = gf.gpt_prefill_workspace_bytes(c)
    assert pw == gf.gpt_workspace_bytes(c) > 0
    Pf = lambda cfg=c, plen=64, tokens=F, cache=CACHE, logits=F, ws=WS, wsb=pw: lib.gpt_prefill(
        ctypes.byref(cfg), ctypes.byref(w), tokens, plen, None, cache, logits, ws, wsb, None)
    assert Pf(plen=0) == gf.GPT_E_INVALID_ARG
    assert Pf(plen=p.seq_len + 64) == gf.GPT_E_INVALID_ARG
    assert Pf(plen=100) == gf.GPT_E_UNSUPPORTED           # bf16 forward needs a multiple of 64
    assert Pf(cache=CACHE + 16) == gf.GPT_E_INVALID_ARG
    assert Pf(logits=None) == gf.GPT_E_INVALID_ARG
    assert Pf(tokens=None) == gf.GPT_E_INVALID_ARG
    assert Pf(wsb=pw - 1) == gf.GPT_E_WORKSPACE
    assert Pf(cfg=gf.make_cfg(gptdata.preset("d24gve"))) == gf.GPT_E_UNSUPPORTED
    S = lambda **kw: lib.gpt_sample(kw.get("logits", F), kw.get("b", 2), kw.get("v", 100), kw.get("k", 5),
                                    kw.get("t", 1.0), kw.get("u", F), kw.get("out", F), None)
    assert S(logits=None) == gf.GPT_E_INVALID_ARG
    assert S(u=None) == gf.GPT_E_INVALID_ARG
    assert S(out=None) == gf.GPT_E_INVALID_ARG
    assert S(b=0) == gf.GPT_E_INVALID_ARG
    assert S(v=0) == gf.GPT_E_INVALID_ARG
    assert S(t=-0.5) == gf.GPT_E_INVALID_ARG
    assert S(t=float("nan")) == gf.GPT_E_INVALID_ARG
    assert S(t=float("inf")) == gf.GPT_E_INVALID_ARG


def test_fwd_loss_timed_argument_errors(lib):
    """The timing record is checked before anything else; a bad one never reaches a launch."""
    c = _cfg()
    w = _weights(c.n_layer)
    need = gf.gpt_workspace_bytes(c)
    F = 0x200000
    ev = (ctypes.c_void_p * 2)(F, F)
    evp = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))

    def call(t, ws=0x10000000):
        return lib.gpt_fwd_loss_timed(ctypes.byref(c), ctypes.byref(w), F, F, F, F, None, ws, need,
                                      None, ctypes.byref(t))
    assert call(gf.gpt_launch_timing(0, 2, evp, evp, 0)) == gf.GPT_E_INVALID_ARG      # no such kind
    assert call(gf.gpt_launch_timing(7, 2, evp, evp, 0)) == gf.GPT_E_INVALID_ARG
    assert call(gf.gpt_launch_timing(gf.GPT_KERNEL_MLP_UP, -1, evp, evp, 0)) == gf.GPT_E_INVALID_ARG
    assert call(gf.gpt_launch_timing(gf.GPT_KERNEL_MLP_UP, 2, None, evp, 0)) == gf.GPT_E_INVALID_ARG
    t = gf.gpt_launch_timing(gf.GPT_KERNEL_MLP_UP, 2, evp, evp, 5)
    assert call(t, ws=None) == gf.GPT_E_WORKSPACE                  # then the usual checks
    assert t.recorded == 0


def test_op_argument_errors(lib):
    F = 0x200000
    assert lib.gpt_op_linear(1, 0, None, F, 10, 10, 64, F, None) == gf.GPT_E_INVALID_ARG
    assert lib.gpt_op_linear(1, 3, F, F, 10, 10, 64, F, None) == gf.GPT_E_INVALID_ARG
    assert lib.gpt_op_linear(1, 0, F, F, 10, 10, 60, F, None) == gf.GPT_E_UNSUPPORTED
    assert lib.gpt_op_attention(1, F, F, F, 1, 100, 2, 2, 128, 8, 0.1, None) == gf.GPT_E_UNSUPPORTED
    assert lib.gpt_op_attention(1, F, F, F, 1, 128, 3, 2, 128, 8, 0.1, None) == gf.GPT_E_INVALID_ARG
    assert lib.gpt_op_attention(1, F, F, F, 1, 128, 2, 2, 80, 8, 0.1, None) == gf.GPT_E_UNSUPPORTED
    assert lib.gpt_op_embed_norm(1, F, F, F, F, F, F, F, 4, 6, 10, 1e-6, F, None) == gf.GPT_E_INVALID_ARG
    assert lib.gpt_op_qk_rope_norm(1, F, 100, F, 4, 4, 1, 256, 1e-6, None) == gf.GPT_E_INVALID_ARG
    assert lib.gpt_op_rope_table(F, 4, 7, 1e5, None) == gf.GPT_E_INVALID_ARG
    # 32-bit limits: RoPE table entries (T * D/2) and one sequence's bf16 q/k rows (< 2^31 bytes)
    assert lib.gpt_op_rope_table(F, 1 << 25, 128, 1e5, None) == gf.GPT_E_UNSUPPORTED
    assert lib.gpt_op_attention(1, F, F, F, 1, 1 << 19, 12, 12, 128, 8, 0.1, None) == gf.GPT_E_UNSUPPORTED
    # fused QKV epilogue (RoPE table given): T % 32 == 0 only (head_dim 64 and 128)
    assert lib.gpt_op_qkv(F, F, F, F, 1, 100, 256, 2, 2, 128, F, 1e-6, F, F, None) == gf.GPT_E_UNSUPPORTED
    assert lib.gpt_op_qkv(F, F, F, F, 1, 100, 256, 2, 2, 64, F, 1e-6, F, F, None) == gf.GPT_E_UNSUPPORTED
    assert lib.gpt_op_lm_head_ce_workspace(1, 16, 1) == 0
    need = lib.gpt_op_lm_head_ce_workspace(1, 16, 100)
    assert need > 0
    assert lib.gpt_op_lm_head_ce(1, F, F, F, F, 16, 64, 100, 15.0, F, F, None, 0x10000000, need - 4,
                                 None) == gf.GPT_E_WORKSPACE
    assert lib.gpt_op_lm_head_ce(1, F, F, None, F, 16, 64, 100, 15.0, F, F, None, 0x10000000, need,
                                 None) == gf.GPT_E_INVALID_ARG


def test_layer_windows_matches_pattern():
    assert gf.layer_windows("SSSL", 1024, 2048, 24) == [1024, 1024, 1024, 2048] * 6
    assert gf.layer_windows("SSSL", 1024, 2048, 12)[-1] == 2048
    assert gf.layer_windows("SSSL", 128, 256, 2) == [128, 256]
    assert gf.layer_windows("SSSL", 1024, 2048, 5) == [1024, 1024, 1024, 2048, 2048]


def test_binding_tensor_checks():
    """The DeviceModel / Decoder methods reject tensors the C functions would read or write out
    of bounds (wrong dtype, size or layout, host memory) before anything is enqueued."""
    import torch
    ok = torch.zeros(6, dtype=torch.int32)
    gf._require(None, "targets", "int32", 6)                 # optional and absent
    gf._require(0x200000, "tokens", "int32", 6)              # raw device address: unchecked
    with pytest.raises(ValueError, match="required"):
        gf._require(None, "tokens", "int32", 6, optional=False)
    with pytest.raises(TypeError):
        gf._require(ok.numpy(), "tokens", "int32", 6)
    with pytest.raises(ValueError, match="int32"):
        gf._require(ok.long(), "tokens", "int32", 6)
    with pytest.raises(ValueError, match="elements"):
        gf._require(ok[:5], "tokens", "int32", 6)
    with pytest.raises(ValueError, match="contiguous"):
        gf._require(torch.zeros((3, 4), dtype=torch.int32)[:, :2], "tokens", "int32", 6)
    with pytest.raises(ValueError, match="GPU"):
        gf._require(ok, "tokens", "int32", 6)


def test_noalloc_refuses_before_any_hip_call(lib):
    """gpt_fwd_loss_noalloc checks the configuration and its workspace size on the host before
    anything else: an invalid configuration reports gpt_validate's status, one whose workspace
    exceeds the fixed array GPT_E_WORKSPACE (the pointers are never dereferenced)."""
    w = gf.gpt_weights()
    big = gf.make_cfg(gptdata.preset("d24"))
    assert gf.gpt_workspace_bytes(big) > gf.GPT_NOALLOC_MAX_BYTES
    assert gf.gpt_fwd_loss_noalloc(big, w, 16, 16, 16, 16, None, 0) == gf.GPT_E_WORKSPACE
    bad = _cfg(head_dim=96)
    assert gf.gpt_fwd_loss_noalloc(bad, w, 16, 16, 16, 16, None, 0) == gf.GPT_E_UNSUPPORTED
    tiny = gf.make_cfg(gptdata.preset("tiny"))
    assert 0 < gf.gpt_workspace_bytes(tiny) <= gf.GPT_NOALLOC_MAX_BYTES
