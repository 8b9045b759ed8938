"""gpt_fwd_loss_noalloc (the library's fixed workspace array instead of a caller workspace)
against gpt_fwd_loss on the same inputs: the same kernels in the same order, so the outputs must
be bit-identical.  Two calls in a row through the no-alloc entry point, the second on a smaller
batch, so the second call runs in an array that still holds the first call's contents."""
import numpy as np
import pytest

import decoder_only_transformer_layer_amd as gf
import gptdata
from gpu_helpers import torch_mod

pytestmark = pytest.mark.gpu


def _outputs(torch, m, tok, tgt, noalloc):
    B, T, V = tok.shape[0], tok.shape[1], m.p.vocab
    loss = torch.full((B, T), float("nan"), dtype=torch.float32, device="cuda")
    mean = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    logits = torch.full((B, T, V), float("nan"), dtype=torch.float32, device="cuda")
    fn = m.forward_noalloc if noalloc else m.forward
    st = fn(tok, tgt, loss, mean, logits)
    torch.cuda.synchronize()
    assert st == gf.GPT_OK, gf.gpt_status_string(st)
    return loss.cpu().numpy(), mean.cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry(dtype):
    torch = torch_mod()
    p = gptdata.Preset(name="noalloc", n_layer=3, d_model=256, n_head=4, n_kv_head=2, head_dim=128,
                       mlp_dim=1024, vocab=1000, seq_len=320 if dtype == "bf16" else 200, batch=2,
                       dtype=dtype, short_window=100, lambda_range=(0.9, 1.1), mu_range=(0.0, 0.2),
                       seed=61)
    w, tok, tgt = gptdata.make_inputs(p, ignore_frac=0.1)
    for batch in (2, 1):  # the second call: a smaller input in the same array
        m = gf.DeviceModel(p, w, batch=batch)
        assert m.ws_bytes <= gf.GPT_NOALLOC_MAX_BYTES
        t_tok = torch.from_numpy(np.ascontiguousarray(tok[:batch])).cuda()
        t_tgt = torch.from_numpy(np.ascontiguousarray(tgt[:batch])).cuda()
        ref = _outputs(torch, m, t_tok, t_tgt, noalloc=False)
        got = _outputs(torch, m, t_tok, t_tgt, noalloc=True)
        print(f"  {dtype} batch {batch}: mean loss {float(got[1][0]):.6f}")
        for r, g in zip(ref, got):
            assert np.array_equal(r, g, equal_nan=True)
        assert np.isfinite(got[1][0])
