#!/usr/bin/env python3
"""Forward+loss throughput of nanochat d24 (T=2048, B=8, bf16) on one MI355X.

One step = one gpt_fwd_loss call over a batch of B*T synthetic tokens resident in HBM:
embedding, 24 layers, lm_head, softcapped cross-entropy and the mean loss.  The timed region
holds exactly K steps between device synchronisations; the JSON line reports whole-job
tokens/s, the dominant kernel's roofline position and the CPU oracle on a bounded sample of the
same workload.  Per-kernel times come from HIP events that gpt_fwd_loss_timed has the
dispatches themselves stamp (start of a launch's first kernel, end of its last) for every launch
of one kind in the forward pass, over separate measurement steps outside the throughput region.

Inputs are synthetic (seeded uniform token ids, N(0, 1/fan_in) weights) with the shapes of the
pages' workload: 2,048-token packed rows and a 32,768-entry vocabulary.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)


def device_info():
    """The GPU's compute-unit count and maximum shader clock as rocminfo reports them, and the
    dense bf16 MFMA peak they imply (4096 FLOP per CU per clock on gfx950); None if rocminfo is
    not available."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in txt.split("*******")[1:]:
        fields = {}
        for line in agent.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
        if fields.get("Device Type") != "GPU":
            continue
        try:
            cus = int(fields["Compute Unit"])
            mhz = int(fields["Max Clock Freq. (MHz)"].split()[0])
        except (KeyError, ValueError, IndexError):
            return None
        return {"name": fields.get("Marketing Name", ""), "arch": fields.get("Name", ""),
                "compute_units": cus, "max_sclk_mhz": mhz,
                "peak_bf16_tflops_from_clock": round(cus * mhz * 1e6 * 4096 / 1e12, 1)}
    return None


def _attn_flops(p, w, prior=False):
    """Attention FLOPs per token of one layer: QK^T and PV over the visible keys (average over
    positions of min(t+1, w)); the looped prior adds a second QK^T of the same width."""
    T = p.seq_len
    w = min(w, T)
    avg = (w * (w + 1) / 2 + (T - w) * w) / T
    return (6 if prior else 4) * p.n_head * p.head_dim * avg


def live_fraction(p):
    """Share of a nested linear's weights that are live (block lower triangular, inner share
    r = c1/C of both dimensions): 1 - r + r^2; 1 for a dense model."""
    r = getattr(p, "nested_c1", 0) / p.d_model
    return 1.0 - r + r * r if r else 1.0


def flops_per_token(p, windows):
    """Algorithmic forward FLOPs per token: every linear (2 per multiply-add; nested models:
    the live blocks only) plus attention over the visible keys only.  Looped trunk: pass 1
    needs L-1 full layers and the last layer's projection (its q, k), pass 2 all L layers with
    the prior.  Nested models count the lm_head once: the kfront=1 logits are a column prefix
    of the same product."""
    C, H, Hkv, D, F, V = p.d_model, p.n_head, p.n_kv_head, p.head_dim, p.mlp_dim, p.vocab
    live = live_fraction(p)
    qkv = 2 * C * (H + 2 * Hkv) * D * live
    lin = qkv + 2 * (H * D * C + 2 * C * F) * live
    L = p.n_layer
    if getattr(p, "looped", False):
        pass1 = (L - 1) * lin + qkv + sum(_attn_flops(p, w) for w in windows[:-1])
        pass2 = L * lin + sum(_attn_flops(p, w, prior=True) for w in windows)
        return pass1 + pass2 + 2 * C * V
    return L * lin + 2 * C * V + sum(_attn_flops(p, w) for w in windows)


KINDS = {  # gpt_kernel_kind -> name
    1: "qkv", 2: "attention", 3: "attn_out", 4: "mlp_up", 5: "mlp_down", 6: "lm_head",
}


def flops_per_launch(p, windows):
    """Algorithmic FLOPs of one launch of each kind (attention: the mean over its launches)."""
    M, C, H, Hkv, D, F, V = (p.batch * p.seq_len, p.d_model, p.n_head, p.n_kv_head, p.head_dim,
                             p.mlp_dim, p.vocab)
    if getattr(p, "looped", False):
        att = [_attn_flops(p, w) for w in windows[:-1]] + [_attn_flops(p, w, True) for w in windows]
    else:
        att = [_attn_flops(p, w) for w in windows]
    live = live_fraction(p)
    # nested: one lm_head pass gives both logits (the kfront=1 ones are its K-prefix)
    head = 2.0 * M * C * V
    return {1: 2.0 * M * C * (H + 2 * Hkv) * D * live, 2: M * sum(att) / len(att),
            3: 2.0 * M * H * D * C * live, 4: 2.0 * M * C * F * live, 5: 2.0 * M * F * C * live, 6: head}


def measured_traffic(root, kind):
    """HBM bytes per launch of kernel kind `kind` from the committed rocprofv3 PMC record
    (profiles/gemm_traffic.json), or None if the record lacks that kind or the GEMM source has
    changed since the counters were taken (the record stores the source hash)."""
    import hashlib
    path = os.path.join(root, "profiles", "gemm_traffic.json")
    try:
        rec = json.load(open(path))
        csrc = os.path.join(root, "decoder_only_transformer_layer_amd", "csrc")
        h = hashlib.sha256(open(os.path.join(csrc, "k_gemm.hip"), "rb").read()
                           + open(os.path.join(csrc, "common.h"), "rb").read()).hexdigest()
        if h != rec["kernel_source_sha256"]:
            return None
        return rec["kinds"][KINDS[kind]]["hbm_bytes_per_dispatch"]
    except (OSError, KeyError, ValueError):
        return None


def decode_bench(gf, p, model, steps):
    """Time gpt_decode_step for the preset's rows at the last cache position (every layer attends
    over its whole window), eagerly and replayed from a HIP graph.  Algorithmic bytes per step:
    every weight once (the linears, W_U and B rows of W_E) plus the cached keys and values each
    layer attends to."""
    import torch
    B, T, C, H, Hkv, D, F, V, L = (p.batch, p.seq_len, p.d_model, p.n_head, p.n_kv_head, p.head_dim,
                                   p.mlp_dim, p.vocab, p.n_layer)
    d = gf.Decoder(model)
    windows = gf.layer_windows(p.window_pattern, p.short_window, T, L)
    cur = torch.zeros(B, dtype=torch.int32, device="cuda")
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    out = torch.empty((B, V), dtype=torch.float32, device="cuda")
    for _ in range(3):
        if d.step(cur, pos, out) != gf.GPT_OK:
            raise RuntimeError("decode step failed")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        d.step(cur, pos, out)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.step(cur, pos, out)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    es = 2 if p.dtype == "bf16" else 4
    weights = (L * (C * (H + 2 * Hkv) * D + H * D * C + 2 * C * F) + V * C + B * C) * es
    kv = sum(2 * B * Hkv * min(w, T) * D * es for w in windows)
    gbs = (weights + kv) / (graph_ms * 1e-3) / 1e9
    print(f"[bench] decode: {eager_ms:.3f} ms/step eager, {graph_ms:.3f} ms/step graph "
          f"({B} rows at position {T - 1}), {gbs:.0f} GB/s algorithmic", file=sys.stderr, flush=True)
    return {"rows": B, "position": T - 1, "ms_per_step_eager": round(eager_ms, 4),
            "ms_per_step_graph": round(graph_ms, 4), "tokens_per_s_graph": round(B / (graph_ms * 1e-3), 1),
            "bytes_per_step": weights + kv, "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS}


def gemm_compare(gf, p, reps=20):
    """The preset's linear shapes (M = B*T rows) through gpt_op_linear with the plain store
    epilogue and through torch's F.linear (the ROCm dense-GEMM library) on the same bf16 operands
    in the same [out, in] weight layout: a yardstick for the GEMM main loop, outside the
    throughput region."""
    import torch
    M, C, F, V = p.batch * p.seq_len, p.d_model, p.mlp_dim, p.vocab
    qkv = (p.n_head + 2 * p.n_kv_head) * p.head_dim
    shapes = [("qkv", qkv, C), ("attn_out", C, p.n_head * p.head_dim), ("mlp_up", F, C),
              ("mlp_down", C, F), ("lm_head", V, C)]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(0)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def alternate(own, lib, rounds=5):
        # both warmed up, then timed in alternation so that clock ramps and drift hit both alike
        for _ in range(5):
            own()
            lib()
        t_own, t_lib = [], []
        for _ in range(rounds):
            t_own.append(timed(own))
            t_lib.append(timed(lib))
        return statistics.median(t_own), statistics.median(t_lib)

    out = []
    for name, N, K in shapes:
        a = torch.randn(M, K, device=dev, generator=gen).to(torch.bfloat16)
        wt = (torch.randn(N, K, device=dev, generator=gen) / math.sqrt(K)).to(torch.bfloat16)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        if gf.gpt_op_linear(gf.GPT_BF16, 0, a, wt, M, N, K, y) != gf.GPT_OK:
            raise RuntimeError(f"gpt_op_linear failed on {name}")
        ref = torch.nn.functional.linear(a, wt)
        torch.cuda.synchronize()
        rel = ((y.float() - ref.float()).abs().max() / ref.float().abs().max()).item()
        t_own, t_lib = alternate(lambda: gf.gpt_op_linear(gf.GPT_BF16, 0, a, wt, M, N, K, y),
                                 lambda: torch.nn.functional.linear(a, wt))
        fl = 2.0 * M * N * K
        print(f"[bench] gemm {name} {M}x{N}x{K}: own {t_own * 1e3:.1f} us ({fl / t_own / 1e9:.0f} TF/s), "
              f"library {t_lib * 1e3:.1f} us ({fl / t_lib / 1e9:.0f} TF/s), max rel diff {rel:.1e}",
              file=sys.stderr, flush=True)
        out.append({"gemm": name, "M": M, "N": N, "K": K, "own_us": round(t_own * 1e3, 1),
                    "library_us": round(t_lib * 1e3, 1)})
        del a, wt, y, ref
    return out


def cpu_baseline(p, w, tok, tgt, windows, rows, budget_s):
    """The oracle as it stands, in float32 (the dtype it offers for full-size runs), on whole
    rows of the same batch, one after another until `rows` rows are done or `budget_s` seconds
    have passed; its BLAS uses every thread it was given."""
    import numpy as np
    import oracle
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [0]) or None
    except Exception:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    params = {
        "wte": w.value(w.wte), "lm_head": w.value(w.lm_head),
        "resid_lambda": w.resid_lambda, "x0_lambda": w.x0_lambda,
        **{k: [w.value(a) for a in getattr(w, k)] for k in ("wq", "wk", "wv", "wo", "w1", "w2")},
    }
    if getattr(p, "value_embeds", False):
        params.update(ve=[w.value(a) for a in w.ve], ve_gate=[w.value(a) for a in w.ve_gate])
    if getattr(p, "looped", False):
        params.update(pass_emb=w.value(w.pass_emb), gate_logit=w.gate_logit)
    done, t_rows = 0, []
    c0 = time.perf_counter()
    for b in range(min(rows, p.batch)):
        r0 = time.perf_counter()
        oracle.forward(p, params, tok[b:b + 1], tgt[b:b + 1], dtype=np.float32, windows=windows)
        t_rows.append(time.perf_counter() - r0)
        done += 1
        print(f"[bench] cpu oracle: row {b} in {t_rows[-1]:.1f}s", file=sys.stderr, flush=True)
        if time.perf_counter() - c0 > budget_s:
            break
    cdt = time.perf_counter() - c0
    n = done * p.seq_len
    return {"value": round(n / cdt, 2), "unit": "tokens/s", "cores": blas or affinity or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{done} of {p.batch} rows x {p.seq_len} tokens ({n} tokens), float32 NumPy oracle, "
                      f"{cdt:.1f}s",
            "cpu_count": os.cpu_count(), "cpu_affinity": affinity, "blas_threads": blas,
            "seconds": round(cdt, 2), "seconds_per_row": [round(t, 2) for t in t_rows]}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="d24")
    ap.add_argument("--cpu-rows", type=int, default=8,
                    help="at most this many whole rows of the batch for the CPU oracle")
    ap.add_argument("--cpu-budget-s", type=float, default=25.0,
                    help="stop the CPU oracle after the row that passes this many seconds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-steps", type=int, default=3,
                    help="measurement steps per kernel kind for the per-kernel event timing")
    ap.add_argument("--decode-steps", type=int, default=20,
                    help="timed decode steps (one token per row, full cache); 0 skips the decode line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (a known-size reference "
                         "for HBM traffic counters)")
    ap.add_argument("--gemm-compare", action="store_true",
                    help="also time the preset's linear shapes (store epilogue) against torch's "
                         "F.linear")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the forward+loss "
              "path has no cross-GPU step; rows shard over GPUs with no communication.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decoder_only_transformer_layer_amd as gf
    import gptdata

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads and writes exactly 1 GiB
        torch.cuda.synchronize()
        del src, dst
        print("[bench] copy calibration: 1 GiB read + 1 GiB written", file=sys.stderr, flush=True)

    p = gptdata.preset(args.config)
    t0 = time.time()
    w, tok, tgt = gptdata.make_inputs(p)
    print(f"[bench] inputs {args.config} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    windows = gf.layer_windows(p.window_pattern, p.short_window, p.seq_len, p.n_layer)
    model = gf.DeviceModel(p, w)
    dev = torch.device("cuda:0")
    t_tok = torch.from_numpy(tok).to(dev)
    t_tgt = torch.from_numpy(tgt).to(dev)
    B, T = p.batch, p.seq_len
    loss = torch.empty((B, T), dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    nested = bool(getattr(p, "nested_c1", 0))
    if nested:  # both losses of the nested model (full and kfront=1) come from every step
        loss1 = torch.empty((B, T), dtype=torch.float32, device=dev)
        mean1 = torch.empty(1, dtype=torch.float32, device=dev)

    def fwd(timing=None):
        if nested:
            return model.forward_nested(t_tok, t_tgt, loss, mean, None, loss1, mean1, None, stream, timing)
        return model.forward(t_tok, t_tgt, loss, mean, None, stream, timing=timing)

    def step():
        st = fwd()
        if st != gf.GPT_OK:
            raise RuntimeError(gf.gpt_status_string(st))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done, mean loss {mean.item():.4f}"
          + (f", kfront=1 mean loss {mean1.item():.4f}" if nested else ""), file=sys.stderr, flush=True)

    # One event before every call and one after the last, all on the forward's stream: the first
    # and the last bracket the whole region (the reported mean), consecutive pairs give each call.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evs[i].record(stream)
        step()
    evs[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_call = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = per_call[len(per_call) // 2] if len(per_call) % 2 else \
        0.5 * (per_call[len(per_call) // 2 - 1] + per_call[len(per_call) // 2])
    ms_min = per_call[0]
    tok_s = B * T / (ms / 1e3)
    fpt = flops_per_token(p, windows)
    assert gf.gpt_device_status(model.ws_ptr) == gf.GPT_OK
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}; per call "
          f"median {ms_median:.3f}, min {ms_min:.3f}), {tok_s:,.0f} tok/s, {fpt * tok_s / 1e12:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    # Per-kernel time inside the forward pass: kernel start/end stamps on HIP events, for every
    # launch of one kind, over separate measurement steps on the forward's own stream.
    L = p.n_layer
    if getattr(p, "looped", False):  # pass 1 stops after its last layer's projection
        per_step = {1: 2 * L, 2: 2 * L - 1, 3: 2 * L - 1, 4: 2 * L - 1, 5: 2 * L - 1, 6: 1}
    else:  # nested: one pair covers both row blocks of a step, one lm_head pass both losses
        per_step = {1: L, 2: L, 3: L, 4: L, 5: L, 6: 1}
    fpl = flops_per_launch(p, windows)
    kern = {}
    for kind in KINDS:
        n = per_step[kind] * args.kernel_steps
        evb = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        eve = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evb + eve:
            e.record(stream)  # creates the underlying hipEvent_t
        torch.cuda.synchronize()
        for i in range(args.kernel_steps):  # one slice of event pairs per step
            sl = slice(i * per_step[kind], (i + 1) * per_step[kind])
            t = gf.launch_timing(kind, evb[sl], eve[sl])
            st = fwd(t)
            if st != gf.GPT_OK:
                raise RuntimeError(gf.gpt_status_string(st))
            assert t.recorded == per_step[kind]
        torch.cuda.synchronize()
        us = [b.elapsed_time(e) * 1e3 for b, e in zip(evb, eve)]
        avg = sum(us) / len(us)
        kern[KINDS[kind]] = {"kind": kind, "avg_us": round(avg, 2), "launches_per_step": per_step[kind],
                             "us_per_step": round(avg * per_step[kind], 1),
                             "tflops": round(fpl[kind] / (avg * 1e-6) / 1e12, 1)}
    dom = max(kern.values(), key=lambda k: k["us_per_step"])
    dk = dom["kind"]
    k_tflops = fpl[dk] / (dom["avg_us"] * 1e-6) / 1e12
    print("[bench] per-kernel (in the forward, HIP events): " + ", ".join(
        f"{n} {k['avg_us']:.1f} us x{k['launches_per_step']} ({k['tflops']:.0f} TF/s)" for n, k in kern.items()),
        file=sys.stderr, flush=True)

    traffic = measured_traffic(ROOT, dk)
    traffic_src = ("stored: HBM bytes per dispatch from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                   "over this kernel source, profiles/gemm_traffic.json" if traffic is not None else
                   "none: no counter record for this kernel source")

    dec = None
    if args.decode_steps > 0 and not nested and not getattr(p, "looped", False) and not p.value_embeds:
        dec = decode_bench(gf, p, model, args.decode_steps)

    gcmp = gemm_compare(gf, p) if args.gemm_compare and p.dtype == "bf16" else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p, w, tok, tgt, windows, args.cpu_rows, args.cpu_budget_s)

    out = {
        "metric": "forward+loss tokens/sec at d24 T=2048 bf16; % of MFMA bf16 peak",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "ms_per_step_min": round(ms_min, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded uniform token ids, N(0,1/fan_in) weights",
        "pct_mfma_peak": round(100.0 * fpt * tok_s / (PEAK_BF16_TFLOPS * 1e12), 2),
        "config": {"workload": f"nanochat {args.config} forward+loss", "batch": B, "seq_len": T,
                   "n_layer": p.n_layer, "d_model": p.d_model, "n_head": p.n_head, "vocab": p.vocab,
                   "flops_per_token": round(fpt), "windows": "SSSL short 1024, last layer full"},
        "roofline": {"bound": "mfma", "kernel": KINDS[dk],
                     "achieved": round(k_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "avg_launch_us": dom["avg_us"], "flops_per_launch": fpl[dk]},
        "kernels": kern,
        "decode": dec,
        "gemm_vs_library": gcmp,
        "cpu_baseline": cpu,
        "device": device_info(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
