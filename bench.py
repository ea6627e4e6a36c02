#!/usr/bin/env python3
"""Throughput of one GPT-2 training step on one MI355X.

A step is the whole hot path over one batch of synthetic tokens:
zero_grad, forward with the fused softmax cross-entropy, backward, global
gradient-norm clip and AdamW -- all through the C ABI of libgpt2.so.

  python bench.py [--steps K] [--warmup W] [--workload gpt2-124m|gpt2-xl|sft]

Prints ONE JSON line.  value = tokens per second over the K timed steps
(inputs already resident in device memory).  roofline = the kernel with the
most time of the two largest, timed live with HIP events on the library's
stream during the timed steps, against the bf16 dense matrix-core peak: in a
training step the grouped weight-gradient GEMM (2*B*T flops per gradient
element it produces), in a forward-only pass the lm_head forward GEMM
(2*B*T*Vp*C flops).  cpu_baseline = the CPU oracle (numpy) on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    "gpt2-124m": dict(model="gpt2-124m", B=16, T=1024, data="zipf", lr=6e-4, wd=0.1,
                      desc="GPT-2 124M training step (fwd + bwd + clip + AdamW), bf16, B=16, "
                           "T=1024, Zipf(1.1) token ids with end-of-text separators"),
    "sft": dict(model="gpt2-124m", B=16, T=1024, data="sft", lr=2e-5, wd=0.0,
                desc="GPT-2 124M masked fine-tuning step, bf16, B=16, T=1024, prompt targets -1"),
    "gpt2-xl": dict(model="gpt2-xl", B=8, T=1024, data="zipf", lr=6e-4, wd=0.1,
                    desc="GPT-2 XL-shape training step (L=48, C=1600, H=25), bf16, B=8, T=1024"),
    "gpt2-124m-eval": dict(model="gpt2-124m", B=16, T=1024, data="zipf", lr=None, wd=0.0,
                           eval=True,
                           desc="GPT-2 124M evaluation pass (forward + losses + per-sequence "
                                "mean losses, no gradient), bf16, B=16, T=1024, Zipf ids"),
    "gpt2-124m-accum": dict(model="gpt2-124m", B=16, T=1024, data="zipf", accum=32, lr=None,
                            wd=0.1,
                            desc="GPT-2 124M full optimizer step: 32 micro-batches of 16x1024 "
                                 "(524,288 tokens) with gradient accumulation, clip 1.0, AdamW, "
                                 "lr warmup 715 steps then cosine 6e-4 -> 6e-5"),
    "gpt2-124m-fusedhead": dict(model="gpt2-124m", B=16, T=1024, data="zipf", lr=6e-4, wd=0.1,
                                head_chunk=4096,
                                desc="GPT-2 124M training step, bf16, B=16, T=1024, Zipf ids, with "
                                     "the fused lm_head + cross-entropy (no logits tensor; the "
                                     "backward recomputes logits in slices of 4096 vocabulary "
                                     "columns, a recomputation MFU does not count)"),
    "gpt2-124m-eval-fusedhead": dict(model="gpt2-124m", B=16, T=1024, data="zipf", lr=None,
                                     wd=0.0, eval=True, head_chunk=4096,
                                     desc="GPT-2 124M evaluation pass, bf16, B=16, T=1024, Zipf "
                                          "ids, fused lm_head + cross-entropy (no logits tensor)"),
    "gpt2-124m-generate-cached": dict(model="gpt2-124m", B=8, T=32, data="zipf", lr=None, wd=0.0,
                                      gen=96, top_k=50, cached=True,
                                      desc="GPT-2 124M sampling loop with a key/value cache, bf16: "
                                           "8 sequences, 32-token Zipf prompts, 96 new tokens "
                                           "each, temperature 1, top-k 50; the prompt is "
                                           "computed once, each new token runs the blocks for "
                                           "its own position; value = new tokens per second"),
    "gpt2-124m-generate": dict(model="gpt2-124m", B=8, T=32, data="zipf", lr=None, wd=0.0,
                               gen=96, top_k=50,
                               desc="GPT-2 124M sampling loop, bf16: 8 sequences, 32-token Zipf "
                                    "prompts, 96 new tokens each, temperature 1, top-k 50, the "
                                    "whole cropped context recomputed per token (no key/value "
                                    "cache); value = new tokens per second"),
}

METRIC = "training tokens/sec + MFU, GPT-2 124M bf16 B=16 T=1024 on one MI355X"

# HBM traffic per launch of the two largest kernels of the GPT-2 124M step at
# B=16, T=1024, from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE)
# over `bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-probe`, each
# scaled by what the same counter reads for a 1 GiB device copy (fetch x2.000,
# write x1.000); profiles/gpt2_124m_b16_hbm_traffic.md.
#   grouped weight gradients: 9,616,575,529 B read + 483,135,872 B written
#   lm_head forward GEMM:     1,876,437,836 B read + 1,648,361,472 B written
# Remove an entry whenever its kernel changes, until it is measured again.
TRAFFIC_BYTES = {("gpt2-124m", "WGRAD"): 10099711401,
                 ("gpt2-124m", "LMHEAD_FWD"): 3524799308,
                 ("gpt2-124m-eval", "LMHEAD_FWD"): 3524799308}


def flops_per_token(d, T):
    L, C, Vp = d["n_layer"], d["n_embd"], d["padded_vocab_size"]
    causal = 6 * (12 * L * C * C + C * Vp) + 6 * L * C * T
    n_nonemb = 12 * L * C * C + 13 * L * C + 2 * C
    nanogpt = 6 * n_nonemb + 12 * L * C * T
    return causal, nanogpt


def cpu_baseline(d, wl, seconds_hint=20.0):
    """The oracle as it stands, on one sequence of the workload (B=1, full T):
    forward, backward, clip and AdamW over every parameter."""
    import numpy as np
    import oracle
    import synthetic
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) \
            if threadpoolctl.threadpool_info() else 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        blas = "unknown"
    cfg = oracle.Config(**d)
    T = wl["T"]
    flat = synthetic.init_params(d, seed=42)
    if wl["data"] == "sft":
        idx, tgt = synthetic.sft_batch(1, T, seed=1004)
    else:
        idx, tgt = synthetic.zipf_batch(1, T, seed=1002)
    m, v = np.zeros_like(flat), np.zeros_like(flat)
    t0 = time.perf_counter()
    if wl.get("gen"):
        n = 4
        uni = synthetic.uniforms((1, n), seed=99).astype(np.float64)
        t0 = time.perf_counter()
        oracle.generate(flat, idx, n, 1.0, wl["top_k"], uni, cfg)
        dt = time.perf_counter() - t0
        return {"value": round(n / dt, 3), "unit": "new tokens/s", "cores": int(threads),
                "kind": "oracle", "blas": blas,
                "sample": f"{n} new tokens of 1 sequence after a {T}-token prompt; {dt:.1f} s"}
    if wl.get("eval"):
        _, cache = oracle.forward(flat, idx, tgt, cfg)
        oracle.sequence_losses(cache["row_loss"], tgt)
        what = "forward + losses + per-sequence mean losses"
    else:
        lr = wl["lr"] if wl["lr"] is not None else 6e-4 / 715
        oracle.train_step(flat, m, v, 1, [(idx, tgt)], cfg, lr=lr, weight_decay=wl["wd"])
        what = "one full step (fwd+bwd+clip+AdamW over all params)"
    dt = time.perf_counter() - t0
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "blas": blas,
            "sample": f"{what} on 1 x {T} tokens of the same workload; {dt:.1f} s"}


def library_gemm(torch, BT, d):
    """The platform's bf16 GEMM (torch.mm, fp32 accumulation, bf16 out, no
    epilogue) on the matrix products of one step, timed with events over 10
    calls after 3 warm-up calls; one line per shape on stderr."""
    C, Vp = d["n_embd"], d["padded_vocab_size"]
    shapes = [  # (product, M, N, K, layout of C[M,N] = A B): nt = B given as (N, K)
        ("lm_head forward", BT, Vp, C, "nt"), ("qkv forward", BT, 3 * C, C, "nt"),
        ("proj forward", BT, C, C, "nt"), ("fc forward", BT, 4 * C, C, "nt"),
        ("fcproj forward", BT, C, 4 * C, "nt"), ("lm_head dX", BT, C, Vp, "nn"),
        ("qkv dX", BT, C, 3 * C, "nn"), ("proj dX", BT, C, C, "nn"),
        ("fc dX", BT, C, 4 * C, "nn"), ("fcproj dX", BT, 4 * C, C, "nn"),
        ("lm_head dW", Vp, C, BT, "tn"), ("qkv dW", 3 * C, C, BT, "tn"),
        ("proj dW", C, C, BT, "tn"), ("fc dW", 4 * C, C, BT, "tn"),
        ("fcproj dW", C, 4 * C, BT, "tn")]
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(0)
    for name, M, N, K, lay in shapes:
        def rnd(*shape):
            return torch.randn(shape, device=dev, dtype=torch.bfloat16, generator=g)
        if lay == "nt":
            A, Bm = rnd(M, K), rnd(N, K).t()
        elif lay == "nn":
            A, Bm = rnd(M, K), rnd(K, N)
        else:
            A, Bm = rnd(K, M).t(), rnd(K, N)
        for _ in range(3):
            torch.mm(A, Bm)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.mm(A, Bm)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 100.0
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        print(f"library gemm {name}: {M}x{N}x{K} {lay} {us:.1f} us {tf:.1f} TFLOP/s "
              f"({tf / 2500.0:.3f} of 2.5 PF)", file=sys.stderr, flush=True)
        del A, Bm
    torch.cuda.empty_cache()


def library_attention(torch, B, T, d):
    """The platform's fused causal attention (torch SDPA restricted to its
    flash and memory-efficient backends; the math path is never used) in
    bf16 on (B, n_head, T, head width), forward and forward + backward timed
    with events over 10 calls after 3 warm-up calls; one line per backend on
    stderr, flops counted as causal (half the score matrix)."""
    import torch.nn.functional as F
    from torch.nn.attention import sdpa_kernel, SDPBackend
    H, D = d["n_head"], d["n_embd"] // d["n_head"]
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(0)
    fl = 4.0 * B * H * T * T * D / 2
    for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            q, k, v, do = (torch.randn((B, H, T, D), device=dev, dtype=torch.bfloat16,
                                       generator=g) for _ in range(4))
            q.requires_grad_(), k.requires_grad_(), v.requires_grad_()
            with sdpa_kernel([be]):
                for _ in range(3):
                    F.scaled_dot_product_attention(q, k, v, is_causal=True).backward(do)
                torch.cuda.synchronize()
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record()
                for _ in range(10):
                    F.scaled_dot_product_attention(q, k, v, is_causal=True)
                e[1].record()
                for _ in range(10):
                    F.scaled_dot_product_attention(q, k, v, is_causal=True).backward(do)
                e[2].record()
                torch.cuda.synchronize()
            fwd = e[0].elapsed_time(e[1]) * 100.0
            bwd = e[1].elapsed_time(e[2]) * 100.0 - fwd
            print(f"library attention {be.name}: {B}x{H}x{T}x{D} causal forward {fwd:.1f} us "
                  f"{fl / fwd / 1e6:.1f} TFLOP/s, backward {bwd:.1f} us "
                  f"{2.5 * fl / bwd / 1e6:.1f} TFLOP/s", file=sys.stderr, flush=True)
            del q, k, v, do
        except RuntimeError as ex:
            print(f"library attention {be.name}: unavailable ({str(ex)[:120]})", file=sys.stderr,
                  flush=True)
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2-124m", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every launch site")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run three 1 GiB device copies (calibrates HBM byte counters)")
    ap.add_argument("--library-ref", action="store_true",
                    help="first time the platform's bf16 GEMM (torch.mm) on the step's GEMM "
                         "shapes and its fused attention (torch SDPA, flash and memory-efficient "
                         "backends) on the step's attention shape, printed to stderr: reference "
                         "points, not part of the step")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synthetic
    from decoder_only_transformer_03_amd import gpt2 as G

    wl = WORKLOADS[args.workload]
    d = synthetic.model_dims(wl["model"])
    B, T = wl["B"], wl["T"]
    fused = wl.get("head_chunk", 0)
    cfg = G.make_config(max_batch=B, precision="bf16", head_chunk=fused, **d)
    model = G.GPT2(cfg, device="cuda:0")
    model.set_params(synthetic.init_params(d, seed=42))
    if args.library_ref:
        library_gemm(torch, B * T, d)
        library_attention(torch, B, T, d)
    if args.copy_probe:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    accum = wl.get("accum", 1)
    if wl["data"] == "sft":
        batches = [synthetic.sft_batch(B, T, seed=1004)]
    elif accum > 1:
        batches = [synthetic.zipf_batch(B, T, seed=10030 + i) for i in range(accum)]
    else:
        batches = [synthetic.zipf_batch(B, T, seed=1002)]
    dev = [(torch.tensor(i, dtype=torch.int32, device="cuda:0"),
            torch.tensor(t, dtype=torch.int32, device="cuda:0")) for i, t in batches]
    opt_step = [0]

    seq_loss = torch.zeros((B,), dtype=torch.float32, device="cuda:0")
    n_gen = wl.get("gen", 0)
    if n_gen:
        gen_u = torch.tensor(synthetic.uniforms((B, n_gen), seed=99), device="cuda:0")
        gen_out = torch.zeros((B, T + n_gen), dtype=torch.int32, device="cuda:0")

    def step():
        if n_gen:
            gen = model.generate_cached if wl.get("cached") else model.generate
            gen(dev[0][0], n_gen, gen_u, gen_out, 1.0, wl["top_k"])
            return
        if wl.get("eval"):
            model.eval(dev[0][0], dev[0][1], seq_loss=seq_loss)
            return
        model.zero_grad()
        for di, dt in dev:
            model.forward(di, dt)
            model.backward(1.0 / len(dev))
        lr = wl["lr"] if wl["lr"] is not None else G.gpt2_lr_at(opt_step[0])
        model.adamw_step(lr, 0.9, 0.95, 1e-8, wl["wd"], 1.0)
        opt_step[0] += 1

    for _ in range(args.warmup):
        step()
    model.sync()
    stream = torch.cuda.current_stream()
    model.timing_begin(["LMHEAD_FWD", "WGRAD"])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    sites = model.timing_end()
    loss = model.get_loss()
    norm = model.get_grad_norm()
    model.sync()
    ms_step = ms_total / args.steps
    tokens = B * n_gen if n_gen else B * T * accum
    tok_s = tokens * args.steps / (ms_total / 1e3)
    f_causal, f_nano = flops_per_token(d, T)
    if wl.get("eval"):  # forward only: a third of the training step's work
        f_causal, f_nano = f_causal / 3.0, f_nano / 3.0
    if n_gen:  # model flops are not the measure of a recomputing sampling loop
        f_causal = f_nano = 0.0

    # the roofline kernel: whichever of the lm_head forward GEMM and the
    # grouped weight-gradient GEMM took longer over the timed steps
    grouped_elems, _, _ = model.wgrad_layout()
    cands = {"LMHEAD_FWD": 2.0 * B * T * d["padded_vocab_size"] * d["n_embd"],
             "WGRAD": 2.0 * B * T * grouped_elems}
    timed = [k for k in cands if sites.get(k, (0.0, 0))[1] and cands[k] > 0]
    site = max(timed, key=lambda k: sites[k][0]) if timed else "LMHEAD_FWD"
    k_ms, k_n = sites.get(site, (0.0, 0))
    k_avg = k_ms / max(k_n, 1)
    k_flops = cands[site]
    achieved = k_flops / (k_avg / 1e3) / 1e12 if k_avg > 0 else 0.0

    breakdown = None
    if args.breakdown:
        model.timing_begin(None)
        for _ in range(2):
            step()
        br = model.timing_end()
        breakdown = {k: round(v[0] / 2, 4) for k, v in sorted(br.items(), key=lambda x: -x[1][0])}

    names = {"WGRAD": "weight gradients of every block" + ("" if fused else " and the lm_head") +
                      ", one grouped GEMM launch (gemm_kernel<256,256,TT,fp32 out,grouped>: written "
                      "after zero_grad, accumulated by later micro-batches)",
             "LMHEAD_FWD": "lm_head forward GEMM with the log-sum-exp epilogue "
                           "(gemm_kernel<256,256,NT,lse>)" if fused else
                           "lm_head forward GEMM (gemm_kernel<256,256,NT,store bf16>)"}
    roofline = {"kernel": names[site], "site": site,
                "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": TRAFFIC_BYTES.get((args.workload, site)),
                "avg_launch_ms": round(k_avg, 4), "launches": k_n,
                "flops_per_launch": k_flops}
    out = {
        "metric": METRIC if args.workload == "gpt2-124m" else
                  f"tokens/sec + MFU, {args.workload} on one MI355X",
        "value": round(tok_s, 1),
        "unit": "new tokens/s" if n_gen else "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "global_batch": B * accum, "seq_len": T,
                   "micro_batches": accum,
                   "precision": "bf16 matmuls, fp32 master weights and optimizer state"},
        "mfu": round(tok_s * f_causal / (PEAK_BF16_TFLOPS * 1e12), 4),
        "mfu_nanogpt_count": round(tok_s * f_nano / (PEAK_BF16_TFLOPS * 1e12), 4),
        "gflop_per_token": round(f_causal / 1e9, 4),
        "loss_last_step": round(loss, 5),
        "grad_norm_last_step": round(norm, 5),
        "host_wall_s": round(wall, 3),
        "roofline": None if n_gen else roofline,
    }
    if breakdown:
        out["site_ms_per_step"] = breakdown
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
