"""Generation path against the oracle: the last-position lm_head, the
temperature / top-k / multinomial draw, and the sampling loop with its
context crop ("GPT-2 from Scratch", The full model; A generation loop).

The draw is an integer decided by floating point: the kernel sums fp32
exponentials in its own order, the oracle fp64 ones.  A GPU token is accepted
when it is the oracle's token, or when u lies within 1e-5 of the boundary
between the oracle's token and the GPU's (there both are correct draws).
Top-k is checked exactly: the GPU token is always among the oracle's kept
entries (ties at the k-th value included).  fp32 logits within 1e-4 of the
oracle's; bf16 (GPT-2 124M) logits within 2e-2 of the largest.  The loop is
checked step by step: every drawn token is a valid draw for the oracle's
logits of the GPU's own cropped context at that step."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gpt2_oracle as O
import synthetic
from decoder_only_transformer_03_amd import gpt2 as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BAND = 1e-5


def dev(a, dtype):
    return torch.tensor(np.ascontiguousarray(a), dtype=dtype, device=DEV)


def oracle_draw_info(logits, temperature, top_k, u):
    """Per row: the oracle token, the kept mask and the cumulative
    probabilities (fp64)."""
    x = np.asarray(logits, np.float64) / temperature
    V = x.shape[1]
    keep = np.ones_like(x, bool)
    if top_k and top_k > 0:
        k = min(top_k, V)
        kth = np.sort(x, axis=1)[:, V - k][:, None]
        keep = x >= kth
    tok = O.sample_next(logits, temperature, top_k, u)
    p = np.where(keep, np.exp(x - x.max(axis=1, keepdims=True)), 0.0)
    cdf = np.cumsum(p / p.sum(axis=1, keepdims=True), axis=1)
    return tok, keep, cdf


def check_draws(got, logits, temperature, top_k, u, band=BAND):
    tok, keep, cdf = oracle_draw_info(logits, temperature, top_k, u)
    exact = 0
    for b in range(len(got)):
        g = int(got[b])
        assert 0 <= g < logits.shape[1] and keep[b, g], (b, g)
        if g == tok[b]:
            exact += 1
            continue
        # a different token is a correct draw only if u sits on the boundary
        lo = cdf[b, g - 1] if g > 0 else 0.0
        hi = cdf[b, g]
        assert lo - band <= u[b] <= hi + band, (b, g, tok[b], u[b], lo, hi)
    return exact


@pytest.fixture(scope="module")
def tiny():
    d = synthetic.model_dims("tiny")
    m = G.GPT2(G.make_config(max_batch=4, precision="fp32", **d), device=DEV)
    flat = synthetic.init_params(d, seed=21)
    m.set_params(flat)
    return d, flat, m


@pytest.mark.parametrize("V,ld,temperature,top_k,grid", [
    (512, 512, 1.0, 0, None), (512, 512, 0.7, 50, None), (512, 512, 1.3, 1, None),
    (512, 512, 1.0, 7, 0.5),                          # ties at the k-th value
    (50304, 50304, 1.0, 50, None), (50304, 50304, 0.8, 0, None),
    (50257, 50304, 1.0, 200, 0.25), (50304, 50304, 1.0, 50304, None),
    (3, 4, 1.0, 2, None), (53248, 53248, 1.0, 5, None),
    (50304, 50304, 1.0, 2000, None)])                 # k above the 1024 threads' maxima
def test_sample_matches_oracle(tiny, V, ld, temperature, top_k, grid):
    _, _, m = tiny
    B = 64
    full = synthetic.logit_rows(B, ld, seed=V + top_k, grid=grid)
    u = synthetic.uniforms(B, seed=V + 7)
    u[:4] = [0.0, 0.5, 0.999999, 1e-7]
    tokens = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    m.sample(dev(full, torch.float32), dev(u, torch.float32), tokens, temperature, top_k, V=V)
    got = tokens.cpu().numpy()
    exact = check_draws(got, full[:, :V], temperature, top_k, u.astype(np.float64))
    print(f"\nV={V} ld={ld} T={temperature} k={top_k}: {exact}/{B} identical to the oracle")
    assert exact >= B - 2
    if top_k == 1 and grid is None:
        assert np.array_equal(got, (full[:, :V] / temperature).argmax(axis=1))
    # the same inputs give the same tokens
    again = torch.zeros_like(tokens)
    m.sample(dev(full, torch.float32), dev(u, torch.float32), again, temperature, top_k, V=V)
    assert np.array_equal(again.cpu().numpy(), got)


def test_sample_rejects_bad_arguments(tiny):
    _, _, m = tiny
    lg = torch.zeros((2, 512), dtype=torch.float32, device=DEV)
    u = torch.zeros((2,), dtype=torch.float32, device=DEV)
    t = torch.zeros((2,), dtype=torch.int32, device=DEV)
    for kw in (dict(temperature=0.0), dict(temperature=-1.0), dict(V=600)):
        with pytest.raises(G.GPT2Error) as e:
            m.sample(lg, u, t, **{"temperature": 1.0, **kw})
        assert e.value.status == G.GPT2_E_ARG
    big = torch.zeros((1, 53252), dtype=torch.float32, device=DEV)
    with pytest.raises(G.GPT2Error):
        m.sample(big, u[:1], t[:1])


def test_forward_last_fp32(tiny):
    d, flat, m = tiny
    cfg = O.Config(**d)
    for B, T in ((3, 37), (1, 1), (4, 64)):
        idx, _ = synthetic.uniform_batch(B, T, 512, seed=300 + T)
        out = torch.zeros((B, d["padded_vocab_size"]), dtype=torch.float32, device=DEV)
        m.forward_last(dev(idx, torch.int32), out)
        got = out.cpu().numpy().astype(np.float64)
        ref = O.last_logits(flat, idx, cfg).astype(np.float64)
        err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        print(f"\nforward_last fp32 B={B} T={T}: maxrel {err:.2e}")
        assert err < 1e-4
    with pytest.raises(G.GPT2Error) as e:
        m.backward(1.0)
    assert e.value.status == G.GPT2_E_STATE


@pytest.mark.parametrize("T0,n_new,temperature,top_k", [(60, 10, 0.8, 40), (3, 5, 1.0, 0),
                                                        (70, 4, 1.2, 1), (5, 0, 1.0, 10)])
def test_generate_fp32_step_by_step(tiny, T0, n_new, temperature, top_k):
    """The prompt is copied; every drawn token is a valid draw for the
    oracle's logits of the GPU's own context cropped to the last block_size
    tokens (T0 + n_new crosses block_size = 64 in the first case, the prompt
    is longer than it in the third)."""
    d, flat, m = tiny
    cfg = O.Config(**d)
    B = 3
    rng = np.random.default_rng(T0 * 31 + n_new)
    prompt = rng.integers(0, 512, size=(B, T0)).astype(np.int32)
    uni = synthetic.uniforms((B, max(n_new, 1)), seed=T0 + n_new)[:, :n_new]
    out = torch.full((B, T0 + n_new), -7, dtype=torch.int32, device=DEV)
    m.generate(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), out, temperature, top_k)
    got = out.cpu().numpy()
    assert np.array_equal(got[:, :T0], prompt)
    exact = 0
    for s in range(n_new):
        ctx = got[:, :T0 + s][:, -cfg.block_size:]
        lg = O.last_logits(flat, ctx, cfg)
        exact += check_draws(got[:, T0 + s], lg, temperature, top_k, uni[:, s].astype(np.float64))
    assert exact >= B * n_new - 1
    if exact == B * n_new:
        ref = O.generate(flat, prompt, n_new, temperature, top_k, uni.astype(np.float64), cfg)
        assert np.array_equal(got, ref)
    # deterministic
    out2 = torch.zeros_like(out)
    m.generate(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), out2, temperature, top_k)
    assert torch.equal(out, out2)


def test_generate_bf16_124m():
    """GPT-2 124M bf16: last-position logits of a long context against the
    oracle; a greedy loop whose every token is a maximum of the oracle's
    logits up to the bf16 tolerance; a top-50 loop whose every token is among
    the oracle's top 50 up to that tolerance."""
    d = synthetic.model_dims("gpt2-124m")
    cfg = O.Config(**d)
    flat = synthetic.init_params(d, seed=42)
    B = 2
    m = G.GPT2(G.make_config(max_batch=B, precision="bf16", **d), device=DEV)
    try:
        m.set_params(flat)
        idx, _ = synthetic.zipf_batch(B, 300, seed=77)
        out = torch.zeros((B, d["padded_vocab_size"]), dtype=torch.float32, device=DEV)
        m.forward_last(dev(idx, torch.int32), out)
        got = out.cpu().numpy().astype(np.float64)
        ref = O.last_logits(flat, idx, cfg).astype(np.float64)
        tol = 2e-2 * np.max(np.abs(ref))
        assert np.max(np.abs(got - ref)) < tol
        prompt = idx[:, :24].astype(np.int32)
        n_new = 4
        uni = synthetic.uniforms((B, n_new), seed=5)
        res = {}
        for k in (1, 50):
            o = torch.zeros((B, 24 + n_new), dtype=torch.int32, device=DEV)
            m.generate(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), o, 1.0, k)
            res[k] = o.cpu().numpy()
    finally:
        m.close()
    for k, seq in res.items():
        assert np.array_equal(seq[:, :24], prompt)
        for s in range(n_new):
            lg = O.last_logits(flat, seq[:, :24 + s], cfg).astype(np.float64)
            t = seq[:, 24 + s]
            kth = np.sort(lg, axis=1)[:, -k]
            for b in range(B):
                assert lg[b, t[b]] >= kth[b] - tol, (k, s, b)
    print(f"\nbf16 124M: forward_last maxabs {np.max(np.abs(got - ref)):.3e} (tol {tol:.3e})")


def test_generate_same_with_fused_head_config(tiny):
    """A model configured with the fused lm_head runs the same last-position
    head when generating: identical tokens for identical inputs."""
    d, flat, m = tiny
    m2 = G.GPT2(G.make_config(max_batch=4, precision="fp32", head_chunk=128, **d), device=DEV)
    m2.set_params(flat)
    B, T0, n_new = 3, 40, 6
    prompt = np.random.default_rng(8).integers(0, 512, size=(B, T0)).astype(np.int32)
    uni = synthetic.uniforms((B, n_new), seed=9)
    outs = []
    for mm in (m, m2):
        o = torch.zeros((B, T0 + n_new), dtype=torch.int32, device=DEV)
        mm.generate(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), o, 0.9, 30)
        outs.append(o.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("T0,n_new,temperature,top_k", [(60, 10, 0.8, 40), (3, 5, 1.0, 0),
                                                        (70, 4, 1.2, 1), (2, 70, 1.0, 20),
                                                        (5, 0, 1.0, 10)])
def test_generate_cached_fp32(tiny, T0, n_new, temperature, top_k):
    """gpt2_generate_cached: the prompt is copied; every drawn token is a
    valid draw for the oracle's logits of its own context cropped to the last
    block_size tokens -- decoded against the key/value cache while the
    sequence is shorter than block_size (64), recomputed once the window
    shifts (the first and fourth cases cross it, the third starts past it);
    with no draw on a CDF boundary the tokens are those of gpt2_generate and
    of the oracle's loop."""
    d, flat, m = tiny
    cfg = O.Config(**d)
    B = 3
    rng = np.random.default_rng(T0 * 17 + n_new)
    prompt = rng.integers(0, 512, size=(B, T0)).astype(np.int32)
    uni = synthetic.uniforms((B, max(n_new, 1)), seed=T0 + 3 * n_new)[:, :n_new]
    out = torch.full((B, T0 + n_new), -7, dtype=torch.int32, device=DEV)
    m.generate_cached(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), out, temperature,
                      top_k)
    got = out.cpu().numpy()
    assert np.array_equal(got[:, :T0], prompt)
    exact = 0
    for s in range(n_new):
        ctx = got[:, :T0 + s][:, -cfg.block_size:]
        lg = O.last_logits(flat, ctx, cfg)
        exact += check_draws(got[:, T0 + s], lg, temperature, top_k, uni[:, s].astype(np.float64))
    assert exact >= B * n_new - 1
    if exact == B * n_new:
        ref = O.generate(flat, prompt, n_new, temperature, top_k, uni.astype(np.float64), cfg)
        assert np.array_equal(got, ref)
        full = torch.zeros_like(out)
        m.generate(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), full, temperature,
                   top_k)
        assert np.array_equal(full.cpu().numpy(), got)
    out2 = torch.zeros_like(out)
    m.generate_cached(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), out2, temperature,
                      top_k)
    assert torch.equal(out, out2)


def test_generate_cached_bf16_124m():
    """GPT-2 124M bf16, greedy: every token decoded against the cache is a
    maximum of the oracle's logits of its context up to the bf16 tolerance,
    and the tokens equal the recomputing loop's up to the first step where
    the oracle's two best logits are within that tolerance of each other."""
    d = synthetic.model_dims("gpt2-124m")
    cfg = O.Config(**d)
    flat = synthetic.init_params(d, seed=42)
    B, T0, n_new = 2, 24, 12
    m = G.GPT2(G.make_config(max_batch=B, precision="bf16", **d), device=DEV)
    try:
        m.set_params(flat)
        idx, _ = synthetic.zipf_batch(B, T0, seed=78)
        prompt = idx.astype(np.int32)
        uni = synthetic.uniforms((B, n_new), seed=6)
        outs = []
        for fn in (m.generate_cached, m.generate):
            o = torch.zeros((B, T0 + n_new), dtype=torch.int32, device=DEV)
            fn(dev(prompt, torch.int32), n_new, dev(uni, torch.float32), o, 1.0, 1)
            outs.append(o.cpu().numpy())
    finally:
        m.close()
    cached, full = outs
    assert np.array_equal(cached[:, :T0], prompt)
    tol = None
    for s in range(n_new):
        lg = O.last_logits(flat, cached[:, :T0 + s], cfg).astype(np.float64)
        tol = 2e-2 * np.max(np.abs(lg)) if tol is None else tol
        top2 = np.sort(lg, axis=1)[:, -2:]
        for b in range(B):
            t = cached[b, T0 + s]
            assert lg[b, t] >= top2[b, 1] - tol, (s, b)
        if not np.array_equal(cached[:, :T0 + s + 1], full[:, :T0 + s + 1]):
            # the loops may part only where the choice is within rounding
            assert np.any(top2[:, 1] - top2[:, 0] < 2 * tol), s
            break
    print(f"\nbf16 124M cached greedy: {np.sum(cached == full)} of {cached.size} tokens equal")


def maxrel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def test_prefill_decode_fp32(tiny):
    """gpt2_prefill + gpt2_decode, one position per call up to block_size: the
    logits of every position within 1e-5 of the oracle's last-position logits
    of the same context (measured: 5e-7; the tokens fed are fixed, not
    drawn); the calls that do not continue the kept sequences, or run past
    block_size, are refused."""
    d, flat0, m = tiny
    flat = synthetic.perturb_vectors(d, flat0, seed=5)
    m.set_params(flat)
    cfg = O.Config(**d)
    B, T0, Vp = 3, 5, d["padded_vocab_size"]
    seq = np.random.default_rng(31).integers(0, d["vocab_size"], size=(B, cfg.block_size))
    seq = seq.astype(np.int32)
    lg = torch.zeros((B, Vp), dtype=torch.float32, device=DEV)
    m.prefill(dev(seq[:, :T0], torch.int32), lg)
    worst = maxrel(lg.cpu().numpy().astype(np.float64), O.last_logits(flat, seq[:, :T0], cfg))
    for p in range(T0, cfg.block_size):
        m.decode(dev(seq[:, p], torch.int32), p, lg)
        ref = O.last_logits(flat, seq[:, :p + 1], cfg)
        worst = max(worst, maxrel(lg.cpu().numpy().astype(np.float64), ref))
    print(f"\nfp32 prefill + {cfg.block_size - T0} decode steps: worst maxrel {worst:.2e}")
    assert worst < 1e-5
    tok = dev(seq[:, 0], torch.int32)
    with pytest.raises(G.GPT2Error) as e:  # the cache is full
        m.decode(tok, cfg.block_size, lg)
    assert e.value.status == G.GPT2_E_SHAPE
    m.prefill(dev(seq[:, :T0], torch.int32), lg)
    for bad_p in (T0 - 1, T0 + 1):
        with pytest.raises(G.GPT2Error) as e:
            m.decode(tok, bad_p, lg)
        assert e.value.status == G.GPT2_E_STATE
    with pytest.raises(G.GPT2Error) as e:  # another batch
        m.decode(tok[:2], T0, lg)
    assert e.value.status == G.GPT2_E_STATE
    m.set_params(flat0)  # the kept keys and values are stale now (and the fixture's again)
    with pytest.raises(G.GPT2Error) as e:
        m.decode(tok, T0, lg)
    assert e.value.status == G.GPT2_E_STATE


@pytest.mark.parametrize("model,B,n_dec", [("gpt2-124m", 2, 8), ("gpt2-124m", 16, 2),
                                           ("gpt2-124m", 17, 2), ("xl-width", 3, 4)])
def test_prefill_decode_bf16(model, B, n_dec):
    """bf16, the decoding kernels themselves, with LayerNorm gains and all
    biases away from the init's ones and zeros: at B <= 16 each LayerNorm runs
    inside the few-rows GEMM that reads it (ln_1 -> qkv, ln_2 -> fc, ln_f ->
    lm_head), the projections add the residual in the few-rows kernel and
    the decode attention appends to the cache; B = 17 takes the separate
    LayerNorm and the K-split GEMMs.  The XL width (2 blocks of C = 1600, 25
    heads) normalises 1600-wide rows in the fused prologue and runs the
    fcproj's K = 6400 in two batches of loads per wavefront.  Every
    position's logits against the oracle's last-position logits of the same
    context, within 1.2e-2 of the largest.  Measured: 124M 2.8e-3 for the
    prompt's full forward (the first position checked) and 3.0e-3 to 3.8e-3
    for the decoded positions (5.7e-3 to 7.8e-3 with the init's vectors);
    XL width 4.9e-3 to 5.8e-3.  The bound is about twice the largest."""
    if model == "xl-width":
        d = dict(synthetic.model_dims("gpt2-xl"), n_layer=2)
    else:
        d = synthetic.model_dims(model)
    cfg = O.Config(**d)
    flat = synthetic.perturb_vectors(d, synthetic.init_params(d, seed=42), seed=7)
    T0, Vp = 24, d["padded_vocab_size"]
    seq, _ = synthetic.zipf_batch(B, T0 + n_dec, seed=90 + B)
    seq = seq.astype(np.int32)
    m = G.GPT2(G.make_config(max_batch=B, precision="bf16", **d), device=DEV)
    try:
        m.set_params(flat)
        lg = torch.zeros((B, Vp), dtype=torch.float32, device=DEV)
        got = []
        m.prefill(dev(seq[:, :T0], torch.int32), lg)
        got.append(lg.cpu().numpy().astype(np.float64))
        for p in range(T0, T0 + n_dec - 1):
            m.decode(dev(seq[:, p], torch.int32), p, lg)
            got.append(lg.cpu().numpy().astype(np.float64))
    finally:
        m.close()
    for i, g in enumerate(got):
        ref = O.last_logits(flat, seq[:, :T0 + i], cfg).astype(np.float64)
        err = maxrel(g, ref)
        print(f"\nbf16 {model} B={B} position {T0 + i - 1}: maxrel {err:.2e}")
        assert err < 1.2e-2
