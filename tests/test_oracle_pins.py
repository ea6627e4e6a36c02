"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the fact it checks.  None of them re-types the oracle's own
formula: they use printed values (tests/golden/pages_values.json), closed
forms, invariants, finite differences and independent library routines
(torch CPU autograd and torch.optim.AdamW, the calls the pages make).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import gpt2_oracle as O
import synthetic

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def cfg_of(name, **over):
    d = synthetic.model_dims(name)
    d.update(over)
    return O.Config(**d), d


# --------------------------------------------------------------------------
# parameter layout
# --------------------------------------------------------------------------

def test_param_count_matches_printed_124m():
    cfg, _ = cfg_of("gpt2-124m", padded_vocab_size=50257)
    n = O.num_params(cfg)
    assert n == GOLD["param_count_124m_v50257"]["value"]
    # the untied model would have one more V x C matrix
    assert GOLD["tie_saving_124m"]["value"] == 50257 * 768
    # 12 blocks of mask buffers (T_max x T_max) are the miscount the page warns about
    assert GOLD["mask_buffer_miscount_124m"]["value"] == 12 * 1024 * 1024
    # block weights ~ 12 C^2 plus about ten thousand biases/LN
    blk = sum(int(np.prod(s)) for nm, s in O.param_specs(cfg) if nm.startswith("h.0."))
    assert 0 < blk - GOLD["per_block_weights_12C2_124m"]["value"] < 11000


def test_param_count_padded_and_other_sizes():
    assert O.num_params(cfg_of("gpt2-124m")[0]) == 124_475_904
    assert O.num_params(cfg_of("tiny")[0]) == 470_528
    xl = cfg_of("gpt2-xl", padded_vocab_size=50257)[0]
    assert round(O.num_params(xl) / 1e6) == 1558          # "gpt2-xl ... 1558M"
    assert len(O.param_specs(cfg_of("gpt2-124m")[0])) == 148
    assert GOLD["padded_vocab"]["value"] % GOLD["padded_vocab"]["multiple_of"] == 0


def test_generator_layout_agrees_with_oracle():
    for name in ("tiny", "gpt2-124m"):
        cfg, d = cfg_of(name)
        flat = synthetic.init_params(d, seed=1)
        assert flat.size == O.num_params(cfg)
        P = O.unflatten(flat, cfg)
        for nm, t in P.items():
            if nm.endswith("ln_1.weight") or nm.endswith("ln_2.weight") or nm == "ln_f.weight":
                assert np.all(t == 1.0), nm
            elif nm.endswith(".bias"):
                assert np.all(t == 0.0), nm


def test_init_statistics_match_printed():
    cfg, d = cfg_of("gpt2-124m")
    P = O.unflatten(synthetic.init_params(d, seed=0), cfg)
    assert abs(P["wte"].std() - 0.02) < 2e-4
    assert abs(P["h.3.attn.c_attn.weight"].std() - 0.02) < 2e-4
    g = GOLD["residual_init_std_L12"]
    assert abs(P["h.0.attn.c_proj.weight"].std() - g["value"]) < g["tol"]
    assert abs(P["h.5.mlp.c_proj.weight"].std() - g["value"]) < g["tol"]
    assert abs(P["h.5.mlp.c_fc.weight"].std() - 0.02) < 2e-4
    assert abs(1 / math.sqrt(768) - GOLD["xavier_scale_C768"]["value"]) < GOLD["xavier_scale_C768"]["tol"]


def test_residual_toy_growth():
    # 100 unit-variance additions grow the running std to about 10
    rng = np.random.default_rng(0)
    x = np.zeros(200000)
    for _ in range(100):
        x += rng.standard_normal(x.size)
    g = GOLD["residual_toy_std_100_additions"]
    assert abs(x.std() - g["value"]) / g["value"] < g["rel_tol"]


# --------------------------------------------------------------------------
# forward: shapes, initial loss, mask, causal invariance
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def p124_v50257():
    cfg, d = cfg_of("gpt2-124m", padded_vocab_size=50257)
    return cfg, synthetic.init_params(d, seed=42)


def test_debug_shapes(p124_v50257):
    cfg, flat = p124_v50257
    g = GOLD["debug_shapes_124m"]
    idx, _ = synthetic.zipf_batch(g["B"], g["T"], seed=3)
    _, cache = O.forward(flat, idx, None, cfg)
    assert list(cache["layers"][0]["x_mid"].shape) == g["residual"]
    assert list(cache["x_final"].shape) == g["residual"]
    lc = cache["layers"][0]
    assert list(O.attention_probs(lc["q"], lc["k"]).shape) == g["scores"]
    assert list(cache["logits"].shape) == g["logits"]


def test_initial_loss_near_ln_v(p124_v50257):
    cfg, flat = p124_v50257
    idx, tgt = synthetic.zipf_batch(2, 64, seed=5)
    loss, cache = O.forward(flat, idx, tgt, cfg)
    g = GOLD["initial_loss_v50257"]
    assert abs(math.log(50257) - g["value"]) < 0.005
    assert abs(math.log(50304) - GOLD["initial_loss_v50304"]["value"]) < GOLD["initial_loss_v50304"]["tol"]
    # printed band: ln V give or take 0.1, "10.9 with a bit of init noise", "~11" observed;
    # the upward bias is about var(logits)/2 (logit std ~ 0.02 sqrt(C) at init)
    z = cache["z"].reshape(-1, 768).astype(np.float64)
    W = O.unflatten(flat, cfg)["wte"].astype(np.float64)
    logits = z @ W.T
    var_logit = float((logits ** 2).mean())
    m = logits.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
    assert math.log(50257) - 0.05 < loss < math.log(50257) + 0.3
    # for near-Gaussian logits the log-partition is ln V + var/2 to second order
    assert abs(lse.mean() - (math.log(50257) + var_logit / 2)) < 0.01


def test_zero_embedding_gives_exact_uniform_loss():
    cfg, d = cfg_of("tiny")
    flat = synthetic.init_params(d, seed=1)
    O.unflatten(flat, cfg)["wte"][:] = 0.0
    idx, tgt = synthetic.uniform_batch(2, 16, 512, seed=2)
    loss, cache = O.forward(flat, idx, tgt, cfg)
    assert abs(float(loss) - math.log(512)) < 1e-5
    rows = cache["dlogits"].reshape(-1, 512)
    assert np.allclose(rows.sum(axis=1), 0.0, atol=1e-9)


def test_mask_direction_and_row_sums():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 3, 7, 16))
    k = rng.standard_normal((2, 3, 7, 16))
    P = O.attention_probs(q, k)
    assert np.all(P[..., np.triu_indices(7, 1)[0], np.triu_indices(7, 1)[1]] == 0.0)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-12)
    # first query can only see itself
    assert np.all(P[..., 0, 0] == 1.0)


def test_attention_single_position_returns_v():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((2, 4, 1, 32)) for _ in range(3))
    Oo, lse = O.causal_attention_fwd(q, k, v)
    assert np.array_equal(Oo, v)


def test_attention_matches_brute_force_loops():
    rng = np.random.default_rng(2)
    B, H, T, hd = 1, 2, 5, 4
    q, k, v = (rng.standard_normal((B, H, T, hd)) for _ in range(3))
    Oo, _ = O.causal_attention_fwd(q, k, v)
    ref = np.zeros_like(q)
    for h in range(H):
        for i in range(T):
            w = [math.exp(sum(q[0, h, i, d] * k[0, h, j, d] for d in range(hd)) / math.sqrt(hd))
                 for j in range(i + 1)]
            zsum = sum(w)
            for d in range(hd):
                ref[0, h, i, d] = sum(w[j] * v[0, h, j, d] for j in range(i + 1)) / zsum
    assert np.allclose(Oo, ref, rtol=0, atol=1e-12)


def test_causal_invariance_bit_exact():
    cfg, d = cfg_of("tiny")
    flat = synthetic.init_params(d, seed=7)
    idx, _ = synthetic.uniform_batch(2, 32, 512, seed=8)
    _, c1 = O.forward(flat, idx, None, cfg)
    t = 12
    idx2 = idx.copy()
    idx2[:, t + 1:] = (idx2[:, t + 1:] + 17) % 512
    _, c2 = O.forward(flat, idx2, None, cfg)
    assert np.array_equal(c1["logits"][:, :t + 1], c2["logits"][:, :t + 1])
    assert not np.array_equal(c1["logits"][:, t + 1:], c2["logits"][:, t + 1:])


# --------------------------------------------------------------------------
# GELU
# --------------------------------------------------------------------------

def test_gelu_tanh_close_to_erf_and_odd_identity():
    x = np.linspace(-10, 10, 200001)
    erf = 0.5 * x * (1 + np.array([math.erf(t / math.sqrt(2)) for t in x]))
    assert np.max(np.abs(O.gelu_tanh(x) - erf)) < GOLD["gelu_tanh_vs_erf_max_abs"]["value"]
    assert np.allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, atol=1e-12)
    assert O.gelu_tanh(np.array(0.0)) == 0.0
    # derivative by central differences
    xs = np.linspace(-6, 6, 1001)
    h = 1e-6
    fd = (O.gelu_tanh(xs + h) - O.gelu_tanh(xs - h)) / (2 * h)
    assert np.allclose(O.gelu_tanh_grad(xs), fd, atol=1e-8)


# --------------------------------------------------------------------------
# cross-entropy
# --------------------------------------------------------------------------

def test_cross_entropy_ignore_and_rows():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((6, 11))
    tgt = np.array([1, -1, 10, 0, -1, 5])
    loss, dl, row, n = O.cross_entropy(logits.copy(), tgt)
    assert n == 4
    assert np.all(dl[[1, 4]] == 0.0)
    assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-15)
    ref = np.mean([math.log(sum(math.exp(v) for v in logits[i])) - logits[i, tgt[i]]
                   for i in (0, 2, 3, 5)])
    assert abs(loss - ref) < 1e-12
    loss0, dl0, _, n0 = O.cross_entropy(logits.copy(), np.full(6, -1))
    assert n0 == 0 and loss0 == 0.0 and np.all(dl0 == 0.0)


# --------------------------------------------------------------------------
# gradients: central differences (fp64) and the tied embedding
# --------------------------------------------------------------------------

def _loss64(flat, idx, tgt, cfg):
    loss, _ = O.forward(flat, idx, tgt, cfg)
    return float(loss)


def test_gradcheck_every_tensor_fp64():
    cfg, d = cfg_of("tiny", vocab_size=500)
    flat = synthetic.init_params(d, seed=11, dtype=np.float64)
    # non-trivial LN / bias values so that no gradient is structurally tiny
    rng = np.random.default_rng(12)
    flat += rng.standard_normal(flat.size) * 0.01
    idx, tgt = synthetic.uniform_batch(2, 16, 500, seed=13)
    tgt[0, 3] = -1
    loss, cache = O.forward(flat, idx, tgt, cfg)
    g = O.backward(flat, cache, cfg)
    h = 1e-5
    off = 0
    for name, shape in O.param_specs(cfg):
        n = int(np.prod(shape))
        for j in rng.choice(n, size=3, replace=False):
            i = off + int(j)
            if name == "wpe" and i - off >= 16 * d["n_embd"]:
                continue
            old = flat[i]
            flat[i] = old + h
            lp = _loss64(flat, idx, tgt, cfg)
            flat[i] = old - h
            lm = _loss64(flat, idx, tgt, cfg)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            # central differences carry ~eps*loss/h = 1e-10 of rounding noise
            assert abs(g[i] - fd) <= 1e-5 * abs(fd) + 2e-9, (name, int(j), g[i], fd)
        off += n


def test_tied_embedding_gradient_has_both_parts():
    cfg, d = cfg_of("tiny", vocab_size=500)
    flat = synthetic.init_params(d, seed=21, dtype=np.float64)
    idx, tgt = synthetic.uniform_batch(1, 8, 500, seed=22)
    present = int(idx[0, 0])
    absent = next(t for t in range(500) if t not in set(idx.reshape(-1).tolist()))
    padded = 505                                    # id >= V: only the lm_head touches it
    loss, cache = O.forward(flat, idx, tgt, cfg)
    g = O.unflatten(O.backward(flat, cache, cfg), cfg)["wte"]
    # the lm_head part alone: dlogits^T z
    head = cache["dlogits"].T @ cache["z"].reshape(-1, d["n_embd"])
    assert np.allclose(g[absent], head[absent], atol=1e-15)
    assert np.allclose(g[padded], head[padded], atol=1e-15)
    assert np.max(np.abs(g[present] - head[present])) > 1e-3 * np.max(np.abs(head[present]))
    # finite differences on one element of each row
    W = O.unflatten(flat, cfg)["wte"]
    for row in (present, absent, padded):
        c = 7
        old = W[row, c]
        W[row, c] = old + 1e-5
        lp = _loss64(flat, idx, tgt, cfg)
        W[row, c] = old - 1e-5
        lm = _loss64(flat, idx, tgt, cfg)
        W[row, c] = old
        fd = (lp - lm) / 2e-5
        assert abs(g[row, c] - fd) <= 1e-6 * max(abs(fd), 1e-9) + 1e-11, (row, g[row, c], fd)


def test_key_bias_gradient_is_zero():
    # softmax is shift invariant per row, so the key bias cannot change the loss
    cfg, d = cfg_of("tiny")
    flat = synthetic.init_params(d, seed=31, dtype=np.float64)
    flat += np.random.default_rng(32).standard_normal(flat.size) * 0.02
    idx, tgt = synthetic.uniform_batch(2, 16, 512, seed=33)
    loss, cache = O.forward(flat, idx, tgt, cfg)
    G = O.unflatten(O.backward(flat, cache, cfg), cfg)
    C = d["n_embd"]
    for l in range(d["n_layer"]):
        b = G[f"h.{l}.attn.c_attn.bias"]
        assert np.max(np.abs(b[C:2 * C])) <= 1e-10 * np.max(np.abs(b[:C]))


def test_accumulation_equals_big_batch_fp64():
    cfg, d = cfg_of("tiny")
    flat = synthetic.init_params(d, seed=41, dtype=np.float64)
    idx, tgt = synthetic.uniform_batch(4, 16, 512, seed=42)
    loss_big, cache = O.forward(flat, idx, tgt, cfg)
    g_big = O.backward(flat, cache, cfg)
    g_acc = np.zeros_like(flat)
    losses = []
    for b in range(4):
        l, c = O.forward(flat, idx[b:b + 1], tgt[b:b + 1], cfg)
        O.backward(flat, c, cfg, loss_scale=0.25, grads=g_acc)
        losses.append(float(l))
    assert abs(np.mean(losses) - float(loss_big)) < 1e-13
    assert np.max(np.abs(g_acc - g_big)) <= 1e-12 * np.max(np.abs(g_big))


# --------------------------------------------------------------------------
# optimizer
# --------------------------------------------------------------------------

def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(5)
    p = rng.standard_normal(1000)
    g = rng.standard_normal(1000)
    decay = (np.arange(1000) < 600).astype(np.float64)
    m, v = np.zeros(1000), np.zeros(1000)
    p1 = p.copy()
    lr, wd, eps = 6e-4, 0.1, 1e-8
    O.adamw_update(p1, g, m, v, 1, lr, 0.9, 0.95, eps, wd, decay)
    expect = p * (1 - lr * wd * decay) - lr * g / (np.abs(g) + eps)
    assert np.allclose(p1, expect, rtol=0, atol=1e-15)


def test_clip_scales_to_unit_norm_and_reports_preclip():
    rng = np.random.default_rng(6)
    cfg, d = cfg_of("tiny")
    n = O.num_params(cfg)
    p = rng.standard_normal(n)
    g = rng.standard_normal(n) * 0.05
    pre = float(np.linalg.norm(g))
    assert pre > 1
    norm = O.clip_and_adamw(p, g, np.zeros(n), np.zeros(n), 1, 6e-4, cfg=cfg)
    assert abs(norm - pre) < 1e-9 * pre
    assert abs(np.linalg.norm(g) - 1.0) < 1e-6
    g2 = rng.standard_normal(n) * 1e-4
    g2c = g2.copy()
    O.clip_and_adamw(rng.standard_normal(n), g2c, np.zeros(n), np.zeros(n), 1, 6e-4, cfg=cfg)
    assert np.array_equal(g2, g2c)               # norm below 1: untouched


def test_lr_schedule_printed_properties():
    s = GOLD["lr_schedule"]
    f = lambda t: O.lr_at(t, s["max_lr"], s["min_lr"], s["warmup"], s["max_steps"])
    assert abs(f(s["warmup"]) - s["max_lr"]) < 1e-15
    assert abs(f(s["max_steps"]) - s["min_lr"]) < 1e-15
    mid = (s["warmup"] + s["max_steps"]) // 2
    assert abs(f(mid) - 0.5 * (s["max_lr"] + s["min_lr"])) < 1e-12
    assert abs(f(0) - s["max_lr"] / s["warmup"]) < 1e-15
    assert abs(f(s["warmup"] - 1) - s["max_lr"]) < 1e-15
    assert f(s["max_steps"] + 5) == s["min_lr"]
    assert abs(s["min_lr"] - 0.1 * s["max_lr"]) < 1e-15
    # monotone decay after warmup
    vals = [f(t) for t in range(s["warmup"], s["max_steps"] + 1)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


# --------------------------------------------------------------------------
# end to end: overfitting one batch
# --------------------------------------------------------------------------

def test_overfit_single_batch():
    cfg, d = cfg_of("tiny")
    p = synthetic.init_params(d, seed=51)
    m, v = np.zeros_like(p), np.zeros_like(p)
    idx, tgt = synthetic.uniform_batch(2, 16, 512, seed=52)
    first = None
    for t in range(1, 121):
        loss, norm, _ = O.train_step(p, m, v, t, [(idx, tgt)], cfg, lr=3e-3)
        first = loss if first is None else first
    assert first > 6.0
    assert loss < 0.05, loss


def test_sequence_losses_pins():
    """Per-sequence mean over valid targets: a hand-worked case (mean of the
    two middle losses, an all-ignored sequence scoring 0, gaps skipped), and
    on a real forward pass the count-weighted mean of the sequences' scores
    is the batch loss."""
    rl = np.array([[1.0, 2.0, 3.0, 4.0], [0.0, 0.0, 0.0, 0.0], [5.0, 0.0, 7.0, 0.0]])
    tg = np.array([[-1, 5, 6, -1], [-1, -1, -1, -1], [1, -1, 2, -1]])
    assert O.sequence_losses(rl, tg).tolist() == [2.5, 0.0, 6.0]
    d = synthetic.model_dims("tiny")
    cfg = O.Config(**d)
    flat = synthetic.init_params(d, seed=42).astype(np.float64)
    idx, tgt = synthetic.uniform_batch(3, 16, 512, seed=7)
    tgt[0, :10] = -1
    tgt[2, :] = -1
    loss, cache = O.forward(flat, idx, tgt, cfg)
    seq = O.sequence_losses(cache["row_loss"], tgt)
    n = (tgt != -1).sum(axis=1)
    assert seq[2] == 0.0
    assert abs((seq * n).sum() / n.sum() - float(loss)) < 1e-12


# ----------------------------------------------------------------------------
# Sampling and the generation loop ("GPT-2 from Scratch", A generation loop)
# ----------------------------------------------------------------------------

def test_sample_inverse_cdf_on_uniform_logits():
    """Equal logits: every token has probability 1/V, so the draw is
    floor(u V) -- pins the index order and the strict 'exceeds u' boundary."""
    V = 10
    u = np.array([0.0, 0.05, 0.0999, 0.1, 0.55, 0.9999])
    got = O.sample_next(np.zeros((len(u), V)), 1.0, None, u)
    assert list(got) == [0, 0, 0, 1, 5, 9]


def test_sample_top1_is_argmax():
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(16, 300))
    for u in (0.0, 0.3, 0.999999):
        got = O.sample_next(logits, 0.7, 1, np.full(16, u))
        assert np.array_equal(got, logits.argmax(axis=1))


def test_sample_frequencies_match_truncated_softmax():
    """Over a fine grid of u, token i is drawn for a fraction of the grid
    equal to its probability: softmax(logits / temperature) restricted to the
    top-k entries and renormalised (closed form, to 1/N)."""
    logits = np.array([[2.0, -1.0, 0.5, 3.0, 0.0, 1.5]])
    N = 60000
    u = (np.arange(N) + 0.5) / N
    for temp, k in ((1.0, None), (0.5, 3), (2.0, 4)):
        x = logits[0] / temp
        keep = np.argsort(-x)[:k] if k else np.arange(6)
        p = np.zeros(6)
        p[keep] = np.exp(x[keep] - x.max())
        p /= p.sum()
        got = np.array([O.sample_next(logits, temp, k, np.array([ui]))[0] for ui in u[::37]])
        freq = np.bincount(got, minlength=6) / len(got)
        assert np.max(np.abs(freq - p)) < 2.0 * 37 / N + 1e-12, (temp, k, freq, p)
        assert np.all(freq[p == 0] == 0)


def test_sample_topk_keeps_ties_at_the_threshold():
    """k = 2 with the 2nd-largest value repeated: every entry equal to the
    k-th largest stays, so 4 of 5 entries are drawable."""
    logits = np.array([[3.0, 1.0, 1.0, 1.0, 0.0]])
    e = math.exp(1.0)
    p_top = math.exp(3.0) / (math.exp(3.0) + 3 * e)
    assert O.sample_next(logits, 1.0, 2, np.array([p_top - 1e-9]))[0] == 0
    assert O.sample_next(logits, 1.0, 2, np.array([p_top + 1e-9]))[0] == 1
    assert O.sample_next(logits, 1.0, 2, np.array([1.0 - 1e-12]))[0] == 3


def test_sample_temperature_divides_logits():
    rng = np.random.default_rng(11)
    logits = rng.normal(size=(64, 50))
    u = rng.random(64)
    for temp in (0.3, 1.7):
        a = O.sample_next(logits, temp, 10, u)
        b = O.sample_next(logits / temp, 1.0, 10, u)
        assert np.array_equal(a, b)
    # a colder distribution concentrates on the argmax
    cold = O.sample_next(logits, 1e-3, None, u)
    assert np.array_equal(cold, logits.argmax(axis=1))


def test_generate_crops_to_the_last_block():
    """The context is cropped to its last block_size tokens, so tokens that
    have left the window cannot change what is drawn next; greedy (top-1)
    steps are the argmax of the last position's logits."""
    d = synthetic.model_dims("tiny")
    cfg = O.Config(**d)
    flat = synthetic.init_params(d, seed=3)
    rng = np.random.default_rng(4)
    prompt = rng.integers(0, 512, size=(2, d["block_size"] + 6))
    uni = rng.random((2, 3))
    a = O.generate(flat, prompt, 3, 0.9, 40, uni, cfg)
    b = O.generate(flat, prompt[:, 6:], 3, 0.9, 40, uni, cfg)
    assert a.shape == (2, d["block_size"] + 9)
    assert np.array_equal(a[:, -3:], b[:, -3:])
    assert np.array_equal(a[:, :-3], prompt)
    # a change inside the window does change the logits
    p2 = prompt.copy()
    p2[:, -1] = (p2[:, -1] + 1) % 512
    assert not np.allclose(O.last_logits(flat, p2[:, -64:], cfg), O.last_logits(flat, prompt[:, -64:], cfg))
    g = O.generate(flat, prompt[:, :10], 2, 1.0, 1, uni, cfg)
    assert g[0, 10] == O.last_logits(flat, prompt[:1, :10], cfg)[0].argmax()
    assert np.array_equal(O.generate(flat, prompt[:, :10], 0, 1.0, None, uni, cfg), prompt[:, :10])


# --------------------------------------------------------------------------
# seeded initialisation: the counter-based normal stream and the init recipe
# --------------------------------------------------------------------------

# Known-answer vectors of Philox4x32 with 10 rounds, as published with the
# generator (Salmon, Moraes, Dror, Shaw, SC 2011; the Random123 library's
# known-answer tests): (counter, key) -> output words.
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


def test_philox_known_answers():
    for ctr, key, want in PHILOX_KAT:
        got = O.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
        assert [int(x) for x in got] == list(want)


def test_normal_stream_is_standard_normal():
    """2^20 draws: mean, variance and the Kolmogorov-Smirnov distance against
    the normal CDF; each pair of a block shares one radius (Box-Muller's
    z_a^2 + z_b^2 = -2 ln u_a) and the two halves of a block are independent."""
    from scipy import stats
    n = 1 << 20
    z = O.normal_stream(np.arange(n), seed=1234)
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    r2 = (z[0::4] ** 2 + z[1::4] ** 2)
    assert stats.kstest(r2, "expon", args=(0, 2)).pvalue > 1e-3     # chi-square with 2 dof
    assert abs(np.corrcoef(z[0::4], z[2::4])[0, 1]) < 5 / math.sqrt(n / 4)
    # counter-based: any subset of indices gives the same numbers
    sub = np.array([0, 3, 4, 99999, n - 1])
    assert np.array_equal(O.normal_stream(sub, seed=1234), z[sub])
    assert not np.allclose(O.normal_stream(sub, seed=1235), z[sub])


def test_seeded_init_follows_the_recipe():
    """"GPT-2 from Scratch", Initialization: weights N(0, 0.02), both c_proj
    weights N(0, 0.02/sqrt(2L)), biases 0, LayerNorm gains 1 and shifts 0."""
    cfg, d = cfg_of("tiny")
    p = O.init_params(cfg, seed=42)
    assert p.size == O.num_params(cfg)
    P = O.unflatten(p, cfg)
    L = cfg.n_layer
    for name, x in P.items():
        if x.ndim == 2:
            std = 0.02 / math.sqrt(2 * L) if name.endswith("c_proj.weight") else 0.02
            n = x.size
            assert abs(x.std() - std) < 6 * std / math.sqrt(2 * n), name
            assert abs(x.mean()) < 6 * std / math.sqrt(n), name
        elif name.endswith(("ln_1.weight", "ln_2.weight")) or name == "ln_f.weight":
            assert np.all(x == 1.0), name
        else:
            assert np.all(x == 0.0), name
    sub = np.array([0, 5, 1000, p.size - 1, O.num_params(cfg) // 2])
    assert np.array_equal(O.init_params(cfg, seed=42, elems=sub), p[sub])
