"""The bf16 step comparison (bf16_check.compare_step) on the CPU, with the
tiny model's exact and bf16-rounded oracle steps standing in for the
reference and the noise model, and a synthetic "GPU" gradient: it accepts a
step whose gradients carry noise of the rounded oracle's size, and it rejects
one whose gradient has a single wrong row -- the wte row of a token absent
from the batch, a small row inside a large tensor, which a per-tensor check
would let through -- or a few flipped signs."""
import numpy as np
import pytest

from oracle import gpt2_oracle as O
import synthetic
import bf16_check as BC

LR, WD = 6e-4, 0.1


@pytest.fixture(scope="module")
def tiny_step():
    d = synthetic.model_dims("tiny")
    cfg = O.Config(**d)
    p0 = synthetic.init_params(d, seed=42)
    idx, tgt = synthetic.uniform_batch(4, 64, 512, seed=1001)
    # a token that never occurs in the batch: its wte row gets only the
    # lm_head part of the gradient, far smaller than the rows of used tokens
    absent = sorted(set(range(d["vocab_size"])) - set(idx.ravel().tolist()))
    assert len(absent) >= 2
    _, cache = O.forward(p0.copy(), idx, tgt, cfg)
    g_ref = O.backward(p0.copy(), cache, cfg)
    _, cache = O.forward(p0.copy(), idx, tgt, cfg, rnd=O.bf16_round)
    g_emul = O.backward(p0.copy(), cache, cfg)
    return cfg, d, p0, g_ref, g_emul, absent


def _step(cfg, p0, g):
    p = p0.astype(np.float32).copy()
    gg = g.astype(np.float32).copy()
    norm = O.clip_and_adamw(p, gg, np.zeros_like(p), np.zeros_like(p), 1, LR, cfg=cfg,
                            weight_decay=WD)
    return p, norm


def _noisy(cfg, g_ref, g_emul, scale, seed):
    """g_ref plus the rounded oracle's noise, scaled, with a random sign per
    element: another noise draw of the same size at every element."""
    rng = np.random.default_rng(seed)
    e = g_emul.astype(np.float64) - g_ref
    sign = rng.choice([-1.0, 1.0], size=e.size)
    return (g_ref + scale * sign * e).astype(np.float32)


def _compare(cfg, p0, g_gpu, g_ref, g_emul):
    p_gpu, n_gpu = _step(cfg, p0, g_gpu)
    p_ref, n_ref = _step(cfg, p0, g_ref)
    return BC.compare_step(O, cfg, p0=p0, g_gpu=g_gpu, g_ref=g_ref, g_emul=g_emul, p_gpu=p_gpu,
                           p_ref=p_ref, norm_gpu=n_gpu, norm_ref=n_ref, lr=LR, wd=WD, t=1,
                           verbose=False)


def test_accepts_exact_and_rounding_sized_noise(tiny_step):
    cfg, d, p0, g_ref, g_emul, _ = tiny_step
    fails, st = _compare(cfg, p0, g_ref.copy(), g_ref, g_emul)
    assert fails == [] and st["worst"]["grad"] == 0.0
    fails, st = _compare(cfg, p0, _noisy(cfg, g_ref, g_emul, 2.0, seed=1), g_ref, g_emul)
    assert fails == [], fails
    assert st["below_frac"] < BC.MAX_BELOW


def test_rejects_one_wrong_rare_token_row(tiny_step):
    cfg, d, p0, g_ref, g_emul, absent = tiny_step
    C = d["n_embd"]
    a, b = absent[0], absent[1]
    g_gpu = _noisy(cfg, g_ref, g_emul, 2.0, seed=2)
    wte = g_gpu[:d["padded_vocab_size"] * C].reshape(-1, C)
    ref_wte = g_ref[:d["padded_vocab_size"] * C].reshape(-1, C)
    # the row is tiny within wte: the tensor's normwise error stays in bounds
    assert np.linalg.norm(ref_wte[a]) < 0.05 * np.linalg.norm(ref_wte, axis=1).max()
    wte[a] = ref_wte[b]                      # same scale, wrong values
    fails, st = _compare(cfg, p0, g_gpu, g_ref, g_emul)
    assert st["worst"]["grad"] < BC.TOL_GRAD  # the per-tensor check alone would pass
    assert any(f.startswith(f"wte: row {a} ") for f in fails), fails


def test_rejects_sign_flips_of_determined_elements(tiny_step):
    """A wrong sign on a few elements well above the floor moves them by 2 lr."""
    cfg, d, p0, g_ref, g_emul, _ = tiny_step
    g_gpu = g_ref.copy()
    name, shape, sl, _ = [x for x in BC.tensor_slices(O, cfg) if x[0] == "h.0.mlp.c_proj.weight"][0]
    x = g_gpu[sl]
    big = np.argsort(-np.abs(x))[: x.size // 100]   # 1% of the largest elements
    x[big] = -x[big]
    fails, _ = _compare(cfg, p0, g_gpu, g_ref, g_emul)
    assert any(f.startswith(name + ": parameter error") for f in fails), fails


def test_key_bias_third_is_not_compared(tiny_step):
    cfg, d, p0, g_ref, g_emul, _ = tiny_step
    C = d["n_embd"]
    g_gpu = g_ref.copy()
    _, _, sl, keep = [x for x in BC.tensor_slices(O, cfg) if x[0] == "h.1.attn.c_attn.bias"][0]
    g_gpu[sl][C:2 * C] = 1e-3                  # noise there is arbitrary by construction
    assert not keep[C:2 * C].any()
    fails, _ = _compare(cfg, p0, g_gpu, g_ref, g_emul)
    assert fails == [], fails


@pytest.mark.parametrize("with_means", [False, True])
def test_second_step_from_shared_state(tiny_step, with_means):
    """t = 2 from a common (p, m, v): a step with rounding-sized gradient
    noise passes; a moment vector off by 10% in one tensor fails (with and
    without the sequence-mean split of the c_attn.weight rows)."""
    cfg, d, p0, g_ref0, _, _ = tiny_step
    p1, m1, v1 = p0.astype(np.float32).copy(), np.zeros_like(p0), np.zeros_like(p0)
    O.clip_and_adamw(p1, g_ref0.copy(), m1, v1, 1, LR, cfg=cfg, weight_decay=WD)
    idx, tgt = synthetic.uniform_batch(4, 64, 512, seed=2002)
    _, cache = O.forward(p1.copy(), idx, tgt, cfg)
    means = BC.seq_means(cache) if with_means else None
    g_ref = O.backward(p1.copy(), cache, cfg)
    _, cache = O.forward(p1.copy(), idx, tgt, cfg, rnd=O.bf16_round)
    g_emul = O.backward(p1.copy(), cache, cfg)
    g_gpu = _noisy(cfg, g_ref, g_emul, 2.0, seed=3)

    def step(g):
        p, m, v = p1.copy(), m1.copy(), v1.copy()
        n = O.clip_and_adamw(p, g.copy(), m, v, 2, LR, cfg=cfg, weight_decay=WD)
        return p, m, v, n

    pa, ma, va, na = step(g_gpu)
    pr, mr, vr, nr = step(g_ref)
    kw = dict(p0=p1, g_gpu=g_gpu, g_ref=g_ref, g_emul=g_emul, p_gpu=pa, p_ref=pr, norm_gpu=na,
              norm_ref=nr, lr=LR, wd=WD, t=2, m0=m1, v0=v1, m_gpu=ma, m_ref=mr, v_gpu=va,
              v_ref=vr, seq_means=means, verbose=False)
    fails, _ = BC.compare_step(O, cfg, **kw)
    assert fails == [], fails
    _, _, sl, _ = [x for x in BC.tensor_slices(O, cfg) if x[0] == "h.0.mlp.c_fc.weight"][0]
    mb = ma.copy()
    mb[sl] *= 1.1
    fails, _ = BC.compare_step(O, cfg, **dict(kw, m_gpu=mb))
    assert any(f.startswith("h.0.mlp.c_fc.weight: moments error") for f in fails), fails


@pytest.fixture(scope="module")
def tiny_means():
    d = synthetic.model_dims("tiny")
    cfg = O.Config(**d)
    p0 = synthetic.init_params(d, seed=42)
    idx, tgt = synthetic.uniform_batch(4, 64, 512, seed=1001)
    _, cache = O.forward(p0.copy(), idx, tgt, cfg)
    return BC.seq_means(cache)


def _key_rows(cfg, name="h.1.attn.c_attn.weight"):
    C = cfg.n_embd
    _, shape, sl, _ = [x for x in BC.tensor_slices(O, cfg) if x[0] == name][0]
    return sl, shape, C


def test_key_row_error_along_sequence_means(tiny_step, tiny_means):
    """With the sequence means given, a c_attn.weight row's error is split:
    along the span of the means (where a bf16 sum of dK over each sequence
    leaves its rounding, the exact sum being zero) it is judged per third
    against the rounded oracle's error in that span, across it row by row.
    An error along the span within that budget passes; the same error
    turned across the span, at three times the row allowance, fails as a
    row; and an error along the span at three times the budget fails the
    span check."""
    cfg, d, p0, g_ref, g_emul, _ = tiny_step
    sl, shape, C = _key_rows(cfg)
    rows = lambda g: g[sl].reshape(shape)
    Q, _ = np.linalg.qr(tiny_means[1].T)
    ref = rows(g_ref).astype(np.float64)
    de = rows(g_emul).astype(np.float64) - ref
    se = np.linalg.norm(de[C:2 * C] @ Q)
    budget = BC.F_SPAN * se + 1e-3 * np.linalg.norm(ref[C:2 * C])
    e_rows = np.linalg.norm(de[C:2 * C] - (de[C:2 * C] @ Q) @ Q.T, axis=1)
    allowance = (BC.F_ROW * np.median(e_rows) +
                 BC.ROW_SLACK * np.median(np.linalg.norm(ref, axis=1)))
    r = C + 5
    rng = np.random.default_rng(5)
    x = rng.standard_normal(C)
    x -= Q @ (Q.T @ x)
    across = x / np.linalg.norm(x)

    def with_error(vec):
        g = g_ref.copy()
        rows(g)[r] += vec.astype(np.float32)
        return _compare_means(cfg, p0, g, g_ref, g_emul, tiny_means)[0]

    assert with_error(0.5 * budget * Q[:, 0]) == []
    fails = with_error(3.0 * allowance * across)
    assert any(f.startswith("h.1.attn.c_attn.weight: row %d " % r) for f in fails), fails
    fails = with_error(3.0 * budget * Q[:, 0])
    assert any(f.startswith("h.1.attn.c_attn.weight: k rows along the sequence means")
               for f in fails), fails


def _compare_means(cfg, p0, g_gpu, g_ref, g_emul, means):
    p_gpu, n_gpu = _step(cfg, p0, g_gpu)
    p_ref, n_ref = _step(cfg, p0, g_ref)
    return BC.compare_step(O, cfg, p0=p0, g_gpu=g_gpu, g_ref=g_ref, g_emul=g_emul, p_gpu=p_gpu,
                           p_ref=p_ref, norm_gpu=n_gpu, norm_ref=n_ref, lr=LR, wd=WD, t=1,
                           seq_means=means, verbose=False)


def test_rounding_noise_passes_with_sequence_means(tiny_step, tiny_means):
    cfg, d, p0, g_ref, g_emul, _ = tiny_step
    fails, _ = _compare_means(cfg, p0, _noisy(cfg, g_ref, g_emul, 2.0, seed=7), g_ref, g_emul,
                              tiny_means)
    assert fails == [], fails
