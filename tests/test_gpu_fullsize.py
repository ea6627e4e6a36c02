"""Parity at the full workload sizes, in the launch configuration the
benchmark times (GPT-2 124M bf16 B=16 T=1024; the masked fine-tuning batch;
the XL shape at B=8), on outputs the oracle can compute one by one.

Every sequence of a batch is processed independently, and the loss at
position t depends only on tokens 0..t (causal attention), so the oracle's
forward pass over one sampled sequence -- or over its first P tokens --
gives the per-position losses the GPU computed for that sequence inside the
full batch.  Those are compared within 5e-3 of the largest per-position
loss.  Properties that hold at any size are checked
over the whole batch: the mean loss equals the sum of per-position losses
over the number of valid targets; reversing the order of the sequences
permutes the per-position losses bit for bit; ignored targets give exactly
zero loss and exactly zero logit-gradient rows; the reported pre-clip norm is
the norm of the gradients the GPU holds; and the AdamW update equals the
closed form of its first step applied to those gradients."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gpt2_oracle as O
import synthetic
from decoder_only_transformer_03_amd import gpt2 as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LR, B1, B2, EPS, WD, CLIP = 6e-4, 0.9, 0.95, 1e-8, 0.1, 1.0


def dev_ids(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.int32, device=DEV)


def oracle_position_losses(d, flat, idx, tgt, rows, prefix):
    """Per-position losses of sequences `rows`, first `prefix` positions."""
    cfg = O.Config(**d)
    _, cache = O.forward(flat, idx[rows, :prefix], tgt[rows, :prefix], cfg)
    return cache["row_loss"].reshape(len(rows), prefix).astype(np.float64)


def check_rows(gpu_rows, ref_rows, what):
    err = float(np.max(np.abs(gpu_rows - ref_rows)) / max(np.max(np.abs(ref_rows)), 1e-30))
    print(f"{what}: per-position loss maxrel {err:.2e}")
    assert err < 5e-3, what


def check_adamw_closed_form(m, flat, d, lr, wd, norm):
    """Step 1 of AdamW on the GPU's own gradients: m_hat = c g, v_hat = (c g)^2,
    so p1 = p0 (1 - lr wd [2-D]) - lr c g / (|c g| + eps), c the clip
    coefficient from the pre-clip norm."""
    g = m.get(G.GPT2_GRADS).astype(np.float64)
    p1 = m.get(G.GPT2_PARAMS).astype(np.float64)
    n64 = float(np.sqrt(np.sum(g * g)))
    assert abs(norm - n64) <= 1e-5 * n64, (norm, n64)
    c = min(1.0, CLIP / (n64 + 1e-6))
    cfg = O.Config(**d)
    decay = np.zeros(g.size, bool)
    off = 0
    for name, shape in O.param_specs(cfg):
        n = int(np.prod(shape))
        decay[off:off + n] = len(shape) >= 2
        off += n
    p0 = flat.astype(np.float64)
    gc = c * g
    expect = p0 * np.where(decay, 1.0 - lr * wd, 1.0) - lr * gc / (np.abs(gc) + EPS)
    err = float(np.max(np.abs(p1 - expect)))
    print(f"AdamW closed form on own grads: max |diff| {err:.2e} (lr {lr:g})")
    # fp32 update arithmetic on values of size <= 1: a few ulps of the largest
    assert err < 1e-6


@pytest.fixture(scope="module")
def m124():
    d = synthetic.model_dims("gpt2-124m")
    flat = synthetic.init_params(d, seed=42)
    cfg = G.make_config(max_batch=16, precision="bf16", **d)
    m = G.GPT2(cfg, device=DEV)
    m.set_params(flat)
    return d, flat, m


def test_124m_b16_sampled_sequences(m124):
    d, flat, m = m124
    B, T = 16, 1024
    idx, tgt = synthetic.zipf_batch(B, T, seed=1002)
    m.zero_grad()
    loss = m.forward(dev_ids(idx), dev_ids(tgt), want_loss=True)
    rl = m.activation("ROW_LOSS", 0, B * T).astype(np.float64).reshape(B, T)
    n_valid = int(np.sum(tgt != -1))
    assert abs(loss - rl.sum() / n_valid) <= 1e-5 * abs(loss)
    rows = [0, 7, 15]
    ref = oracle_position_losses(d, flat, idx, tgt, rows, T)
    check_rows(rl[rows], ref, "124M B=16 sequences 0, 7, 15")
    ref_mean = ref.sum() / np.sum(tgt[rows] != -1)
    gpu_mean = rl[rows].sum() / np.sum(tgt[rows] != -1)
    assert abs(gpu_mean - ref_mean) < 5e-3
    m.backward(1.0)
    norm = m.adamw_step(LR, B1, B2, EPS, WD, CLIP, want_norm=True)
    check_adamw_closed_form(m, flat, d, LR, WD, norm)


def test_124m_b16_sequence_order_bit_exact(m124):
    d, flat, m = m124
    m.set_params(flat)
    B, T = 16, 1024
    idx, tgt = synthetic.zipf_batch(B, T, seed=1002)
    m.forward(dev_ids(idx), dev_ids(tgt), want_loss=True)
    a = m.activation("ROW_LOSS", 0, B * T).reshape(B, T)
    m.forward(dev_ids(idx[::-1]), dev_ids(tgt[::-1]), want_loss=True)
    b = m.activation("ROW_LOSS", 0, B * T).reshape(B, T)
    assert np.array_equal(a, b[::-1])


def test_sft_b16_masked_targets(m124):
    d, flat, m = m124
    m.set_params(flat)
    B, T = 16, 1024
    idx, tgt = synthetic.sft_batch(B, T, seed=1004)
    Vp = d["padded_vocab_size"]
    m.zero_grad()
    loss = m.forward(dev_ids(idx), dev_ids(tgt), want_loss=True)
    rl = m.activation("ROW_LOSS", 0, B * T).astype(np.float64).reshape(B, T)
    ignored = tgt == -1
    n_valid = int((~ignored).sum())
    assert np.all(rl[ignored] == 0.0)
    assert abs(loss - rl.sum() / n_valid) <= 1e-5 * abs(loss)
    # dlogits of sequence 0 (written over the logits by the fused kernel)
    dl = m.activation("LOGITS", 0, T * Vp).reshape(T, Vp)
    assert np.all(dl[ignored[0]] == 0.0)
    valid = dl[~ignored[0]].astype(np.float64)
    # each valid row is (softmax - onehot) / n_valid: sums to 0, one entry < 0
    # (the bf16 rounding of the one entry near -1/n_valid dominates: 2^-9 of it)
    assert np.max(np.abs(valid.sum(axis=1))) < 5e-3 / n_valid
    assert np.all(np.sum(valid < 0, axis=1) == 1)
    rows = [0, 9]
    ref = oracle_position_losses(d, flat, idx, tgt, rows, T)
    assert np.all(ref[ignored[rows]] == 0.0)
    check_rows(rl[rows], ref, "SFT B=16 sequences 0, 9")
    m.backward(1.0)
    norm = m.adamw_step(2e-5, B1, B2, EPS, 0.0, CLIP, want_norm=True)
    check_adamw_closed_form(m, flat, d, 2e-5, 0.0, norm)


@pytest.mark.parametrize("kind", ["zipf", "sft"])
def test_124m_b16_fused_head(kind):
    """The fused lm_head + cross-entropy (vocabulary slices of 4096 columns)
    on the benchmark's batch and on the masked fine-tuning batch: sampled
    sequences' per-position losses against the oracle, ignored targets at
    exactly zero loss, the batch loss the mean of the per-position losses,
    and the AdamW closed form on the GPU's own gradients."""
    d = synthetic.model_dims("gpt2-124m")
    flat = synthetic.init_params(d, seed=42)
    B, T = 16, 1024
    if kind == "zipf":
        idx, tgt = synthetic.zipf_batch(B, T, seed=1002)
        rows, lr, wd = [4, 11], LR, WD
    else:
        idx, tgt = synthetic.sft_batch(B, T, seed=1004)
        rows, lr, wd = [3, 9], 2e-5, 0.0
    cfg = G.make_config(max_batch=B, precision="bf16", head_chunk=4096, **d)
    m = G.GPT2(cfg, device=DEV)
    try:
        m.set_params(flat)
        m.zero_grad()
        loss = m.forward(dev_ids(idx), dev_ids(tgt), want_loss=True)
        rl = m.activation("ROW_LOSS", 0, B * T).astype(np.float64).reshape(B, T)
        ignored = tgt == -1
        assert np.all(rl[ignored] == 0.0)
        assert abs(loss - rl.sum() / np.sum(~ignored)) <= 1e-5 * abs(loss)
        m.backward(1.0)
        norm = m.adamw_step(lr, B1, B2, EPS, wd, CLIP, want_norm=True)
        check_adamw_closed_form(m, flat, d, lr, wd, norm)
    finally:
        m.close()
    ref = oracle_position_losses(d, flat, idx, tgt, rows, T)
    check_rows(rl[rows], ref, f"fused head, {kind} B=16 sequences {rows}")


def test_xl_b8_sampled_prefixes():
    """XL shape (48 layers, C=1600, 25 heads of 64), B=8, T=1024: the first
    256 positions of sequences 0 and 5 against the oracle."""
    d = synthetic.model_dims("gpt2-xl")
    B, T, P = 8, 1024, 256
    flat = synthetic.init_params(d, seed=42)
    idx, tgt = synthetic.zipf_batch(B, T, seed=1005)
    cfg = G.make_config(max_batch=B, precision="bf16", **d)
    m = G.GPT2(cfg, device=DEV)
    try:
        m.set_params(flat)
        m.zero_grad()
        loss = m.forward(dev_ids(idx), dev_ids(tgt), want_loss=True)
        rl = m.activation("ROW_LOSS", 0, B * T).astype(np.float64).reshape(B, T)
        assert abs(loss - rl.sum() / np.sum(tgt != -1)) <= 1e-5 * abs(loss)
        m.backward(1.0)
        norm = m.adamw_step(LR, B1, B2, EPS, WD, CLIP, want_norm=True)
        g = m.get(G.GPT2_GRADS).astype(np.float64)
        assert np.all(np.isfinite(g))
        n64 = float(np.sqrt(np.sum(g * g)))
        assert abs(norm - n64) <= 1e-5 * n64
        del g
    finally:
        m.close()
    rows = [0, 5]
    ref = oracle_position_losses(d, flat, idx, tgt, rows, P)
    check_rows(rl[rows, :P], ref, "XL B=8 sequences 0, 5 (first 256 positions)")
