"""The oracle against torch's CPU library routines, which are the calls the
pages make (F.layer_norm, F.gelu(approximate='tanh'),
F.scaled_dot_product_attention(is_causal=True), F.cross_entropy with
ignore_index=-1, autograd, clip_grad_norm_ and torch.optim.AdamW with two
parameter groups).  Everything runs in float64 so that agreement is to
rounding level; an error anywhere in the oracle's forward, backward or update
(a dropped term, a sign, a transposed operand) shows up here."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import torch.nn.functional as F

from oracle import gpt2_oracle as O
import synthetic


def torch_model_loss(P, idx, tgt, cfg):
    """GPT-2 forward written with torch.nn.functional on named tensors."""
    B, T = idx.shape
    C, H = cfg.n_embd, cfg.n_head
    x = F.embedding(idx, P["wte"]) + P["wpe"][:T]
    for l in range(cfg.n_layer):
        p = f"h.{l}."
        u = F.layer_norm(x, (C,), P[p + "ln_1.weight"], P[p + "ln_1.bias"], eps=1e-5)
        qkv = F.linear(u, P[p + "attn.c_attn.weight"], P[p + "attn.c_attn.bias"])
        q, k, v = qkv.split(C, dim=2)
        q, k, v = (t.view(B, T, H, C // H).transpose(1, 2) for t in (q, k, v))
        y = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        y = y.transpose(1, 2).contiguous().view(B, T, C)
        x = x + F.linear(y, P[p + "attn.c_proj.weight"], P[p + "attn.c_proj.bias"])
        u2 = F.layer_norm(x, (C,), P[p + "ln_2.weight"], P[p + "ln_2.bias"], eps=1e-5)
        h = F.gelu(F.linear(u2, P[p + "mlp.c_fc.weight"], P[p + "mlp.c_fc.bias"]), approximate="tanh")
        x = x + F.linear(h, P[p + "mlp.c_proj.weight"], P[p + "mlp.c_proj.bias"])
    z = F.layer_norm(x, (C,), P["ln_f.weight"], P["ln_f.bias"], eps=1e-5)
    logits = F.linear(z, P["wte"])
    return F.cross_entropy(logits.view(-1, logits.size(-1)), tgt.view(-1), ignore_index=-1)


def _torch_params(flat, cfg):
    out = {}
    for name, arr in O.unflatten(flat, cfg).items():
        out[name] = torch.tensor(arr, dtype=torch.float64, requires_grad=True)
    return out


@pytest.mark.parametrize("masked", [False, True])
def test_forward_backward_match_torch_fp64(masked):
    d = synthetic.model_dims("tiny")
    d["vocab_size"] = 500
    cfg = O.Config(**d)
    flat = synthetic.init_params(d, seed=3, dtype=np.float64)
    flat += np.random.default_rng(4).standard_normal(flat.size) * 0.01
    idx, tgt = synthetic.uniform_batch(3, 24, 500, seed=5)
    if masked:
        tgt[:, :10] = -1
        tgt[2, 15:] = -1
    loss, cache = O.forward(flat, idx, tgt, cfg)
    g = O.backward(flat, cache, cfg, loss_scale=0.5)

    P = _torch_params(flat, cfg)
    tl = torch_model_loss(P, torch.tensor(idx), torch.tensor(tgt), cfg)
    (0.5 * tl).backward()
    assert abs(float(loss) - tl.item()) < 1e-12
    G = O.unflatten(g, cfg)
    for name, t in P.items():
        ref = t.grad.numpy()
        err = np.max(np.abs(G[name] - ref))
        assert err <= 1e-11 * max(np.max(np.abs(ref)), 1e-12), (name, err)


def test_fp32_oracle_close_to_fp64():
    d = synthetic.model_dims("tiny")
    cfg = O.Config(**d)
    flat = synthetic.init_params(d, seed=6)
    idx, tgt = synthetic.uniform_batch(4, 64, 512, seed=7)
    l32, c32 = O.forward(flat, idx, tgt, cfg)
    g32 = O.backward(flat, c32, cfg)
    l64, c64 = O.forward(flat.astype(np.float64), idx, tgt, cfg)
    g64 = O.backward(flat.astype(np.float64), c64, cfg)
    assert abs(float(l32) - float(l64)) < 1e-5 * float(l64)
    off = 0
    for name, shape in O.param_specs(cfg):
        n = int(np.prod(shape))
        a, b = g32[off:off + n], g64[off:off + n]
        off += n
        if name.endswith("attn.c_attn.bias"):
            b = b.copy(); a = a.copy()
            a[128:256] = 0; b[128:256] = 0      # analytically zero slice (key bias)
        assert np.max(np.abs(a - b)) <= 1e-4 * np.max(np.abs(b)), name


def test_clip_and_adamw_match_torch():
    d = synthetic.model_dims("tiny")
    cfg = O.Config(**d)
    rng = np.random.default_rng(8)
    flat = synthetic.init_params(d, seed=9, dtype=np.float64)
    grads = rng.standard_normal(flat.size) * 0.02            # global norm >> 1: clip active
    P = _torch_params(flat, cfg)
    specs = O.param_specs(cfg)
    off = 0
    for name, shape in specs:
        n = int(np.prod(shape))
        P[name].grad = torch.tensor(grads[off:off + n].reshape(shape))
        off += n
    params = list(P.values())
    groups = [{"params": [p for p in params if p.dim() >= 2], "weight_decay": 0.1},
              {"params": [p for p in params if p.dim() < 2], "weight_decay": 0.0}]
    opt = torch.optim.AdamW(groups, lr=6e-4, betas=(0.9, 0.95), eps=1e-8, foreach=False)
    m, v = np.zeros_like(flat), np.zeros_like(flat)
    p_or = flat.copy()
    for t in range(1, 4):
        g_t = grads * (1.0 + 0.1 * t)
        off = 0
        for name, shape in specs:
            n = int(np.prod(shape))
            P[name].grad = torch.tensor(g_t[off:off + n].reshape(shape))
            off += n
        tn = torch.nn.utils.clip_grad_norm_(params, 1.0).item()
        opt.step()
        on = O.clip_and_adamw(p_or, g_t.copy(), m, v, t, 6e-4, cfg=cfg)
        assert abs(tn - on) < 1e-12 * on
    ref = np.concatenate([P[name].detach().numpy().reshape(-1) for name, _ in specs])
    assert np.max(np.abs(p_or - ref)) < 1e-15 + 1e-12 * np.max(np.abs(ref))


def test_layernorm_and_gelu_match_torch():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((5, 7, 96)) * 3 + 1
    w, b = rng.standard_normal(96), rng.standard_normal(96)
    y, _, _ = O.layernorm_fwd(x, w, b)
    ref = F.layer_norm(torch.tensor(x), (96,), torch.tensor(w), torch.tensor(b), eps=1e-5).numpy()
    assert np.max(np.abs(y - ref)) < 1e-12
    z = rng.standard_normal(10000) * 4
    assert np.max(np.abs(O.gelu_tanh(z) - F.gelu(torch.tensor(z), approximate="tanh").numpy())) < 1e-12


def test_bf16_round_matches_torch_conversion():
    """The oracle's bf16 rounding is torch's float32 -> bfloat16 conversion:
    nearest, ties to even (exact halfway cases both ways), NaN and infinities
    kept, values past the largest bf16 to infinity."""
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, np.nan, 3.3895314e38, 3.39e38, 1e-40], np.float32),
        # halfway cases: the dropped 16 bits are exactly 0x8000, kept lsb 0 and 1
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x3F807FFF], np.uint32).view(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = O.bf16_round(x)
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all(), x[~same][:5]


def test_bf16_placement_stays_near_the_exact_step():
    """The bf16-rounded step (R8) is a perturbation of the exact one: loss
    within 1e-3 relative, every gradient tensor within 3e-2 normwise; and the
    exact rounding hook leaves the computation unchanged."""
    d = synthetic.model_dims("tiny")
    d = dict(d, n_head=2)
    cfg = O.Config(**d)
    flat = synthetic.init_params(d, seed=4)
    idx, tgt = synthetic.uniform_batch(2, 64, 512, seed=5)
    l0, c0 = O.forward(flat.copy(), idx, tgt, cfg)
    g0 = O.backward(flat.copy(), c0, cfg)
    l1, c1 = O.forward(flat.copy(), idx, tgt, cfg, rnd=O.exact)
    assert l1 == l0 and np.array_equal(O.backward(flat.copy(), c1, cfg), g0)
    lb, cb = O.forward(flat.copy(), idx, tgt, cfg, rnd=O.bf16_round)
    gb = O.backward(flat.copy(), cb, cfg)
    assert abs(lb - l0) < 1e-3 * l0
    assert not np.array_equal(gb, g0)
    off = 0
    for name, shape in O.param_specs(cfg):
        n = int(np.prod(shape))
        a, b = gb[off:off + n].astype(np.float64), g0[off:off + n].astype(np.float64)
        if np.linalg.norm(b) > 0 and not name.endswith("c_attn.bias"):
            assert np.linalg.norm(a - b) / np.linalg.norm(b) < 3e-2, name
        off += n
