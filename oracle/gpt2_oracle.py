"""Plain CPU oracle for one GPT-2 training step (forward, backward, clip, AdamW).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package's smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library: it has its own parameter layout, its own maths, and it imports
nothing from this repository.

Every function is the textbook definition written out in numpy, in the dtype
of its inputs (float32 for parity, float64 for gradient checks).  Sources, by
page title and section:

* "GPT-2 from Scratch" (lumen chapter): "The config", "Embeddings",
  "CausalSelfAttention", "The MLP and GPT-2's GELU", "The Block: pre-LN and
  residuals", "The full model", "Weight tying", "Initialization",
  "AdamW, and weight decay on matrices only", "Warmup and cosine decay",
  "Gradient clipping", "How to scale up" (accumulation).
* "Let's reproduce GPT-2 (124M)" (synopsis): weight tying, residual init
  scaling, padded vocabulary, GPT-3 optimizer settings, loss/k accumulation.
* "Pretraining and fine-tuning nanoGPT-124M from scratch": padded vocab
  50,304, loss masking with target -1.

Readings where the pages are silent or garbled (each is listed with its reason
in the design notes):
  R1  GELU is the tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
      of Hendrycks & Gimpel; the page's formula did not survive extraction.
  R2  LayerNorm uses the biased variance over C and eps = 1e-5 inside the
      square root.
  R3  The loss is the mean over positions whose target is not -1; with no
      valid position the loss is 0 and the gradient is 0.
  R4  Padded vocabulary columns take part in the softmax like real ones.
  R5  Clip coefficient min(1, max_norm / (norm + 1e-6)); the pre-clip norm is
      what is reported.
  R6  AdamW: decoupled decay p <- p (1 - lr wd) on tensors with dim >= 2,
      then the moment updates, bias correction with t starting at 1, eps added
      to sqrt(v_hat).
  R7  Sampling ("GPT-2 from Scratch", A generation loop): the logits of the
      last position are divided by the temperature; top-k keeps every entry
      not below the k-th largest value (entries tied with it stay); the
      multinomial draw is the inverse CDF of a caller-supplied uniform u in
      [0, 1) over the vocabulary in index order: the smallest i whose
      cumulative probability exceeds u (if rounding leaves none, the last
      entry with non-zero probability).  The context is cropped to its last
      block_size tokens before every forward pass.
  R8  bf16 placement ("Let's reproduce GPT-2 (124M)", the bf16 autocast step:
      products in bf16, weights, LayerNorm and the loss in fp32): with
      rnd=bf16_round, forward/backward round every product operand, weights
      included, and the activations and gradients a mixed-precision step
      stores in bf16; accumulation, LayerNorm, softmax, the residual stream
      and parameter gradients stay fp32.  This only models the rounding
      noise of such a step; the reference is the exact computation.
The backward pass is the chain rule of the forward pass; it is pinned by
central differences and by torch autograd in the CPU tests.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------
# configuration and parameter layout
# ("GPT-2 from Scratch", "The config" / "The full model")
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    n_layer: int
    n_head: int
    n_embd: int
    vocab_size: int
    padded_vocab_size: int
    block_size: int


def param_specs(cfg: Config):
    """Canonical tensor order and shapes: wte, wpe, per block (ln_1, c_attn,
    c_proj, ln_2, c_fc, mlp c_proj), ln_f.  Weights are (out, in) as for a
    torch Linear; wte doubles as the lm_head weight (weight tying)."""
    C, Vp = cfg.n_embd, cfg.padded_vocab_size
    specs = [("wte", (Vp, C)), ("wpe", (cfg.block_size, C))]
    for l in range(cfg.n_layer):
        p = f"h.{l}."
        specs += [
            (p + "ln_1.weight", (C,)), (p + "ln_1.bias", (C,)),
            (p + "attn.c_attn.weight", (3 * C, C)), (p + "attn.c_attn.bias", (3 * C,)),
            (p + "attn.c_proj.weight", (C, C)), (p + "attn.c_proj.bias", (C,)),
            (p + "ln_2.weight", (C,)), (p + "ln_2.bias", (C,)),
            (p + "mlp.c_fc.weight", (4 * C, C)), (p + "mlp.c_fc.bias", (4 * C,)),
            (p + "mlp.c_proj.weight", (C, 4 * C)), (p + "mlp.c_proj.bias", (C,)),
        ]
    specs += [("ln_f.weight", (C,)), ("ln_f.bias", (C,))]
    return specs


def num_params(cfg: Config) -> int:
    return sum(int(np.prod(s)) for _, s in param_specs(cfg))


def unflatten(flat: np.ndarray, cfg: Config) -> dict:
    """Views of the flat vector, one per named tensor (no copies)."""
    out, off = {}, 0
    for name, shape in param_specs(cfg):
        n = int(np.prod(shape))
        out[name] = flat[off:off + n].reshape(shape)
        off += n
    assert off == flat.size, (off, flat.size)
    return out


def decay_mask(cfg: Config, dtype=np.float32) -> np.ndarray:
    """1 on tensors with dim >= 2 (matrices and embeddings), 0 on biases and
    LayerNorm parameters ("AdamW, and weight decay on matrices only")."""
    parts = [np.full(int(np.prod(s)), 1.0 if len(s) >= 2 else 0.0, dtype=dtype)
             for _, s in param_specs(cfg)]
    return np.concatenate(parts)


# ----------------------------------------------------------------------------
# seeded initialisation ("GPT-2 from Scratch", Initialization: 0.02, and the
# residual scaling), from a counter-based normal stream
# ----------------------------------------------------------------------------

_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
    random numbers: as easy as 1, 2, 3", SC 2011).  counter: (n, 4) words,
    key: 2 words (uint32 values).  Per round, words 0 and 2 are multiplied by
    0xD2511F53 and 0xCD9E8D57 into 64-bit products; the new state is
    (hi(w2 M1) ^ w1 ^ k0, lo(w2 M1), hi(w0 M0) ^ w3 ^ k1, lo(w0 M0)); then the
    key advances by the Weyl increments 0x9E3779B9 and 0xBB67AE85 (mod 2^32).
    Returns (n, 4) uint64 arrays holding the 32-bit output words."""
    c = np.asarray(counter, dtype=np.uint64).reshape(-1, 4) & _U32
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    x0, x1, x2, x3 = (c[:, i].copy() for i in range(4))
    for _ in range(10):
        p0 = x0 * np.uint64(0xD2511F53)                    # < 2^64: exact in uint64
        p1 = x2 * np.uint64(0xCD9E8D57)
        hi0, lo0 = p0 >> np.uint64(32), p0 & _U32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _U32
        x0, x1, x2, x3 = hi1 ^ x1 ^ np.uint64(k0), lo1, hi0 ^ x3 ^ np.uint64(k1), lo0
        k0 = (k0 + 0x9E3779B9) & 0xFFFFFFFF
        k1 = (k1 + 0xBB67AE85) & 0xFFFFFFFF
    return np.stack([x0, x1, x2, x3], axis=1)


def normal_stream(elems, seed):
    """Standard normal number e of the stream of `seed`, for each e in
    `elems` (fp64).  Block b = e // 4 is the Philox counter (b mod 2^32,
    b // 2^32, 0, 0) under the key (seed mod 2^32, seed // 2^32); each output
    word x becomes the uniform (floor(x / 2^9) + 1/2) / 2^23 in (0, 1); the
    pairs (u0, u1) and (u2, u3) go through Box and Muller's transform,
    r = sqrt(-2 ln u_a), (r cos 2 pi u_b, r sin 2 pi u_b); element 4b + j takes
    output j of its block."""
    e = np.asarray(elems, dtype=np.int64).reshape(-1)
    b = (e // 4).astype(np.uint64)
    ctr = np.zeros((e.size, 4), dtype=np.uint64)
    ctr[:, 0] = b & _U32
    ctr[:, 1] = b >> np.uint64(32)
    x = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    u = ((x >> np.uint64(9)).astype(np.float64) + 0.5) / 2.0 ** 23
    j = e % 4
    a = np.where(j < 2, u[:, 0], u[:, 2])                  # radius uniform of the pair
    t = np.where(j < 2, u[:, 1], u[:, 3])                  # angle uniform of the pair
    r = np.sqrt(-2.0 * np.log(a))
    return np.where(j % 2 == 0, r * np.cos(2.0 * np.pi * t), r * np.sin(2.0 * np.pi * t))


def init_std(cfg: Config):
    """Per tensor of param_specs: the standard deviation of its normal init,
    or None with the constant it starts at.  Weights and embeddings 0.02; the
    two c_proj weights of a block (the projections back into the residual
    stream) 0.02 / sqrt(2 n_layer); biases and LayerNorm shifts 0; LayerNorm
    gains 1."""
    out = []
    for name, shape in param_specs(cfg):
        if len(shape) == 2:
            resid = name.endswith("c_proj.weight")
            out.append((0.02 / math.sqrt(2 * cfg.n_layer) if resid else 0.02, None))
        else:
            out.append((None, 1.0 if name.endswith("ln_1.weight") or name.endswith("ln_2.weight")
                        or name == "ln_f.weight" else 0.0))
    return out


def init_params(cfg: Config, seed, elems=None):
    """The seeded initial parameter vector (fp64), or only its elements at the
    flat indices `elems`: element e of a normal tensor is std * normal number e
    of the seed's stream (e counts over the whole canonical vector)."""
    n = num_params(cfg)
    idx = np.arange(n) if elems is None else np.asarray(elems, dtype=np.int64)
    out = np.empty(idx.size)
    off = 0
    for (name, shape), (std, const) in zip(param_specs(cfg), init_std(cfg)):
        cnt = int(np.prod(shape))
        sel = (idx >= off) & (idx < off + cnt)
        if std is None:
            out[sel] = const
        else:
            out[sel] = std * normal_stream(idx[sel], seed)
        off += cnt
    return out


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------

def layernorm_fwd(x, w, b, eps=1e-5):
    """y = (x - mean) / sqrt(var + eps) * w + b over the last axis (R2)."""
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = xc * rstd
    return xhat * w + b, xhat, rstd


def layernorm_bwd(dy, xhat, rstd, w):
    """Chain rule of layernorm_fwd: returns dx, dw, db."""
    C = xhat.shape[-1]
    dxhat = dy * w
    mean_d = dxhat.sum(axis=-1, keepdims=True) / C
    mean_dx = (dxhat * xhat).sum(axis=-1, keepdims=True) / C
    dx = rstd * (dxhat - mean_d - xhat * mean_dx)
    red = tuple(range(dy.ndim - 1))
    return dx, (dy * xhat).sum(axis=red), dy.sum(axis=red)


_GELU_A = math.sqrt(2.0 / math.pi)
_GELU_C = 0.044715


def gelu_tanh(x):
    """R1: the tanh approximation of GELU ("The MLP and GPT-2's GELU")."""
    return 0.5 * x * (1.0 + np.tanh(_GELU_A * (x + _GELU_C * x ** 3)))


def gelu_tanh_grad(x):
    """d/dx of gelu_tanh."""
    th = np.tanh(_GELU_A * (x + _GELU_C * x ** 3))
    return 0.5 * (1.0 + th) + 0.5 * x * (1.0 - th * th) * _GELU_A * (1.0 + 3.0 * _GELU_C * x * x)


def softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# rounding of operands: exact (the reference), or bf16 where the bf16
# placement reading puts it (used only to size the rounding noise a bf16
# computation carries)
# ----------------------------------------------------------------------------

def exact(x):
    """No rounding: the reference computation."""
    return x


def bf16_round(x):
    """fp32 -> bf16 -> fp32, round to nearest, ties to even, NaN kept NaN:
    the conversion autocast applies to matrix-product operands ("Let's
    reproduce GPT-2 (124M)", the bf16 autocast step)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out)


# ----------------------------------------------------------------------------
# causal self-attention ("CausalSelfAttention")
# ----------------------------------------------------------------------------

def causal_attention_fwd(q, k, v, rnd=exact):
    """q, k, v: (B, H, T, hd).  S = q k^T / sqrt(hd), entries j > i set to
    -inf, P = row softmax, O = P v.  Also returns the row log-sum-exp of the
    masked, scaled scores so that the backward pass can rebuild P.  rnd
    rounds the probabilities as the operand of the product with v."""
    B, H, T, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    O = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=q.dtype)
    for b in range(B):                         # one batch row at a time bounds memory
        s = np.matmul(q[b], np.swapaxes(k[b], -1, -2)) * q.dtype.type(scale)
        s[:, mask] = -np.inf
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=-1, keepdims=True)
        O[b] = np.matmul(rnd(e), v[b]) / z
        lse[b] = (m + np.log(z))[..., 0]
    return O, lse


def attention_probs(q, k):
    """The full P (B, H, T, T) for small inputs (used by the invariant tests)."""
    hd = q.shape[-1]
    T = q.shape[-2]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * q.dtype.type(1.0 / math.sqrt(hd))
    s[..., np.triu(np.ones((T, T), dtype=bool), k=1)] = -np.inf
    return softmax_rows(s)


def causal_attention_bwd(dO, q, k, v, lse, rnd=exact, O=None):
    """Gradients of O = softmax(mask(q k^T/sqrt(hd))) v with P rebuilt from
    the saved log-sum-exp: dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dP P)),
    dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd).  rnd rounds P and dS as
    product operands.  Given the (stored) output O, the row term is formed as
    rowsum(dO O) instead, the same number in exact arithmetic
    (rowsum(dP P) = dO . (P V))."""
    B, H, T, hd = q.shape
    scale = q.dtype.type(1.0 / math.sqrt(hd))
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        s = np.matmul(q[b], np.swapaxes(k[b], -1, -2)) * scale
        s[:, mask] = -np.inf
        P = np.exp(s - lse[b][..., None])
        dv[b] = np.matmul(np.swapaxes(rnd(P), -1, -2), dO[b])
        dP = np.matmul(dO[b], np.swapaxes(v[b], -1, -2))
        if O is None:
            D = (dP * P).sum(axis=-1, keepdims=True)
        else:
            D = (dO[b] * O[b]).sum(axis=-1, keepdims=True)
        dS = rnd(P * (dP - D))
        dq[b] = np.matmul(dS, k[b]) * scale
        dk[b] = np.matmul(np.swapaxes(dS, -1, -2), q[b]) * scale
    return dq, dk, dv


# ----------------------------------------------------------------------------
# cross-entropy with ignore_index = -1 (R3, R4)
# ----------------------------------------------------------------------------

def cross_entropy(logits, targets):
    """logits (N, Vp), targets (N,) with -1 = ignored.  Returns the mean loss
    over valid rows, d(loss)/d(logits), the per-row losses and n_valid."""
    valid = targets != -1
    n_valid = int(valid.sum())
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    rows = np.nonzero(valid)[0]
    row_loss = np.zeros(logits.shape[0], dtype=logits.dtype)
    row_loss[rows] = lse[rows] - logits[rows, targets[rows]]
    dlogits = e                                # reuse the buffer: softmax in place
    dlogits /= z
    dlogits[rows, targets[rows]] -= 1.0
    dlogits[~valid] = 0.0
    if n_valid == 0:
        return logits.dtype.type(0.0), np.zeros_like(logits), row_loss, 0
    dlogits /= logits.dtype.type(n_valid)
    loss = row_loss.sum(dtype=np.float64) / n_valid
    return logits.dtype.type(loss), dlogits, row_loss, n_valid


# ----------------------------------------------------------------------------
# the model ("The full model", "The Block: pre-LN and residuals")
# ----------------------------------------------------------------------------

def forward(flat_params, idx, targets, cfg: Config, keep_logits=False, rnd=exact):
    """Returns (loss, cache).  idx and targets are (B, T) integer arrays;
    targets may be None (then loss is None and logits are kept).

    rnd (default: exact) is applied to every matrix-product operand and to
    the activations a mixed-precision step keeps in bf16 (LayerNorm outputs,
    qkv, attention output, GELU output and derivative, logits and their
    gradient, the gradients flowing into products); bf16_round gives the bf16
    placement of reading R8 -- a model of that computation's rounding noise,
    not a reference.  The backward pass applies the same rnd."""
    P = unflatten(flat_params, cfg)
    r = rnd
    dt = flat_params.dtype
    B, T = idx.shape
    assert T <= cfg.block_size
    C, H = cfg.n_embd, cfg.n_head
    hd = C // H
    x = P["wte"][idx] + P["wpe"][np.arange(T)]
    cache = {"idx": idx, "targets": targets, "layers": [], "B": B, "T": T, "rnd": rnd}
    for l in range(cfg.n_layer):
        p = f"h.{l}."
        lc = {"x_in": x}
        u, lc["xhat1"], lc["rstd1"] = layernorm_fwd(x, P[p + "ln_1.weight"], P[p + "ln_1.bias"])
        u = r(u)
        lc["u1"] = u
        qkv = r(u @ r(P[p + "attn.c_attn.weight"]).T + P[p + "attn.c_attn.bias"])
        q, k, v = (qkv[..., i * C:(i + 1) * C].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
                   for i in range(3))
        O, lse = causal_attention_fwd(np.ascontiguousarray(q), np.ascontiguousarray(k),
                                      np.ascontiguousarray(v), rnd=r)
        y = r(O.transpose(0, 2, 1, 3).reshape(B, T, C))
        lc.update(q=q, k=k, v=v, lse=lse, y=y, qkv=qkv)
        x = x + (y @ r(P[p + "attn.c_proj.weight"]).T + P[p + "attn.c_proj.bias"])
        lc["x_mid"] = x
        u2, lc["xhat2"], lc["rstd2"] = layernorm_fwd(x, P[p + "ln_2.weight"], P[p + "ln_2.bias"])
        u2 = r(u2)
        lc["u2"] = u2
        h = u2 @ r(P[p + "mlp.c_fc.weight"]).T + P[p + "mlp.c_fc.bias"]
        g = r(gelu_tanh(h))
        lc.update(h=h, g=g)
        x = x + (g @ r(P[p + "mlp.c_proj.weight"]).T + P[p + "mlp.c_proj.bias"])
        cache["layers"].append(lc)
    cache["x_final"] = x
    z, cache["xhatf"], cache["rstdf"] = layernorm_fwd(x, P["ln_f.weight"], P["ln_f.bias"])
    z = r(z)
    cache["z"] = z
    logits = r(z.reshape(B * T, C) @ r(P["wte"]).T)          # tied lm_head, no bias
    if targets is None:
        cache["logits"] = logits.reshape(B, T, -1)
        return None, cache
    loss, dlogits, row_loss, n_valid = cross_entropy(logits, targets.reshape(-1))
    cache.update(dlogits=r(dlogits), row_loss=row_loss, n_valid=n_valid)
    if keep_logits:
        cache["logits"] = logits.reshape(B, T, -1)
    return loss, cache


def backward(flat_params, cache, cfg: Config, loss_scale=1.0, grads=None):
    """Accumulates loss_scale * d(loss)/d(params) into `grads` (flat, same
    layout) and returns it.  The tied wte receives both the lm_head and the
    embedding contribution."""
    P = unflatten(flat_params, cfg)
    dt = flat_params.dtype
    r = cache["rnd"]
    if grads is None:
        grads = np.zeros_like(flat_params)
    G = unflatten(grads, cfg)
    B, T = cache["B"], cache["T"]
    C, H = cfg.n_embd, cfg.n_head
    hd = C // H
    s = dt.type(loss_scale)
    dlogits = cache["dlogits"] * s                             # (B*T, Vp)
    z = cache["z"].reshape(B * T, C)
    G["wte"] += dlogits.T @ z                                  # lm_head part of the tie
    dz = (dlogits @ r(P["wte"])).reshape(B, T, C)
    dx, dw, db = layernorm_bwd(dz, cache["xhatf"], cache["rstdf"], P["ln_f.weight"])
    G["ln_f.weight"] += dw
    G["ln_f.bias"] += db
    for l in reversed(range(cfg.n_layer)):
        p = f"h.{l}."
        lc = cache["layers"][l]
        # x_out = x_mid + c_proj(gelu(c_fc(ln_2(x_mid))))
        W2 = P[p + "mlp.c_proj.weight"]
        dxr = r(dx)
        G[p + "mlp.c_proj.weight"] += dxr.reshape(-1, C).T @ lc["g"].reshape(-1, 4 * C)
        G[p + "mlp.c_proj.bias"] += dx.sum(axis=(0, 1))
        dg = dxr @ r(W2)
        dh = dg * r(gelu_tanh_grad(lc["h"]))
        G[p + "mlp.c_fc.bias"] += dh.sum(axis=(0, 1))
        dh = r(dh)
        G[p + "mlp.c_fc.weight"] += dh.reshape(-1, 4 * C).T @ lc["u2"].reshape(-1, C)
        du2 = dh @ r(P[p + "mlp.c_fc.weight"])
        d, dw, db = layernorm_bwd(du2, lc["xhat2"], lc["rstd2"], P[p + "ln_2.weight"])
        G[p + "ln_2.weight"] += dw
        G[p + "ln_2.bias"] += db
        dx = dx + d
        # x_mid = x_in + c_proj(attn(ln_1(x_in)))
        dxr = r(dx)
        G[p + "attn.c_proj.weight"] += dxr.reshape(-1, C).T @ lc["y"].reshape(-1, C)
        G[p + "attn.c_proj.bias"] += dx.sum(axis=(0, 1))
        dy = r(dxr @ r(P[p + "attn.c_proj.weight"])).reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        # with rounding, the row term of the softmax backward comes from the
        # stored (rounded) output, as a computation that keeps only that has it
        y_heads = None if r is exact else np.ascontiguousarray(
            lc["y"].reshape(B, T, H, hd).transpose(0, 2, 1, 3))
        dq, dk, dv = causal_attention_bwd(np.ascontiguousarray(dy), lc["q"], lc["k"], lc["v"],
                                          lc["lse"], rnd=r, O=y_heads)
        dqkv = np.concatenate([a.transpose(0, 2, 1, 3).reshape(B, T, C) for a in (dq, dk, dv)],
                              axis=-1)
        G[p + "attn.c_attn.bias"] += dqkv.sum(axis=(0, 1))
        dqkv = r(dqkv)
        G[p + "attn.c_attn.weight"] += dqkv.reshape(-1, 3 * C).T @ lc["u1"].reshape(-1, C)
        du = dqkv @ r(P[p + "attn.c_attn.weight"])
        d, dw, db = layernorm_bwd(du, lc["xhat1"], lc["rstd1"], P[p + "ln_1.weight"])
        G[p + "ln_1.weight"] += dw
        G[p + "ln_1.bias"] += db
        dx = dx + d
    # x = wte[idx] + wpe[0:T]
    np.add.at(G["wte"], cache["idx"].reshape(-1), dx.reshape(-1, C))
    G["wpe"][:T] += dx.sum(axis=0)
    return grads


# ----------------------------------------------------------------------------
# optimizer ("Gradient clipping", "AdamW, ...", "Warmup and cosine decay")
# ----------------------------------------------------------------------------

def grad_norm(grads):
    """Global L2 norm over every parameter, the tied tensor counted once."""
    return float(np.sqrt(np.sum(grads.astype(np.float64) ** 2)))


def clip_coefficient(norm, max_norm):
    """R5."""
    return min(1.0, max_norm / (norm + 1e-6))


def adamw_update(params, grads, m, v, t, lr, beta1, beta2, eps, weight_decay, decay):
    """One AdamW step in place (R6).  `decay` is the per-element 0/1 mask of
    decayed tensors, `t` the 1-based step count.  grads must already be
    clipped."""
    dt = params.dtype.type
    params *= (1.0 - dt(lr) * dt(weight_decay) * decay).astype(params.dtype)
    m *= dt(beta1)
    m += dt(1.0 - beta1) * grads
    v *= dt(beta2)
    v += dt(1.0 - beta2) * grads * grads
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    params -= dt(lr / bc1) * m / (np.sqrt(v) / dt(math.sqrt(bc2)) + dt(eps))
    return params, m, v


def clip_and_adamw(params, grads, m, v, t, lr, beta1=0.9, beta2=0.95, eps=1e-8,
                   weight_decay=0.1, max_norm=1.0, decay=None, cfg=None):
    """Global-norm clip then AdamW; returns the pre-clip norm.  `grads` is
    scaled in place by the clip coefficient."""
    if decay is None:
        decay = decay_mask(cfg, params.dtype)
    norm = grad_norm(grads)
    c = clip_coefficient(norm, max_norm)
    grads *= grads.dtype.type(c)
    adamw_update(params, grads, m, v, t, lr, beta1, beta2, eps, weight_decay, decay)
    return norm


def sequence_losses(row_loss, targets):
    """Mean loss of each sequence over its positions with a target ("GPT-2
    from Scratch", Measuring held-out loss; the per-candidate score of a
    multiple-choice evaluation in "Build-GPT-2", Evaluation): row_loss and
    targets are (B, T); positions with target -1 carry no loss and are not
    counted.  A sequence with no target scores 0."""
    row_loss = np.asarray(row_loss, dtype=np.float64).reshape(targets.shape)
    valid = np.asarray(targets) != -1
    out = np.zeros(targets.shape[0])
    for b in range(targets.shape[0]):
        n = int(valid[b].sum())
        out[b] = row_loss[b][valid[b]].sum() / n if n else 0.0
    return out


def last_logits(flat_params, idx, cfg: Config):
    """Logits of the last position of each sequence, (B, Vp) ("GPT-2 from
    Scratch", The full model: without targets only the last position goes
    through the lm_head)."""
    _, cache = forward(flat_params, idx, None, cfg)
    return cache["logits"][:, -1, :]


def sample_next(logits, temperature, top_k, u):
    """One draw per row (R7).  logits (B, V), u (B,) uniforms in [0, 1);
    top_k None or <= 0 keeps everything.  Returns int64 tokens (B,)."""
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    B, V = x.shape
    if top_k is not None and top_k > 0:
        k = min(int(top_k), V)
        kth = np.sort(x, axis=1)[:, V - k][:, None]        # k-th largest per row
        x = np.where(x < kth, -np.inf, x)
    p = np.exp(x - x.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    cdf = np.cumsum(p, axis=1)
    out = np.empty(B, dtype=np.int64)
    for b in range(B):
        i = int(np.searchsorted(cdf[b], u[b], side="right"))   # first cdf > u
        if i >= V:
            i = int(np.nonzero(p[b] > 0)[0][-1])
        out[b] = i
    return out


def generate(flat_params, idx, n_new, temperature, top_k, uniforms, cfg: Config):
    """The pages' sampling loop (R7): n_new times, crop the running sequences
    to their last block_size tokens, take the last position's logits, draw
    with uniforms[:, step], append.  idx (B, T0); returns (B, T0 + n_new)."""
    seq = np.asarray(idx, dtype=np.int64).copy()
    for s in range(n_new):
        ctx = seq[:, -cfg.block_size:]
        nxt = sample_next(last_logits(flat_params, ctx, cfg), temperature, top_k, uniforms[:, s])
        seq = np.concatenate([seq, nxt[:, None]], axis=1)
    return seq


def lr_at(t, eta_max, eta_min, t_w, t_max):
    """Learning rate of optimizer step t (0-based) ("GPT-2 from Scratch",
    Warmup and cosine decay).  Three phases:
      ramp    t < t_w:           a straight line from zero, eta_max (t+1)/t_w,
                                 so the last ramp step reaches eta_max;
      cosine  t_w <= t <= t_max: eta_min + (eta_max - eta_min) (1 + cos(pi s))/2
                                 with s = (t - t_w)/(t_max - t_w) going from 0 to 1
                                 (eta_max at t_w, eta_min at t_max, their mean
                                 halfway); s = 0 when t_max = t_w;
      floor   t > t_max:         eta_min."""
    if t < t_w:
        return eta_max * (t + 1) / t_w
    if t <= t_max:
        span = t_max - t_w
        s = (t - t_w) / span if span > 0 else 0.0
        return eta_min + (eta_max - eta_min) * (1.0 + math.cos(math.pi * s)) / 2.0
    return eta_min


def train_step(params, m, v, t, micro_batches, cfg, lr, beta1=0.9, beta2=0.95, eps=1e-8,
               weight_decay=0.1, max_norm=1.0):
    """One optimizer step over a list of (idx, targets) micro-batches with the
    loss of each divided by their count ("How to scale up").  Updates params,
    m, v in place; returns (mean loss, pre-clip norm, grads)."""
    k = len(micro_batches)
    grads = np.zeros_like(params)
    losses = []
    for idx, tgt in micro_batches:
        loss, cache = forward(params, idx, tgt, cfg)
        backward(params, cache, cfg, loss_scale=1.0 / k, grads=grads)
        losses.append(float(loss))
    norm = clip_and_adamw(params, grads, m, v, t, lr, beta1, beta2, eps, weight_decay,
                          max_norm, cfg=cfg)
    return sum(losses) / k, norm, grads
