"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the training step.  It only draws the
random numbers a run starts from: token ids and targets, and the initial
parameter vector (the random draws of the initialization recipe, passed to
both the oracle and the HIP library as data).

Recipes (sources by page title and section):

* Model shapes: "GPT-2 from Scratch", "The config" (124M: L=12, H=12, C=768,
  block 1024; XL: L=48, H=25, C=1600); vocabulary 50,257 padded to 50,304
  ("Let's reproduce GPT-2 (124M)", FlashAttention and vocabulary padding;
  "Pretraining and fine-tuning nanoGPT-124M", Architecture).
* Initial parameters: "GPT-2 from Scratch", "Initialization": every weight and
  embedding N(0, 0.02), both c_proj weights N(0, 0.02/sqrt(2 L)), biases 0;
  LayerNorm gain 1 and shift 0 (torch's LayerNorm default, which the page's
  nn.LayerNorm uses).
* Pretraining tokens stand in for the pages' FineWeb-Edu shards (no dataset
  is available): ids drawn from a truncated Zipf law, P(id = r - 1) ~ r^-1.1
  for ranks r = 1..50257, with each position independently replaced by the
  end-of-text id 50256 with probability 1/600 (document separators, about one
  per 600 tokens).  A row of T+1 ids gives idx = row[:T], targets = row[1:]
  ("GPT-2 from Scratch", "The data loader with the shift-by-one").
* Fine-tuning rows stand in for the Alpaca pairs: a prompt of uniform length
  32..256, a response of uniform length 64..512, the end-of-text id, then
  end-of-text padding; targets are -1 except where the next token is a
  response token or the closing end-of-text ("Pretraining and fine-tuning
  nanoGPT-124M", Supervised fine-tuning, loss masking).
* Sampling inputs ("GPT-2 from Scratch", A generation loop): the uniforms a
  multinomial draw consumes, U[0, 1) per row and step; stand-alone logit rows
  N(0, scale), optionally rounded to a coarse grid so that many entries tie
  (top-k thresholds with ties).
"""
from __future__ import annotations

import numpy as np

EOT = 50256

# name -> (n_layer, n_head, n_embd, vocab_size, padded_vocab_size, block_size)
MODELS = {
    "tiny": (2, 4, 128, 512, 512, 64),
    "gpt2-124m": (12, 12, 768, 50257, 50304, 1024),
    "gpt2-xl": (48, 25, 1600, 50257, 50304, 1024),
}


def model_dims(name):
    n_layer, n_head, n_embd, V, Vp, block = MODELS[name]
    return dict(n_layer=n_layer, n_head=n_head, n_embd=n_embd, vocab_size=V,
                padded_vocab_size=Vp, block_size=block)


def _layout(d):
    """(shape, kind) per tensor in the canonical order; kind is one of
    'w' (N(0,0.02)), 'wr' (residual projection), 'b' (zeros), 'g' (ones)."""
    C, Vp, L = d["n_embd"], d["padded_vocab_size"], d["n_layer"]
    out = [((Vp, C), "w"), ((d["block_size"], C), "w")]
    for _ in range(L):
        out += [((C,), "g"), ((C,), "b"),
                ((3 * C, C), "w"), ((3 * C,), "b"),
                ((C, C), "wr"), ((C,), "b"),
                ((C,), "g"), ((C,), "b"),
                ((4 * C, C), "w"), ((4 * C,), "b"),
                ((C, 4 * C), "wr"), ((C,), "b")]
    out += [((C,), "g"), ((C,), "b")]
    return out


def init_params(d, seed=42, dtype=np.float32):
    """Flat initial parameter vector in the canonical order."""
    rng = np.random.default_rng(seed)
    std_r = 0.02 / np.sqrt(2.0 * d["n_layer"])
    parts = []
    for shape, kind in _layout(d):
        n = int(np.prod(shape))
        if kind == "w":
            parts.append(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
        elif kind == "wr":
            parts.append(rng.standard_normal(n, dtype=np.float32) * np.float32(std_r))
        elif kind == "b":
            parts.append(np.zeros(n, np.float32))
        else:
            parts.append(np.ones(n, np.float32))
    return np.concatenate(parts).astype(dtype, copy=False)


def perturb_vectors(d, flat, seed, scale=0.1):
    """A copy of flat with every LayerNorm gain at 1 + scale N(0,1) and every
    bias (LayerNorm and linear) at scale N(0,1), in place of the init's ones
    and zeros: parameters a trained model could hold, on which a wrong use of
    a gain or a bias shows from the first step."""
    rng = np.random.default_rng(seed)
    out = np.array(flat, copy=True)
    off = 0
    for shape, kind in _layout(d):
        n = int(np.prod(shape))
        if kind == "g":
            out[off:off + n] = 1.0 + scale * rng.standard_normal(n)
        elif kind == "b":
            out[off:off + n] = scale * rng.standard_normal(n)
        off += n
    assert off == out.size
    return out


def uniform_batch(B, T, vocab, seed):
    """ids uniform in [0, vocab); returns (idx, targets) int64 (B, T)."""
    rng = np.random.default_rng(seed)
    row = rng.integers(0, vocab, size=(B, T + 1), dtype=np.int64)
    return row[:, :T].copy(), row[:, 1:].copy()


_zipf_cdf_cache = {}


def _zipf_cdf(n, s):
    key = (n, s)
    if key not in _zipf_cdf_cache:
        w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(w)
        _zipf_cdf_cache[key] = c / c[-1]
    return _zipf_cdf_cache[key]


def zipf_ids(shape, seed, vocab=50257, s=1.1, sep_id=EOT, sep_p=1.0 / 600.0):
    rng = np.random.default_rng(seed)
    u = rng.random(shape)
    ids = np.searchsorted(_zipf_cdf(vocab, s), u, side="right").astype(np.int64)
    ids = np.minimum(ids, vocab - 1)
    sep = rng.random(shape) < sep_p
    ids[sep] = sep_id
    return ids


def zipf_batch(B, T, seed, vocab=50257):
    row = zipf_ids((B, T + 1), seed, vocab=vocab)
    return row[:, :T].copy(), row[:, 1:].copy()


def sft_batch(B, T, seed, vocab=50257):
    """Masked fine-tuning rows; returns (idx, targets) with -1 on ignored."""
    rng = np.random.default_rng(seed)
    idx = np.empty((B, T), np.int64)
    tgt = np.empty((B, T), np.int64)
    for b in range(B):
        lp = int(rng.integers(32, 257))
        lr = int(rng.integers(64, 513))
        stream = np.full(T + 1, EOT, np.int64)
        body = zipf_ids(lp + lr, int(rng.integers(0, 2 ** 31)), vocab=vocab, sep_p=0.0)
        n = min(lp + lr, T + 1)
        stream[:n] = body[:n]
        if lp + lr < T + 1:
            stream[lp + lr] = EOT
        idx[b] = stream[:T]
        t = np.arange(T)
        keep = (t + 1 >= lp) & (t + 1 <= lp + lr)
        tgt[b] = np.where(keep, stream[1:], -1)
    return idx, tgt


def config_batch(config, B, T, seed):
    """The token batch of a named workload."""
    if config == "tiny":
        return uniform_batch(B, T, 512, seed)
    if config == "sft":
        return sft_batch(B, T, seed)
    return zipf_batch(B, T, seed)


def uniforms(shape, seed):
    """U[0, 1) draws, float32 (the random numbers the sampling step uses)."""
    return np.random.default_rng(seed).random(shape).astype(np.float32)


def logit_rows(B, V, seed, scale=2.0, grid=None):
    """(B, V) float32 logits, N(0, scale); with `grid`, rounded to multiples
    of it (ties)."""
    x = np.random.default_rng(seed).normal(0.0, scale, size=(B, V))
    if grid:
        x = np.round(x / grid) * grid
    return x.astype(np.float32)
