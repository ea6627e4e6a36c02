"""ctypes binding of libgpt2.so (include/gpt2.h, include/gpt2_ops.h).

Argument marshalling only: every step of the training step runs in the HIP
library.  torch supplies the device workspace and the stream.  The library
must have been built (``python -m decoder_only_transformer_03_amd.build``);
loading fails loudly otherwise -- there is no fallback.
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2.so")

GPT2_OK, GPT2_E_ARG, GPT2_E_SHAPE, GPT2_E_RANGE, GPT2_E_STATE, GPT2_E_HIP = 0, -1, -2, -3, -4, -5
GPT2_FP32, GPT2_BF16 = 0, 1
GPT2_PARAMS, GPT2_GRADS, GPT2_ADAM_M, GPT2_ADAM_V = 0, 1, 2, 3
SITES = ["EMBED_FWD", "LN_FWD", "QKV_FWD", "ATTN_FWD", "PROJ_FWD", "FC_FWD", "FCPROJ_FWD",
         "LMHEAD_FWD", "XENT", "LMHEAD_DX", "LMHEAD_DW", "LN_BWD", "FCPROJ_DX", "FCPROJ_DW", "FC_DX",
         "FC_DW", "PROJ_DX", "PROJ_DW", "ATTN_BWD", "QKV_DX", "QKV_DW", "BIAS_GRAD", "EMBED_BWD",
         "GRAD_NORM", "ADAMW", "ZERO_GRAD", "LMHEAD_RECOMP", "WEIGHT_T", "WGRAD",
         "WGRAD_TAIL"]
ACT = {n: i for i, n in enumerate([
    "X_IN", "LN1", "QKV", "ATTN_Y", "LSE", "X_MID", "LN2", "FC_DGELU", "FC_GELU", "LNF", "LOGITS",
    "ROW_LOSS"])}
STATUS_NAMES = {0: "GPT2_OK", -1: "GPT2_E_ARG", -2: "GPT2_E_SHAPE", -3: "GPT2_E_RANGE",
                -4: "GPT2_E_STATE", -5: "GPT2_E_HIP"}


class gpt2_config(ct.Structure):
    _fields_ = [("n_layer", ct.c_int32), ("n_head", ct.c_int32), ("n_embd", ct.c_int32),
                ("vocab_size", ct.c_int32), ("padded_vocab_size", ct.c_int32),
                ("block_size", ct.c_int32), ("max_batch", ct.c_int32), ("precision", ct.c_int32),
                ("head_chunk", ct.c_int32)]


class GPT2Error(RuntimeError):
    def __init__(self, status, msg=""):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m decoder_only_transformer_03_amd.build`")
        L = ct.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ct.c_void_p, ct.c_int, ct.c_int64, ct.c_float, ct.c_size_t
        cfgp = ct.POINTER(gpt2_config)
        sig = {
            "gpt2_num_params": (sz, [cfgp]),
            "gpt2_workspace_bytes": (i32, [cfgp, ct.POINTER(sz)]),
            "gpt2_init": (i32, [cfgp, vp, sz, vp, ct.c_uint64, ct.POINTER(vp)]),
            "gpt2_lr_at": (i32, [i64, ct.c_double, ct.c_double, i64, i64, ct.POINTER(ct.c_double)]),
            "gpt2_set_params": (i32, [vp, vp, sz, i32]),
            "gpt2_get": (i32, [vp, i32, vp, sz, i32]),
            "gpt2_set_state": (i32, [vp, i32, vp, sz, i32]),
            "gpt2_get_step": (i32, [vp, ct.POINTER(i64)]),
            "gpt2_set_step": (i32, [vp, i64]),
            "gpt2_forward": (i32, [vp, vp, vp, i32, i32, ct.POINTER(f32)]),
            "gpt2_eval": (i32, [vp, vp, vp, i32, i32, vp, ct.POINTER(f32)]),
            "gpt2_forward_last": (i32, [vp, vp, i32, i32, vp]),
            "gpt2_sample": (i32, [vp, vp, ct.c_long, i32, i32, f32, i32, vp, vp]),
            "gpt2_generate": (i32, [vp, vp, i32, i32, i32, f32, i32, vp, vp]),
            "gpt2_generate_cached": (i32, [vp, vp, i32, i32, i32, f32, i32, vp, vp]),
            "gpt2_prefill": (i32, [vp, vp, i32, i32, vp]),
            "gpt2_decode": (i32, [vp, vp, i32, i32, vp]),
            "gpt2_get_loss": (i32, [vp, ct.POINTER(f32)]),
            "gpt2_zero_grad": (i32, [vp]),
            "gpt2_backward": (i32, [vp, f32]),
            "gpt2_adamw_step": (i32, [vp, f32, f32, f32, f32, f32, f32, ct.POINTER(f32)]),
            "gpt2_get_grad_norm": (i32, [vp, ct.POINTER(f32)]),
            "gpt2_sync": (i32, [vp]),
            "gpt2_last_error": (ct.c_char_p, [vp]),
            "gpt2_destroy": (None, [vp]),
            "gpt2_get_activation": (i32, [vp, i32, i32, vp, sz]),
            "gpt2_timing_begin": (i32, [vp, ct.c_uint64]),
            "gpt2_timing_end": (i32, [vp, ct.POINTER(ct.c_double), ct.POINTER(ct.c_int32)]),
            "gpt2_wgrad_layout": (i32, [vp, ct.POINTER(i64), ct.POINTER(i64), ct.POINTER(i64)]),
            "gpt2_op_gemm": (i32, [i32, i32, i32, i32, vp, ct.c_long, i32, vp, ct.c_long, i32, vp,
                                   ct.c_long, f32, i32, i32, vp]),
            "gpt2_op_gemm_epi": (i32, [i32, i32, i32, vp, ct.c_long, vp, ct.c_long, i32, vp, vp,
                                       ct.c_long, vp, vp, ct.c_long, i32, vp]),
            "gpt2_op_attention_fwd": (i32, [i32, vp, vp, vp, i32, i32, i32, i32, vp]),
            "gpt2_op_attention_bwd": (i32, [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]),
            "gpt2_op_attention_bwd_noalloc": (i32, [i32, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                    vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


EXPORTED = ["gpt2_num_params", "gpt2_workspace_bytes", "gpt2_init", "gpt2_lr_at", "gpt2_set_params",
            "gpt2_get",
            "gpt2_set_state", "gpt2_get_step", "gpt2_set_step", "gpt2_forward", "gpt2_eval",
            "gpt2_forward_last", "gpt2_sample", "gpt2_generate", "gpt2_generate_cached",
            "gpt2_prefill", "gpt2_decode", "gpt2_get_loss",
            "gpt2_zero_grad", "gpt2_backward", "gpt2_adamw_step", "gpt2_get_grad_norm",
            "gpt2_sync", "gpt2_last_error", "gpt2_destroy", "gpt2_get_activation",
            "gpt2_timing_begin", "gpt2_timing_end", "gpt2_wgrad_layout",
            "gpt2_op_gemm", "gpt2_op_gemm_epi", "gpt2_op_attention_fwd", "gpt2_op_attention_bwd",
            "gpt2_op_attention_bwd_noalloc"]


def make_config(n_layer, n_head, n_embd, vocab_size, padded_vocab_size, block_size, max_batch,
                precision, head_chunk=0):
    """head_chunk > 0 selects the fused lm_head + cross-entropy (no logits
    tensor; the backward recomputes the logits head_chunk columns at a time)."""
    if isinstance(precision, str):
        precision = {"fp32": GPT2_FP32, "bf16": GPT2_BF16}[precision]
    return gpt2_config(n_layer, n_head, n_embd, vocab_size, padded_vocab_size, block_size,
                       max_batch, precision, head_chunk)


def gpt2_num_params(cfg: gpt2_config) -> int:
    return int(lib().gpt2_num_params(ct.byref(cfg)))


def gpt2_workspace_bytes(cfg: gpt2_config) -> int:
    n = ct.c_size_t(0)
    st = lib().gpt2_workspace_bytes(ct.byref(cfg), ct.byref(n))
    if st != GPT2_OK:
        raise GPT2Error(st, "invalid config")
    return n.value


def _ptr(x):
    """Device or host address of a torch tensor or numpy array."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    assert x.is_contiguous()
    return x.data_ptr()


class GPT2:
    """A handle plus its torch-allocated workspace and stream.

    Methods map one to one onto the C functions of the same names."""

    def __init__(self, cfg: gpt2_config, device="cuda", stream=None, seed=0):
        """seed: the parameters start from gpt2_init's seeded initialisation."""
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.n_params = gpt2_num_params(cfg)
        if self.n_params == 0:
            raise GPT2Error(GPT2_E_ARG, "invalid config")
        nbytes = gpt2_workspace_bytes(cfg)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        h = ct.c_void_p()
        st = lib().gpt2_init(ct.byref(cfg), self.workspace.data_ptr(), nbytes,
                             self.stream.cuda_stream, int(seed), ct.byref(h))
        if st != GPT2_OK:
            raise GPT2Error(st, "gpt2_init failed")
        self.h = h

    def _check(self, st):
        if st != GPT2_OK:
            msg = lib().gpt2_last_error(self.h)
            raise GPT2Error(st, msg.decode() if msg else "")

    def close(self):
        if getattr(self, "h", None):
            lib().gpt2_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # --- state -----------------------------------------------------------
    def set_params(self, flat):
        on_dev = not isinstance(flat, np.ndarray)
        if not on_dev:
            flat = np.ascontiguousarray(flat, dtype=np.float32)
        self._check(lib().gpt2_set_params(self.h, _ptr(flat), self.n_params, int(on_dev)))

    def get(self, which=GPT2_PARAMS) -> np.ndarray:
        out = np.empty(self.n_params, np.float32)
        self._check(lib().gpt2_get(self.h, which, out.ctypes.data, self.n_params, 0))
        return out

    def set_state(self, which, flat):
        flat = np.ascontiguousarray(flat, dtype=np.float32)
        self._check(lib().gpt2_set_state(self.h, which, flat.ctypes.data, self.n_params, 0))

    def get_step(self) -> int:
        t = ct.c_int64(0)
        self._check(lib().gpt2_get_step(self.h, ct.byref(t)))
        return t.value

    def set_step(self, t: int):
        self._check(lib().gpt2_set_step(self.h, int(t)))

    # --- the step ----------------------------------------------------------
    def forward(self, idx, targets=None, want_loss=False):
        """idx, targets: int32 device tensors of shape (B, T)."""
        B, T = idx.shape
        loss = ct.c_float(0.0)
        st = lib().gpt2_forward(self.h, _ptr(idx), _ptr(targets), B, T,
                                ct.byref(loss) if want_loss else None)
        self._check(st)
        return loss.value if want_loss else None

    def eval(self, idx, targets, seq_loss=None, want_loss=False):
        """Forward pass and losses only (no gradient).  idx, targets: int32
        device tensors (B, T); seq_loss: optional float32 device tensor (B,)
        that receives each sequence's mean loss over its valid targets."""
        B, T = idx.shape
        loss = ct.c_float(0.0)
        st = lib().gpt2_eval(self.h, _ptr(idx), _ptr(targets), B, T,
                             _ptr(seq_loss) if seq_loss is not None else None,
                             ct.byref(loss) if want_loss else None)
        self._check(st)
        return loss.value if want_loss else None

    # --- generation --------------------------------------------------------
    def forward_last(self, idx, logits):
        """Last-position logits of each sequence: idx int32 (B, T) device
        tensor; logits float32 (B, padded_vocab_size) device tensor."""
        B, T = idx.shape
        self._check(lib().gpt2_forward_last(self.h, _ptr(idx), B, T, _ptr(logits)))

    def sample(self, logits, uniform, tokens, temperature=1.0, top_k=0, V=None):
        """One draw per row of logits (float32 (B, ld) device tensor, first V
        columns) with the caller's uniforms (float32 (B,)) into tokens (int32
        (B,)); top_k <= 0 keeps every entry."""
        B, ld = logits.shape
        self._check(lib().gpt2_sample(self.h, _ptr(logits), ld, B, ld if V is None else V,
                                      float(temperature), int(top_k), _ptr(uniform), _ptr(tokens)))

    def generate(self, prompt, n_new, uniforms, out, temperature=1.0, top_k=0):
        """prompt int32 (B, T0); uniforms float32 (B, n_new); out int32
        (B, T0 + n_new), all device tensors."""
        B, T0 = prompt.shape
        self._check(lib().gpt2_generate(self.h, _ptr(prompt), B, T0, int(n_new), float(temperature),
                                        int(top_k), _ptr(uniforms), _ptr(out)))

    def generate_cached(self, prompt, n_new, uniforms, out, temperature=1.0, top_k=0):
        """generate with a key/value cache (same arguments and draws)."""
        B, T0 = prompt.shape
        self._check(lib().gpt2_generate_cached(self.h, _ptr(prompt), B, T0, int(n_new),
                                               float(temperature), int(top_k), _ptr(uniforms),
                                               _ptr(out)))

    def prefill(self, idx, logits):
        """idx int32 (B, T); logits float32 (B, padded vocab), device tensors:
        the prompt's keys and values kept, the logits of its last position."""
        B, T = idx.shape
        self._check(lib().gpt2_prefill(self.h, _ptr(idx), B, T, _ptr(logits)))

    def decode(self, tok, p, logits):
        """tok int32 (B,), the tokens at position p; logits as in prefill."""
        self._check(lib().gpt2_decode(self.h, _ptr(tok), tok.shape[0], int(p), _ptr(logits)))

    def get_loss(self) -> float:
        loss = ct.c_float(0.0)
        self._check(lib().gpt2_get_loss(self.h, ct.byref(loss)))
        return loss.value

    def zero_grad(self):
        self._check(lib().gpt2_zero_grad(self.h))

    def backward(self, loss_scale=1.0):
        self._check(lib().gpt2_backward(self.h, float(loss_scale)))

    def adamw_step(self, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_grad_norm=1.0,
                   want_norm=False):
        n = ct.c_float(0.0)
        self._check(lib().gpt2_adamw_step(self.h, lr, beta1, beta2, eps, weight_decay,
                                          max_grad_norm, ct.byref(n) if want_norm else None))
        return n.value if want_norm else None

    def get_grad_norm(self) -> float:
        n = ct.c_float(0.0)
        self._check(lib().gpt2_get_grad_norm(self.h, ct.byref(n)))
        return n.value

    def sync(self):
        self._check(lib().gpt2_sync(self.h))

    def timing_begin(self, sites=None):
        """Start recording event pairs around launches of the named sites (all if None)."""
        mask = (1 << len(SITES)) - 1 if sites is None else sum(1 << SITES.index(n) for n in sites)
        self._check(lib().gpt2_timing_begin(self.h, mask))

    def timing_end(self):
        """{site: (total_ms, launches)} for the sites that ran."""
        ms = (ct.c_double * len(SITES))()
        cnt = (ct.c_int32 * len(SITES))()
        self._check(lib().gpt2_timing_end(self.h, ms, cnt))
        return {n: (ms[i], cnt[i]) for i, n in enumerate(SITES) if cnt[i]}

    def wgrad_layout(self):
        """(grouped_elems, tail_elems, grouped_tiles): weight-gradient elements
        produced by the grouped launch and by the split-K tail, and the grouped
        launch's output tiles (all 0 when products run one at a time)."""
        g, t, n = ct.c_int64(0), ct.c_int64(0), ct.c_int64(0)
        self._check(lib().gpt2_wgrad_layout(self.h, ct.byref(g), ct.byref(t), ct.byref(n)))
        return g.value, t.value, n.value

    def activation(self, name, layer, count):
        out = np.empty(count, np.float32)
        self._check(lib().gpt2_get_activation(self.h, ACT[name], layer, out.ctypes.data, count))
        return out


def gpt2_lr_at(step, eta_max=6e-4, eta_min=6e-5, warmup_steps=715, max_steps=19073):
    """Learning rate of optimizer step `step` (0-based) from the library's
    schedule (linear warmup, then cosine decay to eta_min at max_steps)."""
    lr = ct.c_double(0.0)
    _st(lib().gpt2_lr_at(int(step), float(eta_max), float(eta_min), int(warmup_steps),
                         int(max_steps), ct.byref(lr)), "gpt2_lr_at")
    return lr.value


def _st(st, what):
    if st != GPT2_OK:
        raise GPT2Error(st, what)


def gpt2_op_gemm(dtype, M, N, K, A, lda, a_trans, B, ldb, b_trans, C, ldc, alpha=1.0, mode=0,
                 split_k=0, stream=None):
    _st(lib().gpt2_op_gemm(dtype, M, N, K, _ptr(A), lda, int(a_trans), _ptr(B), ldb, int(b_trans),
                           _ptr(C), ldc, alpha, mode, split_k,
                           stream.cuda_stream if stream is not None else None), "gpt2_op_gemm")


def gpt2_op_gemm_epi(M, N, K, A, lda, B, ldb, epi, bias, R, ldr, C, C2, ldc, out_dtype,
                     stream=None):
    _st(lib().gpt2_op_gemm_epi(M, N, K, _ptr(A), lda, _ptr(B), ldb, epi, _ptr(bias), _ptr(R), ldr,
                               _ptr(C), _ptr(C2), ldc, out_dtype,
                               stream.cuda_stream if stream is not None else None),
        "gpt2_op_gemm_epi")


def gpt2_op_attention_fwd(dtype, qkv, y, lse, B, T, H, hd, stream=None):
    _st(lib().gpt2_op_attention_fwd(dtype, _ptr(qkv), _ptr(y), _ptr(lse), B, T, H, hd,
                                    stream.cuda_stream if stream is not None else None),
        "gpt2_op_attention_fwd")


def gpt2_op_attention_bwd(dtype, qkv, y, lse, dy, dqkv, dbuf, B, T, H, hd, stream=None):
    _st(lib().gpt2_op_attention_bwd(dtype, _ptr(qkv), _ptr(y), _ptr(lse), _ptr(dy), _ptr(dqkv),
                                    _ptr(dbuf), B, T, H, hd,
                                    stream.cuda_stream if stream is not None else None),
        "gpt2_op_attention_bwd")


def gpt2_op_attention_bwd_noalloc(dtype, qkv, y, lse, dy, dqkv, B, T, H, hd, stream=None):
    """gpt2_op_attention_bwd with the library's fixed device scratch (no dbuf)."""
    _st(lib().gpt2_op_attention_bwd_noalloc(dtype, _ptr(qkv), _ptr(y), _ptr(lse), _ptr(dy),
                                            _ptr(dqkv), B, T, H, hd,
                                            stream.cuda_stream if stream is not None else None),
        "gpt2_op_attention_bwd_noalloc")
