"""Comparison of a bf16 GPU training step with the fp32 oracle's step.

Everything that decides which elements are compared, and how strictly, comes
from the oracle's side: the GPU output under test enters only as the thing
being measured.  Two oracle runs serve: the exact step (the reference, g_ref)
and the same step with every product operand and every bf16-stored
activation rounded to bf16 (the oracle's rnd=bf16_round, the bf16 placement
reading; g_emul).  Their difference is the rounding noise a bf16 step
carries, row by row: rows whose gradient cancels to a small norm keep the
noise of the terms they sum, so their relative error is large in any bf16
computation -- most of all the value rows of c_attn.weight.

Gradients.  Per tensor, normwise within TOL_GRAD.  Per output row of every
matrix, the GPU's error may be F_ROW times the row's noise scale -- the
rounded oracle's error in that row, or the median of those errors over the
row's group (the q, k and v thirds of c_attn.weight, else the matrix), the
larger -- plus ROW_SLACK of the tensor's median row norm.  The GPU's and the
rounded oracle's errors are independent draws of rounding noise of the same
size -- over the rows their ratio has a median of 0.9 to 1.1 on the GPT-2
124M steps -- but some rows carry essentially one random number: the key
rows, for instance, since sum_j dK_j = 0 exactly, err by (the rounding left
in that sum) x (the part all positions' LayerNorm outputs share).  Two such
draws can differ by any factor, so a single row of the rounded oracle is not
a bound; the group median is.  One wrong row -- a rare token's wte row, say,
whose error is of the order of its norm -- still fails on its own even when
its tensor's overall error is small.

Parameters after AdamW step t = 1.  Adam's first step is lr * g / (|g| + eps),
i.e. lr * sign(g) for every |g| >> eps: elements whose gradient sign agrees
move identically, and an element whose sign flips differs by 2 lr.  A sign is
fixed by a bf16 computation only where |g| clearly exceeds the rounding
noise, so the elements compared are those with |g_ref| above K_FLOOR times
the rms over the element's row of g_emul - g_ref.  Over those, parameters
agree within TOL_PARAM normwise per tensor; the elements below the floor may
differ by at most 2 lr, and may be at most MAX_BELOW of all elements.  How
many fall there depends on the parameters: once the LayerNorm and key biases
give all keys of a head a large common part, the query and key rows of
c_attn.weight carry the rounding noise of two sums that are exactly zero
(each row of dS sums to zero, and so do the key gradients over positions)
times that common part, above most of their exact gradient.  In a 124M step
at B=2, T=1024 with gains and biases drawn around the init's ones and zeros
(0.1 N(0,1) off them) 70-90% of those rows' elements fall under the floor,
11% of all elements; with the init's own ones and zeros, 5%.

Parameters after a step t >= 2 taken from the same state on both sides
(the GPU's parameters and moments copied into the oracle): the previous
moments dominate the update of elements with small gradients, so every
element is compared, TOL_PARAM normwise per tensor, and m and v within
TOL_MOM -- or, where the rounded oracle's own step (its gradient through the
same clip and AdamW from the same state) already deviates by more, within
F_STEP times that deviation.  This matters for tensors that sit near zero
(biases one step after their zero init, whose norm is the size of one
update) and for the query rows of late blocks once the keys share a large
common part: the softmax-backward row term rowsum(dO O) is formed from the
bf16-stored output, and its rounding reaches dQ multiplied by the mean key.

The key third of c_attn.bias has an analytically zero gradient (softmax is
invariant to a per-row shift), so its computed value is rounding noise and
its update is arbitrary: it is left out of every comparison.

The rows of c_attn.weight are sums over positions t of d(q|k|v)[t, row] times
the block's ln_1 output u1[t].  Write u1[t] as its sequence's mean plus the
rest: the part of a row along the sequence means collects, per sequence, the
plain sum of the row's bf16-rounded d(q|k|v) entries -- for the key rows that
sum is exactly zero in exact arithmetic (sum_j dK_j = 0 for every query,
since every row of dS sums to zero), so what a bf16 computation puts there is
rounding noise alone, one random number per row and sequence.  Given the
sequences' means (seq_means, from the exact oracle run), each row is split
into that span and the rest: the rest is compared row by row as above, and
the span part normwise over each third, within F_SPAN times the rounded
oracle's.  On the CPU (stochastic rounding against round-to-nearest on a
GPT-2 124M step) this brings the largest per-row ratio to the group median
from 17.7 down to 3.8.
"""
from __future__ import annotations

import numpy as np

TOL_GRAD = 1.2e-2     # per-tensor normwise gradient error
F_ROW = 12.0          # per-row error: this times the rounded oracle's error in the row ...
ROW_SLACK = 2e-2      # ... plus this times the tensor's median row norm
F_STEP = 6.0          # t >= 2: parameters and moments within this times the rounded oracle's error
K_FLOOR = 8.0         # compared parameters at t = 1: |g_ref| above this times the row's noise rms
TOL_PARAM = 5e-3      # per-tensor normwise parameter error
MAX_BELOW = 0.15      # largest fraction of elements under the floor at t = 1
TOL_MOM = 2e-2        # per-tensor normwise error of m and v at t >= 2
TOL_NORM = 2e-2       # relative error of the pre-clip gradient norm
TOL_ADAMW = 1e-5      # the GPU's own gradients through the oracle's AdamW
F_SPAN = 4.0          # c_attn.weight rows' part along the sequence means, per third


def seq_means(cache):
    """Per block, the per-sequence means of the ln_1 output of an oracle
    forward cache: {block: (B, C)}."""
    out = {}
    for l, lc in enumerate(cache["layers"]):
        u = np.asarray(lc["u1"], np.float64)
        out[l] = u.reshape(cache["B"], cache["T"], -1).mean(axis=1)
    return out


def merge_seq_means(parts):
    """seq_means of several micro-batches, stacked per block."""
    return {l: np.concatenate([p[l] for p in parts]) for l in parts[0]}


def tensor_slices(O, cfg):
    """(name, shape, slice, keep) per tensor; keep masks out the key-bias third."""
    out, off = [], 0
    C = cfg.n_embd
    for name, shape in O.param_specs(cfg):
        n = int(np.prod(shape))
        keep = np.ones(n, bool)
        if name.endswith("attn.c_attn.bias"):
            keep[C:2 * C] = False
        out.append((name, shape, slice(off, off + n), keep))
        off += n
    return out


def _rows(shape):
    return shape[0] if len(shape) == 2 else 1


def _normwise(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def compare_step(O, cfg, *, p0, g_gpu, g_ref, g_emul, p_gpu, p_ref, norm_gpu, norm_ref, lr, wd,
                 t, m0=None, v0=None, m_gpu=None, m_ref=None, v_gpu=None, v_ref=None,
                 beta1=0.9, beta2=0.95, eps=1e-8, clip=1.0, seq_means=None, verbose=True):
    """Compares one bf16 step; returns (failures, stats).  p0, m0, v0: the
    state both sides started the step from (m0, v0 None: zeros, t = 1);
    g_emul: the oracle's gradient of the same step with bf16 rounding;
    seq_means: {block: (sequences, C)} from the exact oracle run (seq_means()),
    or None to compare the c_attn.weight rows whole."""
    fails, stats = [], {}
    if abs(norm_gpu - norm_ref) > TOL_NORM * norm_ref:
        fails.append(f"pre-clip norm {norm_gpu} vs {norm_ref}")
    stats["norm_rel"] = abs(norm_gpu - norm_ref) / norm_ref
    # the GPU's own gradients through the oracle's clip and AdamW
    p_own = p0.astype(np.float32).copy()
    m_own = np.zeros_like(p_own) if m0 is None else m0.astype(np.float32).copy()
    v_own = np.zeros_like(p_own) if v0 is None else v0.astype(np.float32).copy()
    O.clip_and_adamw(p_own, g_gpu.astype(np.float32).copy(), m_own, v_own, t, lr, beta1, beta2,
                     eps, wd, clip, cfg=cfg)
    if m0 is not None:
        # the rounded oracle's gradient through the same clip and AdamW
        p_em = p0.astype(np.float32).copy()
        m_em, v_em = m0.astype(np.float32).copy(), v0.astype(np.float32).copy()
        O.clip_and_adamw(p_em, g_emul.astype(np.float32).copy(), m_em, v_em, t, lr, beta1, beta2,
                         eps, wd, clip, cfg=cfg)
    worst = dict(grad=0.0, grad_emul=0.0, row=0.0, param=0.0, adamw=0.0, mom=0.0)
    where = {}
    row_info = {}
    below = total = 0
    for name, shape, sl, keep in tensor_slices(O, cfg):
        ga, gr = g_gpu[sl].astype(np.float64), g_ref[sl].astype(np.float64)
        ge = g_emul[sl].astype(np.float64)
        pa, pr = p_gpu[sl].astype(np.float64), p_ref[sl].astype(np.float64)
        po = p_own[sl].astype(np.float64)
        eg = _normwise(ga[keep], gr[keep])
        ee = _normwise(ge[keep], gr[keep])
        eo = float(np.max(np.abs(pa[keep] - po[keep])) / max(np.max(np.abs(po[keep])), 1e-30))
        rows = _rows(shape)
        er = 0.0
        if rows > 1:
            ga2, gr2, ge2 = ga.reshape(rows, -1), gr.reshape(rows, -1), ge.reshape(rows, -1)
            rn = np.linalg.norm(gr2, axis=1)
            da, de = ga2 - gr2, ge2 - gr2
            groups = 3 if name.endswith("c_attn.weight") else 1
            if groups == 3 and seq_means is not None:
                # the part along the sequence means: normwise per third
                blk = int(name.split(".")[1])
                Q, _ = np.linalg.qr(np.asarray(seq_means[blk], np.float64).T)
                for part, rs in zip("qkv", np.split(np.arange(rows), 3)):
                    sa = np.linalg.norm(da[rs] @ Q)
                    se = np.linalg.norm(de[rs] @ Q)
                    bound = F_SPAN * se + 1e-3 * np.linalg.norm(gr2[rs])
                    if sa > bound:
                        fails.append(f"{name}: {part} rows along the sequence means, error "
                                     f"{sa:.3e} > {bound:.3e} (rounded oracle {se:.3e})")
                da, de = da - (da @ Q) @ Q.T, de - (de @ Q) @ Q.T
            e_gpu = np.linalg.norm(da, axis=1)
            e_emul = np.linalg.norm(de, axis=1)
            # a row's noise scale: its own rounded error, or the median over
            # its group of rows, whichever is larger (groups: the q, k, v
            # thirds of c_attn.weight, else the whole matrix)
            typical = np.repeat([np.median(x) for x in np.split(e_emul, groups)], rows // groups)
            allowed = F_ROW * np.maximum(e_emul, typical) + ROW_SLACK * np.median(rn)
            ratio = e_gpu / np.maximum(allowed, 1e-30)
            r = int(np.argmax(ratio))
            er = float(ratio[r])
            row_info[name] = (er, r, float(e_gpu[r] / max(rn[r], 1e-30)),
                              float(e_emul[r] / max(rn[r], 1e-30)),
                              float(np.median(e_gpu / np.maximum(e_emul, 1e-30))))
            if er > 1.0:
                fails.append(f"{name}: row {r} gradient error {row_info[name][2]:.3e} of its norm "
                             f"(rounded oracle {row_info[name][3]:.3e})")
        param_bound = TOL_PARAM
        if t == 1 and m0 is None:
            noise = np.sqrt(((ge - gr).reshape(rows, -1) ** 2).mean(axis=1))
            floor = np.repeat(K_FLOOR * noise, gr.size // rows)
            det = (np.abs(gr) > floor) & keep
            und = (~det) & keep
            ep = _normwise(pa[det], pr[det]) if det.any() else 0.0
            dmax = float(np.max(np.abs(pa[und] - pr[und]), initial=0.0))
            if dmax > 2.0 * lr * 1.001 + 1e-7:
                fails.append(f"{name}: below-floor element moved {dmax:.3e} > 2 lr")
            below += int(und.sum())
        else:
            ep = _normwise(pa[keep], pr[keep])
            ep_em = _normwise(p_em[sl][keep].astype(np.float64), pr[keep])
            em = max(_normwise(m_gpu[sl][keep].astype(np.float64), m_ref[sl][keep]),
                     _normwise(v_gpu[sl][keep].astype(np.float64), v_ref[sl][keep]))
            em_em = max(_normwise(m_em[sl][keep].astype(np.float64), m_ref[sl][keep]),
                        _normwise(v_em[sl][keep].astype(np.float64), v_ref[sl][keep]))
            if em > max(TOL_MOM, F_STEP * em_em):
                fails.append(f"{name}: moments error {em:.3e} (rounded oracle {em_em:.3e})")
            worst["mom"] = max(worst["mom"], em)
            param_bound = max(TOL_PARAM, F_STEP * ep_em)
        total += int(keep.sum())
        if eg > TOL_GRAD:
            fails.append(f"{name}: gradient error {eg:.3e}")
        if ep > param_bound:
            fails.append(f"{name}: parameter error {ep:.3e} (bound {param_bound:.3e})")
        if eo > TOL_ADAMW:
            fails.append(f"{name}: AdamW on own gradients {eo:.3e}")
        for k, v in (("grad", eg), ("grad_emul", ee), ("row", er), ("param", ep), ("adamw", eo)):
            if v > worst[k]:
                worst[k], where[k] = v, name
    frac = below / max(total, 1)
    if frac > MAX_BELOW:
        fails.append(f"below-floor fraction {frac:.3e}")
    stats.update(worst=worst, where=where, below_frac=frac, rows=row_info)
    if verbose:
        print("bf16 step t=%d: norm rel %.2e; worst grad %.2e (%s; rounded oracle %.2e), "
              "row %.2f (%s), param %.2e (%s), adamw %.1e, moments %.2e; below-floor %.3e" % (
                  t, stats["norm_rel"], worst["grad"], where.get("grad"), worst["grad_emul"],
                  worst["row"], where.get("row"), worst["param"], where.get("param"),
                  worst["adamw"], worst["mom"], frac))
        top = sorted(row_info.items(), key=lambda kv: -kv[1][0])[:4]
        print("  worst rows (error / allowed, row, gpu error / norm, rounded-oracle error / norm, "
              "median gpu / rounded over rows): " +
              "; ".join(f"{k} {v[0]:.2f} r{v[1]} {v[2]:.2e} {v[3]:.2e} {v[4]:.2f}" for k, v in top))
    return fails, stats
