"""fp64 definitions of the ops (test infrastructure; see the package docstring).

Notation: T tokens, d hidden, D head_dim, F ffn, V vocabulary, H lm-head input width.
Inputs may be numpy arrays or CPU torch tensors of any float dtype; they are widened
to float64 exactly before any arithmetic.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor: widen exactly (bf16/fp32 -> fp64)
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(a, dtype=np.int64)


# ---------------------------------------------------------------------------
# RMSNorm — [FastLLM] 三 技术架构, "Transformer Block 结构" (normalization:
# LayerNorm / RMSNorm) and 训练配置示例 (normalization type rms_norm, epsilon 1e-5);
# [LF] "当前已实现的 kernels" (npu_fused_rmsnorm); [HFK] "Liger" (fused RMSNorm).
# Reading: eps inside the root; y = x * r * w with no (1+w) offset, no bias and no
# mean subtraction.
# ---------------------------------------------------------------------------
def rmsnorm_fwd(x, w, eps):
    """y[t,j] = x[t,j] * r[t] * w[j],  r[t] = 1/sqrt(mean_j x[t,j]^2 + eps).

    Returns (y [T,d], rstd [T])."""
    x = _f64(x)
    w = _f64(w)
    ms = np.mean(x * x, axis=-1)
    rstd = 1.0 / np.sqrt(ms + eps)
    y = x * rstd[..., None] * w
    return y, rstd


def rmsnorm_bwd(dy, x, w, eps):
    """Gradients of y = rmsnorm_fwd(x, w, eps) for upstream dy.

    With g = w*dy and r as above, differentiating y_j = x_j r w_j, where
    dr/dx_k = -r^3 x_k / d, gives
        dx[t,k] = r g_k - r^3 x_k * (1/d) sum_j g_j x_j
        dw[j]   = sum_t dy[t,j] x[t,j] r[t]
    Returns (dx [T,d], dw [d])."""
    dy = _f64(dy)
    x = _f64(x)
    w = _f64(w)
    d = x.shape[-1]
    _, r = rmsnorm_fwd(x, w, eps)
    g = dy * w
    c = np.sum(g * x, axis=-1) / d
    dx = r[..., None] * g - (r ** 3 * c)[..., None] * x
    dw = np.sum(dy * x * r[..., None], axis=tuple(range(x.ndim - 1)))
    return dx, dw


# ---------------------------------------------------------------------------
# LayerNorm — [FastLLM] 三 技术架构, "Transformer Block 结构": the block normalisation is
# LayerNorm or RMSNorm; the same page's environment section names Apex's
# fast_layer_norm kernels.  No formula is printed; the reading is the textbook layer
# normalisation over the last axis with a learned scale and bias, the biased (1/d)
# variance, and eps inside the root (as for RMSNorm).
# ---------------------------------------------------------------------------
def layernorm_fwd(x, w, b, eps):
    """y[t,j] = (x[t,j] - mu[t]) r[t] w[j] + b[j],  mu = mean_j x,
    r = 1/sqrt(mean_j (x - mu)^2 + eps).  Returns (y, mu [T], rstd [T])."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    mu = np.mean(x, axis=-1)
    xc = x - mu[..., None]
    rstd = 1.0 / np.sqrt(np.mean(xc * xc, axis=-1) + eps)
    return xc * rstd[..., None] * w + b, mu, rstd


def layernorm_bwd(dy, x, w, eps):
    """Gradients of layernorm_fwd for upstream dy.  With xh = (x - mu) r and g = w dy,
        dx = r (g - mean_j g - xh mean_j(g xh)),  dw = sum_t dy xh,  db = sum_t dy.
    Returns (dx, dw, db)."""
    dy, x, w = _f64(dy), _f64(x), _f64(w)
    mu = np.mean(x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(np.mean((x - mu) ** 2, axis=-1, keepdims=True) + eps)
    xh = (x - mu) * r
    g = dy * w
    dx = r * (g - np.mean(g, axis=-1, keepdims=True)
              - xh * np.mean(g * xh, axis=-1, keepdims=True))
    axes = tuple(range(x.ndim - 1))
    return dx, np.sum(dy * xh, axis=axes), np.sum(dy, axis=axes)


# ---------------------------------------------------------------------------
# RoPE — [FastLLM] 三 技术架构, "Transformer Block 结构" (attention + RoPE) and
# 训练配置示例 (rotary type default, theta; heads / head_groups / head_size);
# [LF] npu_fused_rope; [HFK] "Liger" (rope).
# Readings: half-split pairing (element i pairs with i + D/2, the layout of the
# HF-format checkpoints these pages load); frequencies theta^(-2i/D) over the full
# head dim; no scaling variants; the angle pos*freq is formed in fp64.
# ---------------------------------------------------------------------------
def rope_angles(pos, D, theta):
    """a[t,i] = pos[t] * theta^(-2i/D) for i in [0, D/2)."""
    pos = _i64(pos).astype(np.float64)
    i = np.arange(D // 2, dtype=np.float64)
    freq = np.power(float(theta), -2.0 * i / D)
    return pos[:, None] * freq[None, :]


def _rotate(x, a):
    # x [T, heads, D], a [T, D/2]: rotate each pair (x_i, x_{i+D/2}) by angle a_i.
    D = x.shape[-1]
    h = D // 2
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_fwd(q, k, pos, theta):
    """Rotate every Q head and every K head of token t by the angles of pos[t].

    q [T,Hq,D], k [T,Hkv,D] -> (q', k').  GQA grouping does not enter the rotation."""
    q = _f64(q)
    k = _f64(k)
    a = rope_angles(pos, q.shape[-1], theta)
    return _rotate(q, a), _rotate(k, a)


def rope_bwd(dq, dk, pos, theta):
    """Transpose of rope_fwd: rotate the gradients by the negated angles."""
    dq = _f64(dq)
    dk = _f64(dk)
    a = rope_angles(pos, dq.shape[-1], theta)
    return _rotate(dq, -a), _rotate(dk, -a)


# ---------------------------------------------------------------------------
# SwiGLU — [FastLLM] 三 技术架构, "Transformer Block 结构" (gated MLP with SiLU) and
# 训练配置示例 (mlp gated: true, activation: silu); [LF] npu_fused_swiglu;
# [HFK] "Liger" (swiglu).  Reading: h = silu(gate) * up, silu(x) = x * sigmoid(x).
# ---------------------------------------------------------------------------
def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = _f64(x)
    return x * _sigmoid(x)


def swiglu_fwd(gate, up):
    """h = gate * sigmoid(gate) * up, elementwise."""
    g = _f64(gate)
    u = _f64(up)
    return g * _sigmoid(g) * u


def swiglu_bwd(dh, gate, up):
    """d/dg [g s(g) u] = u (s + g s (1 - s)) = u s (1 + g (1 - s));  d/du = g s(g).

    Returns (dgate, dup)."""
    dh = _f64(dh)
    g = _f64(gate)
    u = _f64(up)
    s = _sigmoid(g)
    dg = dh * u * s * (1.0 + g * (1.0 - s))
    du = dh * g * s
    return dg, du


# ---------------------------------------------------------------------------
# Other MLP activations — [FastLLM] 三 技术架构, "支持的 MLP 变体": dense MLPs, gated or
# not, with SiLU, GeLU or ReLU.  Readings: GeLU is the exact form x Phi(x) (Phi the
# standard normal CDF, via erf), not the tanh approximation; a gated MLP computes
# act(gate) * up as SwiGLU does; the derivative of ReLU at 0 is taken as 0.
# ---------------------------------------------------------------------------
ACTS = ("silu", "gelu", "relu")


def _erf(x):
    from scipy.special import erf  # the error function, double precision
    return erf(x)


def act_value(x, act):
    """act(x) elementwise for act in ACTS."""
    x = _f64(x)
    if act == "silu":
        return silu(x)
    if act == "gelu":
        return x * 0.5 * (1.0 + _erf(x / np.sqrt(2.0)))
    if act == "relu":
        return np.maximum(x, 0.0)
    raise ValueError(act)


def act_deriv(x, act):
    """d act(x) / dx elementwise."""
    x = _f64(x)
    if act == "silu":
        s = _sigmoid(x)
        return s * (1.0 + x * (1.0 - s))
    if act == "gelu":
        return 0.5 * (1.0 + _erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)
    if act == "relu":
        return (x > 0.0).astype(np.float64)
    raise ValueError(act)


def glu_fwd(gate, up, act):
    """h = act(gate) * up."""
    return act_value(gate, act) * _f64(up)


def glu_bwd(dh, gate, up, act):
    """(dgate, dup) = (dh * up * act'(gate), dh * act(gate))."""
    dh, up = _f64(dh), _f64(up)
    return dh * up * act_deriv(gate, act), dh * act_value(gate, act)


def act_fwd(x, act):
    """y = act(x) (non-gated MLP activation)."""
    return act_value(x, act)


def act_bwd(dy, x, act):
    """dx = dy * act'(x)."""
    return _f64(dy) * act_deriv(x, act)


# ---------------------------------------------------------------------------
# Cross-entropy with ignore_index and z-loss — [FastLLM] 三 技术架构, "损失函数体系"
# (Cross-Entropy; Z-Loss "prevents over-confidence"), and the Triton kernel list of
# 整体框架结构 (entropy_loss.py, z_loss.py); [HFK] "Liger" (cross_entropy).
# Readings: mean over non-ignored rows (N = number of valid targets); z-loss is
# c_z * mean_valid(lse^2) added to the loss; a target outside [0, V) that is not
# ignore_index is counted as bad and treated as ignored; N = 0 gives loss 0 and
# all-zero gradients; ignored rows get exactly zero gradient.
# ---------------------------------------------------------------------------
def _valid_mask(tg, V, ignore_index):
    inr = (tg >= 0) & (tg < V)
    valid = inr & (tg != ignore_index)
    bad = (~inr) & (tg != ignore_index)
    return valid, bad


def xent_rows(z, tg, valid, n_valid, z_loss, dloss):
    """Per-row pieces for rows z [R,V] (fp64) with targets tg [R] and valid mask.

    logsumexp in the plain two-pass form: m = max_j z_j, lse = m + log sum_j exp(z_j - m).
      loss_t = lse - z[t, y_t] + c_z * lse^2
      dz[t]  = (dloss / N) * (softmax(z_t) * (1 + 2 c_z lse) - onehot(y_t))
    Rows with valid=False get loss 0 (excluded) and dz = 0.
    Returns (loss_rows [R], zterm_rows [R], lse [R], dz [R,V])."""
    R, V = z.shape
    m = np.max(z, axis=1)
    lse = m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))
    yt = np.where(valid, tg, 0)
    zy = z[np.arange(R), yt]
    zterm = z_loss * lse * lse
    loss_rows = np.where(valid, lse - zy + zterm, 0.0)
    zterm = np.where(valid, zterm, 0.0)
    dz = np.zeros_like(z)
    if n_valid > 0:
        scale = dloss / n_valid
        p = np.exp(z - lse[:, None])
        g = p * (1.0 + 2.0 * z_loss * lse)[:, None]
        g[np.arange(R), yt] -= 1.0
        dz = np.where(valid[:, None], scale * g, 0.0)
    return loss_rows, zterm, lse, dz


def xent_fwd_bwd(logits, targets, ignore_index=-100, z_loss=0.0, dloss=1.0):
    """Mean cross-entropy (+ z-loss) over valid rows, and its logit gradient.

    Returns dict(loss, z_loss, n_valid, n_bad, lse [T], dlogits [T,V])."""
    z = _f64(logits)
    tg = _i64(targets)
    T, V = z.shape
    valid, bad = _valid_mask(tg, V, ignore_index)
    n = int(valid.sum())
    loss_rows, zterm, lse, dz = xent_rows(z, tg, valid, n, z_loss, dloss)
    loss = float(loss_rows.sum() / n) if n else 0.0
    zl = float(zterm.sum() / n) if n else 0.0
    return dict(loss=loss, z_loss=zl, n_valid=n, n_bad=int(bad.sum()), lse=lse,
                dlogits=dz)


# ---------------------------------------------------------------------------
# Soft-target cross-entropy (distillation) — [FastLLM] 三 技术架构, "损失函数体系": label
# entropy and distillation losses next to the hard-label cross-entropy, computed by the
# framework's fused entropy-loss kernel.  No formula is printed; the reading is the
# cross-entropy of the student's softmax against the teacher's softmax (temperature 1),
# averaged over the rows a mask keeps; the KL divergence (cross-entropy minus the
# teacher's entropy, same gradient) is returned beside it.
# ---------------------------------------------------------------------------
def _log_softmax(z):
    m = np.max(z, axis=-1, keepdims=True)
    return z - m - np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True))


def distill_fwd_bwd(logits, teacher, row_mask=None, dloss=1.0):
    """p = softmax(teacher), q = softmax(logits) per row; over the N rows with a
    nonzero mask (all rows if None):
        loss = (1/N) sum_t -sum_v p log q,   kl = (1/N) sum_t sum_v p (log p - log q),
        dlogits = dloss (q - p) / N  (zero rows where the mask is 0; N = 0: all zero)."""
    z, zt = _f64(logits), _f64(teacher)
    T = z.shape[0]
    keep = np.ones(T, dtype=bool) if row_mask is None else (_i64(row_mask) != 0)
    n = int(keep.sum())
    lq, lp = _log_softmax(z), _log_softmax(zt)
    p = np.exp(lp)
    ce = -np.sum(p * lq, axis=-1)
    kl = np.sum(p * (lp - lq), axis=-1)
    d = np.zeros_like(z)
    if n:
        d[keep] = dloss * (np.exp(lq[keep]) - p[keep]) / n
    return dict(loss=float(ce[keep].sum() / n) if n else 0.0,
                kl=float(kl[keep].sum() / n) if n else 0.0, n_valid=n, dlogits=d)


# ---------------------------------------------------------------------------
# Fused linear cross-entropy — [HFK] "Liger" (fused_linear_cross_entropy: the lm-head
# projection and the loss fused so that large vocabularies stay feasible in memory).
# Definition: the composition xent(H W^T) with dH = dZ W and dW = dZ^T H, where dZ
# is the cross-entropy gradient above.  Reading: no bias, softcap or temperature.
# The optional row chunking below only bounds host memory; rows are independent, so
# it does not change the result beyond fp64 summation order.
# ---------------------------------------------------------------------------
def flce_fwd_bwd(hidden, weight, targets, ignore_index=-100, z_loss=0.0, dloss=1.0,
                 chunk=None, dh_rows=None, dw_rows=None, n_norm=None, abs_products=False):
    """Returns dict(loss, z_loss, n_valid, n_bad, dhidden, dweight).

    dh_rows / dw_rows: optional index arrays; when given only those rows of dH
    ([len, H]) and of dW ([len, H]) are formed (for sampled checks at large sizes).
    n_norm: the N that the mean and the gradient scale divide by, when these rows are
    one block of a larger batch (default: this call's valid count); the block results
    then add up to the batch's.
    abs_products: also return dhidden_abs = |dZ| |W| and dweight_abs = |dZ|^T |H| for
    the same rows (the scale of each output's rounding errors, for error bounds)."""
    Hm = _f64(hidden)
    W = _f64(weight)
    tg = _i64(targets)
    T = Hm.shape[0]
    V = W.shape[0]
    valid, bad = _valid_mask(tg, V, ignore_index)
    n = int(valid.sum())
    nn = n if n_norm is None else int(n_norm)
    chunk = T if chunk is None else int(chunk)
    want_dh = np.arange(T) if dh_rows is None else np.asarray(dh_rows)
    want_dw = None if dw_rows is None else np.asarray(dw_rows)
    dH = np.zeros((len(want_dh), Hm.shape[1]))
    dW = np.zeros((V if want_dw is None else len(want_dw), Hm.shape[1]))
    dH_abs = np.zeros_like(dH) if abs_products else None
    dW_abs = np.zeros_like(dW) if abs_products else None
    loss_sum = 0.0
    z_sum = 0.0
    pos_in_dh = {int(r): i for i, r in enumerate(want_dh)}
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        Z = Hm[c0:c1] @ W.T
        lr, zt, _, dZ = xent_rows(Z, tg[c0:c1], valid[c0:c1], nn, z_loss, dloss)
        loss_sum += lr.sum()
        z_sum += zt.sum()
        rows = [r for r in range(c0, c1) if r in pos_in_dh]
        if rows:
            sel = np.array(rows) - c0
            dH[[pos_in_dh[r] for r in rows]] = dZ[sel] @ W
            if abs_products:
                dH_abs[[pos_in_dh[r] for r in rows]] = np.abs(dZ[sel]) @ np.abs(W)
        dZ_sel = dZ if want_dw is None else dZ[:, want_dw]
        dW += dZ_sel.T @ Hm[c0:c1]
        if abs_products:
            dW_abs += np.abs(dZ_sel).T @ np.abs(Hm[c0:c1])
    out = dict(loss=float(loss_sum / nn) if nn else 0.0,
               z_loss=float(z_sum / nn) if nn else 0.0,
               n_valid=n, n_bad=int(bad.sum()), dhidden=dH, dweight=dW)
    if abs_products:
        out.update(dhidden_abs=dH_abs, dweight_abs=dW_abs)
    return out


# ---------------------------------------------------------------------------
# AdamW step — [FastLLM] 关键实现细节, "Triton Adam 优化器": one fused pass over a
# parameter tensor that scales the gradient (a device scalar), updates both moments,
# applies weight decay and the parameter update, and does nothing at all while a
# device no-op flag is set; the host supplies step_size, bias_correction and
# decay_factor.  The page prints the kernel's signature but no formula, so the reading
# is the textbook AdamW with decoupled weight decay (Loshchilov & Hutter) in the
# bias-corrected form whose host scalars those names describe:
#   step_size = lr / (1 - beta1^t), bias_correction = sqrt(1 - beta2^t),
#   decay_factor = 1 - lr * weight_decay.
# ---------------------------------------------------------------------------
def adamw_scalars(lr, beta1, beta2, weight_decay, step):
    """Host scalars of step t (t >= 1): (step_size, bias_correction, decay_factor)."""
    step_size = lr / (1.0 - beta1 ** step)
    bias_correction = float(np.sqrt(1.0 - beta2 ** step))
    decay_factor = 1.0 - lr * weight_decay
    return step_size, bias_correction, decay_factor


def adamw_step(p, g, m, v, step_size, beta1, beta2, bias_correction, decay_factor, eps,
               grad_scale=1.0, noop=False):
    """One AdamW update of one tensor, elementwise:
        g' = grad_scale * g
        m' = beta1 m + (1 - beta1) g'
        v' = beta2 v + (1 - beta2) g'^2
        p' = decay_factor p - step_size m' / (sqrt(v') / bias_correction + eps)
    With noop set nothing changes.  Returns (p', m', v')."""
    p, g, m, v = _f64(p), _f64(g), _f64(m), _f64(v)
    if noop:
        return p.copy(), m.copy(), v.copy()
    gs = grad_scale * g
    m1 = beta1 * m + (1.0 - beta1) * gs
    v1 = beta2 * v + (1.0 - beta2) * gs * gs
    p1 = decay_factor * p - step_size * m1 / (np.sqrt(v1) / bias_correction + eps)
    return p1, m1, v1
