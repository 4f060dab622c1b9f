"""Tolerance checks of the GPU-vs-oracle parity tests.

The stated contract is "fp32: max relative error <= 1e-5; bf16: max absolute error
<= 2e-2 with fp32 accumulation; scalar loss: relative error <= 1e-4; masking and
position resets bit-exact".  Read literally, the bf16 bound cannot hold for outputs of
magnitude >= 8 (half a bf16 ulp there is 0.03125) and says nothing about gradients of
size 1/N; and a plain elementwise relative error is unbounded at zero crossings.  So:

  bf16:  (i)  |g - r| <= 2e-2 * max(1, |r|)              elementwise
         (ii) max|g - r| / max|r| <= 2e-2                 normwise
  fp32:  |g - r| / max(|r|, rms(r)) <= 1e-5               elementwise
  loss:  |g - r| / |r| <= 1e-4  (|g - r| <= 1e-6 when r == 0)

and, for outputs that the kernels round to bf16 exactly once from an fp32 value, the
much tighter check

  bf16 single rounding:  |g - r| <= (2^-8 + 3e-5) |r| + 1e-5 rms(r)

(half a bf16 ulp is at most 2^-8 |r|; 3e-5 |r| covers the fp32 arithmetic before the
rounding; the rms floor covers cancellation in the fp32 arithmetic).

Where the exact result is the difference of two terms much larger than itself, no fp32
evaluation gets within 1e-5 of the result, only of the terms: the input gradient of
RMSNorm / LayerNorm, dx = r (g - c) - r^3 xc mean(g xc), cancels where r^2 xc^2 is
close to 1 for every column (a one-column RMSNorm row, a two-column LayerNorm row whose
values nearly agree, so that its variance is of the order of eps).  There the relative
bounds take A = |r (g - c)| + |r^3 xc mean(g xc)| (norm_dx_terms) in place of |r|.
LayerNorm's row is also centred with an fp32 mean, a few units of 2^-24 max|x| off the
exact one, which moves xc, and r with it, by up to 2^-24 max|x| r relative: negligible
for rows whose spread is of the order of their values, but for a row of nearly equal
values r max|x| is large.  Sixteen such units against the 1e-5 bound make LayerNorm's
A = (|r (g - c)| + |r^3 xc mean(g xc)|) (1 + 0.1 r max|x|):

  fp32:  |g - r| / max(|r|, rms(r), A) <= 1e-5
  bf16 single rounding:  |g - r| <= 2^-8 |r| + 3e-5 max(|r|, A) + 1e-5 rms(r)

For rows that do not cancel, A is |r| or close to it.

The same centring moves LayerNorm's output y = xc r w + b by up to 16 units of
2^-24 |w| r max|x|, and y is itself a sum that can cancel (xc r w against b), so y takes
A = |xc r w| + |b| + 0.1 |w| r max|x| (layernorm_y_terms).

The weight gradients dw_j = sum_t dy_tj xc_tj r_t (RMSNorm: xc = x) are sums over the
rows of terms of either sign; their fp32 rounding, and their size, go with the root sum
of squares of the terms, which a sum that cancels (a one-column row's terms are about
+-|dy|) can fall far below.  So dw takes A_j = sqrt(sum_t (dy_tj xc_tj r_t)^2) beside |r|
and rms(r); for LayerNorm plus 0.1 sqrt(sum_t (dy_tj r_t max_k |x_tk|)^2), the centring
error of each row's term (16 units of 2^-24 |dy| r max|x|, rows rounding independently)
(norm_dw_terms).  For a sum that does not cancel, A_j is about |dw_j|; the centring part
is negligible unless some row's values nearly agree, where r max|x| reaches 1/sqrt(eps).

The cross-entropy gradient's target column, s (p (1 + 2 c lse) - 1) with s = dloss/N, is
the difference of two terms of size |s| when p is near 1 (a confident row; a one-class
row has p = 1, and with no z-loss the exact result is 0).  Its fp32 evaluation is within a
few units of 2^-24 of those terms, not of their difference, so the single-rounding bound
takes A = |s| (p |1 + 2 c lse| + [column = target]) (xent_dz_terms); elsewhere A = |r|.

The fused linear cross-entropy's weight and hidden gradients are products dZ X of the
logit gradient with an exact bf16 operand X (W for dH, H for dW).  The kernel's dZ
carries two bf16 roundings (exp(z - m) stored in bf16, then dZ itself), each at most
2^-8 relative, so it is within (2^-7 + 2^-16) |dz| of the exact one; the fp32 logits,
logsumexp and accumulation add far less than 2^-9 relative (fp32 sums of a few
thousand terms).  Hence, elementwise, with A = |dz| |X| the product of the absolute
values (the oracle returns it):

  product gradient:  |g - r| <= (2^-7 + 2^-9) A + [output rounded to bf16] (2^-8 + 3e-5) |r|
                                + 1e-6 rms(A)

In the fused linear cross-entropy the same target column, s (p (1 + 2 c lse) - 1), is formed
in fp32 before dZ is rounded; its error is a few units of 2^-24 of terms of size at most
3 |s| (for c |lse| <= 1/2), not of |dz|, and it reaches dH through the target's row of W
and dW through the rows of H that target it.  The product bound therefore adds
2^-20 B, B = 3 |s| |W[target]| for a dH row and the sum of 3 |s| |H[r]| over the rows r
that target the entry for a dW row (flce_target_terms); a single-class head, where every
dz is that column and p = 1, needs it.

The AdamW moment update m' = beta1 m + (1 - beta1) g' is a sum of two terms of either
sign, exact only to a few units of 2^-24 of |beta1 m| + |(1 - beta1) g'|, and the
parameter update p' = decay p - step m' / (sqrt(v')/bc + eps) carries that error of m'
beside its own two terms; a tensor of one element has no rms floor to absorb a cancelling
one.  So m' takes A = |beta1 m| + |(1 - beta1) g'| and p' takes
A = |decay p| + |step| A_m / (sqrt(v')/bc + eps) (adamw_terms); v' is a sum of two
non-negative terms.

A softmax value computed in fp32 is relative-accurate only to a few units of 2^-24 of the
magnitudes of its logit and logsumexp, so the cross-entropy softmax term and the
distillation softmaxes take the factor max(1, 0.03 (|z| + |lse|)), and the distillation
bound a floor of 2^-125 |s| for softmax values below fp32's normal range.  The KL,
sum p (zt - z) + lse_z - lse_t, is a difference of terms of size
A = mean over rows of (sum p |zt - z| + |lse_z - lse_t|) (kl_terms): its bound is
1e-4 |KL| + 1e-5 A.  Where a term size applies, the bf16 elementwise and normwise legs
take it as well (+ 3e-5 A; normwise against max(max|r|, max A)).

The distillation gradient dz = s (q - p) (s = dloss/N) is the difference of two fp32
softmax values, each within a few 1e-6 relative of the exact one (fp32 exponentials of
arguments up to ~40 in size, fp32 logsumexps), then rounded once:

  softmax difference:  |g - r| <= [bf16] (2^-8 + 3e-5) |r| + 1e-5 |s| (q + p)
"""
from __future__ import annotations

import numpy as np


def _np(a):
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _report(name, mask, g, r, bound):
    idx = np.argwhere(mask)
    i = tuple(idx[0])
    return (f"{name}: {len(idx)} element(s) out of tolerance; first at {i}: "
            f"gpu={g[i]!r} oracle={r[i]!r} |diff|={abs(g[i] - r[i]):.3e} bound={bound[i]:.3e}")


def norm_dx_terms(dy, x, w, eps, layer):
    """Per element, |r (g - c)| + |r^3 xc mean(g xc)| for the input gradient of RMSNorm
    (layer False: c = 0, xc = x) or LayerNorm (c = mean(g), xc = x - mean(x)), g = w dy,
    r = 1/sqrt(mean(xc^2) + eps): the sizes of the two terms dx is the difference of;
    for LayerNorm times 1 + 0.1 r max|x| (the centring by an fp32 mean)."""
    dy, x, w = _np(dy), _np(x), _np(w).reshape(1, -1)
    g = dy * w
    xc = x - x.mean(axis=1, keepdims=True) if layer else x
    c = g.mean(axis=1, keepdims=True) if layer else 0.0
    r = 1.0 / np.sqrt((xc * xc).mean(axis=1, keepdims=True) + eps)
    m = (g * xc).mean(axis=1, keepdims=True)
    a = np.abs(r * (g - c)) + np.abs(r ** 3 * xc * m)
    if layer:
        a = a * (1.0 + 0.1 * r * np.abs(x).max(axis=1, keepdims=True))
    return a


def norm_dw_terms(dy, x, eps, layer):
    """Per column, sqrt(sum_t (dy_tj xc_tj r_t)^2), and for LayerNorm (layer True) plus
    0.1 sqrt(sum_t (dy_tj r_t max_k |x_tk|)^2): the term sizes of the weight gradient of
    RMSNorm (xc = x) or LayerNorm (xc = x - mean(x)), r = 1/sqrt(mean(xc^2) + eps)."""
    dy, x = _np(dy), _np(x)
    xc = x - x.mean(axis=1, keepdims=True) if layer else x
    r = 1.0 / np.sqrt((xc * xc).mean(axis=1, keepdims=True) + eps)
    t = dy * xc * r
    a = np.sqrt(np.sum(t * t, axis=0))
    if layer:
        e = dy * (r * np.abs(x).max(axis=1, keepdims=True))
        a = a + 0.1 * np.sqrt(np.sum(e * e, axis=0))
    return a


def layernorm_y_terms(x, w, b, eps):
    """Per element, |xc r w| + |b| + 0.1 |w| r max|x|: the term sizes of LayerNorm's
    output, the last one the centring of the row by an fp32 mean."""
    x, w, b = _np(x), _np(w).reshape(1, -1), _np(b).reshape(1, -1)
    xc = x - x.mean(axis=1, keepdims=True)
    r = 1.0 / np.sqrt((xc * xc).mean(axis=1, keepdims=True) + eps)
    return np.abs(xc * r * w) + np.abs(b) + 0.1 * np.abs(w) * r * np.abs(x).max(axis=1, keepdims=True)


def xent_dz_terms(z, targets, valid, lse, z_loss, dloss, n_valid):
    """Per element, |s| (p |1 + 2 c lse| max(1, 0.03 (|z| + |lse|)) + [column = target]) on
    valid rows (0 elsewhere), s = dloss / n_valid, p = exp(z - lse) from the oracle's lse:
    the sizes of the terms the cross-entropy gradient is the difference of, the softmax
    term widened for logits whose magnitude limits fp32's relative accuracy."""
    z, lse = _np(z), _np(lse).reshape(-1, 1)
    tg = np.asarray(targets, dtype=np.int64)
    valid = np.asarray(valid, dtype=bool)
    if n_valid <= 0:
        return np.zeros_like(z)
    s = abs(dloss / n_valid)
    # p = exp(z - lse) in fp32 is relative-accurate only to a few units of 2^-24 of
    # |z| + |lse| (the rounding of lse and of the exponent's argument)
    mag = np.maximum(1.0, 0.03 * (np.abs(z) + np.abs(lse)))
    a = s * np.exp(z - lse) * np.abs(1.0 + 2.0 * z_loss * lse) * mag
    rows = np.nonzero(valid)[0]
    a[rows, tg[rows]] += s
    return np.where(valid[:, None], a, 0.0)


def check_bf16(g, r, name="out", single_rounding=False, scale=None):
    g, r = _np(g), _np(r)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU output"
    d = np.abs(g - r)
    b1 = 2e-2 * np.maximum(1.0, np.abs(r))
    if scale is not None:
        b1 = b1 + 3e-5 * _np(scale)  # the fp32 error of a difference of larger terms
    assert np.all(d <= b1), _report(name + " [bf16 elementwise]", d > b1, g, r, b1)
    mr = np.max(np.abs(r)) if r.size else 0.0
    if scale is not None and r.size:
        mr = max(mr, float(np.max(_np(scale))))  # a difference of larger terms: their size
    if r.size and mr > 0:
        assert np.max(d) / mr <= 2e-2, f"{name}: normwise {np.max(d) / mr:.3e} > 2e-2"
    if single_rounding and r.size:
        rms = np.sqrt(np.mean(r * r))
        big = np.abs(r) if scale is None else np.maximum(np.abs(r), _np(scale))
        b2 = 2.0 ** -8 * np.abs(r) + 3e-5 * big + 1e-5 * rms
        assert np.all(d <= b2), _report(name + " [bf16 single rounding]", d > b2, g, r, b2)
    return float(np.max(d)) if d.size else 0.0


def flce_target_terms(X, targets, n_valid, dloss, rows, kind):
    """B of the fused linear cross-entropy's product bound for the requested rows:
    kind "dh": 3 |s| |W[t_r]| for each token row r (X = W; 0 for rows that are ignored);
    kind "dw": the sum over valid rows r with t_r = v of 3 |s| |H[r]| for each vocabulary
    row v (X = H); s = dloss / n_valid."""
    X = np.abs(_np(X))
    tg = np.asarray(targets, dtype=np.int64).reshape(-1)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    out = np.zeros((len(rows), X.shape[1]))
    if n_valid <= 0:
        return out
    s3 = 3.0 * abs(dloss / n_valid)
    if kind == "dh":
        V = X.shape[0]
        for i, r in enumerate(rows):
            if 0 <= tg[r] < V:
                out[i] = s3 * X[tg[r]]
    else:
        at = {int(v): i for i, v in enumerate(rows)}
        for r in range(len(tg)):
            i = at.get(int(tg[r]))
            if i is not None:
                out[i] += s3 * X[r]
    return out


def adamw_terms(p, g, m, v, step_size, beta1, beta2, bias_correction, decay_factor, eps,
                grad_scale=1.0):
    """(A_p, A_m): the term sizes of the AdamW parameter and first-moment updates."""
    p, g, m, v = _np(p), _np(g), _np(m), _np(v)
    gs = grad_scale * g
    a_m = np.abs(beta1 * m) + np.abs((1.0 - beta1) * gs)
    v1 = beta2 * v + (1.0 - beta2) * gs * gs
    den = np.sqrt(v1) / bias_correction + eps
    a_p = np.abs(decay_factor * p) + abs(step_size) * a_m / den
    return a_p, a_m


def check_product_grad(g, r, absprod, name="out", rounded_out=True, target=None):
    """target: B of the target column's fp32 error (flce_target_terms), if any."""
    g, r, a = _np(g), _np(r), _np(absprod)
    assert g.shape == r.shape == a.shape, (name, g.shape, r.shape, a.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU output"
    if not r.size:
        return 0.0
    d = np.abs(g - r)
    bound = (2.0 ** -7 + 2.0 ** -9) * a + 1e-6 * np.sqrt(np.mean(a * a))
    if target is not None:
        bound = bound + 2.0 ** -20 * _np(target)
    if rounded_out:
        bound = bound + (2.0 ** -8 + 3e-5) * np.abs(r)
    assert np.all(d <= bound), _report(name + " [product of rounded dZ]", d > bound, g, r, bound)
    return float(np.max(d / np.where(bound > 0, bound, 1.0)))


def check_softmax_diff(g, r, qp_scaled, name="out", rounded_out=True):
    g, r, a = _np(g), _np(r), _np(qp_scaled)
    assert g.shape == r.shape == a.shape, (name, g.shape, r.shape, a.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU output"
    if not r.size:
        return 0.0
    d = np.abs(g - r)
    bound = 1e-5 * np.abs(a) + (2.0 ** -8 + 3e-5 if rounded_out else 2.0 ** -23) * np.abs(r)
    assert np.all(d <= bound), _report(name + " [softmax difference]", d > bound, g, r, bound)
    return float(np.max(d / np.where(bound > 0, bound, 1.0)))


def check_f32(g, r, name="out", rel=1e-5, scale=None):
    g, r = _np(g), _np(r)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU output"
    if not r.size:
        return 0.0
    rms = np.sqrt(np.mean(r * r))
    den = np.maximum(np.abs(r), rms)
    if scale is not None:
        den = np.maximum(den, _np(scale))
    den = np.where(den > 0, den, 1.0)
    e = np.abs(g - r) / den
    bound = np.full_like(e, rel)
    assert np.all(e <= rel), _report(name + " [fp32 relative]", e > rel, g, r, bound * den)
    return float(np.max(e))


def check(g, r, dtype, name="out", single_rounding=False, scale=None):
    """scale: the term sizes A of an output that is a difference of larger terms."""
    if dtype == "bf16":
        return check_bf16(g, r, name, single_rounding, scale)
    return check_f32(g, r, name, scale=scale)


def kl_terms(z, zt, keep):
    """Mean over the kept rows of sum_v p_v |zt_v - z_v| + |lse_z - lse_t| (p the teacher's
    softmax): the sizes of the terms the KL divergence is the sum of."""
    z, zt = _np(z), _np(zt)
    keep = np.asarray(keep, dtype=bool)
    if not keep.any():
        return 0.0
    z, zt = z[keep], zt[keep]

    def lse(x):
        m = x.max(1, keepdims=True)
        return m + np.log(np.exp(x - m).sum(1, keepdims=True))

    lz, lt = lse(z), lse(zt)
    p = np.exp(zt - lt)
    return float(np.mean((p * np.abs(zt - z)).sum(1) + np.abs(lz - lt)[:, 0]))


def check_loss(g, r, name="loss", rel=1e-4, scale=None):
    """scale: the size of the terms a scalar is the sum of, when they can cancel (the KL of
    two close distributions); it adds 1e-5 of it to the bound."""
    g = float(g)
    r = float(r)
    extra = 0.0 if scale is None else 1e-5 * float(scale)
    if r == 0.0:
        assert abs(g) <= 1e-6 + extra, f"{name}: gpu={g} oracle=0"
    else:
        assert abs(g - r) <= rel * abs(r) + extra, \
            f"{name}: gpu={g!r} oracle={r!r} rel={abs(g - r) / abs(r):.3e}"
