"""Pins for the fp64 RMSNorm oracle: closed forms, invariants, an independent library
routine and central finite differences.  No GPU."""
import math

import numpy as np
import torch

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_hand_worked_row():
    # x = (3, 4), eps = 0: mean square 12.5, r = 1/sqrt(12.5); with w = (1, 2)
    # y = (3/sqrt(12.5), 8/sqrt(12.5)) = (0.848528137..., 2.262741699...).
    y, r = oracle.rmsnorm_fwd(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    assert abs(r[0] - 1 / math.sqrt(12.5)) < 1e-15
    assert abs(y[0, 0] - 0.8485281374238570) < 1e-14
    assert abs(y[0, 1] - 2.2627416997969521) < 1e-14


def test_unit_weight_rms_closed_form():
    x = rng(1).standard_normal((5, 33)) * 3.0
    eps = 1e-2
    y, _ = oracle.rmsnorm_fwd(x, np.ones(33), eps)
    ms = np.mean(x * x, axis=1)
    rms_y = np.sqrt(np.mean(y * y, axis=1))
    # RMS(y) = sqrt(ms / (ms + eps)), within eps/(2 ms) of 1
    assert np.max(np.abs(rms_y - np.sqrt(ms / (ms + eps)))) < 1e-12
    assert np.all(np.abs(rms_y - 1) <= eps / (2 * ms) + 1e-12)
    y0, _ = oracle.rmsnorm_fwd(x, np.ones(33), 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(y0 * y0, axis=1)) - 1)) < 1e-13


def test_zero_row_and_constant_row():
    eps = 1e-5
    y, r = oracle.rmsnorm_fwd(np.zeros((1, 16)), np.full(16, 2.0), eps)
    assert np.all(y == 0) and abs(r[0] - eps ** -0.5) < 1e-9 * eps ** -0.5
    c = 0.37
    w = rng(2).standard_normal(16)
    y, _ = oracle.rmsnorm_fwd(np.full((1, 16), c), w, eps)
    assert np.max(np.abs(y[0] - c / math.sqrt(c * c + eps) * w)) < 1e-14


def test_scale_invariance_without_eps():
    x = rng(3).standard_normal((4, 20))
    w = rng(4).standard_normal(20)
    a, _ = oracle.rmsnorm_fwd(x, w, 0.0)
    b, _ = oracle.rmsnorm_fwd(17.5 * x, w, 0.0)
    assert np.max(np.abs(a - b)) < 1e-13


def test_matches_torch_rms_norm_f64():
    x = rng(5).standard_normal((6, 48))
    w = 1 + 0.1 * rng(6).standard_normal(48)
    for eps in (1e-6, 1e-5, 0.3):
        y, _ = oracle.rmsnorm_fwd(x, w, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(w), eps)
        assert np.max(np.abs(y - ref.numpy())) < 1e-13


def _fd(f, a, h=1e-6):
    g = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        ap = a.copy(); ap[i] += h
        am = a.copy(); am[i] -= h
        g[i] = (f(ap) - f(am)) / (2 * h)
    return g


def test_backward_finite_differences():
    r = rng(7)
    T, d, eps = 3, 7, 1e-3
    x = r.standard_normal((T, d))
    w = 1 + 0.1 * r.standard_normal(d)
    dy = r.standard_normal((T, d))
    dx, dw = oracle.rmsnorm_bwd(dy, x, w, eps)
    fx = _fd(lambda xx: np.sum(oracle.rmsnorm_fwd(xx, w, eps)[0] * dy), x)
    fw = _fd(lambda ww: np.sum(oracle.rmsnorm_fwd(x, ww, eps)[0] * dy), w)
    assert np.max(np.abs(dx - fx)) < 1e-8
    assert np.max(np.abs(dw - fw)) < 1e-8


def test_backward_matches_torch_autograd_f64():
    r = rng(8)
    x = torch.from_numpy(r.standard_normal((9, 40))).requires_grad_()
    w = torch.from_numpy(1 + 0.1 * r.standard_normal(40)).requires_grad_()
    dy = r.standard_normal((9, 40))
    y = torch.nn.functional.rms_norm(x, (40,), w, 1e-6)
    y.backward(torch.from_numpy(dy))
    dx, dw = oracle.rmsnorm_bwd(dy, x.detach().numpy(), w.detach().numpy(), 1e-6)
    assert np.max(np.abs(dx - x.grad.numpy())) < 1e-12
    assert np.max(np.abs(dw - w.grad.numpy())) < 1e-12


def test_backward_orthogonality_identity():
    # <dx, x> = r * eps/(ms+eps) * <w*dy, x> per row (0 when eps = 0)
    r_ = rng(9)
    x = r_.standard_normal((5, 64)) * 0.01  # small ms so eps matters
    w = 1 + 0.1 * r_.standard_normal(64)
    dy = r_.standard_normal((5, 64))
    eps = 1e-4
    dx, _ = oracle.rmsnorm_bwd(dy, x, w, eps)
    ms = np.mean(x * x, axis=1)
    r = 1 / np.sqrt(ms + eps)
    lhs = np.sum(dx * x, axis=1)
    rhs = r * eps / (ms + eps) * np.sum(w * dy * x, axis=1)
    assert np.max(np.abs(lhs - rhs)) < 1e-10 * np.max(np.abs(rhs))


def test_accepts_torch_bf16_exactly():
    x = torch.randn(3, 8, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    y, _ = oracle.rmsnorm_fwd(x, torch.ones(8, dtype=torch.bfloat16), 1e-6)
    ref = torch.nn.functional.rms_norm(x.double(), (8,), None, 1e-6)
    assert np.max(np.abs(y - ref.numpy())) < 1e-14
