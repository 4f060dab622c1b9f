"""Pins for the fp64 LayerNorm oracle.  No GPU."""
import numpy as np
import torch

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_hand_worked_row():
    # x = (1, 2, 3, 6): mean 3, deviations (-2, -1, 0, 3), variance 14/4 = 3.5
    x = np.array([[1.0, 2.0, 3.0, 6.0]])
    y, mu, r = oracle.layernorm_fwd(x, np.ones(4), np.zeros(4), 0.0)
    assert mu[0] == 3.0 and abs(r[0] - 1 / np.sqrt(3.5)) < 1e-16
    assert np.max(np.abs(y[0] - np.array([-2.0, -1.0, 0.0, 3.0]) / np.sqrt(3.5))) < 1e-15


def test_normalised_rows_and_affine():
    x = rng(0).standard_normal((7, 300)) * 3 + 5
    y, _, _ = oracle.layernorm_fwd(x, np.ones(300), np.zeros(300), 0.0)
    assert np.max(np.abs(y.mean(-1))) < 1e-13 and np.max(np.abs(y.var(-1) - 1)) < 1e-12
    w = rng(1).standard_normal(300)
    b = rng(2).standard_normal(300)
    y2, _, _ = oracle.layernorm_fwd(x, w, b, 0.0)
    assert np.max(np.abs(y2 - (y * w + b))) < 1e-12


def test_shift_and_scale_invariance():
    x = rng(3).standard_normal((4, 64))
    w, b = rng(4).standard_normal(64), rng(5).standard_normal(64)
    y, _, _ = oracle.layernorm_fwd(x, w, b, 0.0)
    ys, _, _ = oracle.layernorm_fwd(x + 17.0, w, b, 0.0)
    yk, _, _ = oracle.layernorm_fwd(3.5 * x, w, b, 0.0)
    assert np.max(np.abs(ys - y)) < 1e-12 and np.max(np.abs(yk - y)) < 1e-12


def test_matches_torch_layer_norm_f64():
    x = rng(6).standard_normal((9, 130)) * 2 - 1
    w, b = 1 + 0.1 * rng(7).standard_normal(130), rng(8).standard_normal(130)
    y, mu, r = oracle.layernorm_fwd(x, w, b, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (130,), torch.from_numpy(w),
                                         torch.from_numpy(b), 1e-5).numpy()
    assert np.max(np.abs(y - ref)) < 1e-13


def test_backward_against_torch_autograd_f64():
    x = torch.from_numpy(rng(9).standard_normal((6, 50)) * 2 + 0.5).requires_grad_()
    w = torch.from_numpy(1 + 0.2 * rng(10).standard_normal(50)).requires_grad_()
    b = torch.from_numpy(rng(11).standard_normal(50)).requires_grad_()
    dy = rng(12).standard_normal((6, 50))
    torch.nn.functional.layer_norm(x, (50,), w, b, 1e-5).backward(torch.from_numpy(dy))
    dx, dw, db = oracle.layernorm_bwd(dy, x.detach(), w.detach(), 1e-5)
    assert np.max(np.abs(dx - x.grad.numpy())) < 1e-12
    assert np.max(np.abs(dw - w.grad.numpy())) < 1e-12
    assert np.max(np.abs(db - b.grad.numpy())) < 1e-12


def test_backward_invariants_and_finite_differences():
    x = rng(13).standard_normal((3, 20))
    w, dy = rng(14).standard_normal(20), rng(15).standard_normal((3, 20))
    dx, dw, db = oracle.layernorm_bwd(dy, x, w, 1e-5)
    # dx is orthogonal to the constant vector (the mean is removed), db = sum_t dy
    assert np.max(np.abs(dx.sum(-1))) < 1e-12
    assert np.array_equal(db, dy.sum(0))
    # central differences of sum(dy * y) in x
    b = np.zeros(20)
    h = 1e-6
    for t, j in ((0, 0), (1, 7), (2, 19)):
        xp, xm = x.copy(), x.copy()
        xp[t, j] += h
        xm[t, j] -= h
        fp = np.sum(dy * oracle.layernorm_fwd(xp, w, b, 1e-5)[0])
        fm = np.sum(dy * oracle.layernorm_fwd(xm, w, b, 1e-5)[0])
        assert abs((fp - fm) / (2 * h) - dx[t, j]) < 1e-6
