"""Pins for the fp64 SwiGLU oracle.  No GPU."""
import numpy as np
import torch

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_gate_zero():
    u = rng(0).standard_normal(10)
    dh = rng(1).standard_normal(10)
    assert np.all(oracle.swiglu_fwd(np.zeros(10), u) == 0)
    dg, du = oracle.swiglu_bwd(dh, np.zeros(10), u)
    assert np.max(np.abs(dg - dh * u / 2)) < 1e-15 and np.all(du == 0)


def test_silu_odd_part_identity():
    x = rng(2).standard_normal(100) * 5
    assert np.max(np.abs(oracle.silu(x) - oracle.silu(-x) - x)) < 1e-12


def test_saturation_no_nan():
    g = np.array([100.0, -100.0, 800.0, -800.0])
    u = np.array([1.5, 1.5, -2.0, 3.0])
    h = oracle.swiglu_fwd(g, u)
    assert np.all(np.isfinite(h))
    assert abs(h[0] - 150.0) < 1e-12 and abs(h[1]) < 1e-40 and h[2] == -1600.0
    dg, du = oracle.swiglu_bwd(np.ones(4), g, u)
    assert np.all(np.isfinite(dg)) and np.all(np.isfinite(du))
    assert abs(dg[0] - 1.5) < 1e-12 and abs(du[0] - 100.0) < 1e-12


def test_matches_torch_silu_f64():
    g = rng(3).standard_normal(1000) * 4
    u = rng(4).standard_normal(1000)
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
    assert np.max(np.abs(oracle.swiglu_fwd(g, u) - ref)) < 1e-13


def test_backward_matches_autograd_and_finite_differences():
    r = rng(5)
    g = r.standard_normal((4, 9)) * 3
    u = r.standard_normal((4, 9))
    dh = r.standard_normal((4, 9))
    dg, du = oracle.swiglu_bwd(dh, g, u)
    gt = torch.from_numpy(g).requires_grad_()
    ut = torch.from_numpy(u).requires_grad_()
    (torch.nn.functional.silu(gt) * ut).backward(torch.from_numpy(dh))
    assert np.max(np.abs(dg - gt.grad.numpy())) < 1e-12
    assert np.max(np.abs(du - ut.grad.numpy())) < 1e-12
    h = 1e-6
    fd_g = (oracle.swiglu_fwd(g + h, u) - oracle.swiglu_fwd(g - h, u)) / (2 * h) * dh
    fd_u = (oracle.swiglu_fwd(g, u + h) - oracle.swiglu_fwd(g, u - h)) / (2 * h) * dh
    assert np.max(np.abs(dg - fd_g)) < 1e-8 and np.max(np.abs(du - fd_u)) < 1e-8
