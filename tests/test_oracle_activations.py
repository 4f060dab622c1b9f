"""Pins for the fp64 GeLU / ReLU / gated-MLP oracle.  No GPU."""
import numpy as np
import pytest
import torch

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_gelu_matches_torch_exact_f64():
    x = rng(0).standard_normal(2000) * 4
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.max(np.abs(oracle.act_value(x, "gelu") - ref)) < 1e-14


def test_gelu_odd_part_and_known_values():
    x = rng(1).standard_normal(500) * 3
    g = oracle.act_value(x, "gelu")
    assert np.max(np.abs(g - oracle.act_value(-x, "gelu") - x)) < 1e-13  # Phi(x)+Phi(-x)=1
    assert oracle.act_value(np.array([0.0]), "gelu")[0] == 0.0
    # x Phi(x) at x = 1: Phi(1) = 0.8413447460685429
    assert abs(oracle.act_value(np.array([1.0]), "gelu")[0] - 0.8413447460685429) < 1e-15


def test_relu_and_its_derivative_convention():
    x = np.array([-2.0, -0.0, 0.0, 1e-300, 3.0])
    assert np.array_equal(oracle.act_value(x, "relu"), np.array([0.0, 0.0, 0.0, 1e-300, 3.0]))
    assert np.array_equal(oracle.act_deriv(x, "relu"), np.array([0.0, 0.0, 0.0, 1.0, 1.0]))


@pytest.mark.parametrize("act", ["silu", "gelu", "relu"])
def test_derivatives_against_torch_autograd_f64(act):
    x = torch.from_numpy(rng(2).standard_normal(300) * 3 + 0.01).requires_grad_()
    fn = {"silu": torch.nn.functional.silu, "relu": torch.relu,
          "gelu": lambda t: torch.nn.functional.gelu(t, approximate="none")}[act]
    fn(x).sum().backward()
    assert np.max(np.abs(oracle.act_deriv(x.detach(), act) - x.grad.numpy())) < 1e-13


@pytest.mark.parametrize("act", ["silu", "gelu"])
def test_derivative_finite_differences(act):
    x = rng(3).standard_normal(50) * 2
    h = 1e-6
    fd = (oracle.act_value(x + h, act) - oracle.act_value(x - h, act)) / (2 * h)
    assert np.max(np.abs(fd - oracle.act_deriv(x, act))) < 1e-8


@pytest.mark.parametrize("act", ["silu", "gelu", "relu"])
def test_gated_and_plain_forms(act):
    g, u, dh = (rng(4 + i).standard_normal((5, 40)) for i in range(3))
    h = oracle.glu_fwd(g, u, act)
    assert np.array_equal(h, oracle.act_value(g, act) * u)
    dg, du = oracle.glu_bwd(dh, g, u, act)
    assert np.array_equal(du, dh * oracle.act_value(g, act))
    assert np.array_equal(oracle.act_bwd(dh * u, g, act), dg)  # gate path = plain act
    if act == "silu":
        assert np.max(np.abs(h - oracle.swiglu_fwd(g, u))) < 1e-15
