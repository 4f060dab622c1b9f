"""Pins for the fp64 cross-entropy (+ z-loss, ignore_index) oracle.  No GPU."""
import math

import numpy as np
import torch

import oracle

IGN = -100


def rng(seed=0):
    return np.random.default_rng(seed)


def test_hand_worked_two_class_row():
    # logits (0, ln 3), target 1: softmax = (1/4, 3/4), loss = -ln(3/4) = ln(4/3),
    # gradient = softmax - onehot = (1/4, -1/4).
    out = oracle.xent_fwd_bwd(np.array([[0.0, math.log(3.0)]]), np.array([1]))
    assert abs(out["loss"] - math.log(4.0 / 3.0)) < 1e-15
    assert np.max(np.abs(out["dlogits"] - np.array([[0.25, -0.25]]))) < 1e-15
    assert abs(out["lse"][0] - math.log(4.0)) < 1e-15


def test_uniform_logits_give_log_v():
    for V in (4096, 151936, 128256, 49152):
        z = np.full((3, V), 1.75)
        t = np.array([0, V - 1, 17])
        out = oracle.xent_fwd_bwd(z, t)
        assert abs(out["loss"] - math.log(V)) < 1e-10
        # with z-loss the lse is c + log V, so loss = log V + cz (c + log V)^2
        outz = oracle.xent_fwd_bwd(z, t, z_loss=1e-4)
        assert abs(outz["loss"] - (math.log(V) + 1e-4 * (1.75 + math.log(V)) ** 2)) < 1e-10
        assert abs(outz["z_loss"] - 1e-4 * (1.75 + math.log(V)) ** 2) < 1e-12


def test_gradient_row_sums_and_ignored_rows():
    r = rng(0)
    z = r.standard_normal((6, 50)) * 2
    t = np.array([3, IGN, 49, 0, IGN, 7])
    out = oracle.xent_fwd_bwd(z, t, z_loss=0.0, dloss=1.0)
    assert out["n_valid"] == 4
    s = out["dlogits"].sum(axis=1)
    assert np.max(np.abs(s)) < 1e-15
    assert np.all(out["dlogits"][[1, 4]] == 0)
    c = 3e-3
    outz = oracle.xent_fwd_bwd(z, t, z_loss=c, dloss=2.0)
    sz = outz["dlogits"].sum(axis=1)
    expect = 2 * c * outz["lse"] * 2.0 / 4
    valid = t != IGN
    assert np.max(np.abs(sz[valid] - expect[valid])) < 1e-15
    assert np.all(outz["dlogits"][~valid] == 0)


def test_loss_nonnegative_and_dominant_target():
    z = rng(1).standard_normal((5, 30))
    t = np.arange(5)
    assert oracle.xent_fwd_bwd(z, t)["loss"] >= 0
    z[np.arange(5), t] = 200.0
    assert oracle.xent_fwd_bwd(z, t)["loss"] < 1e-50


def test_matches_torch_cross_entropy_f64():
    r = rng(2)
    z = r.standard_normal((12, 97)) * 3
    t = r.integers(0, 97, 12)
    t[[2, 5, 6]] = IGN
    zt = torch.from_numpy(z).requires_grad_()
    ref = torch.nn.functional.cross_entropy(zt, torch.from_numpy(t), ignore_index=IGN)
    ref.backward()
    out = oracle.xent_fwd_bwd(z, t)
    assert abs(out["loss"] - ref.item()) < 1e-13
    assert np.max(np.abs(out["dlogits"] - zt.grad.numpy())) < 1e-15


def test_z_loss_gradient_matches_autograd_with_library_logsumexp():
    r = rng(3)
    z = r.standard_normal((8, 40)) * 3
    t = r.integers(0, 40, 8)
    t[1] = IGN
    c, dl = 1e-2, 1.5
    zt = torch.from_numpy(z).requires_grad_()
    tt = torch.from_numpy(t)
    keep = tt != IGN
    lse = torch.logsumexp(zt, dim=1)
    total = torch.nn.functional.cross_entropy(zt, tt, ignore_index=IGN) + c * (lse[keep] ** 2).mean()
    (dl * total).backward()
    out = oracle.xent_fwd_bwd(z, t, z_loss=c, dloss=dl)
    assert abs(out["loss"] - total.item()) < 1e-13
    assert np.max(np.abs(out["dlogits"] - zt.grad.numpy())) < 1e-14


def test_finite_differences_with_z_loss_and_ignore():
    r = rng(4)
    T, V = 4, 16
    z = r.standard_normal((T, V)) * 2
    t = np.array([1, IGN, 15, 4])
    c, dl = 5e-2, 0.7
    g = oracle.xent_fwd_bwd(z, t, z_loss=c, dloss=dl)["dlogits"]
    h = 1e-6
    fd = np.zeros_like(z)
    for i in range(T):
        for j in range(V):
            zp = z.copy(); zp[i, j] += h
            zm = z.copy(); zm[i, j] -= h
            fd[i, j] = dl * (oracle.xent_fwd_bwd(zp, t, z_loss=c)["loss"]
                             - oracle.xent_fwd_bwd(zm, t, z_loss=c)["loss"]) / (2 * h)
    assert np.max(np.abs(g - fd)) < 1e-8


def test_all_ignored_and_bad_targets():
    z = rng(5).standard_normal((3, 10))
    out = oracle.xent_fwd_bwd(z, np.array([IGN, IGN, IGN]))
    assert out["n_valid"] == 0 and out["loss"] == 0.0 and np.all(out["dlogits"] == 0)
    out = oracle.xent_fwd_bwd(z, np.array([10, -1, 3]))
    assert out["n_bad"] == 2 and out["n_valid"] == 1
    assert np.all(out["dlogits"][:2] == 0)
    ref = oracle.xent_fwd_bwd(z[2:], np.array([3]))
    assert abs(out["loss"] - ref["loss"]) < 1e-15


def test_random_logits_lse_statistics():
    # logits iid N(0, s^2): E[exp z] = exp(s^2/2), so lse ~ log V + s^2/2 for large V
    V, s = 128256, 3.0
    z = rng(6).standard_normal((4, V)) * s
    lse = oracle.xent_fwd_bwd(z, np.zeros(4, np.int64))["lse"]
    assert np.all(np.abs(lse - (math.log(V) + s * s / 2)) < 0.15)
