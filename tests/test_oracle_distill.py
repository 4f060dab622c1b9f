"""Pins for the fp64 soft-target (distillation) cross-entropy oracle.  No GPU."""
import numpy as np
import torch

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_matches_torch_soft_cross_entropy_and_kl_f64():
    z = rng(0).standard_normal((13, 300)) * 3
    zt = rng(1).standard_normal((13, 300)) * 2
    r = oracle.distill_fwd_bwd(z, zt)
    zz = torch.from_numpy(z).requires_grad_()
    p = torch.softmax(torch.from_numpy(zt), -1)
    ce = torch.nn.functional.cross_entropy(zz, p)  # probability targets, mean over rows
    ce.backward()
    kl = torch.nn.functional.kl_div(torch.log_softmax(torch.from_numpy(z), -1),
                                    torch.log_softmax(torch.from_numpy(zt), -1),
                                    reduction="batchmean", log_target=True)
    assert abs(r["loss"] - ce.item()) < 1e-12
    assert abs(r["kl"] - kl.item()) < 1e-12
    assert np.max(np.abs(r["dlogits"] - zz.grad.numpy())) < 1e-15


def test_hard_target_limit_is_the_cross_entropy():
    # a teacher with a 1000-logit margin is one-hot in fp64: the hard-label cross-entropy
    z = rng(2).standard_normal((9, 64)) * 2
    y = rng(3).integers(0, 64, 9)
    zt = np.zeros((9, 64))
    zt[np.arange(9), y] = 1000.0
    r = oracle.distill_fwd_bwd(z, zt)
    h = oracle.xent_fwd_bwd(z, y)
    assert abs(r["loss"] - h["loss"]) < 1e-13
    assert np.max(np.abs(r["dlogits"] - h["dlogits"])) < 1e-15
    assert abs(r["kl"] - r["loss"]) < 1e-13  # the teacher's entropy is 0


def test_teacher_equals_student():
    z = rng(4).standard_normal((5, 100))
    r = oracle.distill_fwd_bwd(z, z.copy())
    assert abs(r["kl"]) < 1e-14 and np.max(np.abs(r["dlogits"])) < 1e-18
    # the cross-entropy is then the entropy of softmax(z)
    lq = z - z.max(-1, keepdims=True)
    lq -= np.log(np.exp(lq).sum(-1, keepdims=True))
    assert abs(r["loss"] - np.mean(-np.sum(np.exp(lq) * lq, -1))) < 1e-13


def test_mask_and_gradient_sums():
    z = rng(5).standard_normal((10, 50))
    zt = rng(6).standard_normal((10, 50))
    mask = np.array([1, 0, 1, 1, 0, 1, 0, 0, 1, 1], dtype=np.uint8)
    r = oracle.distill_fwd_bwd(z, zt, mask, dloss=2.0)
    sub = oracle.distill_fwd_bwd(z[mask == 1], zt[mask == 1], dloss=2.0)
    assert r["n_valid"] == 6 and abs(r["loss"] - sub["loss"]) < 1e-14
    assert np.all(r["dlogits"][mask == 0] == 0)
    assert np.max(np.abs(r["dlogits"][mask == 1] - sub["dlogits"])) < 1e-16
    assert np.max(np.abs(r["dlogits"].sum(-1))) < 1e-15  # each gradient row sums to 0
    none = oracle.distill_fwd_bwd(z, zt, np.zeros(10, dtype=np.uint8))
    assert none["loss"] == 0.0 and none["n_valid"] == 0 and np.all(none["dlogits"] == 0)


def test_finite_differences():
    z = rng(7).standard_normal((3, 12))
    zt = rng(8).standard_normal((3, 12))
    d = oracle.distill_fwd_bwd(z, zt)["dlogits"]
    h = 1e-6
    for t, j in ((0, 0), (1, 5), (2, 11)):
        zp, zm = z.copy(), z.copy()
        zp[t, j] += h
        zm[t, j] -= h
        fd = (oracle.distill_fwd_bwd(zp, zt)["loss"] - oracle.distill_fwd_bwd(zm, zt)["loss"]) / (2 * h)
        assert abs(fd - d[t, j]) < 1e-8
