"""Pins for the fp64 AdamW oracle.  No GPU."""
import numpy as np
import torch

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_first_step_closed_form():
    # zero moments, t = 1: step_size * m' = lr * g and sqrt(v') / bias_correction = |g|,
    # so p' = (1 - lr wd) p - lr g / (|g| + eps)
    p = rng(0).standard_normal(1000)
    g = rng(1).standard_normal(1000) * 1e-3
    lr, b1, b2, wd, eps = 3e-4, 0.9, 0.95, 0.1, 1e-8
    ss, bc, df = oracle.adamw_scalars(lr, b1, b2, wd, 1)
    p1, m1, v1 = oracle.adamw_step(p, g, np.zeros(1000), np.zeros(1000), ss, b1, b2, bc, df, eps)
    ref = (1 - lr * wd) * p - lr * g / (np.abs(g) + eps)
    assert np.max(np.abs(p1 - ref)) < 1e-15
    assert np.max(np.abs(m1 - 0.1 * g)) < 1e-18 and np.max(np.abs(v1 - 0.05 * g * g)) < 1e-20
    # the update moves against the gradient
    assert np.all(np.sign(p1 - (1 - lr * wd) * p) == -np.sign(g))


def test_noop_changes_nothing():
    a = [rng(i).standard_normal(50) for i in range(4)]
    a[3] = np.abs(a[3])
    out = oracle.adamw_step(*a, 1e-3, 0.9, 0.999, 0.5, 0.99, 1e-8, grad_scale=7.0, noop=True)
    for x, y in zip(out, (a[0], a[2], a[3])):
        assert np.array_equal(x, y)


def test_grad_scale_is_a_gradient_multiplier():
    p, g, m = (rng(i).standard_normal(100) for i in range(3))
    v = np.abs(rng(3).standard_normal(100))
    args = (1e-3, 0.9, 0.999, 0.3, 0.999, 1e-8)
    a = oracle.adamw_step(p, g, m, v, *args, grad_scale=0.125)
    b = oracle.adamw_step(p, 0.125 * g, m, v, *args)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-15 * np.max(np.abs(y))


def test_zero_lr_keeps_parameters():
    p, g, m = (rng(i).standard_normal(100) for i in range(3))
    v = np.abs(rng(3).standard_normal(100))
    ss, bc, df = oracle.adamw_scalars(0.0, 0.9, 0.999, 0.1, 3)
    p1, m1, v1 = oracle.adamw_step(p, g, m, v, ss, 0.9, 0.999, bc, df, 1e-8)
    assert np.array_equal(p1, p)
    assert np.max(np.abs(m1 - (0.9 * m + 0.1 * g))) < 1e-15


def test_matches_torch_adamw_f64():
    # torch.optim.AdamW (decoupled weight decay, bias-corrected) in fp64 over five steps,
    # with different gradients each step; an L2-coupled decay (torch.optim.Adam with
    # weight_decay) must not match
    lr, b1, b2, wd, eps = 1e-3, 0.9, 0.95, 0.1, 1e-8
    p0 = rng(10).standard_normal(257)
    grads = [rng(20 + t).standard_normal(257) * 10 ** (-t) for t in range(5)]
    pt = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([pt], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    p, m, v = p0.copy(), np.zeros(257), np.zeros(257)
    for t, g in enumerate(grads, start=1):
        pt.grad = torch.from_numpy(g.copy())
        opt.step()
        ss, bc, df = oracle.adamw_scalars(lr, b1, b2, wd, t)
        p, m, v = oracle.adamw_step(p, g, m, v, ss, b1, b2, bc, df, eps)
        st = opt.state[pt]
        for mine, ref in ((p, pt.detach().numpy()), (m, st["exp_avg"].numpy()),
                          (v, st["exp_avg_sq"].numpy())):
            assert np.max(np.abs(mine - ref)) <= 1e-13 * np.max(np.abs(ref))
    q = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt2 = torch.optim.Adam([q], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    for g in grads:
        q.grad = torch.from_numpy(g.copy())
        opt2.step()
    assert np.max(np.abs(p - q.detach().numpy())) > 1e-6


def test_synthetic_inputs_shapes_and_signs():
    from reduction_rmsnorm_fwd_amd import synth
    i = synth.adamw_inputs([3, 0, 70], seed=4)
    assert [t.numel() for t in i["params"]] == [3, 0, 70]
    assert all(t.dtype == torch.float32 for k in i for t in i[k])
    assert all(bool((t >= 0).all()) for t in i["exp_avg_sqs"])
    j = synth.adamw_inputs([3, 0, 70], seed=4)
    assert all(torch.equal(a, b) for k in i for a, b in zip(i[k], j[k]))
