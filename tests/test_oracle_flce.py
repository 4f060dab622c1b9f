"""Pins for the fp64 fused-linear-cross-entropy oracle.  No GPU."""
import math

import numpy as np
import torch

import oracle

IGN = -100


def rng(seed=0):
    return np.random.default_rng(seed)


def test_zero_weight_closed_form():
    # W = 0: every logit is 0, lse = log V, softmax = 1/V, so
    # loss = log V + c log^2 V, dH = 0, dW = (1/N) sum_valid ((1+2c log V)/V - onehot)^T h
    r = rng(0)
    T, Hd, V, c = 6, 5, 11, 1e-2
    Hm = r.standard_normal((T, Hd))
    t = np.array([0, 3, IGN, 10, 3, 7])
    out = oracle.flce_fwd_bwd(Hm, np.zeros((V, Hd)), t, z_loss=c)
    L = math.log(V)
    assert abs(out["loss"] - (L + c * L * L)) < 1e-13
    assert np.all(out["dhidden"] == 0)
    valid = t != IGN
    N = valid.sum()
    expect = np.zeros((V, Hd))
    for i in np.nonzero(valid)[0]:
        expect += np.outer(np.full(V, (1 + 2 * c * L) / V), Hm[i])
        expect[t[i]] -= Hm[i]
    expect /= N
    assert np.max(np.abs(out["dweight"] - expect)) < 1e-14


def test_matches_torch_autograd_f64():
    r = rng(1)
    T, Hd, V, c, dl = 9, 12, 23, 1e-3, 1.3
    Hm = r.standard_normal((T, Hd))
    W = r.standard_normal((V, Hd)) * 0.3
    t = r.integers(0, V, T)
    t[[0, 4]] = IGN
    ht = torch.from_numpy(Hm).requires_grad_()
    wt = torch.from_numpy(W).requires_grad_()
    tt = torch.from_numpy(t)
    z = ht @ wt.T
    lse = torch.logsumexp(z, dim=1)
    total = torch.nn.functional.cross_entropy(z, tt, ignore_index=IGN) + c * (lse[tt != IGN] ** 2).mean()
    (dl * total).backward()
    out = oracle.flce_fwd_bwd(Hm, W, t, z_loss=c, dloss=dl)
    assert abs(out["loss"] - total.item()) < 1e-13
    assert np.max(np.abs(out["dhidden"] - ht.grad.numpy())) < 1e-14
    assert np.max(np.abs(out["dweight"] - wt.grad.numpy())) < 1e-14


def test_finite_differences():
    r = rng(2)
    T, Hd, V, c = 4, 8, 16, 2e-2
    Hm = r.standard_normal((T, Hd))
    W = r.standard_normal((V, Hd)) * 0.5
    t = np.array([2, IGN, 15, 0])
    out = oracle.flce_fwd_bwd(Hm, W, t, z_loss=c)
    h = 1e-6

    def loss(Hx, Wx):
        return oracle.flce_fwd_bwd(Hx, Wx, t, z_loss=c)["loss"]

    for (i, j) in [(0, 0), (2, 7), (3, 3), (1, 5)]:
        Hp = Hm.copy(); Hp[i, j] += h
        Hn = Hm.copy(); Hn[i, j] -= h
        assert abs((loss(Hp, W) - loss(Hn, W)) / (2 * h) - out["dhidden"][i, j]) < 1e-8
    for (i, j) in [(0, 0), (15, 7), (2, 3), (9, 1)]:
        Wp = W.copy(); Wp[i, j] += h
        Wn = W.copy(); Wn[i, j] -= h
        assert abs((loss(Hm, Wp) - loss(Hm, Wn)) / (2 * h) - out["dweight"][i, j]) < 1e-8


def test_chunking_and_sampled_rows_do_not_change_results():
    r = rng(3)
    T, Hd, V = 13, 6, 19
    Hm = r.standard_normal((T, Hd))
    W = r.standard_normal((V, Hd))
    t = r.integers(0, V, T)
    t[5] = IGN
    a = oracle.flce_fwd_bwd(Hm, W, t, z_loss=1e-4)
    for ch in (1, 4, 5):
        b = oracle.flce_fwd_bwd(Hm, W, t, z_loss=1e-4, chunk=ch)
        assert abs(a["loss"] - b["loss"]) < 1e-13
        assert np.max(np.abs(a["dweight"] - b["dweight"])) < 1e-14
        assert np.max(np.abs(a["dhidden"] - b["dhidden"])) < 1e-14
    rows_h = np.array([12, 0, 5])
    rows_w = np.array([3, 18])
    s = oracle.flce_fwd_bwd(Hm, W, t, z_loss=1e-4, chunk=4, dh_rows=rows_h, dw_rows=rows_w)
    assert np.max(np.abs(s["dhidden"] - a["dhidden"][rows_h])) < 1e-14
    assert np.max(np.abs(s["dweight"] - a["dweight"][rows_w])) < 1e-14


def test_equals_xent_of_the_product():
    r = rng(4)
    Hm = r.standard_normal((5, 4))
    W = r.standard_normal((7, 4))
    t = np.array([0, 6, 2, IGN, 1])
    a = oracle.flce_fwd_bwd(Hm, W, t, z_loss=1e-3)
    b = oracle.xent_fwd_bwd(Hm @ W.T, t, z_loss=1e-3)
    assert abs(a["loss"] - b["loss"]) < 1e-14
    assert np.max(np.abs(a["dhidden"] - b["dlogits"] @ W)) < 1e-14


def test_row_blocks_with_the_batch_normaliser_add_up_to_the_batch():
    # rows are independent once N is fixed: blocks normalised by the batch's N sum to
    # the batch's loss and dW, and give the batch's dH rows (the full-size GPU parity
    # test maps blocks over threads this way)
    r = rng(5)
    T, Hd, V, c = 17, 6, 13, 1e-3
    Hm = r.standard_normal((T, Hd))
    W = r.standard_normal((V, Hd)) * 0.4
    t = r.integers(0, V, T)
    t[[1, 8, 9]] = IGN
    a = oracle.flce_fwd_bwd(Hm, W, t, z_loss=c, dloss=0.7)
    N = a["n_valid"]
    loss = zl = 0.0
    dW = np.zeros_like(a["dweight"])
    for b0 in (0, 5, 11):
        b1 = {0: 5, 5: 11, 11: T}[b0]
        b = oracle.flce_fwd_bwd(Hm[b0:b1], W, t[b0:b1], z_loss=c, dloss=0.7, n_norm=N)
        loss += b["loss"]
        zl += b["z_loss"]
        dW += b["dweight"]
        assert np.max(np.abs(b["dhidden"] - a["dhidden"][b0:b1])) < 1e-15
    assert abs(loss - a["loss"]) < 1e-13 and abs(zl - a["z_loss"]) < 1e-15
    assert np.max(np.abs(dW - a["dweight"])) < 1e-14


def test_abs_products_brute_force():
    # dhidden_abs[i, j] = sum_v |dZ[i, v]| |W[v, j]| and dweight_abs[v, j] =
    # sum_i |dZ[i, v]| |H[i, j]|, written out element by element from the logit gradient
    # of the plain cross-entropy of the product
    r = rng(6)
    T, Hd, V = 4, 3, 5
    Hm = r.standard_normal((T, Hd))
    W = r.standard_normal((V, Hd))
    t = np.array([4, IGN, 0, 2])
    out = oracle.flce_fwd_bwd(Hm, W, t, z_loss=1e-2, abs_products=True,
                              dh_rows=np.array([2, 0]), dw_rows=np.array([1, 4]))
    Z = [[sum(Hm[i, k] * W[v, k] for k in range(Hd)) for v in range(V)] for i in range(T)]
    dZ = oracle.xent_fwd_bwd(np.array(Z), t, z_loss=1e-2)["dlogits"]
    for a, i in enumerate((2, 0)):
        for j in range(Hd):
            e = sum(abs(dZ[i, v]) * abs(W[v, j]) for v in range(V))
            assert abs(out["dhidden_abs"][a, j] - e) < 1e-15
    for a, v in enumerate((1, 4)):
        for j in range(Hd):
            e = sum(abs(dZ[i, v]) * abs(Hm[i, j]) for i in range(T))
            assert abs(out["dweight_abs"][a, j] - e) < 1e-15
    # and the products bound the gradients themselves (triangle inequality)
    assert np.all(np.abs(out["dhidden"]) <= out["dhidden_abs"] + 1e-15)
    assert np.all(np.abs(out["dweight"]) <= out["dweight_abs"] + 1e-15)
