"""Pins for the fp64 RoPE oracle (half-split pairing, frequencies theta^(-2i/D)).
No GPU."""
import numpy as np

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_position_zero_is_identity():
    q = rng(0).standard_normal((3, 4, 16))
    k = rng(1).standard_normal((3, 2, 16))
    a, b = oracle.rope_fwd(q, k, np.zeros(3, np.int64), 1e4)
    assert np.array_equal(a, q) and np.array_equal(b, k)


def test_head_dim_two_is_complex_multiplication():
    # D = 2: the single pair (x0, x1) is rotated by exactly pos radians
    x = rng(2).standard_normal((5, 3, 2))
    pos = np.array([0, 1, 7, 300, 16383])
    out, _ = oracle.rope_fwd(x, x[:, :1], pos, 5e5)
    zc = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos)[:, None]
    assert np.max(np.abs(out[..., 0] - zc.real)) < 1e-12
    assert np.max(np.abs(out[..., 1] - zc.imag)) < 1e-12


def test_frequency_exponent_closed_form():
    # theta = 1e4, D = 8: frequencies 10000^(-2i/8) = 10^-i exactly, i = 0..3; the pair
    # of element i is element i+4.
    D = 8
    pos = np.array([3, 250, 8191])
    x = np.zeros((3, 1, D))
    x[:, 0, :4] = 1.0  # every pair starts at (1, 0)
    out, _ = oracle.rope_fwd(x, x, pos, 1e4)
    for i in range(4):
        ang = pos * 10.0 ** (-i)
        assert np.max(np.abs(out[:, 0, i] - np.cos(ang))) < 1e-12
        assert np.max(np.abs(out[:, 0, i + 4] - np.sin(ang))) < 1e-12


def test_pair_norms_preserved():
    q = rng(3).standard_normal((6, 5, 32))
    pos = rng(4).integers(0, 20000, 6)
    a, _ = oracle.rope_fwd(q, q[:, :1], pos, 1e6)
    n0 = q[..., :16] ** 2 + q[..., 16:] ** 2
    n1 = a[..., :16] ** 2 + a[..., 16:] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12


def test_scores_depend_only_on_relative_position():
    r = rng(5)
    D = 64
    q = r.standard_normal((1, 1, D))
    k = r.standard_normal((1, 1, D))
    for m, n, s in [(5, 2, 100), (0, 40, 1000), (300, 299, 7000)]:
        qa, ka = oracle.rope_fwd(q, k, np.array([m]), 1e4)
        _, kb = oracle.rope_fwd(q, k, np.array([n]), 1e4)
        qs, _ = oracle.rope_fwd(q, k, np.array([m + s]), 1e4)
        _, ks = oracle.rope_fwd(q, k, np.array([n + s]), 1e4)
        assert abs(np.sum(qa * kb) - np.sum(qs * ks)) < 1e-12


def test_backward_is_inverse_and_adjoint():
    r = rng(6)
    q = r.standard_normal((4, 3, 16))
    k = r.standard_normal((4, 1, 16))
    g = r.standard_normal((4, 3, 16))
    pos = np.array([0, 5, 77, 1234])
    fq, fk = oracle.rope_fwd(q, k, pos, 1e4)
    bq, bk = oracle.rope_bwd(fq, fk, pos, 1e4)
    assert np.max(np.abs(bq - q)) < 1e-13 and np.max(np.abs(bk - k)) < 1e-13
    # <R q, g> = <q, R^T g>
    gq, _ = oracle.rope_bwd(g, k, pos, 1e4)
    assert abs(np.sum(fq * g) - np.sum(q * gq)) < 1e-12


def test_backward_finite_differences():
    # rope is linear in q, so the directional derivative of <rope(q), g> along e is
    # <rope(e), g>; compare with <e, rope_bwd(g)> for random directions.
    r = rng(7)
    q = r.standard_normal((2, 2, 8))
    g = r.standard_normal((2, 2, 8))
    pos = np.array([3, 9])
    gq, _ = oracle.rope_bwd(g, g, pos, 1e4)
    for _ in range(5):
        e = r.standard_normal(q.shape)
        h = 1e-6
        fp = np.sum(oracle.rope_fwd(q + h * e, q, pos, 1e4)[0] * g)
        fm = np.sum(oracle.rope_fwd(q - h * e, q, pos, 1e4)[0] * g)
        assert abs((fp - fm) / (2 * h) - np.sum(e * gq)) < 1e-8


def test_packed_documents_equal_separate_runs():
    r = rng(8)
    q = r.standard_normal((7, 2, 8))
    pos = np.array([0, 1, 2, 0, 1, 0, 1])
    a, _ = oracle.rope_fwd(q, q, pos, 1e4)
    for lo, hi in [(0, 3), (3, 5), (5, 7)]:
        b, _ = oracle.rope_fwd(q[lo:hi], q[lo:hi], np.arange(hi - lo), 1e4)
        assert np.array_equal(a[lo:hi], b)
