"""GPU parity on the degenerate shapes of the row ops: rows of one to three columns
(and an all-zero row), a single rotary pair per head and the widest head the rotary
kernel takes, a single hidden unit, one- and two-entry vocabularies, and empty batches."""
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check, check_loss, layernorm_y_terms, norm_dw_terms, xent_dz_terms

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX


def randn(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g)).to(synth.torch_dtype(dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [1, 2, 3])
def test_rmsnorm_tiny_rows(gpu, dtype, d):
    # With eps far below x^2 a one-column row's dx is eps/(x^2+eps) times its two terms,
    # a cancellation no fp32 bound covers; eps 0.5 keeps the gradient well conditioned.
    T, eps = 19, 0.5
    x, dy = randn((T, d), d, dtype), randn((T, d), d + 100, dtype)
    x[3] = 0  # zero row: rstd = eps^-1/2, y = 0, dx = rstd * w * dy
    w = (1 + 0.1 * randn((d,), d + 200, "f32")).to(synth.torch_dtype(dtype))
    xg, wg = x.to(DEV), w.to(DEV)
    y, rstd = gpu.fo_rmsnorm_fwd(xg, wg, eps)
    dx, dw = gpu.fo_rmsnorm_bwd(dy.to(DEV), xg, wg, rstd, eps)
    torch.cuda.synchronize()
    ry, rr = oracle.rmsnorm_fwd(x, w, eps)
    rdx, rdw = oracle.rmsnorm_bwd(dy, x, w, eps)
    check(y.cpu(), ry, dtype, "y", single_rounding=True)
    check(rstd.cpu(), rr, "f32", "rstd")
    check(dx.cpu(), rdx, dtype, "dx", single_rounding=True)
    check(dw.cpu(), rdw, "f32", "dw", scale=norm_dw_terms(dy, x, eps, False))
    assert torch.all(y[3].cpu() == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,hq,hk", [(2, 3, 1), (512, 4, 2)])
def test_rope_single_pair_and_widest_head(gpu, dtype, D, hq, hk):
    # D 2: one pair per head (the scalar path); D 512: the widest head, 16-byte vectors
    T = 21
    q, k = randn((T, hq, D), D, dtype), randn((T, hk, D), D + 1, dtype)
    pos = torch.arange(T, dtype=torch.int64) * 48611  # up to ~1e6
    qg, kg = q.to(DEV), k.to(DEV)
    gpu.fo_rope_fwd(qg, kg, pos.to(DEV), 1e4)
    torch.cuda.synchronize()
    rq, rk = oracle.rope_fwd(q, k, pos, 1e4)
    check(qg.cpu(), rq, dtype, "q", single_rounding=True)
    check(kg.cpu(), rk, dtype, "k", single_rounding=True)
    fq, fk = qg.cpu(), kg.cpu()  # the forward's outputs, the backward's inputs
    gpu.fo_rope_bwd(qg, kg, pos.to(DEV), 1e4)
    torch.cuda.synchronize()
    bq, bk = oracle.rope_bwd(fq, fk, pos, 1e4)
    check(qg.cpu(), bq, dtype, "dq", single_rounding=True)
    check(kg.cpu(), bk, dtype, "dk", single_rounding=True)
    # the round trip returns the inputs to within two roundings
    check(qg.cpu(), q, dtype, "q round trip")
    check(kg.cpu(), k, dtype, "k round trip")


def test_empty_batches(gpu):
    for dt in (torch.float32, torch.bfloat16):
        q = torch.empty(0, 4, 64, dtype=dt, device=DEV)
        k = torch.empty(0, 2, 64, dtype=dt, device=DEV)
        pos = torch.empty(0, dtype=torch.int64, device=DEV)
        gpu.fo_rope_fwd(q, k, pos, 1e4)
        gpu.fo_rope_bwd(q, k, pos, 1e4)
        g = torch.empty(0, 96, dtype=dt, device=DEV)
        h = gpu.fo_swiglu_fwd(g, g)
        dg, du = gpu.fo_swiglu_bwd(h, g, g)
        y, rstd = gpu.fo_rmsnorm_fwd(torch.empty(0, 96, dtype=dt, device=DEV),
                                     torch.ones(96, dtype=dt, device=DEV), 1e-5)
        torch.cuda.synchronize()
        assert h.shape == (0, 96) and dg.shape == (0, 96) and du.shape == (0, 96)
        assert y.shape == (0, 96) and rstd.shape == (0,)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_swiglu_single_unit(gpu, dtype):
    T = 33
    g, u, dh = randn((T, 1), 1, dtype, 3.0), randn((T, 1), 2, dtype), randn((T, 1), 3, dtype)
    h = gpu.fo_swiglu_fwd(g.to(DEV), u.to(DEV))
    dg, du = gpu.fo_swiglu_bwd(dh.to(DEV), g.to(DEV), u.to(DEV))
    torch.cuda.synchronize()
    check(h.cpu(), oracle.swiglu_fwd(g, u), dtype, "h", single_rounding=True)
    rg, ru = oracle.swiglu_bwd(dh, g, u)
    check(dg.cpu(), rg, dtype, "dgate", single_rounding=True)
    check(du.cpu(), ru, dtype, "dup", single_rounding=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2])
@pytest.mark.parametrize("zc", [1e-3, 0.0])
def test_xent_one_and_two_classes(gpu, dtype, V, zc):
    # V 1: p = 1 and lse = z, so the loss is the z-loss alone and dz = 2 c lse / N (with no
    # z-loss, dz = 0: the difference of p = 1 and the one-hot, exact only to the size of
    # those terms, hence the term-size bound)
    T = 17
    z = randn((T, V), V, dtype, 2.0)
    t = torch.randint(0, V, (T,), generator=torch.Generator().manual_seed(V))
    t[4] = IGN
    o = gpu.fo_xent_fwd_bwd(z.to(DEV), t.to(DEV), IGN, zc, 1.0)
    torch.cuda.synchronize()
    r = oracle.xent_fwd_bwd(z, t, IGN, zc, 1.0)
    assert o["n_valid"].item() == r["n_valid"] == T - 1
    check_loss(o["loss"].item(), r["loss"])
    check_loss(o["z_loss"].item(), r["z_loss"], "z_loss")
    check(o["dlogits"].cpu(), r["dlogits"], dtype, "dlogits", single_rounding=True,
          scale=xent_dz_terms(z, t.numpy(), t != IGN, r["lse"], zc, 1.0, r["n_valid"]))
    assert torch.all(o["dlogits"][4].cpu().float() == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [1, 2, 3])
def test_layernorm_tiny_rows(gpu, dtype, d):
    # d 1: the centred row is exactly zero, so y = b exactly; the kernels form g - mean(g)
    # before scaling it, which is exactly 0 in a one-column row, so dx is exactly zero
    # as the reference is; eps 0.5 as for RMSNorm above
    T, eps = 19, 0.5
    td = synth.torch_dtype(dtype)
    x, dy = randn((T, d), d + 7, dtype), randn((T, d), d + 107, dtype)
    x[5] = 0
    w = (1 + 0.1 * randn((d,), d + 207, "f32")).to(td)
    b = (0.1 * randn((d,), d + 307, "f32")).to(td)
    xg, wg = x.to(DEV), w.to(DEV)
    y, mean, rstd = gpu.fo_layernorm_fwd(xg, wg, b.to(DEV), eps)
    dx, dw, db = gpu.fo_layernorm_bwd(dy.to(DEV), xg, wg, mean, rstd)
    torch.cuda.synchronize()
    ry, rmu, rr = oracle.layernorm_fwd(x, w, b, eps)
    rdx, rdw, rdb = oracle.layernorm_bwd(dy, x, w, eps)
    check(y.cpu(), ry, dtype, "y", single_rounding=True, scale=layernorm_y_terms(x, w, b, eps))
    check(mean.cpu(), rmu, "f32", "mean")
    check(rstd.cpu(), rr, "f32", "rstd")
    check(dx.cpu(), rdx, dtype, "dx", single_rounding=True)
    check(dw.cpu(), rdw, "f32", "dw", scale=norm_dw_terms(dy, x, eps, True))
    check(db.cpu(), rdb, "f32", "db")
    if d == 1:
        assert torch.equal(y.cpu(), b.expand(T, 1))
        assert torch.all(dx.cpu() == 0)


@pytest.mark.parametrize("act", ["silu", "gelu", "relu"])
def test_activation_single_unit(gpu, act):
    T = 29
    x, dy = randn((T, 1), 11, "bf16", 3.0), randn((T, 1), 12, "bf16")
    y = gpu.fo_act_fwd(act, x.to(DEV))
    dx = gpu.fo_act_bwd(act, dy.to(DEV), x.to(DEV))
    torch.cuda.synchronize()
    check(y.cpu(), oracle.act_fwd(x, act), "bf16", "y", single_rounding=True)
    check(dx.cpu(), oracle.act_bwd(dy, x, act), "bf16", "dx", single_rounding=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2])
def test_distill_one_and_two_classes(gpu, dtype, V):
    # V 1: both distributions are the point mass, so loss, KL and gradient vanish
    T = 13
    z, zt = randn((T, V), 21 + V, dtype, 2.0), randn((T, V), 31 + V, dtype, 2.0)
    o = gpu.fo_distill_fwd_bwd(z.to(DEV), zt.to(DEV), None, 1.0)
    torch.cuda.synchronize()
    r = oracle.distill_fwd_bwd(z, zt, None, 1.0)
    assert o["n_valid"].item() == r["n_valid"] == T
    check_loss(o["loss"].item(), r["loss"])
    check_loss(o["kl"].item(), r["kl"], "kl")
    check(o["dlogits"].cpu(), r["dlogits"], dtype, "dlogits")
    if V == 1:
        assert abs(o["loss"].item()) <= 1e-6 and abs(o["kl"].item()) <= 1e-6
        assert o["dlogits"].cpu().float().abs().max().item() <= 1e-7
