"""Non-finite inputs propagate to the outputs and nothing traps: NaN and +-Inf are placed
in a few rows (or elements) of otherwise ordinary inputs; wherever the fp64 oracle's
result is non-finite the kernel's is too, and everywhere else the kernel's result is
finite and within the usual bound.  Rows (and, for elementwise ops, elements) that hold
no non-finite input give exactly the values of a call without any."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX
NAN, INF = float("nan"), float("inf")


def rnd(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(dtype)


def agree(g, r, dt, name):
    """Non-finite where the oracle is; finite and within the bound elsewhere."""
    g = g.detach().to("cpu", torch.float64).numpy()
    r = np.asarray(r, dtype=np.float64)
    bad = ~np.isfinite(r)
    assert np.all(~np.isfinite(g[bad])), f"{name}: finite where the oracle is not"
    assert np.all(np.isfinite(g[~bad])), f"{name}: non-finite where the oracle is finite"
    if (~bad).any():
        check(g[~bad], r[~bad], "bf16" if dt == torch.bfloat16 else "f32", name)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rmsnorm(gpu, dtype):
    T, d = 11, 1024
    x, dy, w = rnd((T, d), 1, dtype), rnd((T, d), 2, dtype), (1 + 0.1 * rnd((d,), 3, torch.float32)).to(dtype)
    x[3, 7] = NAN
    x[5, 100] = INF
    dy[8, 9] = -INF
    y, r = gpu.fo_rmsnorm_fwd(x.to(DEV), w.to(DEV), 1e-5)
    dx, dw = gpu.fo_rmsnorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), r, 1e-5)
    torch.cuda.synchronize()
    ry, _ = oracle.rmsnorm_fwd(x, w, 1e-5)
    rdx, rdw = oracle.rmsnorm_bwd(dy, x, w, 1e-5)
    agree(y.cpu(), ry, dtype, "y")
    agree(dx.cpu(), rdx, dtype, "dx")
    agree(dw.cpu(), rdw, torch.float32, "dw")
    clean = [0, 1, 2, 4, 6, 7, 9, 10]
    y0, _ = gpu.fo_rmsnorm_fwd(x[clean].to(DEV), w.to(DEV), 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu()[clean], y0.cpu())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope(gpu, dtype):
    T, D = 9, 128
    q, k = rnd((T, 4, D), 4, dtype), rnd((T, 2, D), 5, dtype)
    q[2, 1, 5] = NAN
    k[6, 0, 70] = INF
    pos = torch.arange(T) * 101
    gq, gk = q.to(DEV), k.to(DEV)
    gpu.fo_rope_fwd(gq, gk, pos.to(DEV), 1e4)
    torch.cuda.synchronize()
    rq, rk = oracle.rope_fwd(q, k, pos, 1e4)
    agree(gq.cpu(), rq, dtype, "q")
    agree(gk.cpu(), rk, dtype, "k")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_swiglu(gpu, dtype):
    T, F = 7, 1408
    g, u, dh = rnd((T, F), 6, dtype), rnd((T, F), 7, dtype), rnd((T, F), 8, dtype)
    g[1, 3], g[2, 4], g[3, 5], u[4, 6], dh[5, 7] = NAN, INF, -INF, INF, NAN
    h = gpu.fo_swiglu_fwd(g.to(DEV), u.to(DEV))
    dg, du = gpu.fo_swiglu_bwd(dh.to(DEV), g.to(DEV), u.to(DEV))
    torch.cuda.synchronize()
    agree(h.cpu(), oracle.swiglu_fwd(g, u), dtype, "h")
    rg, ru = oracle.swiglu_bwd(dh, g, u)
    agree(dg.cpu(), rg, dtype, "dgate")
    agree(du.cpu(), ru, dtype, "dup")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [4096, 128256, 151936])
def test_cross_entropy(gpu, dtype, V):
    # register-resident, LDS-prefetch and streamed rows
    T = 6
    z = rnd((T, V), 9, dtype, 2.0)
    g = torch.Generator().manual_seed(10)
    t = torch.randint(0, V, (T,), generator=g)
    z[1, 17] = NAN
    z[3, (int(t[3]) + 1) % V] = INF
    o = gpu.fo_xent_fwd_bwd(z.to(DEV), t.to(DEV), IGN, 1e-4, 1.0)
    torch.cuda.synchronize()
    r = oracle.xent_fwd_bwd(z, t, IGN, 1e-4, 1.0)
    assert not np.isfinite(r["loss"]) and not np.isfinite(o["loss"].item())
    # the gradient rows of the rows without non-finite logits stay exact: the scale N
    # counts rows, not values
    clean = [0, 2, 4, 5]
    agree(o["dlogits"].cpu()[clean], r["dlogits"][clean], dtype, "dlogits clean rows")
    assert not torch.isfinite(o["dlogits"].cpu()[1]).all()


def test_flce(gpu):
    cfg = synth.flce_small(40, 64, 1000, seed=11, ignore_frac=0.0)
    i = synth.flce_inputs(cfg)
    h = i["hidden"].clone()
    h[7, 3] = NAN
    o = gpu.fo_flce_fwd_bwd(h.to(DEV), i["weight"].to(DEV), i["targets"].to(DEV), IGN,
                            cfg.z_loss, 1.0, chunk_tokens=16)
    torch.cuda.synchronize()
    r = oracle.flce_fwd_bwd(h, i["weight"], i["targets"], IGN, cfg.z_loss, 1.0)
    assert not np.isfinite(r["loss"]) and not np.isfinite(o["loss"].item())
    agree(o["dhidden"].cpu(), r["dhidden"], torch.bfloat16, "dhidden")
    assert not torch.isfinite(o["dweight"].cpu()).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_layernorm_and_distillation(gpu, dtype):
    T, d = 8, 512
    x, dy = rnd((T, d), 12, dtype), rnd((T, d), 13, dtype)
    w, b = (1 + 0.1 * rnd((d,), 14, torch.float32)).to(dtype), (0.1 * rnd((d,), 15, torch.float32)).to(dtype)
    x[2, 9] = NAN
    y, m, s = gpu.fo_layernorm_fwd(x.to(DEV), w.to(DEV), b.to(DEV), 1e-5)
    dx, dw, db = gpu.fo_layernorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), m, s)
    torch.cuda.synchronize()
    ry, _, _ = oracle.layernorm_fwd(x, w, b, 1e-5)
    rdx, rdw, rdb = oracle.layernorm_bwd(dy, x, w, 1e-5)
    agree(y.cpu(), ry, dtype, "layernorm y")
    agree(dx.cpu(), rdx, dtype, "layernorm dx")
    agree(db.cpu(), rdb, torch.float32, "layernorm db")
    z, zt = rnd((T, 5000), 16, dtype, 2.0), rnd((T, 5000), 17, dtype, 2.0)
    zt[4, 11] = INF
    o = gpu.fo_distill_fwd_bwd(z.to(DEV), zt.to(DEV), None)
    torch.cuda.synchronize()
    rr = oracle.distill_fwd_bwd(z, zt, None)
    assert not np.isfinite(rr["loss"]) and not np.isfinite(o["loss"].item())
    clean = [0, 1, 2, 3, 5, 6, 7]
    agree(o["dlogits"].cpu()[clean], rr["dlogits"][clean], dtype, "distill dlogits clean rows")
