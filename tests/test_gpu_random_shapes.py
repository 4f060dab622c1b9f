"""GPU parity on seeded random shapes: widths of any length and alignment, bases off the
16-byte grid, padded row strides, odd head counts and vocabularies, against the fp64
oracle under the same bounds as the targeted tests.  Every case prints its parameters in
the assertion message."""
import sys

import numpy as np
import pytest
import torch

import oracle
from tolerance import (check, check_loss, check_softmax_diff, kl_terms, layernorm_y_terms,
                       norm_dw_terms, norm_dx_terms, xent_dz_terms)
from test_gpu_distill import softmax_sum

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = -100
TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def width(g):
    # short rows, rows around the vector and wave boundaries, and long rows
    return int(g.choice([g.integers(1, 17), g.integers(17, 600), g.integers(600, 4200),
                         g.integers(4200, 9000)]))


def norm_width(g):
    # width(), or rows the norms spread over 2-16 waves (forward) or hand to the
    # workgroup-per-row kernels (backward beyond 16384)
    return width(g) if g.random() < 0.75 else int(g.integers(9000, 40000))


# operand magnitudes: None, or factors one of which scales each operand (drawn per view)
MAGS = None


def view(g, T, n, dt, scale=1.0, shift=0.0):
    """A [T, n] view into a larger buffer: base 0-7 elements off, row stride n + 0-9; the
    view (on the device) and its values (on the host).  With MAGS set, the values are
    scaled by one of its factors, drawn per view."""
    if MAGS is not None:
        f = MAGS[int(g.integers(0, len(MAGS)))]
        scale, shift = scale * f, shift * f
    off, pad = int(g.integers(0, 8)), int(g.integers(0, 10))
    buf = torch.from_numpy(g.standard_normal((T, n + off + pad)) * scale + shift).float().to(TD[dt])
    return buf.to(DEV)[:, off:off + n], buf[:, off:off + n].clone()


def cases(n, seed):
    g = np.random.default_rng(seed)
    return [(int(s), "bf16" if s % 3 else "f32") for s in g.integers(0, 2**31, n)]


@pytest.mark.parametrize("seed,dt", cases(40, 1))
def test_rmsnorm(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T, d = int(g.integers(1, 300)), norm_width(g)
    eps = float(g.choice([1e-6, 1e-5]))
    x, xh = view(g, T, d, dt)
    dy, dyh = view(g, T, d, dt)
    w, wh = view(g, 1, d, dt, 0.1, 1.0)
    y, rstd = gpu.fo_rmsnorm_fwd(x, w[0], eps)
    dx, dw = gpu.fo_rmsnorm_bwd(dy, x, w[0], rstd, eps)
    torch.cuda.synchronize()
    ry, rr = oracle.rmsnorm_fwd(xh, wh[0], eps)
    rdx, rdw = oracle.rmsnorm_bwd(dyh, xh, wh[0], eps)
    tag = f"rmsnorm seed={seed} {dt} T={T} d={d}"
    check(y.cpu(), ry, dt, tag + " y", single_rounding=True)
    check(rstd.cpu(), rr, "f32", tag + " rstd")
    check(dx.cpu(), rdx, dt, tag + " dx", single_rounding=True,
          scale=norm_dx_terms(dyh, xh, wh[0], eps, False))
    check(dw.cpu(), rdw, "f32", tag + " dw", scale=norm_dw_terms(dyh, xh, eps, False))


@pytest.mark.parametrize("seed,dt", cases(30, 2))
def test_layernorm(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T, d = int(g.integers(1, 300)), norm_width(g)
    x, xh = view(g, T, d, dt, 1.0, 0.5)
    dy, dyh = view(g, T, d, dt)
    w, wh = view(g, 1, d, dt, 0.1, 1.0)
    b, bh = view(g, 1, d, dt, 0.1)
    y, mean, rstd = gpu.fo_layernorm_fwd(x, w[0], b[0], 1e-5)
    dx, dw, db = gpu.fo_layernorm_bwd(dy, x, w[0], mean, rstd)
    torch.cuda.synchronize()
    ry, rm, rr = oracle.layernorm_fwd(xh, wh[0], bh[0], 1e-5)
    rdx, rdw, rdb = oracle.layernorm_bwd(dyh, xh, wh[0], 1e-5)
    tag = f"layernorm seed={seed} {dt} T={T} d={d}"
    check(y.cpu(), ry, dt, tag + " y", single_rounding=True,
          scale=layernorm_y_terms(xh, wh[0], bh[0], 1e-5))
    check(mean.cpu(), rm, "f32", tag + " mean")
    check(rstd.cpu(), rr, "f32", tag + " rstd")
    check(dx.cpu(), rdx, dt, tag + " dx", single_rounding=True,
          scale=norm_dx_terms(dyh, xh, wh[0], 1e-5, True))
    check(dw.cpu(), rdw, "f32", tag + " dw", scale=norm_dw_terms(dyh, xh, 1e-5, True))
    check(db.cpu(), rdb, "f32", tag + " db")


@pytest.mark.parametrize("seed,dt", cases(30, 3))
def test_swiglu(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T, F = int(g.integers(1, 200)), width(g)
    gate, gh = view(g, T, F, dt, 2.0)
    up, uh = view(g, T, F, dt)
    dh, dhh = view(g, T, F, dt)
    h = gpu.fo_swiglu_fwd(gate, up)
    dg, du = gpu.fo_swiglu_bwd(dh, gate, up)
    torch.cuda.synchronize()
    rg, ru = oracle.swiglu_bwd(dhh, gh, uh)
    tag = f"swiglu seed={seed} {dt} T={T} F={F}"
    check(h.cpu(), oracle.swiglu_fwd(gh, uh), dt, tag + " h", single_rounding=True)
    check(dg.cpu(), rg, dt, tag + " dgate", single_rounding=True)
    check(du.cpu(), ru, dt, tag + " dup", single_rounding=True)


@pytest.mark.parametrize("seed,dt", cases(30, 4))
def test_rope(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 100))
    nkv = int(g.integers(1, 5))
    nq = nkv * int(g.integers(1, 5))
    D = 2 * int(g.integers(1, 129))
    theta = float(g.choice([1e4, 5e5, 1e6]))
    # packed positions: documents of random lengths, each counting from 0
    pos = np.concatenate([np.arange(n) for n in g.integers(1, 40, T)])[:T]
    pos = torch.from_numpy(pos + int(g.choice([0, 0, 5000]))).long()
    q, qh = view(g, T, nq * D, dt)
    k, kh = view(g, T, nkv * D, dt)
    q3, k3 = q.unflatten(1, (nq, D)), k.unflatten(1, (nkv, D))
    gpu.fo_rope_fwd(q3, k3, pos.to(DEV), theta)
    torch.cuda.synchronize()
    rq, rk = oracle.rope_fwd(qh.unflatten(1, (nq, D)), kh.unflatten(1, (nkv, D)), pos, theta)
    tag = f"rope seed={seed} {dt} T={T} heads={nq}/{nkv} D={D}"
    check(q3.cpu(), rq, dt, tag + " q", single_rounding=True)
    check(k3.cpu(), rk, dt, tag + " k", single_rounding=True)


@pytest.mark.parametrize("seed,dt", cases(30, 5))
def test_cross_entropy(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 48))
    V = int(g.choice([g.integers(1, 600), g.integers(600, 20000), g.integers(20000, 70000)]))
    zc = float(g.choice([0.0, 1e-4, 1e-3]))
    z, zh = view(g, T, V, dt, 2.0)
    t = torch.from_numpy(g.integers(0, V, T)).long()
    t[torch.from_numpy(g.random(T) < 0.2)] = IGN
    if T > 2:
        t[1] = V  # a bad target: counted, treated as ignored
    o = gpu.fo_xent_fwd_bwd(z, t.to(DEV), IGN, zc, 0.7)
    torch.cuda.synchronize()
    r = oracle.xent_fwd_bwd(zh, t, IGN, zc, 0.7)
    tag = f"xent seed={seed} {dt} T={T} V={V}"
    check_loss(o["loss"].item(), r["loss"], tag + " loss")
    check_loss(o["z_loss"].item(), r["z_loss"], tag + " z_loss")
    assert o["n_valid"].item() == r["n_valid"] and o["status"].item() == r["n_bad"], tag
    check(o["dlogits"].cpu(), r["dlogits"], dt, tag + " dlogits", single_rounding=True,
          scale=xent_dz_terms(zh, t.numpy(), (t != IGN) & (t >= 0) & (t < V), r["lse"], zc,
                                0.7, r["n_valid"]))


def wide_rows(g, T, dt, scale):
    """Rows of a large vocabulary: half the cases contiguous with V a multiple of 8 (on the
    16-byte grid: the register-and-LDS and streaming row kernels), the others views off
    the grid with row padding (the element-aligned paths)."""
    if g.random() < 0.5:
        V = 8 * int(g.integers(100000 // 8, 200000 // 8))
        host = torch.from_numpy(g.standard_normal((T, V)) * scale).float().to(TD[dt])
        return host.to(DEV), host, V
    V = int(g.integers(100000, 200000))
    dev_view, host = view(g, T, V, dt, scale)
    return dev_view, host, V


@pytest.mark.parametrize("seed,dt", cases(10, 8))
def test_cross_entropy_wide_vocab(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 9))
    z, zh, V = wide_rows(g, T, dt, 2.0)
    zc = float(g.choice([0.0, 1e-4]))
    t = torch.from_numpy(g.integers(0, V, T)).long()
    t[torch.from_numpy(g.random(T) < 0.2)] = IGN
    o = gpu.fo_xent_fwd_bwd(z, t.to(DEV), IGN, zc, 0.7)
    torch.cuda.synchronize()
    r = oracle.xent_fwd_bwd(zh, t, IGN, zc, 0.7)
    tag = f"xent wide seed={seed} {dt} T={T} V={V}"
    check_loss(o["loss"].item(), r["loss"], tag + " loss")
    check_loss(o["z_loss"].item(), r["z_loss"], tag + " z_loss")
    assert o["n_valid"].item() == r["n_valid"] and o["status"].item() == r["n_bad"], tag
    check(o["dlogits"].cpu(), r["dlogits"], dt, tag + " dlogits", single_rounding=True,
          scale=xent_dz_terms(zh, t.numpy(), (t != IGN) & (t >= 0) & (t < V), r["lse"], zc,
                                0.7, r["n_valid"]))


@pytest.mark.parametrize("seed,dt", cases(8, 9))
def test_distillation_wide_vocab(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 7))
    z, zh, V = wide_rows(g, T, dt, 3.0)
    zt_h = torch.from_numpy(g.standard_normal((T, V)) * 2.0).float().to(TD[dt])
    mask = torch.from_numpy((g.random(T) > 0.2).astype(np.uint8))
    o = gpu.fo_distill_fwd_bwd(z, zt_h.to(DEV), mask.to(DEV), 1.3)
    torch.cuda.synchronize()
    r = oracle.distill_fwd_bwd(zh, zt_h, mask, 1.3)
    tag = f"distill wide seed={seed} {dt} T={T} V={V}"
    assert o["n_valid"].item() == r["n_valid"], tag
    check_loss(o["loss"].item(), r["loss"], tag + " loss")
    keep = mask.numpy() != 0
    check_loss(o["kl"].item(), r["kl"], tag + " kl", scale=kl_terms(zh, zt_h, keep))
    n = max(1, int(keep.sum()))
    check_softmax_diff(o["dlogits"].cpu(), r["dlogits"], softmax_sum(zh, zt_h, keep, 1.3 / n),
                       tag + " dlogits", rounded_out=dt == "bf16")


@pytest.mark.parametrize("seed,dt", cases(24, 6))
def test_distillation(gpu, seed, dt):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 32))
    V = int(g.choice([g.integers(1, 600), g.integers(600, 20000), g.integers(20000, 70000)]))
    z, zh = view(g, T, V, dt, 3.0)
    zt, zth = view(g, T, V, dt, 2.0)
    mask = torch.from_numpy((g.random(T) > 0.2).astype(np.uint8))
    o = gpu.fo_distill_fwd_bwd(z, zt, mask.to(DEV), 1.3)
    torch.cuda.synchronize()
    r = oracle.distill_fwd_bwd(zh, zth, mask, 1.3)
    tag = f"distill seed={seed} {dt} T={T} V={V}"
    assert o["n_valid"].item() == r["n_valid"], tag
    check_loss(o["loss"].item(), r["loss"], tag + " loss")
    keep = mask.numpy() != 0
    check_loss(o["kl"].item(), r["kl"], tag + " kl", scale=kl_terms(zh, zth, keep))
    n = max(1, int(keep.sum()))
    check_softmax_diff(o["dlogits"].cpu(), r["dlogits"], softmax_sum(zh, zth, keep, 1.3 / n),
                       tag + " dlogits", rounded_out=dt == "bf16")


@pytest.mark.parametrize("seed", [int(s) for s in np.random.default_rng(7).integers(0, 2**31, 12)])
def test_fused_linear_cross_entropy(gpu, seed):
    from tolerance import check_bf16, check_product_grad, flce_target_terms
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 160))
    H = 8 * int(g.integers(1, 40))
    V = int(g.choice([g.integers(1, 300), g.integers(300, 5000)]))
    chunk = int(g.choice([0, 16, 64, 100]))
    zc = float(g.choice([0.0, 1e-4]))
    h = torch.from_numpy(g.standard_normal((T, H))).to(torch.bfloat16)
    w = torch.from_numpy(0.05 * g.standard_normal((V, H))).to(torch.bfloat16)
    t = torch.from_numpy(g.integers(0, V, T)).long()
    t[torch.from_numpy(g.random(T) < 0.15)] = IGN
    o = gpu.fo_flce_fwd_bwd(h.to(DEV), w.to(DEV), t.to(DEV), IGN, zc, 1.0, chunk_tokens=chunk)
    torch.cuda.synchronize()
    r = oracle.flce_fwd_bwd(h, w, t, IGN, zc, 1.0, abs_products=True)
    tag = f"flce seed={seed} T={T} H={H} V={V} chunk={chunk}"
    check_loss(o["loss"].item(), r["loss"], tag + " loss")
    check_loss(o["z_loss"].item(), r["z_loss"], tag + " z_loss")
    assert o["n_valid"].item() == r["n_valid"], tag
    check_bf16(o["dhidden"].cpu(), r["dhidden"], tag + " dhidden")
    tn = t.numpy()
    check_product_grad(o["dhidden"].cpu(), r["dhidden"], r["dhidden_abs"], tag + " dhidden",
                       target=flce_target_terms(w, tn, r["n_valid"], 1.0, np.arange(T), "dh"))
    check_product_grad(o["dweight"].cpu(), r["dweight"], r["dweight_abs"], tag + " dweight",
                       rounded_out=False,
                       target=flce_target_terms(h, tn, r["n_valid"], 1.0, np.arange(V), "dw"))


@pytest.mark.parametrize("seed,dt", cases(24, 8))
def test_mlp_activations(gpu, seed, dt):
    g = np.random.default_rng(seed)
    act = str(g.choice(["silu", "gelu", "relu"]))
    T, F = int(g.integers(1, 200)), width(g)
    gate, gh = view(g, T, F, dt, 2.0)
    up, uh = view(g, T, F, dt)
    dh, dhh = view(g, T, F, dt)
    tag = f"{act} seed={seed} {dt} T={T} F={F}"
    h = gpu.fo_glu_fwd(act, gate, up)
    dg, du = gpu.fo_glu_bwd(act, dh, gate, up)
    y = gpu.fo_act_fwd(act, gate)
    dx = gpu.fo_act_bwd(act, dh, gate)
    torch.cuda.synchronize()
    rg, ru = oracle.glu_bwd(dhh, gh, uh, act)
    check(h.cpu(), oracle.glu_fwd(gh, uh, act), dt, tag + " glu h", single_rounding=True)
    check(dg.cpu(), rg, dt, tag + " glu dgate", single_rounding=True)
    check(du.cpu(), ru, dt, tag + " glu dup", single_rounding=True)
    check(y.cpu(), oracle.act_fwd(gh, act), dt, tag + " act y", single_rounding=True)
    check(dx.cpu(), oracle.act_bwd(dhh, gh, act), dt, tag + " act dx", single_rounding=True)


@pytest.mark.parametrize("seed", [int(s) for s in np.random.default_rng(9).integers(0, 2**31, 10)])
def test_adamw(gpu, seed):
    from tolerance import adamw_terms, check_f32
    g = np.random.default_rng(seed)
    n = int(g.integers(1, 40))
    sizes = [int(g.choice([g.integers(1, 9), g.integers(9, 5000), g.integers(5000, 70000)]))
             for _ in range(n)]
    lr, b1, b2, wd, step = 3e-4, 0.9, 0.95, 0.1, int(g.integers(1, 1000))
    ss, bc, df = oracle.adamw_scalars(lr, b1, b2, wd, step)
    f = lambda x: float(np.float32(x))  # noqa: E731
    sc = dict(step_size=f(ss), beta1=f(b1), beta2=f(b2), bias_correction=f(bc),
              decay_factor=f(df), eps=f(1e-8))
    host = {k: [torch.from_numpy(g.standard_normal(s) * sd).float() for s in sizes]
            for k, sd in (("p", 1.0), ("g", 0.1), ("m", 0.01))}
    host["v"] = [torch.from_numpy(np.abs(g.standard_normal(s)) * 1e-4).float() for s in sizes]
    dev = {}
    for k, ts in host.items():  # each tensor 0-3 elements into its buffer (misaligned views)
        dev[k] = []
        for t in ts:
            o = int(g.integers(0, 4))
            buf = torch.empty(t.numel() + o, dtype=torch.float32, device=DEV)
            buf[o:].copy_(t.to(DEV))
            dev[k].append(buf[o:])
    gpu.fo_adamw_step(dev["p"], dev["g"], dev["m"], dev["v"], **sc)
    torch.cuda.synchronize()
    for i in range(n):
        rp, rm, rv = oracle.adamw_step(host["p"][i], host["g"][i], host["m"][i], host["v"][i],
                                       sc["step_size"], sc["beta1"], sc["beta2"],
                                       sc["bias_correction"], sc["decay_factor"], sc["eps"])
        tag = f"adamw seed={seed} tensor {i} of {n}, {sizes[i]} elements"
        ap, am = adamw_terms(host["p"][i], host["g"][i], host["m"][i], host["v"][i],
                             sc["step_size"], sc["beta1"], sc["beta2"], sc["bias_correction"],
                             sc["decay_factor"], sc["eps"])
        check_f32(dev["p"][i].cpu(), rp, tag + " p", scale=ap)
        check_f32(dev["m"][i].cpu(), rm, tag + " m", scale=am)
        check_f32(dev["v"][i].cpu(), rv, tag + " v")


@pytest.mark.parametrize("seed,dt", cases(12, 21))
def test_operands_scaled(gpu, seed, dt, monkeypatch):
    # the same cases with every operand scaled independently by 0.01, 1, 10 or 100
    # (logits to about +-600, norm weights to +-100): the bounds' magnitude terms
    monkeypatch.setattr(sys.modules[__name__], "MAGS", (0.01, 1.0, 10.0, 100.0))
    for fn in (test_rmsnorm, test_layernorm, test_swiglu, test_rope, test_cross_entropy,
               test_distillation, test_mlp_activations):
        fn(gpu, seed, dt)
