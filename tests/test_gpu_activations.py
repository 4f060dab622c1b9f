"""GPU parity of fo_glu_* (gated) and fo_act_* (plain) MLP activations against the fp64
oracle, for SiLU, GeLU and ReLU."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda"
ACTS = ["silu", "gelu", "relu"]


def cfg_of(dtype, T, F, seed=21):
    return synth.Config(0, "act", dtype, T=T, d=8, n_q=1, n_kv=1, head_dim=2, F=F, V=2,
                        eps=1e-5, theta=1e4, logit_std=1, z_loss=0, ignore_frac=0,
                        packed=False, doc_lengths=(T,), seed=seed)


def gated(fo, act, g, u, dh, dt):
    gg, ug, dhg = g.to(DEV), u.to(DEV), dh.to(DEV)
    h = fo.fo_glu_fwd(act, gg, ug)
    dg, du = fo.fo_glu_bwd(act, dhg, gg, ug)
    torch.cuda.synchronize()
    check(h.cpu(), oracle.glu_fwd(g, u, act), dt, "h", single_rounding=True)
    rdg, rdu = oracle.glu_bwd(dh, g, u, act)
    check(dg.cpu(), rdg, dt, "dgate", single_rounding=True)
    check(du.cpu(), rdu, dt, "dup", single_rounding=True)


def plain(fo, act, x, dy, dt):
    xg, dyg = x.to(DEV), dy.to(DEV)
    y = fo.fo_act_fwd(act, xg)
    dx = fo.fo_act_bwd(act, dyg, xg)
    torch.cuda.synchronize()
    check(y.cpu(), oracle.act_fwd(x, act), dt, "y", single_rounding=True)
    check(dx.cpu(), oracle.act_bwd(dy, x, act), dt, "dx", single_rounding=True)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("F", [8, 13, 1001, 4096, 14336])
def test_gated_and_plain_shapes(gpu, act, dtype, F):
    i = synth.swiglu_inputs(cfg_of(dtype, 19, F))
    gated(gpu, act, i["gate"], i["up"], i["dh"], dtype)
    plain(gpu, act, i["gate"], i["dh"], dtype)


@pytest.mark.parametrize("act", ACTS)
def test_halves_of_one_tensor(gpu, act):
    # gate and up as the two halves of a [T, 2F] projection output (row stride 2F)
    T, F = 33, 1024
    g = torch.Generator().manual_seed(5)
    gu = torch.randn(T, 2 * F, generator=g).to(torch.bfloat16)
    dh = torch.randn(T, F, generator=g).to(torch.bfloat16)
    gud = gu.to(DEV)
    h = gpu.fo_glu_fwd(act, gud[:, :F], gud[:, F:])
    dgu = torch.empty_like(gud)
    gpu.fo_glu_bwd(act, dh.to(DEV), gud[:, :F], gud[:, F:], dgate=dgu[:, :F], dup=dgu[:, F:])
    torch.cuda.synchronize()
    check(h.cpu(), oracle.glu_fwd(gu[:, :F], gu[:, F:], act), "bf16", "h", single_rounding=True)
    rdg, rdu = oracle.glu_bwd(dh, gu[:, :F], gu[:, F:], act)
    check(dgu[:, :F].cpu(), rdg, "bf16", "dgate", single_rounding=True)
    check(dgu[:, F:].cpu(), rdu, "bf16", "dup", single_rounding=True)


@pytest.mark.parametrize("act", ACTS)
def test_plain_in_place(gpu, act):
    i = synth.swiglu_inputs(cfg_of("bf16", 40, 2048, seed=3))
    x, dy = i["gate"].to(DEV), i["dh"].to(DEV)
    ref_y = gpu.fo_act_fwd(act, x)
    ref_dx = gpu.fo_act_bwd(act, dy, x)
    x2, dy2 = x.clone(), dy.clone()
    gpu.fo_act_bwd(act, dy2, x, dx=dy2)
    gpu.fo_act_fwd(act, x2, y=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2, ref_y) and torch.equal(dy2, ref_dx)


def test_silu_entry_points_agree(gpu):
    i = synth.swiglu_inputs(cfg_of("bf16", 64, 1536, seed=4))
    g, u, dh = (i[k].to(DEV) for k in ("gate", "up", "dh"))
    a = gpu.fo_glu_fwd("silu", g, u)
    b = gpu.fo_swiglu_fwd(g, u)
    da = gpu.fo_glu_bwd("silu", dh, g, u)
    db = gpu.fo_swiglu_bwd(dh, g, u)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and all(torch.equal(p, q) for p, q in zip(da, db))


@pytest.mark.parametrize("act", ["gelu", "relu"])
def test_full_size_sampled(gpu, act):
    """The Llama-3-8B MLP width (T 8192, F 14336, bf16) in one call; sampled rows."""
    cfg = synth.CONFIGS[3]
    i = synth.swiglu_inputs(cfg)
    g, u, dh = (i[k].to(DEV) for k in ("gate", "up", "dh"))
    h = gpu.fo_glu_fwd(act, g, u)
    dg, du = gpu.fo_glu_bwd(act, dh, g, u)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, cfg.T - 1], np.random.default_rng(7).integers(0, cfg.T, 20)]))
    gs, us, dhs = i["gate"][rows], i["up"][rows], i["dh"][rows]
    check(h[rows].cpu(), oracle.glu_fwd(gs, us, act), "bf16", "h", single_rounding=True)
    rdg, rdu = oracle.glu_bwd(dhs, gs, us, act)
    check(dg[rows].cpu(), rdg, "bf16", "dgate", single_rounding=True)
    check(du[rows].cpu(), rdu, "bf16", "dup", single_rounding=True)
