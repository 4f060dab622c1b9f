"""GPU parity of fo_swiglu_fwd / fo_swiglu_bwd against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(fo, g, u, dh):
    gg, ug, hg = g.to(DEV), u.to(DEV), dh.to(DEV)
    h = fo.fo_swiglu_fwd(gg, ug)
    dg, du = fo.fo_swiglu_bwd(hg, gg, ug)
    torch.cuda.synchronize()
    return h.cpu(), dg.cpu(), du.cpu()


def compare(g, u, dh, dt, got):
    h, dg, du = got
    check(h, oracle.swiglu_fwd(g, u), dt, "h", single_rounding=True)
    rg, ru = oracle.swiglu_bwd(dh, g, u)
    check(dg, rg, dt, "dgate", single_rounding=True)
    check(du, ru, dt, "dup", single_rounding=True)


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 45])
def test_configs_small(gpu, cid, T):
    cfg = synth.scaled(synth.CONFIGS[cid], T)
    i = synth.swiglu_inputs(cfg)
    compare(i["gate"], i["up"], i["dh"], cfg.dtype, run(gpu, i["gate"], i["up"], i["dh"]))


def test_config1_as_stated(gpu):
    # the tiny fp32 block at its stated size: T 256, F 1408, every element
    cfg = synth.CONFIGS[1]
    assert cfg.T == 256
    i = synth.swiglu_inputs(cfg)
    compare(i["gate"], i["up"], i["dh"], cfg.dtype, run(gpu, i["gate"], i["up"], i["dh"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("F", [1409, 7, 8, 513])
def test_unaligned_widths(gpu, dtype, F):
    g = torch.Generator().manual_seed(F)
    td = synth.torch_dtype(dtype)
    a, b, c = (torch.randn(29, F, generator=g).to(td) for _ in range(3))
    compare(a, b, c, dtype, run(gpu, a, b, c))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("F", [1408, 1409, 8192, 8200, 14336, 14337])
def test_halves_of_fused_projection(gpu, dtype, F):
    # gate and up as the two halves of one [T, 2F] tensor (row stride 2F); with an odd F
    # every row of the up half, and every other row of both, starts off the 16-byte grid.
    # Rows of one block or whole blocks (1408, 1409, bf16 8192) take blocks per row; rows
    # of several blocks with a partial last one (bf16 8200, 14336, 14337, fp32 from 8192)
    # one flat space of blocks that run on into the next row
    T = 77 if F < 10000 else 9
    g = torch.Generator().manual_seed(1)
    td = synth.torch_dtype(dtype)
    gu = torch.randn(T, 2 * F, generator=g).to(td)
    dh = torch.randn(T, F, generator=g).to(td)
    gug = gu.to(DEV)
    h = gpu.fo_swiglu_fwd(gug[:, :F], gug[:, F:])
    dgu = torch.empty_like(gug)
    gpu.fo_swiglu_bwd(dh.to(DEV), gug[:, :F], gug[:, F:], dgate=dgu[:, :F], dup=dgu[:, F:])
    torch.cuda.synchronize()
    compare(gu[:, :F], gu[:, F:], dh, dtype, (h.cpu(), dgu[:, :F].cpu(), dgu[:, F:].cpu()))


def test_extreme_gates_finite(gpu):
    g = torch.tensor([[100.0, -100.0, 80.0, -80.0, 0.0, -0.0, 30.0, -30.0]])
    u = torch.full_like(g, 1.5)
    dh = torch.ones_like(g)
    for dt in ("f32", "bf16"):
        td = synth.torch_dtype(dt)
        got = run(gpu, g.to(td), u.to(td), dh.to(td))
        for t in got:
            assert torch.all(torch.isfinite(t))
        compare(g.to(td), u.to(td), dh.to(td), dt, got)


def test_in_place_outputs(gpu):
    cfg = synth.scaled(synth.CONFIGS[3], 33)
    i = synth.swiglu_inputs(cfg)
    g, u, dh = (i[k].to(DEV) for k in ("gate", "up", "dh"))
    ref_h = gpu.fo_swiglu_fwd(g, u)
    ref_dg, ref_du = gpu.fo_swiglu_bwd(dh, g, u)
    g2, u2 = g.clone(), u.clone()
    gpu.fo_swiglu_bwd(dh, g2, u2, dgate=g2, dup=u2)
    g3 = g.clone()
    gpu.fo_swiglu_fwd(g3, u, h=g3)
    torch.cuda.synchronize()
    assert torch.equal(g2, ref_dg) and torch.equal(u2, ref_du) and torch.equal(g3, ref_h)


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size_sampled(gpu, cid):
    cfg = synth.CONFIGS[cid]
    i = synth.swiglu_inputs(cfg)
    h, dg, du = run(gpu, i["gate"], i["up"], i["dh"])
    rows = np.unique(np.concatenate([[0, cfg.T - 1],
                                     np.random.default_rng(cid).integers(0, cfg.T, 14)]))
    compare(i["gate"][rows], i["up"][rows], i["dh"][rows], cfg.dtype,
            (h[rows], dg[rows], du[rows]))


def test_halves_full_size_sampled(gpu):
    # the bench's unaligned line: gate and up as halves of one [8192, 2 x 14337] bf16
    # tensor (strided rows off the 16-byte grid), sampled rows
    T, F = 8192, 14337
    g = torch.Generator().manual_seed(14337)
    gu = torch.randn(T, 2 * F, generator=g).to(torch.bfloat16)
    dh = torch.randn(T, F, generator=g).to(torch.bfloat16)
    gug = gu.to(DEV)
    h = gpu.fo_swiglu_fwd(gug[:, :F], gug[:, F:])
    dgu = torch.empty_like(gug)
    gpu.fo_swiglu_bwd(dh.to(DEV), gug[:, :F], gug[:, F:], dgate=dgu[:, :F], dup=dgu[:, F:])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(2).integers(0, T, 13)]))
    h, dgu = h.cpu(), dgu.cpu()
    compare(gu[rows, :F], gu[rows, F:], dh[rows], "bf16", (h[rows], dgu[rows, :F], dgu[rows, F:]))

