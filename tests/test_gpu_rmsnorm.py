"""GPU parity of fo_rmsnorm_fwd / fo_rmsnorm_bwd against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check, norm_dw_terms, norm_dx_terms

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(fo, x, w, dy, eps, use_rstd=True):
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    y, rstd = fo.fo_rmsnorm_fwd(xg, wg, eps)
    dx, dw = fo.fo_rmsnorm_bwd(dyg, xg, wg, rstd if use_rstd else None, eps)
    torch.cuda.synchronize()
    return y.cpu(), rstd.cpu(), dx.cpu(), dw.cpu()


def compare(x, w, dy, eps, dt, got, rows=None):
    y, rstd, dx, dw = got
    ry, rr = oracle.rmsnorm_fwd(x, w, eps)
    rdx, rdw = oracle.rmsnorm_bwd(dy, x, w, eps)
    sel = slice(None) if rows is None else rows
    check(y[sel], ry[sel], dt, "y", single_rounding=True)
    check(rstd[sel], rr[sel], "f32", "rstd")
    terms = norm_dx_terms(dy, x, w, eps, False)
    check(dx[sel], rdx[sel], dt, "dx", single_rounding=True, scale=terms[sel])
    # dw is an fp32 output: the products of exact inputs summed in fp32
    check(dw, rdw, "f32", "dw", scale=norm_dw_terms(dy, x, eps, False))


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 67])
def test_configs_small(gpu, cid, T):
    cfg = synth.scaled(synth.CONFIGS[cid], T)
    i = synth.rmsnorm_inputs(cfg)
    got = run(gpu, i["x"], i["w"], i["dy"], cfg.eps)
    compare(i["x"], i["w"], i["dy"], cfg.eps, cfg.dtype, got)
    got2 = run(gpu, i["x"], i["w"], i["dy"], cfg.eps, use_rstd=False)
    compare(i["x"], i["w"], i["dy"], cfg.eps, cfg.dtype, got2)


def test_config1_as_stated(gpu):
    # the tiny fp32 block at its stated size: T 256, d 512, eps 1e-6, every row
    cfg = synth.CONFIGS[1]
    assert cfg.T == 256 and cfg.dtype == "f32"
    i = synth.rmsnorm_inputs(cfg)
    compare(i["x"], i["w"], i["dy"], cfg.eps, cfg.dtype, run(gpu, i["x"], i["w"], i["dy"], cfg.eps))


# Row widths at the launch-plan boundaries (VEC = 8 bf16 / 4 fp32 elements per vector):
# tail-only rows (3, 5); vectors plus a tail; the forward's one-wave rows end at 512
# vectors (4096 bf16, 2048 fp32), then 2, 4, 8, 16 waves per row up to 16384 vectors
# (131072 bf16, 65536 fp32; + a tail of VEC - 1: 131079, 65539), past which (131080,
# 65540) the workgroup-per-row kernel takes the row; the backward holds up to 2048 bf16 /
# 4096 fp32 vectors (16384 elements; 16391 bf16 and 16387 fp32 with the longest tail)
# in up to 16 waves and takes the workgroup kernel past that (16388 fp32, 16392 bf16).
WIDE = (3, 5, 13, 1000, 1025, 2049, 4096, 4097, 4099, 4100, 4104, 8, 8191, 8199, 8200, 12288,
        16387, 16388, 16391, 16392, 24577, 65539, 65540, 131072, 131079, 131080)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,d", [(37, d) for d in WIDE] + [(5000, 1027), (300, 12289)])
def test_unaligned_and_wide_rows(gpu, dtype, T, d):
    # every width of WIDE, and batches whose backward workgroups each take several
    # rounds of rows with a tail (T 5000, d 1027; T 300, d 12289 at 16 waves per row)
    cfg = synth.Config(0, "odd", dtype, T=T, d=d, n_q=1, n_kv=1, head_dim=2, F=1, V=2,
                       eps=1e-5, theta=1e4, logit_std=1, z_loss=0, ignore_frac=0,
                       packed=False, doc_lengths=(T,), seed=11)
    i = synth.rmsnorm_inputs(cfg)
    got = run(gpu, i["x"], i["w"], i["dy"], cfg.eps)
    compare(i["x"], i["w"], i["dy"], cfg.eps, dtype, got)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_and_misaligned_rows(gpu, dtype):
    td = synth.torch_dtype(dtype)
    T, d, ld = 50, 256, 264  # ld > d and a multiple of the vector: strided fast path
    g = torch.Generator().manual_seed(3)
    base = torch.randn(T, ld, generator=g).to(td)
    w = (1 + 0.1 * torch.randn(d, generator=g)).to(td)
    dy = torch.randn(T, d, generator=g).to(td)
    for off in (0, 1):  # off=1: base pointer not 16-byte aligned
        xs = base[:, off:off + d]
        xg = base.to(DEV)[:, off:off + d]
        y, rstd = gpu.fo_rmsnorm_fwd(xg, w.to(DEV), 1e-6)
        dx, dw = gpu.fo_rmsnorm_bwd(dy.to(DEV), xg, w.to(DEV), rstd, 1e-6)
        torch.cuda.synchronize()
        compare(xs, w, dy, 1e-6, dtype, (y.cpu(), rstd.cpu(), dx.cpu(), dw.cpu()))


def test_in_place_forward_and_backward(gpu):
    cfg = synth.scaled(synth.CONFIGS[3], 40)
    i = synth.rmsnorm_inputs(cfg)
    xg, wg = i["x"].to(DEV), i["w"].to(DEV)
    ref_y, _ = gpu.fo_rmsnorm_fwd(xg, wg, cfg.eps)
    x2 = xg.clone()
    gpu.fo_rmsnorm_fwd(x2, wg, cfg.eps, y=x2, want_rstd=False)
    dyg = i["dy"].to(DEV)
    ref_dx, ref_dw = gpu.fo_rmsnorm_bwd(dyg, xg, wg, None, cfg.eps)
    dy2 = dyg.clone()
    _, dw2 = gpu.fo_rmsnorm_bwd(dy2, xg, wg, None, cfg.eps, dx=dy2)
    torch.cuda.synchronize()
    assert torch.equal(x2, ref_y) and torch.equal(dy2, ref_dx) and torch.equal(dw2, ref_dw)


def test_empty_batch_zeroes_dw(gpu):
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    dw = torch.full((64,), 7.0, device=DEV)
    gpu.fo_rmsnorm_bwd(x, x, w, None, 1e-5, dx=x, dw=dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_deterministic(gpu):
    cfg = synth.scaled(synth.CONFIGS[4], 3000)
    i = synth.rmsnorm_inputs(cfg)
    a = run(gpu, i["x"], i["w"], i["dy"], cfg.eps)
    b = run(gpu, i["x"], i["w"], i["dy"], cfg.eps)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size_sampled(gpu, cid):
    cfg = synth.CONFIGS[cid]
    i = synth.rmsnorm_inputs(cfg)
    got = run(gpu, i["x"], i["w"], i["dy"], cfg.eps)
    rows = np.unique(np.concatenate([[0, 1, cfg.T - 1],
                                     np.random.default_rng(cid).integers(0, cfg.T, 29)]))
    y, rstd, dx, dw = got
    x, w, dy = i["x"][rows], i["w"], i["dy"][rows]
    ry, rr = oracle.rmsnorm_fwd(x, w, cfg.eps)
    rdx, _ = oracle.rmsnorm_bwd(dy, x, w, cfg.eps)
    check(y[rows], ry, cfg.dtype, "y", single_rounding=True)
    check(rstd[rows], rr, "f32", "rstd")
    check(dx[rows], rdx, cfg.dtype, "dx", single_rounding=True)
    # dw needs every row: oracle over all T in row blocks
    rdw, a2 = np.zeros(cfg.d), np.zeros(cfg.d)
    for r0 in range(0, cfg.T, 2048):
        xb, dyb = i["x"][r0:r0 + 2048], i["dy"][r0:r0 + 2048]
        rdw += oracle.rmsnorm_bwd(dyb, xb, w, cfg.eps)[1]
        a2 += norm_dw_terms(dyb, xb, cfg.eps, False) ** 2
    check(dw, rdw, "f32", "dw", scale=np.sqrt(a2))


def test_unaligned_full_size_sampled(gpu):
    # the bench's unaligned line: Llama-3-8B token count with d = 4097 (bf16, contiguous,
    # so 7 rows in 8 start off the 16-byte grid), sampled rows; dw over every row
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS[3], d=4097)
    i = synth.rmsnorm_inputs(cfg)
    y, rstd, dx, dw = run(gpu, i["x"], i["w"], i["dy"], cfg.eps)
    rows = np.unique(np.concatenate([[0, 1, 2, 7, cfg.T - 1],
                                     np.random.default_rng(4097).integers(0, cfg.T, 27)]))
    x, w, dy = i["x"][rows], i["w"], i["dy"][rows]
    ry, rr = oracle.rmsnorm_fwd(x, w, cfg.eps)
    rdx, _ = oracle.rmsnorm_bwd(dy, x, w, cfg.eps)
    check(y[rows], ry, cfg.dtype, "y", single_rounding=True)
    check(rstd[rows], rr, "f32", "rstd")
    check(dx[rows], rdx, cfg.dtype, "dx", single_rounding=True)
    rdw, a2 = np.zeros(cfg.d), np.zeros(cfg.d)
    for r0 in range(0, cfg.T, 2048):
        xb, dyb = i["x"][r0:r0 + 2048], i["dy"][r0:r0 + 2048]
        rdw += oracle.rmsnorm_bwd(dyb, xb, w, cfg.eps)[1]
        a2 += norm_dw_terms(dyb, xb, cfg.eps, False) ** 2
    check(dw, rdw, "f32", "dw", scale=np.sqrt(a2))



def test_widest_llama_rows_full_size_sampled(gpu):
    # the widest Llama-style layer: T 8192, d 16384 (bf16), whose rows the forward spreads
    # over 4 waves of 8 vectors and the backward over 16 waves (1024-thread workgroups,
    # one row each, dw partials written from registers); sampled rows, dw over every row
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS[3], d=16384)
    i = synth.rmsnorm_inputs(cfg)
    y, rstd, dx, dw = run(gpu, i["x"], i["w"], i["dy"], cfg.eps)
    rows = np.unique(np.concatenate([[0, 1, cfg.T - 1],
                                     np.random.default_rng(16384).integers(0, cfg.T, 29)]))
    x, w, dy = i["x"][rows], i["w"], i["dy"][rows]
    ry, rr = oracle.rmsnorm_fwd(x, w, cfg.eps)
    rdx, _ = oracle.rmsnorm_bwd(dy, x, w, cfg.eps)
    check(y[rows], ry, cfg.dtype, "y", single_rounding=True)
    check(rstd[rows], rr, "f32", "rstd")
    check(dx[rows], rdx, cfg.dtype, "dx", single_rounding=True)
    rdw, a2 = np.zeros(cfg.d), np.zeros(cfg.d)
    for r0 in range(0, cfg.T, 1024):
        xb, dyb = i["x"][r0:r0 + 1024], i["dy"][r0:r0 + 1024]
        rdw += oracle.rmsnorm_bwd(dyb, xb, w, cfg.eps)[1]
        a2 += norm_dw_terms(dyb, xb, cfg.eps, False) ** 2
    check(dw, rdw, "f32", "dw", scale=np.sqrt(a2))
