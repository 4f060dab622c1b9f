"""GPU parity of fo_flce_fwd_bwd against the fp64 oracle, plus its chunking and
masking properties."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from blockwise import map_blocks
from tolerance import check_bf16, check_loss, check_product_grad, flce_target_terms

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX


def run(fo, h, w, t, zc, chunk=0, dwt=torch.float32, dloss=1.0):
    o = fo.fo_flce_fwd_bwd(h.to(DEV), w.to(DEV), t.to(DEV), IGN, zc, dloss, dweight_dtype=dwt,
                           chunk_tokens=chunk)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in o.items()}


def compare(h, w, t, zc, o, dloss=1.0):
    r = oracle.flce_fwd_bwd(h, w, t, IGN, zc, dloss, chunk=256, abs_products=True)
    check_loss(o["loss"].item(), r["loss"])
    check_loss(o["z_loss"].item(), r["z_loss"], "z_loss")
    assert o["n_valid"].item() == r["n_valid"]
    assert o["status"].item() == r["n_bad"]
    tn = t.numpy()
    check_bf16(o["dhidden"], r["dhidden"], "dhidden")
    check_product_grad(o["dhidden"], r["dhidden"], r["dhidden_abs"], "dhidden",
                       target=flce_target_terms(w, tn, r["n_valid"], dloss, np.arange(len(tn)), "dh"))
    check_bf16(o["dweight"], r["dweight"], "dweight")
    check_product_grad(o["dweight"], r["dweight"], r["dweight_abs"], "dweight",
                       rounded_out=o["dweight"].dtype == torch.bfloat16,
                       target=flce_target_terms(h, tn, r["n_valid"], dloss, np.arange(w.shape[0]), "dw"))
    ign = (t == IGN).nonzero().flatten()
    assert torch.all(o["dhidden"][ign].view(torch.int16) == 0)
    return r


@pytest.mark.parametrize("T,H,V,chunk", [
    (1, 64, 100, 0),
    (37, 64, 1000, 16),        # ragged chunks and tiles
    (200, 256, 4097, 64),      # vocabulary not a multiple of the vector
    (300, 512, 8192, 0),
    (200, 128, 1000, 16),      # 13 chunks: dW over four groups, accumulated across them
])
def test_small(gpu, T, H, V, chunk):
    cfg = synth.flce_small(T, H, V, seed=T)
    i = synth.flce_inputs(cfg)
    o = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk)
    compare(i["hidden"], i["weight"], i["targets"], cfg.z_loss, o)


def test_full_width_few_tokens(gpu):
    # the full lm-head shape (H 4096, V 128256) on 520 tokens in 3 ragged chunks
    cfg = synth.flce_small(520, 4096, 128256, seed=5)
    i = synth.flce_inputs(cfg)
    o = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=256)
    compare(i["hidden"], i["weight"], i["targets"], cfg.z_loss, o)


def test_chunk_size_and_dweight_dtype(gpu):
    cfg = synth.flce_small(384, 256, 3000, seed=9)
    i = synth.flce_inputs(cfg)
    a = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=384)
    b = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=128)
    g = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=32)  # 3 dW groups
    c = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=128,
            dwt=torch.bfloat16)
    assert abs(a["loss"].item() - b["loss"].item()) <= 1e-6 * abs(a["loss"].item())
    assert torch.equal(a["dhidden"], b["dhidden"])  # rows do not depend on the chunking
    check_bf16(b["dweight"], a["dweight"].double(), "dweight chunk")
    assert torch.equal(a["dhidden"], g["dhidden"])
    check_bf16(g["dweight"], a["dweight"].double(), "dweight groups")
    assert c["dweight"].dtype == torch.bfloat16
    assert torch.equal(c["dweight"], b["dweight"].to(torch.bfloat16))


def test_all_ignored(gpu):
    cfg = synth.flce_small(50, 64, 300, seed=2, ignore_frac=1.0)
    i = synth.flce_inputs(cfg)
    o = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss)
    assert o["loss"].item() == 0.0 and o["n_valid"].item() == 0
    assert torch.all(o["dhidden"] == 0) and torch.all(o["dweight"] == 0)


def test_deterministic(gpu):
    cfg = synth.flce_small(333, 128, 2000, seed=4)
    i = synth.flce_inputs(cfg)
    a = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=100)
    b = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=100)
    for k in ("loss", "dhidden", "dweight"):
        assert torch.equal(a[k], b[k]), k


def test_bf16_dweight_against_oracle(gpu):
    cfg = synth.flce_small(300, 256, 5000, seed=12)
    i = synth.flce_inputs(cfg)
    o = run(gpu, i["hidden"], i["weight"], i["targets"], cfg.z_loss, chunk=128,
            dwt=torch.bfloat16)
    compare(i["hidden"], i["weight"], i["targets"], cfg.z_loss, o)


def oracle_full_size(h, w, t, zc, dh_rows, dw_rows, block=256):
    """The fp64 oracle over every token of a full-size batch, in row blocks normalised
    by the batch's valid count (blocks then add up to the batch): loss, z-loss, the
    dH rows dh_rows and the dW rows dw_rows, with their absolute-value products."""
    W64 = w.double().numpy()
    n_full = int(((t != IGN) & (t >= 0) & (t < w.shape[0])).sum())
    dh_rows = np.asarray(dh_rows)

    def one(r0, r1):
        mine = dh_rows[(dh_rows >= r0) & (dh_rows < r1)]
        b = oracle.flce_fwd_bwd(h[r0:r1], W64, t[r0:r1], IGN, zc, 1.0, chunk=block,
                                dh_rows=mine - r0, dw_rows=dw_rows, n_norm=n_full,
                                abs_products=True)
        b["rows"] = mine
        return b

    parts = map_blocks(one, h.shape[0], block)
    out = dict(loss=sum(p["loss"] for p in parts), z_loss=sum(p["z_loss"] for p in parts),
               n_valid=n_full, n_bad=sum(p["n_bad"] for p in parts),
               dweight=sum(p["dweight"] for p in parts),
               dweight_abs=sum(p["dweight_abs"] for p in parts))
    where = {int(r): (p, k) for p in parts for k, r in enumerate(p["rows"])}
    out["dhidden"] = np.stack([where[int(r)][0]["dhidden"][where[int(r)][1]] for r in dh_rows])
    out["dhidden_abs"] = np.stack([where[int(r)][0]["dhidden_abs"][where[int(r)][1]]
                                   for r in dh_rows])
    return out


def test_full_size_against_oracle(gpu):
    """The lm-head workload at its stated size (H [8192, 4096], W [128256, 4096], 10%
    ignored targets, z-loss 1e-4), in the launch configuration the bench times, against
    the fp64 oracle over every token: loss and z-loss, the valid and bad counts, 72 dH
    rows (ignored ones included) and 72 dW rows (vocabulary entries that are some valid
    row's target and entries no row targets) under the bound of products of the rounded
    dZ."""
    cfg = synth.CONFIGS[5]
    i = synth.flce_inputs(cfg)
    h, w, t = i["hidden"], i["weight"], i["targets"]
    o = run(gpu, h, w, t, cfg.z_loss)
    g = np.random.default_rng(55)
    tn = t.numpy()
    ign_rows = np.nonzero(tn == IGN)[0]
    dh_rows = np.unique(np.concatenate([[0, 1, cfg.T - 1], g.choice(ign_rows, 8, replace=False),
                                        g.integers(0, cfg.T, 64)]))[:72]
    hit = np.unique(tn[tn != IGN])
    never = np.setdiff1d(np.arange(cfg.V), hit)
    dw_rows = np.unique(np.concatenate([[0, cfg.V - 1], g.choice(hit, 35, replace=False),
                                        g.choice(never, 35, replace=False)]))
    r = oracle_full_size(h, w, t, cfg.z_loss, dh_rows, dw_rows)
    check_loss(o["loss"].item(), r["loss"])
    check_loss(o["z_loss"].item(), r["z_loss"], "z_loss")
    assert o["n_valid"].item() == r["n_valid"] and o["status"].item() == r["n_bad"] == 0
    check_bf16(o["dhidden"][dh_rows], r["dhidden"], "dhidden")
    bh = flce_target_terms(w, tn, r["n_valid"], 1.0, dh_rows, "dh")
    bw = flce_target_terms(h, tn, r["n_valid"], 1.0, dw_rows, "dw")
    check_product_grad(o["dhidden"][dh_rows], r["dhidden"], r["dhidden_abs"], "dhidden", target=bh)
    check_bf16(o["dweight"][dw_rows], r["dweight"], "dweight")
    check_product_grad(o["dweight"][dw_rows], r["dweight"], r["dweight_abs"], "dweight",
                       rounded_out=False, target=bw)
    ign = torch.from_numpy(ign_rows)
    assert torch.all(o["dhidden"][ign].view(torch.int16) == 0)
    # another chunk size (other split-K slices of dH, more dW accumulations): the same
    # loss, and outputs within the same bounds
    o1 = run(gpu, h, w, t, cfg.z_loss, chunk=1024)
    check_loss(o1["loss"].item(), o["loss"].item(), rel=1e-6)
    check_product_grad(o1["dhidden"][dh_rows], r["dhidden"], r["dhidden_abs"], "dhidden c1024",
                       target=bh)
    check_product_grad(o1["dweight"][dw_rows], r["dweight"], r["dweight_abs"], "dweight c1024",
                       rounded_out=False, target=bw)


def test_bad_targets_are_counted_and_ignored(gpu):
    # targets outside [0, V) that are not ignore_index: counted into status, and their
    # rows treated as ignored (no loss, +0.0 dH rows, nothing in dW)
    cfg = synth.flce_small(64, 128, 1000, seed=21)
    i = synth.flce_inputs(cfg)
    t = i["targets"].clone()
    bad = [3, 17, 40]
    t[bad] = torch.tensor([1000, -5, 10**12])
    o = run(gpu, i["hidden"], i["weight"], t, cfg.z_loss)
    r = compare(i["hidden"], i["weight"], t, cfg.z_loss, o)
    assert o["status"].item() == r["n_bad"] == 3
    assert torch.all(o["dhidden"][bad].view(torch.int16) == 0)


@pytest.mark.parametrize("dwt", [torch.float32, torch.bfloat16])
def test_empty_batch(gpu, dwt):
    h = torch.empty(0, 64, dtype=torch.bfloat16)
    w = torch.randn(300, 64).to(torch.bfloat16)
    o = run(gpu, h, w, torch.empty(0, dtype=torch.int64), 1e-4, dwt=dwt)
    assert o["loss"].item() == 0.0 and o["n_valid"].item() == 0 and o["status"].item() == 0
    assert o["dweight"].shape == (300, 64) and torch.all(o["dweight"] == 0)


def test_forward_only_and_one_gradient(gpu):
    # no gradient, dH only and dW only (null outputs through the C ABI): the loss and each
    # gradient bit-identical to the call that forms both
    import ctypes
    cfg = synth.flce_small(300, 256, 3000, seed=31)
    i = synth.flce_inputs(cfg)
    h, w, t = (i[k].to(DEV) for k in ("hidden", "weight", "targets"))
    T, H = h.shape
    V = w.shape[0]
    full = gpu.fo_flce_fwd_bwd(h, w, t, IGN, cfg.z_loss, 1.0, chunk_tokens=128)
    fwd = gpu.fo_flce_fwd_bwd(h, w, t, IGN, cfg.z_loss, 1.0, chunk_tokens=128, grad=False)
    lib = gpu.load()

    def partial(dh, dw):
        o = gpu._scalars(DEV)
        ws = gpu._ws(lib.fo_flce_workspace(T, H, V, 128, gpu.FO_F32), DEV)
        rc = lib.fo_flce_fwd_bwd(gpu.FO_BF16, T, H, V, gpu._ptr(h), gpu._ptr(w), gpu._ptr(t), IGN,
                                 ctypes.c_float(cfg.z_loss), ctypes.c_float(1.0),
                                 gpu._ptr(dh) if dh is not None else None,
                                 gpu._ptr(dw) if dw is not None else None, gpu.FO_F32,
                                 gpu._ptr(o["loss"]), gpu._ptr(o["z_loss"]), gpu._ptr(o["n_valid"]),
                                 gpu._ptr(o["status"]), 128, gpu._ptr(ws), ws.numel(), gpu._stream())
        assert rc == 0, rc
        return o

    dh = torch.empty_like(h)
    dw = torch.empty((V, H), dtype=torch.float32, device=DEV)
    a = partial(dh, None)
    b = partial(None, dw)
    torch.cuda.synchronize()
    for o in (fwd, a, b):
        assert torch.equal(o["loss"].cpu(), full["loss"].cpu())
        assert torch.equal(o["z_loss"].cpu(), full["z_loss"].cpu())
    assert fwd["dhidden"] is None and fwd["dweight"] is None
    assert torch.equal(dh.cpu(), full["dhidden"].cpu())
    assert torch.equal(dw.cpu(), full["dweight"].cpu())
