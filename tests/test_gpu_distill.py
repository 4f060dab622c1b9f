"""GPU parity of fo_distill_fwd_bwd (soft-target cross-entropy) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check, check_loss, check_softmax_diff, kl_terms

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(fo, z, zt, mask, dloss=1.0, want_grad=True):
    o = fo.fo_distill_fwd_bwd(z.to(DEV), zt.to(DEV), None if mask is None else mask.to(DEV),
                              dloss, want_grad=want_grad)
    torch.cuda.synchronize()
    return {k: (v.cpu() if v is not None else None) for k, v in o.items()}


def softmax_sum(z, zt, keep, scale):
    """|scale| (q f_q + p f_p) + a floor of 2^-125 |scale| / 1e-5 on the kept rows (zero
    elsewhere): the error scale of dz.  f = max(1, 0.03 (|x| + |lse|)) per softmax: fp32
    carries a few units of 2^-24 of the magnitudes of the logit and its logsumexp into the
    softmax's relative error; the floor covers softmax values below fp32's normal range."""
    out = np.zeros(tuple(z.shape))
    if keep.any():
        z64, t64 = z.double().numpy()[keep], zt.double().numpy()[keep]

        def soft(x):
            m = x.max(1, keepdims=True)
            e = np.exp(x - m)
            lse = m + np.log(e.sum(1, keepdims=True))
            return e / e.sum(1, keepdims=True) * np.maximum(1.0, 0.03 * (np.abs(x) + np.abs(lse)))

        out[keep] = abs(scale) * (soft(z64) + soft(t64) + 2.0 ** -125 / 1e-5)
    return out


def compare(z, zt, mask, o, dt, dloss=1.0):
    r = oracle.distill_fwd_bwd(z, zt, mask, dloss)
    assert o["n_valid"].item() == r["n_valid"]
    check_loss(o["loss"].item(), r["loss"])
    keep = np.ones(z.shape[0], bool) if mask is None else mask.numpy() != 0
    check_loss(o["kl"].item(), r["kl"], "kl", scale=kl_terms(z, zt, keep))
    if o["dlogits"] is not None:
        check(o["dlogits"], r["dlogits"], dt, "dlogits")
        keep = np.ones(z.shape[0], bool) if mask is None else mask.numpy() != 0
        n = max(1, int(keep.sum()))
        check_softmax_diff(o["dlogits"], r["dlogits"], softmax_sum(z, zt, keep, dloss / n),
                           "dlogits", rounded_out=dt == "bf16")
        if mask is not None:
            dropped = (mask == 0).nonzero().flatten()
            assert torch.all(o["dlogits"][dropped].float() == 0)


def cfg_of(dtype, T, V, seed=31, logit_std=3.0):
    return synth.Config(0, "kd", dtype, T=T, d=8, n_q=1, n_kv=1, head_dim=2, F=1, V=V,
                        eps=1e-5, theta=1e4, logit_std=logit_std, z_loss=0, ignore_frac=0,
                        packed=False, doc_lengths=(T,), seed=seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [100, 1000, 4096, 8199, 12000, 12001, 16384, 16389, 49152, 50257,
                               128256, 151936])
def test_vocab_paths(gpu, dtype, V):
    # Rows off the 16-byte grid (V 100, 8199, 12001, 16389, 50257: 16-byte accesses at
    # element-aligned addresses, the partial last vector element by element) in each of
    # their plans: whole rows in 256 threads keeping up to 4 vectors (bf16 100) or 6
    # (bf16 8199 and 12001), longer rows in 512 threads keeping 8 and streaming the rest
    # (bf16 16389 and up, fp32 8199 and up); aligned rows: 1000/4096
    # (whole rows in 256 threads of up to 4 vectors), 12000/16384 (whole rows in 256
    # threads of up to 8; fp32 16384 and the longer ones: 512 threads keeping 8 vectors
    # per thread of each row and streaming the rest twice)
    T = 6 if V > 50000 else 23
    i = synth.distill_inputs(cfg_of(dtype, T, V))
    o = run(gpu, i["logits"], i["teacher"], i["row_mask"])
    compare(i["logits"], i["teacher"], i["row_mask"], o, dtype)


def test_no_mask_forward_only_and_dloss(gpu):
    i = synth.distill_inputs(cfg_of("bf16", 40, 32000, seed=5))
    o = run(gpu, i["logits"], i["teacher"], None, dloss=0.5)
    compare(i["logits"], i["teacher"], None, o, "bf16", dloss=0.5)
    f = run(gpu, i["logits"], i["teacher"], None, want_grad=False)
    assert f["dlogits"] is None and f["loss"].item() == o["loss"].item()


def test_all_masked(gpu):
    i = synth.distill_inputs(cfg_of("bf16", 12, 5000, seed=6), mask_frac=1.0)
    o = run(gpu, i["logits"], i["teacher"], i["row_mask"])
    assert o["loss"].item() == 0.0 and o["kl"].item() == 0.0 and o["n_valid"].item() == 0
    assert torch.all(o["dlogits"].float() == 0)


def test_teacher_equals_student(gpu):
    i = synth.distill_inputs(cfg_of("f32", 9, 8192, seed=7))
    o = run(gpu, i["logits"], i["logits"].clone(), None)
    assert abs(o["kl"].item()) < 1e-5
    assert o["dlogits"].abs().max().item() < 1e-9


def test_in_place_gradient(gpu):
    i = synth.distill_inputs(cfg_of("bf16", 16, 128256, seed=8))
    zg, tg, mg = i["logits"].to(DEV), i["teacher"].to(DEV), i["row_mask"].to(DEV)
    ref = gpu.fo_distill_fwd_bwd(zg, tg, mg)
    z2 = zg.clone()
    o = gpu.fo_distill_fwd_bwd(z2, tg, mg, dlogits=z2)
    torch.cuda.synchronize()
    assert torch.equal(z2, ref["dlogits"]) and o["loss"].item() == ref["loss"].item()


def test_full_size_sampled(gpu):
    """T 8192 x V 128256 bf16 (the Llama-3-8B lm-head logits) in one call: gradient rows
    sampled against the oracle, the loss against a row-block oracle sum."""
    cfg = synth.scaled(synth.CONFIGS[3], 8192)
    i = synth.distill_inputs(cfg)
    z, zt, mask = i["logits"], i["teacher"], i["row_mask"]
    o = run(gpu, z, zt, mask)
    n = int((mask != 0).sum())
    assert o["n_valid"].item() == n
    rows = np.unique(np.concatenate([[0, cfg.T - 1], np.random.default_rng(9).integers(0, cfg.T, 12)]))
    keep = [r for r in rows if mask[r] != 0]
    rr = oracle.distill_fwd_bwd(z[keep], zt[keep], None, dloss=len(keep) / n)
    check(o["dlogits"][keep], rr["dlogits"], "bf16", "dlogits rows")
    check_softmax_diff(o["dlogits"][keep], rr["dlogits"],
                       softmax_sum(z[keep], zt[keep], np.ones(len(keep), bool), 1.0 / n),
                       "dlogits rows")
    ce = kl = 0.0
    for r0 in range(0, cfg.T, 1024):
        b = oracle.distill_fwd_bwd(z[r0:r0 + 1024], zt[r0:r0 + 1024], mask[r0:r0 + 1024])
        ce += b["loss"] * b["n_valid"]
        kl += b["kl"] * b["n_valid"]
    check_loss(o["loss"].item(), ce / n)
    check_loss(o["kl"].item(), kl / n, "kl")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_rows_in_place(gpu, dtype):
    # a 50257-wide vocabulary (every row at another alignment), gradient written over the
    # student logits: the same bits as out of place
    i = synth.distill_inputs(cfg_of(dtype, 10, 50257, seed=9))
    z, zt, m = i["logits"].to(DEV), i["teacher"].to(DEV), i["row_mask"].to(DEV)
    a = gpu.fo_distill_fwd_bwd(z, zt, m)
    zc = z.clone()
    b = gpu.fo_distill_fwd_bwd(zc, zt, m, dlogits=zc)
    torch.cuda.synchronize()
    assert torch.equal(a["dlogits"].cpu(), b["dlogits"].cpu())
    assert torch.equal(a["loss"].cpu(), b["loss"].cpu()) and torch.equal(a["kl"].cpu(), b["kl"].cpu())
