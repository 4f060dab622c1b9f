"""GPU parity past 2^31 elements per tensor (byte offsets past 4 GiB for bf16).

Every kernel forms row and element offsets in 64 bits (buffer resources are built per
row, per operand panel or per K slice, so their 32-bit ranges stay small whatever the
tensor's size).  These cases put rows on both sides of the 2^31-element mark and at the
very end of such tensors, and check them against the fp64 oracle; the reductions over
every row (the cross-entropy and distillation losses, the norms' dw and db) are checked against
the oracle over row blocks.  One case per kernel family: cross-entropy (in place),
distillation, RMSNorm and LayerNorm forward and backward, RoPE forward and backward,
SwiGLU on contiguous operands and on the halves of a [T, 2F] tensor, the plain GeLU, an
AdamW step over a tensor of more than 2^31 elements, and the fused linear cross-entropy
with an lm-head weight of more than 2^31 elements (its fp32 dW past 8 GiB)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from blockwise import map_blocks
from tolerance import (check, check_bf16, check_loss, check_product_grad, check_softmax_diff,
                       adamw_terms, flce_target_terms, layernorm_y_terms, norm_dw_terms,
                       norm_dx_terms)

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX
BIG = 1 << 31


def sample_rows(n_cols, T, seed, n_random=8):
    """The first and last rows, the rows on both sides of the 2^31-element mark of a
    [T, n_cols] tensor, and a few random ones."""
    r = BIG // n_cols
    fixed = np.array([0, r - 1, r, r + 1, T - 2, T - 1])
    rnd = np.random.default_rng(seed).integers(0, T, n_random)
    return np.unique(np.concatenate([fixed, rnd]).clip(0, T - 1))


def on_host(t, rows):
    return t[torch.from_numpy(rows).to(t.device)].cpu()


@pytest.fixture(autouse=True)
def free_device_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_xent_in_place(gpu):
    # the 151936-entry vocabulary over a 16384-token batch: 2.49e9 bf16 logits (4.98 GB),
    # 10% of the targets ignored, z-loss 1e-4, the gradient written over the logits
    cfg = dataclasses.replace(synth.CONFIGS[2], T=16384, doc_lengths=(16384,),
                              ignore_frac=0.1, z_loss=1e-4)
    i = synth.xent_inputs(cfg)
    z, t = i["logits"], i["targets"]
    assert z.numel() > BIG
    zg = z.to(DEV)
    o = gpu.fo_xent_fwd_bwd(zg, t.to(DEV), IGN, cfg.z_loss, 1.0, dlogits=zg)
    torch.cuda.synchronize()
    n_full = int((t != IGN).sum())
    assert o["n_valid"].item() == n_full and o["status"].item() == 0
    rows = sample_rows(cfg.V, cfg.T, 151936)
    tg = t[rows].numpy()
    valid = tg != IGN
    _, _, _, dz = oracle.xent_rows(z[rows].double().numpy(), tg, valid, n_full, cfg.z_loss, 1.0)
    check(on_host(zg, rows), dz, "bf16", "dlogits", single_rounding=True)
    ign = (t == IGN).nonzero().flatten()[-64:].numpy()  # ignored rows near the end
    assert torch.all(on_host(zg, ign).view(torch.int16) == 0)
    del zg

    def one(r0, r1):
        b = oracle.xent_fwd_bwd(z[r0:r1], t[r0:r1], IGN, cfg.z_loss, 1.0)
        return b["loss"] * b["n_valid"], b["z_loss"] * b["n_valid"], b["n_valid"]

    parts = map_blocks(one, cfg.T, 256)
    assert sum(p[2] for p in parts) == n_full
    check_loss(o["loss"].item(), sum(p[0] for p in parts) / n_full)
    check_loss(o["z_loss"].item(), sum(p[1] for p in parts) / n_full, "z_loss")


def test_distillation(gpu):
    # student and teacher logits of 16384 x 151936 bf16 (two 4.98 GB tensors), 10% of
    # the rows masked, the gradient into a third such tensor
    cfg = dataclasses.replace(synth.CONFIGS[2], T=16384, doc_lengths=(16384,), logit_std=3.0)
    i = synth.distill_inputs(cfg)
    z, zt, mask = i["logits"], i["teacher"], i["row_mask"]
    assert z.numel() > BIG
    o = gpu.fo_distill_fwd_bwd(z.to(DEV), zt.to(DEV), mask.to(DEV), 1.0)
    torch.cuda.synchronize()
    n = int((mask != 0).sum())
    assert o["n_valid"].item() == n
    rows = sample_rows(cfg.V, cfg.T, 3)
    keep = np.array([r for r in rows if mask[r] != 0])
    gone = np.array([r for r in rows if mask[r] == 0] +
                    list((mask == 0).nonzero().flatten()[-8:].numpy()))
    rr = oracle.distill_fwd_bwd(z[keep], zt[keep], None, dloss=len(keep) / n)
    got = on_host(o["dlogits"], keep)
    check(got, rr["dlogits"], "bf16", "dlogits rows")
    z64, t64 = z[keep].double().numpy(), zt[keep].double().numpy()
    q = np.exp(z64 - z64.max(1, keepdims=True))
    p = np.exp(t64 - t64.max(1, keepdims=True))
    qp = (q / q.sum(1, keepdims=True) + p / p.sum(1, keepdims=True)) / n
    check_softmax_diff(got, rr["dlogits"], qp, "dlogits rows")
    assert torch.all(on_host(o["dlogits"], gone).float() == 0)
    del o["dlogits"]

    def one(r0, r1):
        b = oracle.distill_fwd_bwd(z[r0:r1], zt[r0:r1], mask[r0:r1])
        return b["loss"] * b["n_valid"], b["kl"] * b["n_valid"]

    parts = map_blocks(one, cfg.T, 256)
    check_loss(o["loss"].item(), sum(p[0] for p in parts) / n)
    check_loss(o["kl"].item(), sum(p[1] for p in parts) / n, "kl")


def test_rmsnorm_forward_backward(gpu):
    # Llama-3-8B rows (d 4096, bf16) over 524800 tokens: 2.15e9 elements per tensor;
    # dw sums every row
    cfg = dataclasses.replace(synth.CONFIGS[3], T=524800, doc_lengths=(524800,))
    i = synth.rmsnorm_inputs(cfg)
    x, w, dy, eps = i["x"], i["w"], i["dy"], cfg.eps
    assert x.numel() > BIG
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    y, rstd = gpu.fo_rmsnorm_fwd(xg, wg, eps)
    dx, dw = gpu.fo_rmsnorm_bwd(dyg, xg, wg, rstd, eps)
    torch.cuda.synchronize()
    del xg, dyg
    rows = sample_rows(cfg.d, cfg.T, 4096)
    ry, rr = oracle.rmsnorm_fwd(x[rows], w, eps)
    rdx, _ = oracle.rmsnorm_bwd(dy[rows], x[rows], w, eps)
    check(on_host(y, rows), ry, "bf16", "y", single_rounding=True)
    check(on_host(rstd, rows), rr, "f32", "rstd")
    check(on_host(dx, rows), rdx, "bf16", "dx", single_rounding=True,
          scale=norm_dx_terms(dy[rows], x[rows], w, eps, False))
    def one(r0, r1):
        return (oracle.rmsnorm_bwd(dy[r0:r1], x[r0:r1], w, eps)[1],
                norm_dw_terms(dy[r0:r1], x[r0:r1], eps, False))

    parts = map_blocks(one, cfg.T, 4096)
    # the blocks' term sizes combine as their root sum of squares
    check(dw.cpu(), sum(p[0] for p in parts), "f32", "dw",
          scale=np.sqrt(sum(p[1] ** 2 for p in parts)))


@pytest.mark.parametrize("halves", [False, True])
def test_swiglu_forward_backward(gpu, halves):
    # Llama-3-8B MLP width (F 14336, bf16) over 149800 tokens: 2.1475e9 elements per
    # operand; halves: gate and up (and dgate and dup) are the two halves of one
    # [T, 2F] tensor, 4.3e9 elements, rows 57344 bytes apart
    cfg = dataclasses.replace(synth.CONFIGS[3], T=149800, doc_lengths=(149800,))
    i = synth.swiglu_inputs(cfg)
    g, u, dh = i["gate"], i["up"], i["dh"]
    T, F = g.shape
    assert g.numel() > BIG
    if halves:
        gu = torch.empty((T, 2 * F), dtype=g.dtype, device=DEV)
        gu[:, :F] = g.to(DEV)
        gu[:, F:] = u.to(DEV)
        gg, ug = gu[:, :F], gu[:, F:]
        dgu = torch.empty_like(gu)
        dgo, duo = dgu[:, :F], dgu[:, F:]
    else:
        gg, ug = g.to(DEV), u.to(DEV)
        dgo = duo = None
    h = gpu.fo_swiglu_fwd(gg, ug)
    dg, du = gpu.fo_swiglu_bwd(dh.to(DEV), gg, ug, dgate=dgo, dup=duo)
    torch.cuda.synchronize()
    rows = sample_rows(F, T, 14336 + halves)
    if halves:
        rows = np.unique(np.concatenate([rows, sample_rows(2 * F, T, 0, 0)]))
    check(on_host(h, rows), oracle.swiglu_fwd(g[rows], u[rows]), "bf16", "h",
          single_rounding=True)
    rg, ru = oracle.swiglu_bwd(dh[rows], g[rows], u[rows])
    check(on_host(dg, rows), rg, "bf16", "dgate", single_rounding=True)
    check(on_host(du, rows), ru, "bf16", "dup", single_rounding=True)


def test_flce_weight_past_2g_elements(gpu):
    # an lm head of 262208 x 8192 (2.148e9 bf16 weights, 4.3 GB; its fp32 dW 8.6 GB) on
    # 256 tokens, 10% ignored, z-loss 1e-4: loss, dH rows and dW rows on both sides of the
    # 2^31-element mark and at the end, under the bound of products of the rounded dZ
    cfg = synth.flce_small(256, 8192, 262208, seed=77)
    i = synth.flce_inputs(cfg)
    h, w, t = i["hidden"], i["weight"], i["targets"]
    assert w.numel() > BIG
    o = gpu.fo_flce_fwd_bwd(h.to(DEV), w.to(DEV), t.to(DEV), IGN, cfg.z_loss, 1.0)
    torch.cuda.synchronize()
    tn = t.numpy()
    V, H = w.shape
    g = np.random.default_rng(78)
    hit = np.unique(tn[tn != IGN])
    dw_rows = np.unique(np.concatenate([sample_rows(H, V, 79), g.choice(hit, 8, replace=False),
                                        hit[-2:]]))
    dh_rows = np.unique(np.concatenate([[0, cfg.T - 1], np.nonzero(tn == IGN)[0][:4],
                                        g.integers(0, cfg.T, 8)]))
    # the whole batch in one oracle chunk: |W| is formed once for the dH bound
    r = oracle.flce_fwd_bwd(h, w.double().numpy(), t, IGN, cfg.z_loss, 1.0,
                            dh_rows=dh_rows, dw_rows=dw_rows, abs_products=True)
    check_loss(o["loss"].item(), r["loss"])
    check_loss(o["z_loss"].item(), r["z_loss"], "z_loss")
    assert o["n_valid"].item() == r["n_valid"] and o["status"].item() == r["n_bad"] == 0
    gh, gw = on_host(o["dhidden"], dh_rows), on_host(o["dweight"], dw_rows)
    check_bf16(gh, r["dhidden"], "dhidden")
    check_product_grad(gh, r["dhidden"], r["dhidden_abs"], "dhidden",
                       target=flce_target_terms(w, tn, r["n_valid"], 1.0, dh_rows, "dh"))
    check_bf16(gw, r["dweight"], "dweight")
    check_product_grad(gw, r["dweight"], r["dweight_abs"], "dweight", rounded_out=False,
                       target=flce_target_terms(h, tn, r["n_valid"], 1.0, dw_rows, "dw"))
    ign = np.nonzero(tn == IGN)[0]
    assert torch.all(on_host(o["dhidden"], ign).view(torch.int16) == 0)


def test_layernorm_forward_backward(gpu):
    # LayerNorm over the same 524800 x 4096 bf16 rows (x ~ N(1, 1)); dw and db sum every row
    cfg = dataclasses.replace(synth.CONFIGS[3], T=524800, doc_lengths=(524800,))
    i = synth.layernorm_inputs(cfg)
    x, w, b, dy, eps = i["x"], i["w"], i["b"], i["dy"], cfg.eps
    assert x.numel() > BIG
    xg, dyg = x.to(DEV), dy.to(DEV)
    y, mean, rstd = gpu.fo_layernorm_fwd(xg, w.to(DEV), b.to(DEV), eps)
    dx, dw, db = gpu.fo_layernorm_bwd(dyg, xg, w.to(DEV), mean, rstd)
    torch.cuda.synchronize()
    del xg, dyg
    rows = sample_rows(cfg.d, cfg.T, 4097)
    ry, rm, rr = oracle.layernorm_fwd(x[rows], w, b, eps)
    rdx, _, _ = oracle.layernorm_bwd(dy[rows], x[rows], w, eps)
    check(on_host(y, rows), ry, "bf16", "y", single_rounding=True,
          scale=layernorm_y_terms(x[rows], w, b, eps))
    check(on_host(mean, rows), rm, "f32", "mean")
    check(on_host(rstd, rows), rr, "f32", "rstd")
    check(on_host(dx, rows), rdx, "bf16", "dx", single_rounding=True,
          scale=norm_dx_terms(dy[rows], x[rows], w, eps, True))
    def one(r0, r1):
        _, a, c = oracle.layernorm_bwd(dy[r0:r1], x[r0:r1], w, eps)
        return a, c, norm_dw_terms(dy[r0:r1], x[r0:r1], eps, True)

    parts = map_blocks(one, cfg.T, 4096)
    # the blocks' centring term sizes combine as their root sum of squares
    check(dw.cpu(), sum(p[0] for p in parts), "f32", "dw",
          scale=np.sqrt(sum(p[2] ** 2 for p in parts)))
    check(db.cpu(), sum(p[1] for p in parts), "f32", "db")


def test_rope_forward_backward(gpu):
    # Llama-3-8B heads (32 query / 8 key-value heads of 128) over 524800 tokens at
    # positions 0 .. 524799: q of 2.15e9 bf16 elements, rotated in place
    cfg = dataclasses.replace(synth.CONFIGS[3], T=524800, doc_lengths=(524800,))
    i = synth.rope_inputs(cfg)
    q, k, dq, dk, pos = i["q"], i["k"], i["dq"], i["dk"], i["pos"]
    assert q.numel() > BIG
    pg = pos.to(DEV)
    qg, kg = q.to(DEV), k.to(DEV)
    gpu.fo_rope_fwd(qg, kg, pg, cfg.theta)
    rows = sample_rows(cfg.n_q * cfg.head_dim, cfg.T, 5)
    torch.cuda.synchronize()
    rq, rk = oracle.rope_fwd(q[rows], k[rows], pos[rows], cfg.theta)
    check(on_host(qg, rows), rq, "bf16", "q", single_rounding=True)
    check(on_host(kg, rows), rk, "bf16", "k", single_rounding=True)
    del qg, kg
    dqg, dkg = dq.to(DEV), dk.to(DEV)
    gpu.fo_rope_bwd(dqg, dkg, pg, cfg.theta)
    torch.cuda.synchronize()
    oq, ok = oracle.rope_bwd(dq[rows], dk[rows], pos[rows], cfg.theta)
    check(on_host(dqg, rows), oq, "bf16", "dq", single_rounding=True)
    check(on_host(dkg, rows), ok, "bf16", "dk", single_rounding=True)


def test_plain_gelu_forward_backward(gpu):
    # the plain (ungated) GeLU over 149800 x 14336 bf16 (2.1475e9 elements per operand)
    cfg = dataclasses.replace(synth.CONFIGS[3], T=149800, doc_lengths=(149800,))
    i = synth.swiglu_inputs(cfg)
    x, dy = i["gate"], i["dh"]
    assert x.numel() > BIG
    xg = x.to(DEV)
    y = gpu.fo_act_fwd("gelu", xg)
    dx = gpu.fo_act_bwd("gelu", dy.to(DEV), xg)
    torch.cuda.synchronize()
    rows = sample_rows(cfg.F, cfg.T, 6)
    check(on_host(y, rows), oracle.act_fwd(x[rows], "gelu"), "bf16", "y", single_rounding=True)
    check(on_host(dx, rows), oracle.act_bwd(dy[rows], x[rows], "gelu"), "bf16", "dx",
          single_rounding=True)


def test_adamw_tensor_past_2g_elements(gpu):
    # one fp32 tensor of 2^31 + 4099 elements (8.6 GB per array; its last chunk ragged)
    # beside a small one, in one call; sampled elements on both sides of 2^31 and at the end
    sizes = [BIG + 4099, 5000]
    i = synth.adamw_inputs(sizes, 11)
    d = {k: [t.to(DEV) for t in v] for k, v in i.items()}
    ss, bc, df = oracle.adamw_scalars(3e-4, 0.9, 0.95, 0.1, 10)
    f = lambda v: float(np.float32(v))  # noqa: E731  (the fp32 values the kernel receives)
    sc = dict(step_size=f(ss), beta1=f(0.9), beta2=f(0.95), bias_correction=f(bc),
              decay_factor=f(df), eps=f(1e-8))
    gpu.fo_adamw_step(d["params"], d["grads"], d["exp_avgs"], d["exp_avg_sqs"],
                      sc["step_size"], sc["beta1"], sc["beta2"], sc["bias_correction"],
                      sc["decay_factor"], sc["eps"])
    torch.cuda.synchronize()
    g = np.random.default_rng(12)
    for k, n in enumerate(sizes):
        idx = np.unique(np.concatenate([[0, n - 1, n - 4099, min(n - 1, BIG - 1), min(n - 1, BIG)],
                                        g.integers(0, n, 4000)]))
        ti = torch.from_numpy(idx)
        rp, rm, rv = oracle.adamw_step(i["params"][k][ti], i["grads"][k][ti], i["exp_avgs"][k][ti],
                                       i["exp_avg_sqs"][k][ti], sc["step_size"], sc["beta1"],
                                       sc["beta2"], sc["bias_correction"], sc["decay_factor"],
                                       sc["eps"])
        ap, am = adamw_terms(i["params"][k][ti], i["grads"][k][ti], i["exp_avgs"][k][ti],
                             i["exp_avg_sqs"][k][ti], sc["step_size"], sc["beta1"], sc["beta2"],
                             sc["bias_correction"], sc["decay_factor"], sc["eps"])
        check(d["params"][k][ti.to(DEV)].cpu(), rp, "f32", f"p[{k}]", scale=ap)
        check(d["exp_avgs"][k][ti.to(DEV)].cpu(), rm, "f32", f"m[{k}]", scale=am)
        check(d["exp_avg_sqs"][k][ti.to(DEV)].cpu(), rv, "f32", f"v[{k}]")
