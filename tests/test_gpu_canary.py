"""Every output is written inside its own rows and nowhere else: outputs live in views of
larger device buffers (a misaligned lead, row strides wider than the rows, a tail) whose
other elements hold a sentinel bit pattern, and after the call every sentinel is intact.
The shapes are the ones that take the partial-vector, unaligned and ragged-tile paths:
RMSNorm and LayerNorm rows of 4097, cross-entropy and distillation over 50257 classes,
SwiGLU on the halves of a [T, 2F] projection with odd F, RoPE with 5 pairs per head and
gaps between tokens, ragged FLCE chunks and tiles, AdamW tensors of ragged sizes.  The
values are those of the same call on plain tensors, bit for bit."""
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX
SENT = {torch.bfloat16: (torch.int16, 0x7E5B), torch.float32: (torch.int32, 0x7FA5A5A5)}


def canary(shape, dtype, lead, ld=None):
    """(buffer, view): a view of `shape` (rows of ld elements, default contiguous)
    starting `lead` elements into a buffer whose every other element is the sentinel."""
    rows, cols = (shape[0], int(torch.tensor(shape[1:]).prod())) if len(shape) > 1 else (1, shape[0])
    ld = cols if ld is None else ld
    n = lead + (rows - 1) * ld + cols + 37
    it, bits = SENT[dtype]
    buf = torch.full((n,), bits, dtype=it, device=DEV).view(dtype)
    if len(shape) == 1:
        view = buf.as_strided(shape, (1,), lead)
    elif len(shape) == 2:
        view = buf.as_strided(shape, (ld, 1), lead)
    else:
        view = buf.as_strided(shape, (ld, shape[2], 1), lead)
    return buf, view, (rows, cols, ld, lead)


def intact(buf, geom, name):
    rows, cols, ld, lead = geom
    it, bits = SENT[buf.dtype]
    mask = torch.ones(buf.numel(), dtype=torch.bool)
    idx = (lead + torch.arange(rows)[:, None] * ld + torch.arange(cols)[None, :]).flatten()
    mask[idx] = False
    outside = buf.view(it).cpu()[mask]
    bad = (outside != torch.tensor(bits, dtype=it)).nonzero().flatten()
    assert len(bad) == 0, f"{name}: {len(bad)} element(s) outside the output written"


def rnd(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(dtype).to(DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rmsnorm_and_layernorm_rows_of_4097(gpu, dtype):
    T, d = 37, 4097
    x, dy, w, b = rnd((T, d), 1, dtype), rnd((T, d), 2, dtype), rnd((d,), 3, dtype), rnd((d,), 4, dtype)
    y0, r0 = gpu.fo_rmsnorm_fwd(x, w, 1e-5)
    dx0, dw0 = gpu.fo_rmsnorm_bwd(dy, x, w, r0, 1e-5)
    by, y, gy = canary((T, d), dtype, 3, ld=d + 4)
    br, r, gr = canary((T,), torch.float32, 1)
    gpu.fo_rmsnorm_fwd(x, w, 1e-5, y=y, rstd=r)
    bdx, dx, gdx = canary((T, d), dtype, 5, ld=d + 6)
    bdw, dw, gdw = canary((d,), torch.float32, 2)
    gpu.fo_rmsnorm_bwd(dy, x, w, r, 1e-5, dx=dx, dw=dw)
    torch.cuda.synchronize()
    for buf, g, n in ((by, gy, "y"), (br, gr, "rstd"), (bdx, gdx, "dx"), (bdw, gdw, "dw")):
        intact(buf, g, "rmsnorm " + n)
    assert torch.equal(y, y0) and torch.equal(r, r0) and torch.equal(dx, dx0) and torch.equal(dw, dw0)
    ly0, m0, s0 = gpu.fo_layernorm_fwd(x, w, b, 1e-5)
    ldx0, ldw0, ldb0 = gpu.fo_layernorm_bwd(dy, x, w, m0, s0)
    by, y, gy = canary((T, d), dtype, 1, ld=d + 2)
    bm, m, gm = canary((T,), torch.float32, 3)
    gpu.fo_layernorm_fwd(x, w, b, 1e-5, y=y, mean=m, rstd=r)
    bdx, dx, gdx = canary((T, d), dtype, 7, ld=d + 1)
    bdb, db, gdb = canary((d,), torch.float32, 1)
    gpu.fo_layernorm_bwd(dy, x, w, m, r, dx=dx, dw=dw, db=db)
    torch.cuda.synchronize()
    for buf, g, n in ((by, gy, "y"), (bm, gm, "mean"), (bdx, gdx, "dx"), (bdw, gdw, "dw"), (bdb, gdb, "db")):
        intact(buf, g, "layernorm " + n)
    assert torch.equal(y, ly0) and torch.equal(dx, ldx0) and torch.equal(dw, ldw0) and torch.equal(db, ldb0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cross_entropy_and_distillation_over_50257(gpu, dtype):
    T, V = 12, 50257
    z, zt = rnd((T, V), 5, dtype, 2.0), rnd((T, V), 6, dtype, 2.0)
    g = torch.Generator().manual_seed(7)
    t = torch.randint(0, V, (T,), generator=g)
    t[4] = IGN
    t = t.to(DEV)
    a = gpu.fo_xent_fwd_bwd(z, t, IGN, 1e-4, 1.0)
    bd, d, gd = canary((T, V), dtype, 1, ld=V + 3)
    o = gpu.fo_xent_fwd_bwd(z, t, IGN, 1e-4, 1.0, dlogits=d)
    torch.cuda.synchronize()
    intact(bd, gd, "xent dlogits")
    assert torch.equal(d, a["dlogits"]) and torch.equal(o["loss"], a["loss"])
    mask = torch.ones(T, dtype=torch.uint8, device=DEV)
    mask[3] = 0
    k = gpu.fo_distill_fwd_bwd(z, zt, mask)
    bd, d, gd = canary((T, V), dtype, 3, ld=V + 1)
    o = gpu.fo_distill_fwd_bwd(z, zt, mask, dlogits=d)
    torch.cuda.synchronize()
    intact(bd, gd, "distill dlogits")
    assert torch.equal(d, k["dlogits"]) and torch.equal(o["loss"], k["loss"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_swiglu_halves_with_odd_width(gpu, dtype):
    T, F = 9, 14337
    gu, dh = rnd((T, 2 * F), 8, dtype), rnd((T, F), 9, dtype)
    g, u = gu[:, :F], gu[:, F:]
    h0 = gpu.fo_swiglu_fwd(g, u)
    dg0, du0 = gpu.fo_swiglu_bwd(dh, g, u)
    bh, h, gh = canary((T, F), dtype, 1, ld=F + 5)
    gpu.fo_swiglu_fwd(g, u, h=h)
    bg, dgv, gg = canary((T, F), dtype, 2, ld=F + 3)
    bu, duv, gu_ = canary((T, F), dtype, 3, ld=F + 1)
    gpu.fo_swiglu_bwd(dh, g, u, dgate=dgv, dup=duv)
    torch.cuda.synchronize()
    for buf, gm, n in ((bh, gh, "h"), (bg, gg, "dgate"), (bu, gu_, "dup")):
        intact(buf, gm, "swiglu " + n)
    assert torch.equal(h, h0) and torch.equal(dgv, dg0) and torch.equal(duv, du0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_in_place_with_gaps_between_tokens(gpu, dtype):
    T, hq, hk, D = 23, 4, 2, 10
    pos = torch.arange(T, device=DEV) * 37
    bq, q, gq = canary((T, hq, D), dtype, 1, ld=hq * D + 6)
    bk, k, gk = canary((T, hk, D), dtype, 2, ld=hk * D + 3)
    q.copy_(rnd((T, hq, D), 10, dtype))
    k.copy_(rnd((T, hk, D), 11, dtype))
    q0, k0 = q.contiguous(), k.contiguous()
    gpu.fo_rope_fwd(q0, k0, pos, 1e4)
    gpu.fo_rope_fwd(q, k, pos, 1e4)
    torch.cuda.synchronize()
    intact(bq, gq, "rope q")
    intact(bk, gk, "rope k")
    assert torch.equal(q, q0) and torch.equal(k, k0)


def test_flce_ragged_chunks_and_tiles(gpu):
    cfg = synth.flce_small(37, 64, 1000, seed=3)
    i = synth.flce_inputs(cfg)
    h, w, t = i["hidden"].to(DEV), i["weight"].to(DEV), i["targets"].to(DEV)
    a = gpu.fo_flce_fwd_bwd(h, w, t, IGN, cfg.z_loss, 1.0, chunk_tokens=16)
    # dH must be contiguous and 16-byte aligned: the lead is a whole 16-byte vector
    bh, dh, gh = canary((37, 64), torch.bfloat16, 8)
    bw, dw, gw = canary((1000, 64), torch.float32, 4)
    o = gpu.fo_flce_fwd_bwd(h, w, t, IGN, cfg.z_loss, 1.0, chunk_tokens=16, dhidden=dh, dweight=dw)
    torch.cuda.synchronize()
    intact(bh, gh, "flce dhidden")
    intact(bw, gw, "flce dweight")
    assert torch.equal(dh, a["dhidden"]) and torch.equal(dw, a["dweight"])
    assert torch.equal(o["loss"], a["loss"])


def test_adamw_ragged_tensors(gpu):
    sizes = [5000, 4097, 1, 12289]
    st = synth.adamw_inputs(sizes, seed=5)
    bufs = {}
    views = {k: [] for k in st}
    for k in st:
        for j, x in enumerate(st[k]):
            b, v, g = canary((x.numel(),), torch.float32, 1 + (j % 2) * 3)  # misaligned and aligned
            v.copy_(x.to(DEV))
            bufs[(k, j)] = (b, g)
            views[k].append(v)
    hyp = dict(step_size=1e-3, beta1=0.9, beta2=0.95, bias_correction=0.3, decay_factor=0.999, eps=1e-8)
    gpu.fo_adamw_step(views["params"], views["grads"], views["exp_avgs"], views["exp_avg_sqs"], **hyp)
    torch.cuda.synchronize()
    for (k, j), (b, g) in bufs.items():
        intact(b, g, f"adamw {k}[{j}]")
    # misaligned tensors take the element path, aligned ones the vector path: both match
    # the oracle (not necessarily each other bit for bit)
    for j in range(len(sizes)):
        p, m, v = oracle.adamw_step(st["params"][j], st["grads"][j], st["exp_avgs"][j],
                                    st["exp_avg_sqs"][j], **hyp)
        check(views["params"][j].cpu(), p, "f32", f"param {j}")
        check(views["exp_avgs"][j].cpu(), m, "f32", f"exp_avg {j}")
        check(views["exp_avg_sqs"][j].cpu(), v, "f32", f"exp_avg_sq {j}")
