"""GPU parity of fo_flce_fwd_bwd against the fp64 oracle, plus its chunking and
masking properties."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import check, check_bf16, check_loss

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX


def run(fo, h, w, t, zc, chunk=0, dwt=torch.float32, dloss=1.0):
    o = fo.fo_flce_fwd_bwd(h.to(DEV), w.to(DEV), t.to(DEV), IGN, zc, dloss, dweight_dtype=dwt,
                           chunk_tokens=chunk)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in o.items()}


def compare(h, w, t, zc, o, dloss=1.0):
    r = oracle.flce_fwd_bwd(h, w, t, IGN, zc, dloss, chunk=256)
    check_loss(o["loss"].item(), r["loss"])
    check_loss(o["z_loss"].item(), r["z_loss"], "z_loss")
    assert o["n_valid"].item() == r["n_valid"]
    check_bf16(o["dhidden"], r["dhidden"], "dhidden")
    check_bf16(o["dweight"], r["dweight"], "dweight")
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


def test_full_size_sampled(gpu):
    """The lm-head workload at full size, in the launch configuration the bench times.
    dH rows are checked one by one against the oracle (each needs only its own row's
    logits); the loss and dW need every row's logsumexp, so at this size they are
    checked through properties: chunk-size independence and, with z-loss off, the
    vocabulary sum of dW, which vanishes because every softmax-gradient row sums to 0."""
    cfg = synth.CONFIGS[5]
    i = synth.flce_inputs(cfg)
    h, w, t = i["hidden"], i["weight"], i["targets"]
    o = run(gpu, h, w, t, cfg.z_loss)
    n_full = int((t != IGN).sum())
    assert o["n_valid"].item() == n_full
    rows = np.unique(np.concatenate([[0, cfg.T - 1],
                                     np.random.default_rng(5).integers(0, cfg.T, 10)]))
    W64 = w.double().numpy()
    for r in rows:
        z = (W64 @ h[r].double().numpy())[None, :]
        tg = t[r:r + 1].numpy()
        _, _, _, dz = oracle.xent_rows(z, tg, tg != IGN, n_full, cfg.z_loss, 1.0)
        check_bf16(o["dhidden"][r:r + 1], dz @ W64, f"dhidden row {r}")
    ign = (t == IGN).nonzero().flatten()
    assert torch.all(o["dhidden"][ign].view(torch.int16) == 0)
    o0 = run(gpu, h, w, t, 0.0, chunk=1024)
    colsum = o0["dweight"].double().sum(0)
    scale = o0["dweight"].double().abs().sum(0)
    assert torch.all(colsum.abs() <= 1e-3 * scale + 1e-6), float((colsum.abs() / scale).max())
    o1 = run(gpu, h, w, t, 0.0, chunk=0)
    check_loss(o1["loss"].item(), o0["loss"].item(), rel=1e-6)
    check_bf16(o1["dweight"], o0["dweight"].double(), "dweight chunk 1024 vs auto")
