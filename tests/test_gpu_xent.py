"""GPU parity of fo_xent_fwd_bwd against the fp64 oracle, plus its bit-exact
properties (ignored rows, in place, determinism, counters)."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from blockwise import map_blocks
from tolerance import check, check_loss, xent_dz_terms

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX


def run(fo, z, t, zc, dloss=1.0, inplace=False, grad=True):
    zg, tg = z.to(DEV), t.to(DEV)
    o = fo.fo_xent_fwd_bwd(zg, tg, IGN, zc, dloss, dlogits=zg if inplace else None, grad=grad)
    torch.cuda.synchronize()
    return {k: (v.cpu() if v is not None else None) for k, v in o.items()}


def compare(z, t, zc, dt, o, dloss=1.0):
    r = oracle.xent_fwd_bwd(z, t, IGN, zc, dloss)
    check_loss(o["loss"].item(), r["loss"])
    check_loss(o["z_loss"].item(), r["z_loss"], "z_loss")
    assert o["n_valid"].item() == r["n_valid"]
    assert o["status"].item() == r["n_bad"]
    if o["dlogits"] is not None:
        V = z.shape[1]
        check(o["dlogits"], r["dlogits"], dt, "dlogits", single_rounding=True,
              scale=xent_dz_terms(z, t.numpy(), (t != IGN) & (t >= 0) & (t < V), r["lse"], zc,
                                  dloss, r["n_valid"]))
    return r


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 23])
def test_configs_small(gpu, cid, T):
    cfg = synth.scaled(synth.CONFIGS[cid], T)
    i = synth.xent_inputs(cfg)
    t = i["targets"]
    if cid == 4 and T > 1:
        t = t.clone()
        t[::4] = IGN
    compare(i["logits"], t, cfg.z_loss, cfg.dtype, run(gpu, i["logits"], t, cfg.z_loss))


def test_config1_as_stated(gpu):
    # the tiny fp32 block at its stated size: T 256 logits over 4096 classes, N(0, 2^2),
    # uniform targets, every row
    cfg = synth.CONFIGS[1]
    assert cfg.T == 256 and cfg.V == 4096
    i = synth.xent_inputs(cfg)
    compare(i["logits"], i["targets"], cfg.z_loss, cfg.dtype,
            run(gpu, i["logits"], i["targets"], cfg.z_loss))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [4097, 7, 8, 1000, 12000, 12001, 16384, 20000, 32001, 50257,
                               65536, 65544, 131072, 131080, 151936, 163840, 163848, 196608,
                               196616, 81920, 98304, 98312, 200000])
def test_vocab_sizes(gpu, dtype, V):
    # rows off the 16-byte grid (4097, 7, 12001, 32001, 50257: every row starts at another
    # alignment), tiny and register-resident rows (bf16 12000 and 16384: 256 threads of 8
    # vectors, the latter full; bf16 20000 and fp32 12000: 512 threads of 8; fp32 20000,
    # bf16 65536: 512 threads of 16, the latter full; 65544 one vector past it),
    # rows split between registers and LDS (16 vectors per thread in registers and 4 in
    # LDS: bf16 131080, 17 vectors per thread, 151936: 19, 163840: 20; and 8 in LDS:
    # bf16 163848, 21, 196608: 24, the most; fp32 81920: 20, 98304: 24) and streaming
    # rows (longer: bf16 196616, 200000, fp32 98312)
    g = torch.Generator().manual_seed(V)
    T = 9
    z = (2 * torch.randn(T, V, generator=g)).to(synth.torch_dtype(dtype))
    t = torch.randint(0, V, (T,), generator=g)
    t[3] = IGN
    compare(z, t, 1e-4, dtype, run(gpu, z, t, 1e-4, dloss=0.5), dloss=0.5)


def test_ignored_rows_exact_zero_and_garbage_invariance(gpu):
    cfg = synth.scaled(synth.CONFIGS[4], 64)
    i = synth.xent_inputs(cfg)
    z, t = i["logits"].clone(), i["targets"].clone()
    t[[0, 5, 6, 63]] = IGN
    a = run(gpu, z, t, 0.0)
    ign = (t == IGN).nonzero().flatten()
    d = a["dlogits"][ign]
    assert torch.all(d.view(torch.int16) == 0)  # +0.0 bit pattern
    z2 = z.clone()
    z2[ign] = 1234.0  # finite garbage in ignored rows changes nothing
    b = run(gpu, z2, t, 0.0)
    assert torch.equal(a["loss"], b["loss"]) and torch.equal(a["dlogits"], b["dlogits"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_rows_in_place_and_strided(gpu, dtype):
    # a 50257-wide vocabulary (rows start at every alignment) in place, and the same rows
    # as a view with a row stride of 50263 and a misaligned base: the same bits
    g = torch.Generator().manual_seed(50257)
    T, V = 12, 50257
    z = (2 * torch.randn(T, V, generator=g)).to(synth.torch_dtype(dtype))
    t = torch.randint(0, V, (T,), generator=g)
    t[5] = IGN
    a = run(gpu, z, t, 1e-4)
    compare(z, t, 1e-4, dtype, a)
    b = run(gpu, z, t, 1e-4, inplace=True)
    assert torch.equal(a["dlogits"], b["dlogits"]) and torch.equal(a["loss"], b["loss"])
    wide = torch.zeros(T, V + 6, dtype=z.dtype)
    wide[:, 3:3 + V] = z
    zs = wide.to(DEV)[:, 3:3 + V]  # base 6 bytes (bf16) / 12 bytes (fp32) off, ld = V + 6
    c = gpu.fo_xent_fwd_bwd(zs, t.to(DEV), IGN, 1e-4, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(c["dlogits"].cpu(), a["dlogits"]) and torch.equal(c["loss"].cpu(), a["loss"])


def test_in_place_matches_out_of_place(gpu):
    cfg = synth.scaled(synth.CONFIGS[3], 40)
    i = synth.xent_inputs(cfg)
    a = run(gpu, i["logits"], i["targets"], cfg.z_loss)
    b = run(gpu, i["logits"], i["targets"], cfg.z_loss, inplace=True)
    assert torch.equal(a["dlogits"], b["dlogits"]) and torch.equal(a["loss"], b["loss"])


def test_forward_only(gpu):
    cfg = synth.scaled(synth.CONFIGS[2], 17)
    i = synth.xent_inputs(cfg)
    a = run(gpu, i["logits"], i["targets"], 0.0, grad=False)
    assert a["dlogits"] is None
    compare(i["logits"], i["targets"], 0.0, "bf16", a)


def test_all_ignored_and_bad_targets(gpu):
    z = torch.randn(5, 300).to(torch.bfloat16)
    t = torch.full((5,), IGN, dtype=torch.int64)
    a = run(gpu, z, t, 1e-4)
    assert a["loss"].item() == 0.0 and a["n_valid"].item() == 0
    assert torch.all(a["dlogits"].view(torch.int16) == 0)
    t2 = torch.tensor([300, -1, 5, 299, 10**12])
    b = run(gpu, z, t2, 1e-4)
    assert b["status"].item() == 3 and b["n_valid"].item() == 2
    compare(z, t2, 1e-4, "bf16", b)


def test_empty_batch(gpu):
    z = torch.empty(0, 128, dtype=torch.bfloat16)
    o = run(gpu, z, torch.empty(0, dtype=torch.int64), 0.0)
    assert o["loss"].item() == 0.0 and o["n_valid"].item() == 0


def test_deterministic(gpu):
    cfg = synth.scaled(synth.CONFIGS[2], 300)
    i = synth.xent_inputs(cfg)
    a = run(gpu, i["logits"], i["targets"], 1e-4)
    b = run(gpu, i["logits"], i["targets"], 1e-4)
    assert torch.equal(a["loss"], b["loss"]) and torch.equal(a["dlogits"], b["dlogits"])


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size(gpu, cid):
    cfg = synth.CONFIGS[cid]
    i = synth.xent_inputs(cfg)
    o = run(gpu, i["logits"], i["targets"], cfg.z_loss)
    z, t = i["logits"], i["targets"]
    rows = np.unique(np.concatenate([[0, cfg.T - 1],
                                     np.random.default_rng(cid).integers(0, cfg.T, 14)]))
    n_full = int(((t != IGN) & (t >= 0) & (t < cfg.V)).sum())
    # the sampled rows' gradients are scaled by the whole batch's N
    tg = t[rows].numpy()
    valid = (tg != IGN) & (tg >= 0) & (tg < cfg.V)
    _, _, _, dz = oracle.xent_rows(z[rows].double().numpy(), tg, valid, n_full, cfg.z_loss, 1.0)
    check(o["dlogits"][rows], dz, cfg.dtype, "dlogits", single_rounding=True)
    assert o["n_valid"].item() == n_full
    ign = (t == IGN).nonzero().flatten()
    if len(ign):
        assert torch.all(o["dlogits"][ign[:64]].view(torch.int16) == 0)
    # the loss needs every row: the oracle over row blocks (each block's mean times its
    # valid count), on a thread pool
    check_losses_full(o, z, t, cfg.z_loss, n_full)


def check_losses_full(o, z, t, zc, n_full):
    def one(r0, r1):
        b = oracle.xent_fwd_bwd(z[r0:r1], t[r0:r1], IGN, zc, 1.0)
        return b["loss"] * b["n_valid"], b["z_loss"] * b["n_valid"], b["n_valid"], b["n_bad"]

    parts = map_blocks(one, z.shape[0], 256)
    assert sum(p[2] for p in parts) == n_full
    check_loss(o["loss"].item(), sum(p[0] for p in parts) / n_full)
    check_loss(o["z_loss"].item(), sum(p[1] for p in parts) / n_full, "z_loss")
    assert o["status"].item() == sum(p[3] for p in parts)


def test_unaligned_full_size(gpu):
    # the bench's unaligned line: Llama-3-8B logits shape with GPT-2's 50257-entry
    # vocabulary (every row at another alignment), z-loss 1e-4: sampled gradient rows and
    # the loss over every row (oracle in row blocks)
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS[3], V=50257)
    i = synth.xent_inputs(cfg)
    z, t = i["logits"], i["targets"]
    o = run(gpu, z, t, cfg.z_loss)
    rows = np.unique(np.concatenate([[0, 1, cfg.T - 1], np.random.default_rng(50257).integers(0, cfg.T, 13)]))
    n_full = int(((t != IGN) & (t >= 0) & (t < cfg.V)).sum())
    tg = t[rows].numpy()
    valid = (tg != IGN) & (tg >= 0) & (tg < cfg.V)
    _, _, _, dz = oracle.xent_rows(z[rows].double().numpy(), tg, valid, n_full, cfg.z_loss, 1.0)
    check(o["dlogits"][rows], dz, cfg.dtype, "dlogits", single_rounding=True)
    assert o["n_valid"].item() == n_full
    check_losses_full(o, z, t, cfg.z_loss, n_full)
