"""GPU parity of fo_adamw_step against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from reduction_rmsnorm_fwd_amd import synth
from tolerance import adamw_terms, check_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def scalars(step, lr=3e-4, b1=0.9, b2=0.95, wd=0.1, eps=1e-8):
    """The step's host scalars, rounded to the fp32 values the kernel receives."""
    ss, bc, df = oracle.adamw_scalars(lr, b1, b2, wd, step)
    f = lambda x: float(np.float32(x))  # noqa: E731
    return dict(step_size=f(ss), beta1=f(b1), beta2=f(b2), bias_correction=f(bc),
                decay_factor=f(df), eps=f(eps))


def to_dev(ts, offsets=None):
    """Device copies; offsets[i] > 0 places tensor i that many elements into a larger
    buffer (a misaligned but contiguous view)."""
    out = []
    for i, t in enumerate(ts):
        o = offsets[i] if offsets else 0
        buf = torch.empty(t.numel() + o, dtype=torch.float32, device=DEV)
        v = buf[o:]
        v.copy_(t.to(DEV))
        out.append(v)
    return out


def run_and_check(sizes, seed, sc, offsets=None, grad_scale=None, noop=None):
    i = synth.adamw_inputs(sizes, seed)
    d = {k: to_dev(i[k], offsets) for k in i}
    gs = None if grad_scale is None else torch.tensor([grad_scale], dtype=torch.float32, device=DEV)
    nf = None if noop is None else torch.tensor([noop], dtype=torch.int32, device=DEV)
    fo_call(d, sc, gs, nf)
    torch.cuda.synchronize()
    for k in range(len(sizes)):
        rp, rm, rv = oracle.adamw_step(i["params"][k], i["grads"][k], i["exp_avgs"][k],
                                       i["exp_avg_sqs"][k], sc["step_size"], sc["beta1"],
                                       sc["beta2"], sc["bias_correction"], sc["decay_factor"],
                                       sc["eps"], grad_scale=1.0 if grad_scale is None else grad_scale,
                                       noop=bool(noop))
        ap, am = adamw_terms(i["params"][k], i["grads"][k], i["exp_avgs"][k], i["exp_avg_sqs"][k],
                             sc["step_size"], sc["beta1"], sc["beta2"], sc["bias_correction"],
                             sc["decay_factor"], sc["eps"],
                             grad_scale=1.0 if grad_scale is None else grad_scale)
        check_f32(d["params"][k].cpu(), rp, f"p[{k}]", scale=ap)
        check_f32(d["exp_avgs"][k].cpu(), rm, f"m[{k}]", scale=am)
        check_f32(d["exp_avg_sqs"][k].cpu(), rv, f"v[{k}]")
        assert torch.equal(d["grads"][k].cpu(), i["grads"][k])  # gradients are read only
    return i, d


def fo_call(d, sc, gs=None, nf=None):
    import reduction_rmsnorm_fwd_amd as fo
    fo.fo_adamw_step(d["params"], d["grads"], d["exp_avgs"], d["exp_avg_sqs"], noop_flag=nf,
                     grad_scale=gs, **sc)


def test_ragged_sizes(gpu):
    # empty, sub-vector, one vector, around a 4096-element chunk, several chunks + tail
    run_and_check([1, 3, 4, 5, 0, 4095, 4096, 4097, 12289, 100003], seed=1, sc=scalars(7))


def test_many_tensors_several_launches(gpu):
    sizes = [int(x) for x in np.random.default_rng(3).integers(0, 5000, 80)]
    run_and_check(sizes, seed=2, sc=scalars(3))


def test_misaligned_views(gpu):
    sizes = [4097, 1000, 8192, 33]
    run_and_check(sizes, seed=3, sc=scalars(2), offsets=[1, 0, 3, 2])


def test_grad_scale(gpu):
    run_and_check([5000, 77], seed=4, sc=scalars(11), grad_scale=0.125)


def test_noop_flag(gpu):
    i, d = run_and_check([5000, 77], seed=5, sc=scalars(1), noop=1)
    for k in ("params", "exp_avgs", "exp_avg_sqs"):
        for a, b in zip(d[k], i[k]):
            assert torch.equal(a.cpu(), b)  # bit-identical: nothing written
    run_and_check([5000, 77], seed=5, sc=scalars(1), noop=0)


def test_two_consecutive_steps(gpu):
    sizes = [9000, 17]
    i = synth.adamw_inputs(sizes, 6)
    d = {k: to_dev(i[k]) for k in i}
    ref = [(i["params"][k], i["exp_avgs"][k], i["exp_avg_sqs"][k]) for k in range(2)]
    for t in (1, 2):
        sc = scalars(t)
        fo_call(d, sc)
        ref = [oracle.adamw_step(p, i["grads"][k], m, v, sc["step_size"], sc["beta1"],
                                 sc["beta2"], sc["bias_correction"], sc["decay_factor"], sc["eps"])
               for k, (p, m, v) in enumerate(ref)]
    torch.cuda.synchronize()
    for k in range(2):
        check_f32(d["params"][k].cpu(), ref[k][0], "p")
        check_f32(d["exp_avgs"][k].cpu(), ref[k][1], "m")
        check_f32(d["exp_avg_sqs"][k].cpu(), ref[k][2], "v")


def test_full_layer_sampled(gpu):
    """The parameter tensors of one Llama-3-8B decoder layer (218 M elements) in one
    call, as the bench times it; 20000 sampled elements per tensor against the oracle."""
    sizes = [n for _, n in synth.LLAMA3_8B_LAYER_PARAMS]
    i = synth.adamw_inputs(sizes, 7)
    d = {k: to_dev(i[k]) for k in i}
    sc = scalars(100)
    fo_call(d, sc)
    torch.cuda.synchronize()
    g = np.random.default_rng(8)
    for k, n in enumerate(sizes):
        idx = torch.from_numpy(np.unique(np.concatenate([[0, n - 1], g.integers(0, n, 20000)])))
        rp, rm, rv = oracle.adamw_step(i["params"][k][idx], i["grads"][k][idx],
                                       i["exp_avgs"][k][idx], i["exp_avg_sqs"][k][idx],
                                       sc["step_size"], sc["beta1"], sc["beta2"],
                                       sc["bias_correction"], sc["decay_factor"], sc["eps"])
        didx = idx.to(DEV)
        ap, am = adamw_terms(i["params"][k][idx], i["grads"][k][idx], i["exp_avgs"][k][idx],
                             i["exp_avg_sqs"][k][idx], sc["step_size"], sc["beta1"], sc["beta2"],
                             sc["bias_correction"], sc["decay_factor"], sc["eps"])
        check_f32(d["params"][k][didx].cpu(), rp, f"p[{k}]", scale=ap)
        check_f32(d["exp_avgs"][k][didx].cpu(), rm, f"m[{k}]", scale=am)
        check_f32(d["exp_avg_sqs"][k][didx].cpu(), rv, f"v[{k}]")
