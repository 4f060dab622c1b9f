"""Writes tests/golden/oracle_tiny.json: tiny inputs and the fp64 oracle's outputs.

The pages print no worked numeric example for any of the ops, so there are no
page-printed values to store.  This file freezes the oracle's own results on tiny
inputs (inputs included) so that any later change to the oracle's arithmetic shows
up as a failing regression test and has to be justified.  It calls only ``oracle``.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402


def main():
    g = np.random.default_rng(20261202)
    # inputs are chosen on a bf16-representable grid (multiples of 1/64, |x| < 4) so
    # the same values can be fed to the GPU in either dtype
    def grid(*shape):
        return np.round(g.standard_normal(shape) * 64) / 64

    cases = {}
    x, w, dy = grid(3, 8), 1 + grid(8) / 8, grid(3, 8)
    y, r = oracle.rmsnorm_fwd(x, w, 1e-5)
    dx, dw = oracle.rmsnorm_bwd(dy, x, w, 1e-5)
    cases["rmsnorm"] = dict(x=x, w=w, dy=dy, eps=1e-5, y=y, rstd=r, dx=dx, dw=dw)
    q, k, pos = grid(3, 2, 8), grid(3, 1, 8), np.array([0, 1, 700])
    qo, ko = oracle.rope_fwd(q, k, pos, 1e4)
    qb, kb = oracle.rope_bwd(q, k, pos, 1e4)
    cases["rope"] = dict(q=q, k=k, pos=pos, theta=1e4, q_fwd=qo, k_fwd=ko, q_bwd=qb, k_bwd=kb)
    gt, up, dh = grid(2, 6), grid(2, 6), grid(2, 6)
    h = oracle.swiglu_fwd(gt, up)
    dg, du = oracle.swiglu_bwd(dh, gt, up)
    cases["swiglu"] = dict(gate=gt, up=up, dh=dh, h=h, dgate=dg, dup=du)
    z, t = grid(4, 10), np.array([3, -100, 9, 0])
    o = oracle.xent_fwd_bwd(z, t, -100, 1e-2, 1.0)
    cases["xent"] = dict(logits=z, targets=t, ignore_index=-100, z_loss=1e-2, dloss=1.0,
                         loss=o["loss"], z_loss_part=o["z_loss"], n_valid=o["n_valid"],
                         dlogits=o["dlogits"])
    Hm, W, t = grid(4, 8), grid(12, 8) / 4, np.array([11, 0, -100, 5])
    o = oracle.flce_fwd_bwd(Hm, W, t, -100, 1e-3, 1.0)
    cases["flce"] = dict(hidden=Hm, weight=W, targets=t, ignore_index=-100, z_loss=1e-3,
                         dloss=1.0, loss=o["loss"], z_loss_part=o["z_loss"],
                         n_valid=o["n_valid"], dhidden=o["dhidden"], dweight=o["dweight"])

    def enc(v):
        if isinstance(v, np.ndarray):
            return dict(shape=list(v.shape), data=[float(a) if v.dtype.kind == "f" else int(a)
                                                   for a in v.ravel()],
                        kind=v.dtype.kind)
        return v

    out = {name: {k: enc(v) for k, v in c.items()} for name, c in cases.items()}
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
