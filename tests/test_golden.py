"""The oracle still reproduces its frozen tiny-case outputs (regression guard)."""
import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def load():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        raw = json.load(f)

    def dec(v):
        if isinstance(v, dict) and "shape" in v:
            a = np.array(v["data"], dtype=np.float64 if v["kind"] == "f" else np.int64)
            return a.reshape(v["shape"])
        return v
    return {n: {k: dec(v) for k, v in c.items()} for n, c in raw.items()}


def close(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) <= 1e-15 * max(1.0, np.max(np.abs(b)))


def test_golden_reproduced():
    G = load()
    c = G["rmsnorm"]
    y, r = oracle.rmsnorm_fwd(c["x"], c["w"], c["eps"])
    dx, dw = oracle.rmsnorm_bwd(c["dy"], c["x"], c["w"], c["eps"])
    assert close(y, c["y"]) and close(r, c["rstd"]) and close(dx, c["dx"]) and close(dw, c["dw"])
    c = G["rope"]
    qo, ko = oracle.rope_fwd(c["q"], c["k"], c["pos"], c["theta"])
    assert close(qo, c["q_fwd"]) and close(ko, c["k_fwd"])
    c = G["swiglu"]
    assert close(oracle.swiglu_fwd(c["gate"], c["up"]), c["h"])
    c = G["xent"]
    o = oracle.xent_fwd_bwd(c["logits"], c["targets"], c["ignore_index"], c["z_loss"], c["dloss"])
    assert close(o["loss"], c["loss"]) and close(o["dlogits"], c["dlogits"])
    c = G["flce"]
    o = oracle.flce_fwd_bwd(c["hidden"], c["weight"], c["targets"], c["ignore_index"],
                            c["z_loss"], c["dloss"])
    assert close(o["loss"], c["loss"]) and close(o["dweight"], c["dweight"])
