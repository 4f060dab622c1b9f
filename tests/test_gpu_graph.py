"""HIP-graph capture of the step's fused ops.

Every entry point of the step (RMSNorm, RoPE, SwiGLU forward and backward, cross-entropy
with and without a workspace, the fused linear cross-entropy) is captured into one graph
through torch.cuda.graph: the library enqueues kernels only (no allocation, memset, copy
or host synchronisation), so the calls capture as they are.  Each replay must reproduce
the eager results bit for bit (every reduction runs in a fixed order).  Between replays
the program runs the same ops eagerly on other inputs and synchronises, and the captured
inputs are overwritten in place, so a replay that read stale or shared state would
differ."""
import dataclasses

import pytest
import torch

from reduction_rmsnorm_fwd_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Step:
    """Static buffers of one step at a config (layer ops) plus a small lm head."""

    def __init__(self, fo, cfg, seed_shift=0):
        self.fo, self.cfg = fo, cfg
        c = cfg if not seed_shift else dataclasses.replace(cfg, seed=cfg.seed + seed_shift)
        r, ro, sw, xe = (synth.rmsnorm_inputs(c), synth.rope_inputs(c), synth.swiglu_inputs(c),
                         synth.xent_inputs(c))
        fl = synth.flce_inputs(synth.flce_small(96, 64, 1000, seed=5 + seed_shift))
        self.src = {"x": r["x"], "w": r["w"], "dy": r["dy"], "q": ro["q"], "k": ro["k"],
                    "dq": ro["dq"], "dk": ro["dk"], "g": sw["gate"], "u": sw["up"],
                    "dh": sw["dh"], "z": xe["logits"], "hid": fl["hidden"], "wt": fl["weight"]}
        self.pos, self.tg, self.ftg = ro["pos"].to(DEV), xe["targets"].to(DEV), fl["targets"].to(DEV)
        self.buf = {k: v.to(DEV) for k, v in self.src.items()}
        # RoPE works in place: its captured inputs are refreshed from these before each run
        self.rope0 = {k: self.buf[k].clone() for k in ("q", "k", "dq", "dk")}
        T, d, V = cfg.T, cfg.d, cfg.V
        b = self.buf
        self.out = {
            "y": torch.empty_like(b["x"]), "rstd": torch.empty(T, device=DEV),
            "dx": torch.empty_like(b["x"]), "dw": torch.empty(d, device=DEV),
            "h": torch.empty_like(b["g"]), "dg": torch.empty_like(b["g"]),
            "du": torch.empty_like(b["g"]), "dz": torch.empty_like(b["z"]),
            "dz_na": torch.empty_like(b["z"]), "dhid": torch.empty_like(b["hid"]),
            "dwt": torch.empty(b["wt"].shape, dtype=torch.float32, device=DEV),
        }
        self.sc = {n: fo._scalars(DEV) for n in ("xent", "xent_na", "flce")}
        self.ws = {
            "rms": torch.empty(fo.fo_rmsnorm_bwd_workspace(T, d), dtype=torch.uint8, device=DEV),
            "xent": torch.empty(fo.fo_xent_workspace(T, V), dtype=torch.uint8, device=DEV),
            "flce": torch.empty(fo.fo_flce_workspace(96, 64, 1000), dtype=torch.uint8,
                                device=DEV),
        }

    def load(self, other):
        """Overwrite the captured inputs in place with another step's values (a kernel,
        not a memcpy node: torch's elementwise mul by one is exact)."""
        for k, v in other.buf.items():
            torch.mul(v, 1, out=self.buf[k])
        for k in self.rope0:
            torch.mul(other.rope0[k], 1, out=self.rope0[k])
        for k in ("pos", "tg", "ftg"):
            torch.mul(getattr(other, k), 1, out=getattr(self, k))

    def run(self):
        fo, c, b, o = self.fo, self.cfg, self.buf, self.out
        for k, v in self.rope0.items():
            torch.mul(v, 1, out=b[k])
        fo.fo_rmsnorm_fwd(b["x"], b["w"], c.eps, y=o["y"], rstd=o["rstd"])
        fo.fo_rmsnorm_bwd(b["dy"], b["x"], b["w"], o["rstd"], c.eps, dx=o["dx"], dw=o["dw"],
                          ws=self.ws["rms"])
        fo.fo_rope_fwd(b["q"], b["k"], self.pos, c.theta)
        fo.fo_rope_bwd(b["dq"], b["dk"], self.pos, c.theta)
        fo.fo_swiglu_fwd(b["g"], b["u"], h=o["h"])
        fo.fo_swiglu_bwd(b["dh"], b["g"], b["u"], dgate=o["dg"], dup=o["du"])
        fo.fo_xent_fwd_bwd(b["z"], self.tg, -100, c.z_loss, 1.0, dlogits=o["dz"],
                           ws=self.ws["xent"], out=self.sc["xent"])
        fo.fo_xent_fwd_bwd_noalloc(b["z"], self.tg, -100, c.z_loss, 1.0, dlogits=o["dz_na"],
                                   out=self.sc["xent_na"])
        fo.fo_flce_fwd_bwd(b["hid"], b["wt"], self.ftg, -100, 1e-4, 1.0, dhidden=o["dhid"],
                           dweight=o["dwt"], ws=self.ws["flce"], out=self.sc["flce"])

    def results(self):
        r = {k: v.clone() for k, v in self.out.items()}
        r.update({k: self.buf[k].clone() for k in self.rope0})
        for n, s in self.sc.items():
            r.update({f"{n}_{k}": v.clone() for k, v in s.items() if k != "dlogits" and
                      k != "dhidden" and k != "dweight"})
        return r


def same(a, b, tag):
    """Bit-for-bit equality of every output (signed zeros included)."""
    assert a.keys() == b.keys()
    for k in a:
        ab, bb = a[k].reshape(-1).view(torch.uint8), b[k].reshape(-1).view(torch.uint8)
        assert torch.equal(ab, bb), f"{tag}: {k} differs"


@pytest.mark.parametrize("cid", [1, 3, 4])
def test_step_graph_replays_match_eager(gpu, cid):
    cfg = synth.scaled(synth.CONFIGS[cid], 160)
    st = Step(gpu, cfg)
    alt = Step(gpu, cfg, seed_shift=17)
    # eager references on both input sets, then warm-up on a side stream (torch's
    # capture recipe), then capture
    st.run()
    ref = st.results()
    alt.run()
    ref_alt = alt.results()
    assert any(not torch.equal(ref[k], ref_alt[k]) for k in ("y", "dz", "dhid"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work of the same ops (the library's noalloc workspace included) between
        # replays, then the replay on the captured inputs
        alt.run()
        torch.cuda.synchronize()
        same(alt.results(), ref_alt, f"cfg{cid} eager between replays {rep}")
        g.replay()
        torch.cuda.synchronize()
        same(st.results(), ref, f"cfg{cid} replay {rep}")
    # the captured inputs overwritten in place: the replay computes on the new values
    st.load(alt)
    g.replay()
    torch.cuda.synchronize()
    same(st.results(), ref_alt, f"cfg{cid} replay on new inputs")
    del g
