"""Every entry point is stateless: the caller owns every buffer (workspaces included)
and the library keeps nothing between calls, so

  * the same sequence of calls issued on two streams at once, each with its own buffers,
    gives bit for bit what it gives when the two run one after the other;
  * all of them captured into one HIP graph (the library only enqueues kernels: no
    allocation, memset, copy or host synchronisation) replay bit for bit the eager
    results, with eager work on other buffers between the replays.

Every reduction runs in a fixed order, which is what makes bit-for-bit the bar.  The
no-allocation cross-entropy call shares one per-device scratch array between all its
calls, so it appears in the graph case only (two streams would race on it, as its
declaration says)."""
import dataclasses

import pytest
import torch

from reduction_rmsnorm_fwd_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX


def _cfg(cid, T, shift):
    c = synth.scaled(synth.CONFIGS[cid], T)
    return dataclasses.replace(c, seed=c.seed + shift)


class AllOps:
    """Inputs, preallocated outputs and workspaces for one call of every entry point
    (Llama-3-8B-shaped layer ops on 2048 tokens, cross-entropy and distillation over
    32000 classes, a small lm head, an AdamW step over three ragged tensors)."""

    def __init__(self, fo, shift, noalloc=False):
        self.fo, self.noalloc = fo, noalloc
        c3 = _cfg(3, 2048, shift)
        self.eps, self.theta = c3.eps, c3.theta
        nrm, ln, rp, mlp = (synth.rmsnorm_inputs(c3), synth.layernorm_inputs(c3),
                            synth.rope_inputs(c3), synth.swiglu_inputs(c3))
        cx = dataclasses.replace(_cfg(3, 1024, shift), V=32000, ignore_frac=0.1)
        xe = synth.xent_inputs(cx)
        kd = synth.distill_inputs(dataclasses.replace(cx, T=512))
        fl = synth.flce_inputs(synth.flce_small(300, 512, 8192, seed=40 + shift))
        ad = synth.adamw_inputs([100000, 4097, 30000], 50 + shift)
        d = lambda t: t.to(DEV)  # noqa: E731
        self.i = dict(x=d(nrm["x"]), w=d(nrm["w"]), dy=d(nrm["dy"]), lx=d(ln["x"]), lw=d(ln["w"]),
                      lb=d(ln["b"]), ldy=d(ln["dy"]), pos=d(rp["pos"]), g=d(mlp["gate"]),
                      u=d(mlp["up"]), dh=d(mlp["dh"]), z=d(xe["logits"]), tg=d(xe["targets"]),
                      kz=d(kd["logits"]), kt=d(kd["teacher"]), km=d(kd["row_mask"]),
                      hid=d(fl["hidden"]), wt=d(fl["weight"]), ftg=d(fl["targets"]))
        # buffers the calls update in place, and the values they start from each run
        self.orig = dict(q=d(rp["q"]), k=d(rp["k"]), dq=d(rp["dq"]), dk=d(rp["dk"]))
        for n in ("params", "exp_avgs", "exp_avg_sqs"):
            for j, t in enumerate(ad[n]):
                self.orig[f"{n}{j}"] = d(t)
        self.live = {k: torch.empty_like(v) for k, v in self.orig.items()}
        self.grads = [d(t) for t in ad["grads"]]
        i, e = self.i, torch.empty_like
        f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device=DEV)  # noqa: E731
        T, dm = i["x"].shape
        self.o = dict(y=e(i["x"]), rstd=f32(T), dx=e(i["x"]), dw=f32(dm),
                      ly=e(i["lx"]), lmean=f32(T), lrstd=f32(T), ldx=e(i["lx"]), ldw=f32(dm),
                      ldb=f32(dm), h=e(i["g"]), dg=e(i["g"]), du=e(i["g"]), gh=e(i["g"]),
                      gdg=e(i["g"]), gdu=e(i["g"]), ay=e(i["g"]), adx=e(i["g"]),
                      dz=e(i["z"]), kdz=e(i["kz"]), dhid=e(i["hid"]), dwt=f32(tuple(i["wt"].shape)))
        if noalloc:
            self.o["dz_na"] = e(i["z"])
        self.sc = {n: fo._scalars(DEV) for n in ("xent", "xent_na", "flce")}
        self.sc["kd"] = dict(loss=f32(()), kl=f32(()), n_valid=torch.empty((), dtype=torch.int64, device=DEV))
        u8 = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=DEV)  # noqa: E731
        Tx, V = i["z"].shape
        self.ws = dict(rms=u8(fo.fo_rmsnorm_bwd_workspace(T, dm)),
                       ln=u8(fo.fo_layernorm_bwd_workspace(T, dm)),
                       xent=u8(fo.fo_xent_workspace(Tx, V)),
                       kd=u8(fo.fo_distill_workspace(*i["kz"].shape)),
                       flce=u8(fo.fo_flce_workspace(*i["hid"].shape, i["wt"].shape[0])))
        ss = lambda v: float(torch.tensor(v, dtype=torch.float32))  # noqa: E731
        self.adam = (ss(3e-4 / (1 - 0.9 ** 3)), ss(0.9), ss(0.95), ss((1 - 0.95 ** 3) ** 0.5),
                     ss(1 - 3e-4 * 0.1), ss(1e-8))

    def steps(self):
        """The calls, one per step, on the current stream (a generator, so that two sets
        can be interleaved call by call)."""
        fo, i, o, lv, ws, sc = self.fo, self.i, self.o, self.live, self.ws, self.sc
        for k, v in self.orig.items():  # a kernel, not a memcpy node
            torch.mul(v, 1, out=lv[k])
        yield
        fo.fo_rmsnorm_fwd(i["x"], i["w"], self.eps, y=o["y"], rstd=o["rstd"])
        yield
        fo.fo_rmsnorm_bwd(i["dy"], i["x"], i["w"], o["rstd"], self.eps, dx=o["dx"], dw=o["dw"],
                          ws=ws["rms"])
        yield
        fo.fo_layernorm_fwd(i["lx"], i["lw"], i["lb"], self.eps, y=o["ly"], mean=o["lmean"],
                            rstd=o["lrstd"])
        yield
        fo.fo_layernorm_bwd(i["ldy"], i["lx"], i["lw"], o["lmean"], o["lrstd"], dx=o["ldx"],
                            dw=o["ldw"], db=o["ldb"], ws=ws["ln"])
        yield
        fo.fo_rope_fwd(lv["q"], lv["k"], i["pos"], self.theta)
        fo.fo_rope_bwd(lv["dq"], lv["dk"], i["pos"], self.theta)
        yield
        fo.fo_swiglu_fwd(i["g"], i["u"], h=o["h"])
        fo.fo_swiglu_bwd(i["dh"], i["g"], i["u"], dgate=o["dg"], dup=o["du"])
        yield
        fo.fo_glu_fwd("gelu", i["g"], i["u"], h=o["gh"])
        fo.fo_glu_bwd("gelu", i["dh"], i["g"], i["u"], dgate=o["gdg"], dup=o["gdu"])
        fo.fo_act_fwd("silu", i["g"], y=o["ay"])
        fo.fo_act_bwd("silu", i["dh"], i["g"], dx=o["adx"])
        yield
        fo.fo_xent_fwd_bwd(i["z"], i["tg"], IGN, 1e-4, 1.0, dlogits=o["dz"], ws=ws["xent"],
                           out=sc["xent"])
        if self.noalloc:
            fo.fo_xent_fwd_bwd_noalloc(i["z"], i["tg"], IGN, 1e-4, 1.0, dlogits=o["dz_na"],
                                       out=sc["xent_na"])
        yield
        fo.fo_distill_fwd_bwd(i["kz"], i["kt"], i["km"], 1.0, dlogits=o["kdz"], ws=ws["kd"],
                              out=sc["kd"])
        yield
        fo.fo_flce_fwd_bwd(i["hid"], i["wt"], i["ftg"], IGN, 1e-4, 1.0, dhidden=o["dhid"],
                           dweight=o["dwt"], ws=ws["flce"], out=sc["flce"])
        yield
        n = len(self.grads)
        fo.fo_adamw_step([lv[f"params{j}"] for j in range(n)], self.grads,
                         [lv[f"exp_avgs{j}"] for j in range(n)],
                         [lv[f"exp_avg_sqs{j}"] for j in range(n)], *self.adam)

    def run(self):
        for _ in self.steps():
            pass

    def results(self):
        r = {k: v.clone() for k, v in self.o.items()}
        r.update({k: v.clone() for k, v in self.live.items()})
        for n, s in self.sc.items():
            r.update({f"{n}_{k}": v.clone() for k, v in s.items()
                      if k not in ("dlogits", "dhidden", "dweight")})
        return r


def same(a, b, tag):
    """Bit-for-bit equality of every output (signed zeros included)."""
    assert a.keys() == b.keys()
    for k in a:
        ab, bb = a[k].reshape(-1).view(torch.uint8), b[k].reshape(-1).view(torch.uint8)
        assert torch.equal(ab, bb), f"{tag}: {k} differs"


def test_two_streams_match_one_after_the_other(gpu):
    a, b = AllOps(gpu, 0), AllOps(gpu, 11)
    a.run()
    torch.cuda.synchronize()
    ref_a = a.results()
    b.run()
    torch.cuda.synchronize()
    ref_b = b.results()
    assert any(not torch.equal(ref_a[k], ref_b[k]) for k in ("y", "dz", "dhid", "params0"))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority, both
    for rep in range(3):
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        # the two sets interleaved call by call, each on its own stream, so their
        # kernels are in flight together
        ga, gb = a.steps(), b.steps()
        while True:
            with torch.cuda.stream(sa):
                da = next(ga, "end")
            with torch.cuda.stream(sb):
                db = next(gb, "end")
            if da == "end" and db == "end":
                break
        torch.cuda.synchronize()
        same(a.results(), ref_a, f"stream a, round {rep}")
        same(b.results(), ref_b, f"stream b, round {rep}")


def test_every_entry_point_in_one_graph(gpu):
    st, alt = AllOps(gpu, 0, noalloc=True), AllOps(gpu, 23, noalloc=True)
    st.run()
    torch.cuda.synchronize()
    ref = st.results()
    alt.run()
    torch.cuda.synchronize()
    ref_alt = alt.results()
    # the no-allocation call equals the workspace call
    for r in (ref, ref_alt):
        assert torch.equal(r["dz"], r["dz_na"])
        assert all(torch.equal(r[f"xent_{k}"], r[f"xent_na_{k}"]) for k in ("loss", "z_loss", "n_valid", "status"))
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
        alt.run()  # eager work on other buffers (the shared no-allocation scratch too)
        torch.cuda.synchronize()
        same(alt.results(), ref_alt, f"eager between replays {rep}")
        g.replay()
        torch.cuda.synchronize()
        same(st.results(), ref, f"replay {rep}")
    del g
