"""Benchmark of the fused per-token training ops on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input, with
every input already resident in HBM:
  RMSNorm fwd + bwd, RoPE fwd + bwd on Q/K, SwiGLU fwd + bwd, cross-entropy fwd+bwd
  (with z-loss) at the Llama-3-8B layer shapes (T 8192, d 4096, 32 Q / 8 KV heads of
  128, ffn 14336, vocab 128256), and the fused linear cross-entropy of the lm head
  of the same model (H [8192, 4096], W [128256, 4096], 10% ignored targets, z-loss).
`value` is whole-step throughput in tokens/s (8192 tokens per step).  Per op it
reports the time inside the step and in isolation (caches flushed before each call),
the algorithmic bytes (or flops) and the fraction of the MI355X roofline.  The fp64
CPU oracle is timed on a bounded sample of the same step as the baseline.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HBM GB/s & % of peak per fused op (fwd+bwd); xent/FLCE tokens/s"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
FLUSH_BYTES = 1 << 30        # written between isolated calls: beyond L2 and the 256 MB MALL
COPY_BYTES = 1 << 30         # copy probe: 1 GiB read + 1 GiB written
MFMA_PROBE_ITERS = 100000    # MFMA probe rounds per wave (about 12 ms)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_step_llama3-8b.json")


def sources_sha256():
    """Hash of the kernel sources and the C ABI header (same recipe as the one stamped
    into the counter summary when the FETCH_SIZE / WRITE_SIZE runs were taken)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join("reduction_rmsnorm_fwd_amd", "csrc")
    files = sorted([os.path.join(csrc, f) for f in os.listdir(os.path.join(ROOT, csrc))]
                   + [os.path.join("include", "fo.h")])
    for f in files:
        h.update(f.encode())
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """Per-op HBM bytes per call from the committed counter runs, or None when the
    kernels have changed since those counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sources_sha256():
        return None
    return {k: v["traffic_bytes"] for k, v in t.get("per_op", {}).items()}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--iso-reps", type=int, default=50, help="isolated calls per memory-bound op")
    p.add_argument("--iso-reps-flce", type=int, default=10, help="isolated calls of the FLCE")
    p.add_argument("--no-probes", action="store_true",
                   help="skip the copy / MFMA ceiling probes and the unaligned-shape lines")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-next", action="store_true",
                   help="skip the rows after the step (AdamW, LayerNorm, GeLU MLP "
                        "activations, soft-target cross-entropy)")
    p.add_argument("--no-isolated", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-(config, op) records of configs 1-4")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the graph-replayed step of each config record")
    p.add_argument("--config", default="1,2,3,4",
                   help="comma list of the configs (1-4) the per-(config, op) records cover")
    p.add_argument("--only", default="", help="comma list of ops to run (profiling)")
    p.add_argument("--calib-copy", action="store_true",
                   help="first run one plain 1 GiB device copy (counter calibration)")
    a = p.parse_args()
    try:
        a.cids = tuple(int(c) for c in a.config.split(",") if c.strip())
    except ValueError:
        a.cids = (0,)
    if any(c not in (1, 2, 3, 4) for c in a.cids):
        p.error("--config takes configs 1-4 (config 5, the lm-head FLCE, is part of the step)")
    return a


class Workload:
    """Device-resident inputs/outputs of one step and the per-op callables."""

    def __init__(self, fo, synth, torch, only=()):
        self.fo, self.torch = fo, torch
        dev = "cuda"
        c3, c5 = synth.CONFIGS[3], synth.CONFIGS[5]
        self.c3, self.c5 = c3, c5
        T, d = c3.T, c3.d
        self.T = T
        r = synth.rmsnorm_inputs(c3)
        self.x, self.w, self.dy = (r[k].to(dev) for k in ("x", "w", "dy"))
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.rstd = torch.empty(T, dtype=torch.float32, device=dev)
        self.dw = torch.empty(d, dtype=torch.float32, device=dev)
        self.rms_ws = torch.empty(fo.fo_rmsnorm_bwd_workspace(T, d), dtype=torch.uint8, device=dev)
        ro = synth.rope_inputs(c3)
        self.q, self.k, self.dq, self.dk = (ro[k].to(dev) for k in ("q", "k", "dq", "dk"))
        self.pos = ro["pos"].to(dev)
        s = synth.swiglu_inputs(c3)
        self.g, self.u, self.dh = (s[k].to(dev) for k in ("gate", "up", "dh"))
        self.h = torch.empty_like(self.g)
        self.dg = torch.empty_like(self.g)
        self.du = torch.empty_like(self.g)
        xe = synth.xent_inputs(c3)
        self.logits, self.tg = xe["logits"].to(dev), xe["targets"].to(dev)
        self.dlogits = torch.empty_like(self.logits)
        self.xent_ws = torch.empty(fo.fo_xent_workspace(T, c3.V), dtype=torch.uint8, device=dev)
        self.xo = fo._scalars(dev)
        fl = synth.flce_inputs(c5)
        self.H, self.W, self.ftg = (fl[k].to(dev) for k in ("hidden", "weight", "targets"))
        self.dH = torch.empty_like(self.H)
        self.dW = torch.empty(self.W.shape, dtype=torch.float32, device=dev)
        self.flce_ws = torch.empty(fo.fo_flce_workspace(c5.T, c5.flce_H, c5.V, 0, fo.FO_F32),
                                   dtype=torch.uint8, device=dev)
        self.fo_out = fo._scalars(dev)
        self.flce_memory = {}
        self.n_valid_x = int((xe["targets"] != synth.IGNORE_INDEX).sum())
        self.n_valid_f = int((fl["targets"] != synth.IGNORE_INDEX).sum())
        del r, ro, s, xe, fl
        self.ops = self._ops()
        if only:
            self.ops = [o for o in self.ops if o[0] in only]

    def _ops(self):
        fo, c3, c5 = self.fo, self.c3, self.c5
        T, d, b = c3.T, c3.d, 2
        heads = c3.n_q + c3.n_kv
        D, F, V = c3.head_dim, c3.F, c3.V
        n_ign = T - self.n_valid_x
        H5, V5 = c5.flce_H, c5.V
        # algorithmic bytes (what each op must move at least) and flops
        by = {
            "rmsnorm_fwd": 2 * T * d * b + d * b + 4 * T,
            "rmsnorm_bwd": 3 * T * d * b + d * b + 4 * T + 4 * d,
            "rope_fwd": 2 * T * heads * D * b + 8 * T,
            "rope_bwd": 2 * T * heads * D * b + 8 * T,
            "swiglu_fwd": 3 * T * F * b,
            "swiglu_bwd": 5 * T * F * b,
            "xent_fwd_bwd": (2 * self.n_valid_x + n_ign) * V * b + 8 * T,
        }
        flce_flops = 6 * self.n_valid_f * H5 * V5
        return [
            ("rmsnorm_fwd", lambda: fo.fo_rmsnorm_fwd(self.x, self.w, c3.eps, y=self.y, rstd=self.rstd),
             by["rmsnorm_fwd"], "hbm"),
            ("rmsnorm_bwd", lambda: fo.fo_rmsnorm_bwd(self.dy, self.x, self.w, self.rstd, c3.eps,
                                                      dx=self.dx, dw=self.dw, ws=self.rms_ws),
             by["rmsnorm_bwd"], "hbm"),
            ("rope_fwd", lambda: fo.fo_rope_fwd(self.q, self.k, self.pos, c3.theta),
             by["rope_fwd"], "hbm"),
            ("rope_bwd", lambda: fo.fo_rope_bwd(self.dq, self.dk, self.pos, c3.theta),
             by["rope_bwd"], "hbm"),
            ("swiglu_fwd", lambda: fo.fo_swiglu_fwd(self.g, self.u, h=self.h), by["swiglu_fwd"], "hbm"),
            ("swiglu_bwd", lambda: fo.fo_swiglu_bwd(self.dh, self.g, self.u, dgate=self.dg, dup=self.du),
             by["swiglu_bwd"], "hbm"),
            ("xent_fwd_bwd", lambda: fo.fo_xent_fwd_bwd(self.logits, self.tg, -100, c3.z_loss, 1.0,
                                                        dlogits=self.dlogits, ws=self.xent_ws,
                                                        out=self.xo),
             by["xent_fwd_bwd"], "hbm"),
            ("flce_fwd_bwd", lambda: fo.fo_flce_fwd_bwd(self.H, self.W, self.ftg, -100, c5.z_loss, 1.0,
                                                        dhidden=self.dH, dweight=self.dW,
                                                        ws=self.flce_ws, out=self.fo_out),
             flce_flops, "mfma"),
        ]


def flce_memory(fo, torch, wl):
    """Device memory of one fused linear cross-entropy call at the lm-head workload: the
    caller's inputs, outputs and workspace (the library allocates nothing: checked by the
    allocator's count across a call), against the bf16 logits [T, V] the fusion never
    stores."""
    c5 = wl.c5
    T, H, V = c5.T, c5.flce_H, c5.V
    ins = sum(t.numel() * t.element_size() for t in (wl.H, wl.W, wl.ftg))
    outs = sum(t.numel() * t.element_size() for t in (wl.dH, wl.dW))
    ws = wl.flce_ws.numel()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    wl.ops[[o[0] for o in wl.ops].index("flce_fwd_bwd")][1]()
    torch.cuda.synchronize()
    return {"workspace_bytes": ws,
            "full_logits_bf16_bytes": T * V * 2,
            "workspace_frac_of_logits": round(ws / (T * V * 2), 4),
            "input_bytes": ins, "output_bytes": outs,
            "peak_bytes_in_call": ins + outs + ws,
            "bytes_allocated_by_call": torch.cuda.max_memory_allocated() - before}


def measured_peaks(fo, torch, stream, med):
    """Ceilings on this device, same process: the library's streaming copy probe over
    1 GiB (caches flushed before each call) and its register-only MFMA probe."""
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    ts = []
    for r in range(11):
        scratch.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fo.fo_probe_copy(src, dst)
        b.record(stream)
        b.synchronize()
        if r:
            ts.append(a.elapsed_time(b))
    assert torch.equal(dst[:1024], src[:1024])
    copy_gbs = 2 * COPY_BYTES / (med(ts) * 1e-3) / 1e9
    del src, dst, scratch
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(n_cu * 8, dtype=torch.float32, device="cuda")
    ts = []
    flops = 0
    for r in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        flops = fo.fo_probe_mfma(n_cu, MFMA_PROBE_ITERS, out)
        b.record(stream)
        b.synchronize()
        if r:
            ts.append(a.elapsed_time(b))
    mfma_tfs = flops / (med(ts) * 1e-3) / 1e12
    print(f"# probes: copy {copy_gbs:.0f} GB/s, mfma {mfma_tfs:.0f} TFLOP/s", file=sys.stderr,
          flush=True)
    return {"copy_GBps": round(copy_gbs, 1), "copy_bytes": 2 * COPY_BYTES,
            "mfma_TFLOPs": round(mfma_tfs, 1), "mfma_cus": n_cu,
            "note": "fo_probe_copy (16-byte non-temporal, 1 GiB read + 1 GiB written) and "
                    "fo_probe_mfma (v_mfma_f32_32x32x16_bf16 on registers, 2 waves/SIMD)"}


def same_size_copies(fo, torch, stream, med, byte_counts, reps):
    """Per byte count B: the isolated time (caches flushed before each call, median of
    reps) of the library's streaming copy probe moving B/2 bytes in and B/2 out, i.e. the
    ceiling a plain copy of the same size reaches, start-up and drain included."""
    halves = {b: (int(b) // 2) // 16 * 16 for b in byte_counts}
    n = max(halves.values()) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    out = {}
    for b, h in halves.items():
        s_, d_ = src[:h // 4], dst[:h // 4]
        ts = []
        for _ in range(reps):
            scratch.fill_(1.0)
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fo.fo_probe_copy(s_, d_)
            e.record(stream)
            e.synchronize()
            ts.append(a.elapsed_time(e))
        out[b] = med(ts)
    del src, dst, scratch
    return out


ADAMW_LAYERS = 4  # Llama-3-8B decoder layers whose parameters one AdamW call updates


def adamw_line(fo, synth, torch, stream, med, reps, copy_gbs):
    """The fused AdamW step (a row after the step's ops, reported apart from the step):
    one fo_adamw_step call over the fp32 parameters, gradients and moments of
    ADAMW_LAYERS Llama-3-8B decoder layers (9 tensors each, one launch), isolated with
    caches flushed; 28 bytes per element.  The state of one layer is drawn by the seeded
    generator and cloned on the device for the others (values do not change timing)."""
    sizes = [n for _, n in synth.LLAMA3_8B_LAYER_PARAMS]
    one = synth.adamw_inputs(sizes, seed=11)
    base = {k: [t.to("cuda") for t in one[k]] for k in one}
    d = {k: [t.clone() for _ in range(ADAMW_LAYERS) for t in base[k]] for k in base}
    del one, base
    n = sum(t.numel() for t in d["params"])
    sc = dict(step_size=3e-4 / (1 - 0.9 ** 10), beta1=0.9, beta2=0.95,
              bias_correction=(1 - 0.95 ** 10) ** 0.5, decay_factor=1 - 3e-4 * 0.1, eps=1e-8)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    ts = []
    for r in range(reps + 2):
        scratch.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fo.fo_adamw_step(d["params"], d["grads"], d["exp_avgs"], d["exp_avg_sqs"], **sc)
        b.record(stream)
        b.synchronize()
        if r >= 2:
            ts.append(a.elapsed_time(b))
    del scratch
    ms = med(ts)
    byt = 28 * n
    e = {"workload": f"fp32 AdamW step over the parameters of {ADAMW_LAYERS} Llama-3-8B decoder "
                     f"layers ({len(d['params'])} tensors, {n / 1e6:.1f} M elements) in one "
                     "fo_adamw_step call",
         "ms_isolated_median": round(ms, 4), "algorithmic_MB": round(byt / 1e6, 1),
         "GBps": round(byt / (ms * 1e-3) / 1e9, 1),
         "frac_hbm_peak": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if copy_gbs:
        e["frac_measured_copy"] = round(e["GBps"] / copy_gbs, 4)
    del d
    print(f"# adamw: {ms:.3f} ms, {e['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    return e


def layernorm_lines(fo, synth, torch, stream, med, reps, copy_gbs):
    """LayerNorm forward and backward (a row after the step's ops, reported apart from
    the step) at the Llama-3-8B layer shape, isolated with caches flushed.  Algorithmic
    bytes: forward 2Tdb + 2db + 8T (x in, y out, w and b, mean and rstd out); backward
    3Tdb + db + 8T + 8d (dy and x in, dx out, w, the saved statistics, dw and db out)."""
    c3 = synth.CONFIGS[3]
    i = synth.layernorm_inputs(c3)
    x, w, b, dy = (i[k].to("cuda") for k in ("x", "w", "b", "dy"))
    T, d = x.shape
    el = x.element_size()
    y, mean, rstd = fo.fo_layernorm_fwd(x, w, b, c3.eps)
    dx = torch.empty_like(x)
    dw = torch.empty(d, dtype=torch.float32, device="cuda")
    db = torch.empty_like(dw)
    ws = torch.empty(fo.fo_layernorm_bwd_workspace(T, d), dtype=torch.uint8, device="cuda")
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    lines = {}
    for name, fn, byt in (
            ("layernorm_fwd", lambda: fo.fo_layernorm_fwd(x, w, b, c3.eps, y=y, mean=mean, rstd=rstd),
             2 * T * d * el + 2 * d * el + 8 * T),
            ("layernorm_bwd", lambda: fo.fo_layernorm_bwd(dy, x, w, mean, rstd, dx=dx, dw=dw, db=db, ws=ws),
             3 * T * d * el + d * el + 8 * T + 8 * d)):
        ts = []
        for r in range(reps + 2):
            scratch.fill_(1.0)
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            e.record(stream)
            e.synchronize()
            if r >= 2:
                ts.append(a.elapsed_time(e))
        ms = med(ts)
        ent = {"workload": f"T {T}, d {d}, bf16 (Llama-3-8B layer shape)",
               "ms_isolated_median": round(ms, 4), "algorithmic_MB": round(byt / 1e6, 3),
               "GBps": round(byt / (ms * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if copy_gbs:
            ent["frac_measured_copy"] = round(ent["GBps"] / copy_gbs, 4)
        lines[name] = ent
    del scratch
    print("# layernorm lines done", file=sys.stderr, flush=True)
    return lines


def activation_lines(fo, synth, torch, stream, med, reps, copy_gbs):
    """GeLU-gated and plain GeLU MLP activations (rows after the step's ops, reported apart
    from the step) at the Llama-3-8B MLP width (T 8192, F 14336, bf16), isolated with
    caches flushed.  Bytes: gated 3TFb forward, 5TFb backward; plain 2TFb, 3TFb."""
    c3 = synth.CONFIGS[3]
    i = synth.swiglu_inputs(c3)
    g, u, dh = (i[k].to("cuda") for k in ("gate", "up", "dh"))
    T, F = g.shape
    b = g.element_size()
    h = torch.empty_like(g)
    dg, du = torch.empty_like(g), torch.empty_like(g)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    lines = {}
    for name, fn, byt in (
            ("geglu_fwd", lambda: fo.fo_glu_fwd("gelu", g, u, h=h), 3 * T * F * b),
            ("geglu_bwd", lambda: fo.fo_glu_bwd("gelu", dh, g, u, dgate=dg, dup=du), 5 * T * F * b),
            ("gelu_fwd", lambda: fo.fo_act_fwd("gelu", g, y=h), 2 * T * F * b),
            ("gelu_bwd", lambda: fo.fo_act_bwd("gelu", dh, g, dx=dg), 3 * T * F * b)):
        ts = []
        for r in range(reps + 2):
            scratch.fill_(1.0)
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            e.record(stream)
            e.synchronize()
            if r >= 2:
                ts.append(a.elapsed_time(e))
        ms = med(ts)
        ent = {"workload": f"T {T}, F {F}, bf16 (Llama-3-8B MLP width)",
               "ms_isolated_median": round(ms, 4), "algorithmic_MB": round(byt / 1e6, 3),
               "GBps": round(byt / (ms * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if copy_gbs:
            ent["frac_measured_copy"] = round(ent["GBps"] / copy_gbs, 4)
        lines[name] = ent
    del scratch
    print("# activation lines done", file=sys.stderr, flush=True)
    return lines


def distill_line(fo, synth, torch, stream, med, reps, copy_gbs):
    """Soft-target cross-entropy (a row after the step's ops, reported apart from the
    step) on the Llama-3-8B lm-head logits shape (T 8192, V 128256, bf16, 10% of rows
    masked), isolated with caches flushed.  Bytes (3 K + M) V b + T: a kept row reads
    the student and teacher rows and writes its gradient, a masked one only writes zeros
    (K kept rows, M masked), plus the mask."""
    cfg = synth.scaled(synth.CONFIGS[3], 8192)
    i = synth.distill_inputs(cfg)
    z, zt, mask = (i[k].to("cuda") for k in ("logits", "teacher", "row_mask"))
    T, V = z.shape
    dz = torch.empty_like(z)
    ws = torch.empty(fo.fo_distill_workspace(T, V), dtype=torch.uint8, device="cuda")
    out = None
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    ts = []
    for r in range(reps + 2):
        scratch.fill_(1.0)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        out = fo.fo_distill_fwd_bwd(z, zt, mask, dlogits=dz, ws=ws, out=out)
        e.record(stream)
        e.synchronize()
        if r >= 2:
            ts.append(a.elapsed_time(e))
    del scratch
    ms = med(ts)
    kept = int(i["row_mask"].sum())
    byt = (3 * kept + (T - kept)) * V * z.element_size() + T
    ent = {"workload": f"T {T}, V {V}, bf16, 10% of rows masked (Llama-3-8B lm-head logits shape)",
           "ms_isolated_median": round(ms, 4), "algorithmic_MB": round(byt / 1e6, 1),
           "GBps": round(byt / (ms * 1e-3) / 1e9, 1),
           "frac_hbm_peak": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "tokens_per_s": round(T / (ms * 1e-3), 1)}
    if copy_gbs:
        ent["frac_measured_copy"] = round(ent["GBps"] / copy_gbs, 4)
    print(f"# distill: {ms:.3f} ms", file=sys.stderr, flush=True)
    return ent


def iso_times(torch, stream, fn, reps, scratch):
    """Isolated event times (ms) of fn: the 1 GiB scratch written before each call evicts
    L2 and the Infinity Cache, so every call reads its inputs from HBM."""
    fn()
    ts = []
    for _ in range(reps):
        scratch.fill_(1.0)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        e.record(stream)
        e.synchronize()
        ts.append(a.elapsed_time(e))
    return ts


LAUNCH_BOUND_US = 7.0  # ops whose bytes take less than this at 70% of peak: launch-bound


def graph_step(torch, stream, cases, reps, scratch, med):
    """The config's seven layer-op calls as one step, timed eagerly (seven launches from
    the host) and as one captured HIP graph replayed (torch.cuda.graph; the calls use
    preallocated outputs and workspaces, so capture records kernels only), caches flushed
    before each step as for the isolated ops."""
    def eager():
        for _, fn, _ in cases:
            fn()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        eager()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eager()
    torch.cuda.synchronize()
    te = med(iso_times(torch, stream, eager, reps, scratch))
    tg = med(iso_times(torch, stream, g.replay, reps, scratch))
    del g
    return {"ops": [n for n, _, _ in cases], "step_ms_eager": round(te, 4),
            "step_ms_graph": round(tg, 4), "graph_speedup": round(te / tg, 3)}


def config_lines(fo, synth, torch, stream, med, reps, copy_gbs, cids=(1, 2, 3, 4), graph=True):
    """One record per (config, op) for the layer-op configs: the tiny fp32 block (T 256),
    the Qwen2.5-0.5B shapes (T 4096, vocabulary 151936), the Llama-3-8B shapes (T 8192,
    vocabulary 128256, z-loss) and the packed 16k batch (document-reset positions, 25%
    ignored targets): RMSNorm, RoPE and SwiGLU forward and backward, and cross-entropy
    forward+backward, each isolated with caches flushed, against the config's algorithmic
    bytes; fwd+bwd pairs as (bytes_f + bytes_b) / (t_f + t_b).  Ops whose bytes would take
    under LAUNCH_BOUND_US at 70% of the HBM peak are flagged launch_bound (parity cases;
    their rate is not a bandwidth figure).  Each record also carries the isolated time of
    the library's copy probe moving the same bytes (frac_same_size_copy = copy time / op
    time): what a plain copy of that size reaches, start-up and drain included."""
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    out = {}
    for cid in cids:
        cfg = synth.CONFIGS[cid]
        T, d, D, F, V = cfg.T, cfg.d, cfg.head_dim, cfg.F, cfg.V
        heads = cfg.n_q + cfg.n_kv
        r = synth.rmsnorm_inputs(cfg)
        x, w, dy = (r[k].to("cuda") for k in ("x", "w", "dy"))
        b = x.element_size()
        y, rstd = fo.fo_rmsnorm_fwd(x, w, cfg.eps)
        dx = torch.empty_like(x)
        dw = torch.empty(d, dtype=torch.float32, device="cuda")
        rws = torch.empty(fo.fo_rmsnorm_bwd_workspace(T, d), dtype=torch.uint8, device="cuda")
        ro = synth.rope_inputs(cfg)
        q, k, dq, dk, pos = (ro[n].to("cuda") for n in ("q", "k", "dq", "dk", "pos"))
        sw = synth.swiglu_inputs(cfg)
        g, u, dh = (sw[n].to("cuda") for n in ("gate", "up", "dh"))
        h, dg, du = torch.empty_like(g), torch.empty_like(g), torch.empty_like(g)
        xe = synth.xent_inputs(cfg)
        lg, tg = xe["logits"].to("cuda"), xe["targets"].to("cuda")
        dlg = torch.empty_like(lg)
        xws = torch.empty(fo.fo_xent_workspace(T, V), dtype=torch.uint8, device="cuda")
        xo = fo._scalars("cuda")
        n_ign = int((xe["targets"] == synth.IGNORE_INDEX).sum())
        del r, ro, sw, xe
        cases = [
            ("rmsnorm_fwd", lambda: fo.fo_rmsnorm_fwd(x, w, cfg.eps, y=y, rstd=rstd),
             2 * T * d * b + d * b + 4 * T),
            ("rmsnorm_bwd", lambda: fo.fo_rmsnorm_bwd(dy, x, w, rstd, cfg.eps, dx=dx, dw=dw, ws=rws),
             3 * T * d * b + d * b + 4 * T + 4 * d),
            ("rope_fwd", lambda: fo.fo_rope_fwd(q, k, pos, cfg.theta), 2 * T * heads * D * b + 8 * T),
            ("rope_bwd", lambda: fo.fo_rope_bwd(dq, dk, pos, cfg.theta), 2 * T * heads * D * b + 8 * T),
            ("swiglu_fwd", lambda: fo.fo_swiglu_fwd(g, u, h=h), 3 * T * F * b),
            ("swiglu_bwd", lambda: fo.fo_swiglu_bwd(dh, g, u, dgate=dg, dup=du), 5 * T * F * b),
            ("xent_fwd_bwd", lambda: fo.fo_xent_fwd_bwd(lg, tg, -100, cfg.z_loss, 1.0, dlogits=dlg,
                                                        ws=xws, out=xo),
             (2 * (T - n_ign) + n_ign) * V * b + 8 * T),
        ]
        ent = {"workload": f"{cfg.name}: T {T}, d {d}, {cfg.n_q}/{cfg.n_kv} heads x {D}, ffn {F}, "
                           f"vocab {V}, {cfg.dtype}" + (", packed documents" if cfg.packed else "")
                           + (f", {n_ign} ignored targets" if n_ign else "")
                           + (f", z-loss {cfg.z_loss:g}" if cfg.z_loss else ""),
               "ops": {}}
        copy_ms = same_size_copies(fo, torch, stream, med, [byt for _, _, byt in cases], reps)
        for name, fn, byt in cases:
            ts = iso_times(torch, stream, fn, reps, scratch)
            t = med(ts)
            e = {"ms_isolated_median": round(t, 4),
                 "ms_isolated_p10_p90": [round(sorted(ts)[len(ts) // 10], 4),
                                         round(sorted(ts)[(9 * len(ts)) // 10], 4)],
                 "algorithmic_MB": round(byt / 1e6, 3),
                 "GBps": round(byt / (t * 1e-3) / 1e9, 1),
                 "frac_hbm_peak": round(byt / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "launch_bound": byt / (0.7 * HBM_PEAK_GBS * 1e9) * 1e6 < LAUNCH_BOUND_US}
            if copy_gbs:
                e["frac_measured_copy"] = round(e["GBps"] / copy_gbs, 4)
            # the library's copy probe moving the same bytes (half in, half out), isolated
            e["same_size_copy_ms"] = round(copy_ms[byt], 4)
            e["frac_same_size_copy"] = round(copy_ms[byt] / t, 4)
            if name == "xent_fwd_bwd":
                e["tokens_per_s"] = round(T / (t * 1e-3), 1)
            ent["ops"][name] = e
        pairs = {}
        for base in ("rmsnorm", "rope", "swiglu"):
            f_, b_ = ent["ops"][base + "_fwd"], ent["ops"][base + "_bwd"]
            byt = (f_["algorithmic_MB"] + b_["algorithmic_MB"]) * 1e6
            t = (f_["ms_isolated_median"] + b_["ms_isolated_median"]) * 1e-3
            pairs[base] = {"GBps": round(byt / t / 1e9, 1),
                           "frac_hbm_peak": round(byt / t / 1e9 / HBM_PEAK_GBS, 4),
                           "launch_bound": f_["launch_bound"] and b_["launch_bound"]}
        ent["fwd_bwd"] = pairs
        if graph:
            try:
                ent["step_graph"] = graph_step(torch, stream, cases, reps, scratch, med)
            except Exception as e:  # a capture failure must not cost the rest of the line
                torch.cuda.synchronize()
                ent["step_graph"] = {"error": f"{type(e).__name__}: {e}"[:300]}
        out[f"cfg{cid}"] = ent
        del x, w, dy, y, rstd, dx, dw, rws, q, k, dq, dk, pos, g, u, dh, h, dg, du, lg, tg, dlg, xws
        torch.cuda.empty_cache()
        print(f"# config {cid} lines done", file=sys.stderr, flush=True)
    del scratch
    return out


def unaligned_lines(fo, synth, torch, stream, med):
    """Rows that are not a multiple of the 16-byte vector, at the Llama-3-8B token count,
    reported apart from the aligned per-op lines: RMSNorm with d = 4097, SwiGLU with
    F = 14337 (contiguous, and as the halves of one [T, 2F] projection) and cross-entropy
    over a 50257-entry vocabulary (GPT-2's)."""
    import dataclasses
    c3 = synth.CONFIGS[3]
    cu = dataclasses.replace(c3, d=4097, F=14337)
    r = synth.rmsnorm_inputs(cu)
    x, w, dy = (r[k].to("cuda") for k in ("x", "w", "dy"))
    T, d = x.shape
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    dw = torch.empty(d, dtype=torch.float32, device="cuda")
    ws = torch.empty(fo.fo_rmsnorm_bwd_workspace(T, d), dtype=torch.uint8, device="cuda")
    s = synth.swiglu_inputs(cu)
    g, u = s["gate"].to("cuda"), s["up"].to("cuda")
    h = torch.empty_like(g)
    F = g.shape[1]
    b = 2
    # gate and up as the two halves of one [T, 2F] projection with an odd F: strided rows
    # off the 16-byte grid (not walkable as one flat array)
    gu2 = torch.cat([g, u], dim=1)
    g2, u2 = gu2[:, :F], gu2[:, F:]
    dh2 = s["dh"].to("cuda")
    dgu2 = torch.empty_like(gu2)
    cv = dataclasses.replace(c3, V=50257)
    xe = synth.xent_inputs(cv)
    lg, tg = xe["logits"].to("cuda"), xe["targets"].to("cuda")
    dlg = torch.empty_like(lg)
    V = lg.shape[1]
    n_ign = int((xe["targets"] == synth.IGNORE_INDEX).sum())
    xws = torch.empty(fo.fo_xent_workspace(T, V), dtype=torch.uint8, device="cuda")
    xo = fo._scalars("cuda")
    cases = [
        ("rmsnorm_fwd_d4097", lambda: fo.fo_rmsnorm_fwd(x, w, cu.eps, y=y, rstd=rstd),
         2 * T * d * b + d * b + 4 * T),
        ("rmsnorm_bwd_d4097", lambda: fo.fo_rmsnorm_bwd(dy, x, w, rstd, cu.eps, dx=dx, dw=dw, ws=ws),
         3 * T * d * b + d * b + 4 * T + 4 * d),
        ("swiglu_fwd_F14337", lambda: fo.fo_swiglu_fwd(g, u, h=h), 3 * T * F * b),
        ("swiglu_fwd_halves_F14337", lambda: fo.fo_swiglu_fwd(g2, u2, h=h), 3 * T * F * b),
        ("swiglu_bwd_halves_F14337", lambda: fo.fo_swiglu_bwd(dh2, g2, u2, dgate=dgu2[:, :F],
                                                               dup=dgu2[:, F:]), 5 * T * F * b),
        ("xent_fwd_bwd_V50257", lambda: fo.fo_xent_fwd_bwd(lg, tg, -100, cv.z_loss, 1.0, dlogits=dlg,
                                                           ws=xws, out=xo),
         (2 * (T - n_ign) + n_ign) * V * b + 8 * T),
    ]
    res = time_cases(torch, stream, med, cases)
    print("# unaligned lines done", file=sys.stderr, flush=True)
    return res


def time_cases(torch, stream, med, cases, reps=20):
    """Isolated medians (caches flushed before each call) of (name, fn, bytes) cases."""
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    res = {}
    for name, fn, byt in cases:
        t = med(iso_times(torch, stream, fn, reps, scratch))
        res[name] = {"ms_isolated_median": round(t, 4), "algorithmic_MB": round(byt / 1e6, 3),
                     "GBps": round(byt / (t * 1e-3) / 1e9, 1),
                     "frac_hbm_peak": round(byt / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del scratch
    return res


def layout_lines(fo, synth, torch, stream, med):
    """Two layouts of real models at the Llama-3-8B token count, reported apart: RMSNorm
    at the widest Llama width (d 16384, rows over several waves), and SwiGLU on the two
    halves of one fused [T, 2F] gate/up projection (F 14336: strided rows on the 16-byte
    grid)."""
    import dataclasses
    c3 = synth.CONFIGS[3]
    cw = dataclasses.replace(c3, d=16384)
    r = synth.rmsnorm_inputs(cw)
    x, w, dy = (r[k].to("cuda") for k in ("x", "w", "dy"))
    del r
    T, d = x.shape
    y, dx = torch.empty_like(x), torch.empty_like(x)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    dw = torch.empty(d, dtype=torch.float32, device="cuda")
    ws = torch.empty(fo.fo_rmsnorm_bwd_workspace(T, d), dtype=torch.uint8, device="cuda")
    s = synth.swiglu_inputs(c3)
    g, u, dh = (s[k].to("cuda") for k in ("gate", "up", "dh"))
    del s
    F = g.shape[1]
    gu = torch.cat([g, u], dim=1)
    del g, u
    g2, u2 = gu[:, :F], gu[:, F:]
    h = torch.empty(T, F, dtype=gu.dtype, device="cuda")
    dgu = torch.empty_like(gu)
    b = 2
    cases = [
        ("rmsnorm_fwd_d16384", lambda: fo.fo_rmsnorm_fwd(x, w, cw.eps, y=y, rstd=rstd),
         2 * T * d * b + d * b + 4 * T),
        ("rmsnorm_bwd_d16384", lambda: fo.fo_rmsnorm_bwd(dy, x, w, rstd, cw.eps, dx=dx, dw=dw, ws=ws),
         3 * T * d * b + d * b + 4 * T + 4 * d),
        ("swiglu_fwd_halves_F14336", lambda: fo.fo_swiglu_fwd(g2, u2, h=h), 3 * T * F * b),
        ("swiglu_bwd_halves_F14336", lambda: fo.fo_swiglu_bwd(dh, g2, u2, dgate=dgu[:, :F],
                                                               dup=dgu[:, F:]), 5 * T * F * b),
    ]
    fo.fo_rmsnorm_fwd(x, w, cw.eps, y=y, rstd=rstd)
    res = time_cases(torch, stream, med, cases)
    print("# layout lines done", file=sys.stderr, flush=True)
    return res


def gpu_bench(args):
    import torch
    import reduction_rmsnorm_fwd_amd as fo
    from reduction_rmsnorm_fwd_amd import synth

    torch.cuda.set_device(0)
    fo.load()
    if args.calib_copy:
        # a plain copy of known size: 1 GiB read + 1 GiB written, for scaling the
        # FETCH_SIZE / WRITE_SIZE counters of the ops
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        evict = torch.empty(1 << 29, dtype=torch.float32, device="cuda")
        evict.fill_(0.0)  # 2 GiB written after src: src is read cold from HBM below
        torch.cuda.synchronize()
        # device-to-device memcpy: the runtime's plain blit kernel
        dst.untyped_storage().copy_(src.untyped_storage())
        torch.cuda.synchronize()
        del src, dst, evict
    only = tuple(s for s in args.only.split(",") if s)
    t0 = time.time()
    wl = Workload(fo, synth, torch, only)
    print(f"# inputs resident in HBM after {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step(evs=None):
        for i, (_, fn, _, _) in enumerate(wl.ops):
            if evs is not None:
                evs[i][0].record(stream)
            fn()
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)
    if any(o[0] == "flce_fwd_bwd" for o in wl.ops):
        wl.flce_memory = flce_memory(fo, torch, wl)

    nops = len(wl.ops)
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(nops)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    in_step = [[evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]
               for i in range(nops)]
    print(f"# timed {args.steps} steps in {wall:.3f}s", file=sys.stderr, flush=True)

    iso = [None] * nops
    if not args.no_isolated:
        scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        for i, (name, fn, _, bound) in enumerate(wl.ops):
            ts = []
            for _ in range(args.iso_reps if bound == "hbm" else args.iso_reps_flce):
                scratch.fill_(1.0)  # evict L2 and the Infinity Cache
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                b.synchronize()
                ts.append(a.elapsed_time(b))
            iso[i] = ts
        del scratch
        print("# isolated timings done", file=sys.stderr, flush=True)

    def med(v):
        v = sorted(v)
        return v[len(v) // 2]

    peaks = None if args.no_probes else measured_peaks(fo, torch, stream, med)
    hbm_bytes = [work for (_, _, work, bound), t in zip(wl.ops, iso) if bound == "hbm" and t]
    same = (None if args.no_probes or not hbm_bytes
            else same_size_copies(fo, torch, stream, med, hbm_bytes, args.iso_reps))
    unaligned = None if args.no_probes or only else unaligned_lines(fo, synth, torch, stream, med)
    layouts = None if args.no_probes or only else layout_lines(fo, synth, torch, stream, med)
    configs = (None if args.no_configs or only or not args.cids
               else config_lines(fo, synth, torch, stream, med, args.iso_reps,
                                 peaks["copy_GBps"] if peaks else None, args.cids,
                                 graph=not args.no_graph))
    next_ops = None
    if not (args.no_next or only):
        cg = peaks["copy_GBps"] if peaks else None
        next_ops = {"adamw_step": adamw_line(fo, synth, torch, stream, med, 20, cg)}
        next_ops.update(layernorm_lines(fo, synth, torch, stream, med, args.iso_reps, cg))
        next_ops.update(activation_lines(fo, synth, torch, stream, med, args.iso_reps, cg))
        next_ops["distill_fwd_bwd"] = distill_line(fo, synth, torch, stream, med, 10, cg)
    traffic = measured_traffic()
    per_op = {}
    for i, (name, _, work, bound) in enumerate(wl.ops):
        ms = sum(in_step[i]) / len(in_step[i])
        e = {"ms_in_step": round(ms, 4)}
        if iso[i] is not None:
            e["ms_isolated_median"] = round(med(iso[i]), 4)
            e["ms_isolated_p10_p90"] = [round(sorted(iso[i])[len(iso[i]) // 10], 4),
                                        round(sorted(iso[i])[(9 * len(iso[i])) // 10], 4)]
        t_ref = e.get("ms_isolated_median", ms)
        if bound == "hbm":
            e["algorithmic_MB"] = round(work / 1e6, 3)
            e["GBps"] = round(work / (t_ref * 1e-3) / 1e9, 1)
            e["frac_hbm_peak"] = round(work / (t_ref * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            e["GBps_in_step"] = round(work / (ms * 1e-3) / 1e9, 1)
        else:
            e["algorithmic_TFLOP"] = round(work / 1e12, 4)
            e["TFLOPs"] = round(work / (t_ref * 1e-3) / 1e12, 1)
            e["frac_bf16_peak"] = round(work / (t_ref * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
            e["tokens_per_s"] = round(wl.T / (t_ref * 1e-3), 1)
        if name == "xent_fwd_bwd":
            e["tokens_per_s"] = round(wl.T / (t_ref * 1e-3), 1)
        if peaks is not None:
            if bound == "hbm":
                e["frac_measured_copy"] = round(e["GBps"] / peaks["copy_GBps"], 4)
                if same is not None and work in same:
                    e["same_size_copy_ms"] = round(same[work], 4)
                    e["frac_same_size_copy"] = round(same[work] / t_ref, 4)
            else:
                e["frac_measured_mfma"] = round(e["TFLOPs"] / peaks["mfma_TFLOPs"], 4)
        e["traffic_MB"] = round(traffic[name] / 1e6, 1) if traffic and name in traffic else None
        if name == "flce_fwd_bwd":
            e.update(wl.flce_memory)
        per_op[name] = e

    ms_step = wall / args.steps * 1e3
    out = {
        "metric": METRIC,
        "value": round(wl.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3-8b-shaped per-token ops fwd+bwd + lm-head fused linear cross-entropy",
            "tokens_per_step": wl.T,
            "layer_ops": "T 8192, d 4096, 32 Q / 8 KV heads x 128, ffn 14336, eps 1e-5, "
                         "rope theta 5e5, vocab 128256, logits N(0,3^2), z-loss 1e-4",
            "lm_head": "H [8192,4096] N(0,1), W [128256,4096] N(0,0.02^2), 10% ignore_index, "
                       "z-loss 1e-4, dW fp32",
            "parallelism": "single GPU",
        },
        "per_op": per_op,
    }
    # fwd+bwd pairs: (bytes_fwd + bytes_bwd) / (t_fwd + t_bwd), isolated medians
    pairs = {}
    for base in ("rmsnorm", "rope", "swiglu"):
        f, b = per_op.get(base + "_fwd"), per_op.get(base + "_bwd")
        if f and b and "ms_isolated_median" in f and "ms_isolated_median" in b:
            byt = (f["algorithmic_MB"] + b["algorithmic_MB"]) * 1e6
            t = (f["ms_isolated_median"] + b["ms_isolated_median"]) * 1e-3
            pairs[base] = {"GBps": round(byt / t / 1e9, 1),
                           "frac_hbm_peak": round(byt / t / 1e9 / HBM_PEAK_GBS, 4)}
            if peaks is not None:
                pairs[base]["frac_measured_copy"] = round(byt / t / 1e9 / peaks["copy_GBps"], 4)
    if pairs:
        out["fwd_bwd"] = pairs
    if peaks is not None:
        out["measured_peaks"] = peaks
    if next_ops is not None:
        out["next_ops"] = next_ops
    if unaligned is not None:
        out["unaligned"] = unaligned
    if layouts is not None:
        out["layouts"] = layouts
    if configs is not None:
        out["configs"] = configs
    # dominant op of the step: the fused linear cross-entropy (MFMA-bound)
    if "flce_fwd_bwd" in per_op:
        i = [o[0] for o in wl.ops].index("flce_fwd_bwd")
        ms = sum(in_step[i]) / len(in_step[i])
        work = wl.ops[i][2]
        ach = work / (ms * 1e-3) / 1e12
        out["roofline"] = {
            "kernel": "fo_flce_fwd_bwd (per call: per 2048-row chunk the logits and split-K dH "
                      "bf16 MFMA products, ce_apply and the dW product accumulating into the "
                      "fp32 dW; compaction, gather/scatter)",
            "bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic.get("flce_fwd_bwd") if traffic else None,
            "traffic_unit": "bytes per launch",
            "ms_per_launch": round(ms, 4),
        }
        if peaks is not None:
            out["roofline"]["measured_peak"] = peaks["mfma_TFLOPs"]
            out["roofline"]["frac_measured"] = round(ach / peaks["mfma_TFLOPs"], 4)
    return out, wl


def cpu_baseline():
    """The fp64 oracle, as it stands, on a bounded sample of the same step: 4096 of the
    8192 tokens for every layer op and 2048 tokens for the lm head; times are scaled up
    linearly in tokens (every op is per-token) to the step's 8192 tokens."""
    import torch
    import oracle
    from reduction_rmsnorm_fwd_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = os.cpu_count() or 1
    c3, c5 = synth.CONFIGS[3], synth.CONFIGS[5]
    n_layer, n_head = 4096, 2048
    s3 = synth.scaled(c3, n_layer)
    # the layer ops are per token: their oracle calls are mapped over row blocks on a
    # thread pool (numpy releases the GIL inside its loops), at most 16 workers (one
    # GPU's share of the host)
    from concurrent.futures import ThreadPoolExecutor
    workers = max(1, min(16, os.cpu_count() or 1))
    blocks = [(i * n_layer // workers, (i + 1) * n_layer // workers) for i in range(workers)]

    def on_blocks(fn):
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda b: fn(*b), blocks))

    t = {}
    r = synth.rmsnorm_inputs(s3)
    a = time.perf_counter()
    on_blocks(lambda i, j: (oracle.rmsnorm_fwd(r["x"][i:j], r["w"], c3.eps),
                            oracle.rmsnorm_bwd(r["dy"][i:j], r["x"][i:j], r["w"], c3.eps)))
    t["rmsnorm"] = time.perf_counter() - a
    ro = synth.rope_inputs(s3)
    a = time.perf_counter()
    on_blocks(lambda i, j: (oracle.rope_fwd(ro["q"][i:j], ro["k"][i:j], ro["pos"][i:j], c3.theta),
                            oracle.rope_bwd(ro["dq"][i:j], ro["dk"][i:j], ro["pos"][i:j], c3.theta)))
    t["rope"] = time.perf_counter() - a
    s = synth.swiglu_inputs(s3)
    a = time.perf_counter()
    on_blocks(lambda i, j: (oracle.swiglu_fwd(s["gate"][i:j], s["up"][i:j]),
                            oracle.swiglu_bwd(s["dh"][i:j], s["gate"][i:j], s["up"][i:j])))
    t["swiglu"] = time.perf_counter() - a
    xe = synth.xent_inputs(s3)
    a = time.perf_counter()
    on_blocks(lambda i, j: oracle.xent_fwd_bwd(xe["logits"][i:j], xe["targets"][i:j], -100, c3.z_loss, 1.0))
    t["xent"] = time.perf_counter() - a
    fl = synth.flce_inputs(c5)  # the full weight; a token sample of the hidden states
    h = fl["hidden"][:n_head]
    tg = fl["targets"][:n_head]
    a = time.perf_counter()
    oracle.flce_fwd_bwd(h, fl["weight"], tg, -100, c5.z_loss, 1.0)
    t["flce"] = time.perf_counter() - a
    T = c3.T
    est = (t["rmsnorm"] + t["rope"] + t["swiglu"] + t["xent"]) * T / n_layer + t["flce"] * T / n_head
    # the oracle's rate on the same algorithmic work as the GPU lines (sample sizes)
    Ts, d, b = n_layer, c3.d, 2
    heads, D, F, V = c3.n_q + c3.n_kv, c3.head_dim, c3.F, c3.V
    n_ign = int((xe["targets"] == synth.IGNORE_INDEX).sum())
    alg = {
        "rmsnorm": (2 * Ts * d * b + d * b + 4 * Ts) + (3 * Ts * d * b + d * b + 4 * Ts + 4 * d),
        "rope": 2 * (2 * Ts * heads * D * b + 8 * Ts),
        "swiglu": 8 * Ts * F * b,
        "xent": (2 * (Ts - n_ign) + n_ign) * V * b + 8 * Ts,
    }
    n_valid_head = int((tg != synth.IGNORE_INDEX).sum())
    rates = {f"{k}_GBps": round(v / t[k] / 1e9, 3) for k, v in alg.items()}
    rates["flce_TFLOPs"] = round(6 * n_valid_head * c5.flce_H * c5.V / t["flce"] / 1e12, 4)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(T / est, 3), "unit": "tokens/s", "cores": int(max(workers, blas_threads)),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle on {n_layer} of 8192 tokens for RMSNorm/RoPE/SwiGLU/xent "
                  f"and {n_head} tokens for the lm-head FLCE (full 128256x4096 weight), scaled "
                  f"linearly to one 8192-token step; the layer ops' oracle calls mapped over "
                  f"{workers} row blocks on {workers} threads, the FLCE matmuls on "
                  f"{blas_threads} BLAS threads",
        "seconds_measured": round(sum(t.values()), 2),
        "est_seconds_per_step": round(est, 2),
        "per_op_seconds_sample": {k: round(v, 3) for k, v in t.items()},
        "per_op_rate_sample": rates,
        "cpu_model": cpu_model,
        "host_cpus": os.cpu_count(),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the library has no multi-GPU "
                                   "path (every call runs on one device and stream). Run with "
                                   "--gpus 1."}))
        sys.exit(2)
    out, wl = gpu_bench(args)
    del wl
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
