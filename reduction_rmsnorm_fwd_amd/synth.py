"""Seeded synthetic inputs for the fused per-token ops.

This module only draws random numbers and lays them out; it holds none of the
arithmetic of RMSNorm, RoPE, SwiGLU or cross-entropy.  Both the HIP path (bench,
GPU tests) and the fp64 oracle (tests, CPU baseline) take their inputs from here,
so the two sides see exactly the same values.

Workloads stand in for the ones the pages train on:
  * "Fast-LLM: 高效大语言模型训练框架" (xllm-io paper review), section 三 技术架构,
    sub-section 训练配置示例: a Mistral-7B-shaped decoder (hidden 4096, 32 heads / 8
    head groups of size 128, gated SiLU MLP with intermediate 14336, rms_norm
    epsilon 1e-5, rotary theta 1e4, bf16) trained on a ``type: random`` dataset,
    which is what licenses synthetic inputs here.
  * The same page, StarCoder2 case study: 16,384-token context.
  * "LLaMA-Factory Kernels 系统", usage example: Qwen2.5-0.5B.

Every tensor has its own stream ``numpy.random.default_rng([seed, tensor_id, block])``
so any tensor (and any flat block of 2**22 elements of it) can be drawn
independently and in parallel, always giving the same values.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np
import torch

BLOCK = 1 << 22  # elements per independent random stream

# tensor ids: part of every stream key, never reuse one for another tensor
TID = {
    "x": 1, "dy": 2, "w": 3, "q": 4, "k": 5, "dq": 6, "dk": 7,
    "gate": 8, "up": 9, "dh": 10, "logits": 11, "targets": 12, "ignore": 13,
    "docs": 14, "hidden": 15, "weight": 16,
    "param": 17, "grad": 18, "exp_avg": 19, "exp_avg_sq": 20, "bias": 21,
    "teacher": 22, "row_mask": 23,
}


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: shapes, value scales and op hyper-parameters."""
    cid: int
    name: str
    dtype: str            # "f32" or "bf16": storage/compute-output dtype of activations
    T: int                # tokens (rows)
    d: int                # hidden size (RMSNorm)
    n_q: int              # query heads
    n_kv: int             # key/value heads
    head_dim: int
    F: int                # SwiGLU intermediate size
    V: int                # vocabulary
    eps: float
    theta: float
    logit_std: float
    z_loss: float
    ignore_frac: float
    packed: bool          # documents packed with position-id resets
    doc_lengths: tuple = ()   # documents of the unpacked batch (e.g. 2 x 2048)
    seed: int = 0
    # fused linear cross-entropy (lm head) shapes
    flce_H: int = 0
    flce_w_std: float = 0.02


IGNORE_INDEX = -100

CONFIGS = {
    1: Config(1, "tiny-fp32", "f32", T=256, d=512, n_q=8, n_kv=8, head_dim=64, F=1408,
              V=4096, eps=1e-6, theta=1e4, logit_std=2.0, z_loss=0.0, ignore_frac=0.0,
              packed=False, doc_lengths=(256,), seed=0),
    2: Config(2, "qwen2.5-0.5b-bf16", "bf16", T=4096, d=896, n_q=14, n_kv=2, head_dim=64,
              F=4864, V=151936, eps=1e-6, theta=1e6, logit_std=2.0, z_loss=0.0,
              ignore_frac=0.0, packed=False, doc_lengths=(2048, 2048), seed=1),
    3: Config(3, "llama3-8b-bf16", "bf16", T=8192, d=4096, n_q=32, n_kv=8, head_dim=128,
              F=14336, V=128256, eps=1e-5, theta=5e5, logit_std=3.0, z_loss=1e-4,
              ignore_frac=0.0, packed=False, doc_lengths=(8192,), seed=2),
    4: Config(4, "packed-16k-bf16", "bf16", T=16384, d=3072, n_q=24, n_kv=2, head_dim=128,
              F=8192, V=49152, eps=1e-5, theta=1e4, logit_std=2.0, z_loss=0.0,
              ignore_frac=0.25, packed=True, seed=3),
    5: Config(5, "flce-llama3-8b-bf16", "bf16", T=8192, d=4096, n_q=32, n_kv=8,
              head_dim=128, F=14336, V=128256, eps=1e-5, theta=5e5, logit_std=0.0,
              z_loss=1e-4, ignore_frac=0.10, packed=False, doc_lengths=(8192,), seed=4,
              flce_H=4096, flce_w_std=0.02),
}


def scaled(cfg: Config, T: int) -> Config:
    """The same workload with fewer tokens (for oracle-sized parity cases).  An
    unpacked batch of n equal documents stays n documents (the last takes the rest)."""
    n = max(1, min(len(cfg.doc_lengths), T))
    each = T // n
    docs = tuple([each] * (n - 1) + [T - each * (n - 1)])
    return dataclasses.replace(cfg, T=T, doc_lengths=docs)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, tid: int, n: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """n draws of N(mean, std^2) in float32, block-parallel and deterministic."""
    out = np.empty(n, dtype=np.float32)
    nblk = (n + BLOCK - 1) // BLOCK

    def fill(b):
        lo, hi = b * BLOCK, min(n, (b + 1) * BLOCK)
        g = np.random.default_rng([seed, tid, b])
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)
        if mean != 0.0:
            out[lo:hi] += np.float32(mean)

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def _as_torch(a: np.ndarray, dtype: str, shape) -> torch.Tensor:
    t = torch.from_numpy(a.reshape(shape))
    if dtype == "bf16":
        return t.to(torch.bfloat16)  # round-to-nearest-even
    return t


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def doc_lengths_geometric(seed: int, T: int, mean: float = 1024.0, cap: int = 16384):
    """Document lengths ~ Geometric(p=1/mean) on {1,2,...}, capped, concatenated until
    they cover T tokens; the last document is truncated."""
    g = np.random.default_rng([seed, TID["docs"], 0])
    lens = []
    total = 0
    while total < T:
        L = int(min(cap, g.geometric(1.0 / mean)))
        L = min(L, T - total)
        lens.append(L)
        total += L
    return tuple(lens)


def positions(cfg: Config) -> torch.Tensor:
    """Position ids [T] int64: 0..L-1 within each document (reset at each start)."""
    lens = doc_lengths_geometric(cfg.seed, cfg.T) if cfg.packed else cfg.doc_lengths
    if not lens:
        lens = (cfg.T,)
    pos = np.concatenate([np.arange(L, dtype=np.int64) for L in lens])
    assert pos.shape[0] == cfg.T
    return torch.from_numpy(pos)


def targets(cfg: Config, V: int | None = None) -> torch.Tensor:
    """Uniform targets in [0, V); exactly floor(ignore_frac*T) rows set to -100,
    chosen by a seeded permutation independent of document boundaries."""
    V = cfg.V if V is None else V
    g = np.random.default_rng([cfg.seed, TID["targets"], 0])
    t = g.integers(0, V, size=cfg.T, dtype=np.int64)
    n_ign = int(np.floor(cfg.ignore_frac * cfg.T))
    if n_ign:
        gi = np.random.default_rng([cfg.seed, TID["ignore"], 0])
        idx = gi.permutation(cfg.T)[:n_ign]
        t[idx] = IGNORE_INDEX
    return torch.from_numpy(t)


def rmsnorm_inputs(cfg: Config):
    T, d, s = cfg.T, cfg.d, cfg.seed
    x = _as_torch(normal_f32(s, TID["x"], T * d), cfg.dtype, (T, d))
    w = _as_torch(normal_f32(s, TID["w"], d, std=0.1, mean=1.0), cfg.dtype, (d,))
    dy = _as_torch(normal_f32(s, TID["dy"], T * d), cfg.dtype, (T, d))
    return dict(x=x, w=w, dy=dy, eps=cfg.eps)


def layernorm_inputs(cfg: Config):
    """LayerNorm: as RMSNorm's inputs but with rows of nonzero mean (x ~ N(1, 1)) and a
    bias N(0, 0.1^2)."""
    T, d, s = cfg.T, cfg.d, cfg.seed
    x = _as_torch(normal_f32(s, TID["x"], T * d, mean=1.0), cfg.dtype, (T, d))
    w = _as_torch(normal_f32(s, TID["w"], d, std=0.1, mean=1.0), cfg.dtype, (d,))
    b = _as_torch(normal_f32(s, TID["bias"], d, std=0.1), cfg.dtype, (d,))
    dy = _as_torch(normal_f32(s, TID["dy"], T * d), cfg.dtype, (T, d))
    return dict(x=x, w=w, b=b, dy=dy, eps=cfg.eps)


def rope_inputs(cfg: Config):
    T, hq, hk, D, s = cfg.T, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.seed
    q = _as_torch(normal_f32(s, TID["q"], T * hq * D), cfg.dtype, (T, hq, D))
    k = _as_torch(normal_f32(s, TID["k"], T * hk * D), cfg.dtype, (T, hk, D))
    dq = _as_torch(normal_f32(s, TID["dq"], T * hq * D), cfg.dtype, (T, hq, D))
    dk = _as_torch(normal_f32(s, TID["dk"], T * hk * D), cfg.dtype, (T, hk, D))
    return dict(q=q, k=k, dq=dq, dk=dk, pos=positions(cfg), theta=cfg.theta)


def swiglu_inputs(cfg: Config):
    T, F, s = cfg.T, cfg.F, cfg.seed
    g = _as_torch(normal_f32(s, TID["gate"], T * F), cfg.dtype, (T, F))
    u = _as_torch(normal_f32(s, TID["up"], T * F), cfg.dtype, (T, F))
    dh = _as_torch(normal_f32(s, TID["dh"], T * F), cfg.dtype, (T, F))
    return dict(gate=g, up=u, dh=dh)


def xent_inputs(cfg: Config):
    T, V, s = cfg.T, cfg.V, cfg.seed
    z = _as_torch(normal_f32(s, TID["logits"], T * V, std=cfg.logit_std), cfg.dtype, (T, V))
    return dict(logits=z, targets=targets(cfg), ignore_index=IGNORE_INDEX,
                z_loss=cfg.z_loss, dloss=1.0)


def flce_inputs(cfg: Config):
    T, H, V, s = cfg.T, cfg.flce_H, cfg.V, cfg.seed
    assert H > 0, "config has no lm-head shape"
    h = _as_torch(normal_f32(s, TID["hidden"], T * H), "bf16", (T, H))
    w = _as_torch(normal_f32(s, TID["weight"], V * H, std=cfg.flce_w_std), "bf16", (V, H))
    return dict(hidden=h, weight=w, targets=targets(cfg), ignore_index=IGNORE_INDEX,
                z_loss=cfg.z_loss, dloss=1.0)


def flce_small(T: int, H: int, V: int, seed: int, ignore_frac: float = 0.1,
               z_loss: float = 1e-4, w_std: float = 0.02) -> Config:
    """An oracle-sized lm-head workload with the full-size value distributions."""
    return Config(90 + seed, f"flce-{T}x{H}x{V}", "bf16", T=T, d=H, n_q=1, n_kv=1,
                  head_dim=2, F=1, V=V, eps=1e-5, theta=1e4, logit_std=0.0,
                  z_loss=z_loss, ignore_frac=ignore_frac, packed=False,
                  doc_lengths=(T,), seed=seed, flce_H=H, flce_w_std=w_std)


# Parameter tensors of one Llama-3-8B decoder layer (fp32 master copies): q, k, v, o
# projections, gate/up/down of the MLP, the two RMSNorm weights.
LLAMA3_8B_LAYER_PARAMS = (
    ("wq", 4096 * 4096), ("wk", 1024 * 4096), ("wv", 1024 * 4096), ("wo", 4096 * 4096),
    ("w_gate", 14336 * 4096), ("w_up", 14336 * 4096), ("w_down", 4096 * 14336),
    ("attn_norm", 4096), ("mlp_norm", 4096),
)


def adamw_inputs(sizes, seed: int):
    """Optimizer state of a list of fp32 parameter tensors with the given element
    counts: parameters N(0, 0.02^2), gradients N(0, 1e-3^2), first moments
    N(0, 1e-4^2), second moments |N(0, 1e-3^2)| (non-negative, as squares are).
    Tensor i draws from its own streams, keyed by (seed, tensor id, i)."""
    out = dict(params=[], grads=[], exp_avgs=[], exp_avg_sqs=[])
    for i, n in enumerate(sizes):
        key = seed * 100003 + i
        out["params"].append(torch.from_numpy(normal_f32(key, TID["param"], n, std=0.02)))
        out["grads"].append(torch.from_numpy(normal_f32(key, TID["grad"], n, std=1e-3)))
        out["exp_avgs"].append(torch.from_numpy(normal_f32(key, TID["exp_avg"], n, std=1e-4)))
        out["exp_avg_sqs"].append(
            torch.from_numpy(np.abs(normal_f32(key, TID["exp_avg_sq"], n, std=1e-3))))
    return out


def distill_inputs(cfg: Config, mask_frac: float = 0.1, teacher_std: float = 2.0):
    """Soft-target cross-entropy: the config's student logits (as for cross-entropy), a
    teacher's logits N(0, teacher_std^2) of the same shape and dtype, and a row mask that
    drops round(mask_frac * T) rows chosen by a seeded permutation."""
    T, V, s = cfg.T, cfg.V, cfg.seed
    z = _as_torch(normal_f32(s, TID["logits"], T * V, std=cfg.logit_std), cfg.dtype, (T, V))
    zt = _as_torch(normal_f32(s, TID["teacher"], T * V, std=teacher_std), cfg.dtype, (T, V))
    mask = np.ones(T, dtype=np.uint8)
    drop = np.random.default_rng([s, TID["row_mask"]]).permutation(T)[:int(round(mask_frac * T))]
    mask[drop] = 0
    return dict(logits=z, teacher=zt, row_mask=torch.from_numpy(mask), dloss=1.0)
