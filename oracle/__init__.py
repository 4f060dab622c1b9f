"""fp64 CPU oracle for the fused per-token training ops — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct definition of what the HIP
library computes.  It exists to check the library; it is never part of the
product path.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it.  It shares no code with the HIP path (no
kernels, helpers, tables or constants); the only thing both sides use is the
seeded input generator module, which holds no arithmetic of the ops.

All arithmetic is numpy float64 on inputs decoded exactly from the values the GPU
sees (fp32 or bf16 widened to fp64).  The oracle never rounds its outputs.

Pages cited (titles as printed):
  [FastLLM] "Fast-LLM: 高效大语言模型训练框架" (xllm-io paper review)
  [LF]      "LLaMA-Factory Kernels 系统"
  [HFK]     "Kernels（自定义内核）" (transformers docs)
The pages name the ops but print no formula for any of them; each function below
states the textbook reading it implements and the readings taken where the pages
are silent.  Every function is pinned by the ``-m "not gpu"`` tests against closed
forms, invariants, finite differences and independent library routines.  Parity
unpinned by the pages themselves (fixed by a stated reading, pinned only against
that reading): the RoPE pairing convention, the z-loss formula, the position
of eps inside the RMSNorm and LayerNorm roots, the LayerNorm form (biased variance,
scale and bias), the exact (erf) GeLU, the soft-target (distillation) cross-entropy form, and the AdamW
formula behind the Adam kernel's
printed signature.
"""
from .ops import (  # noqa: F401
    rmsnorm_fwd, rmsnorm_bwd,
    layernorm_fwd, layernorm_bwd,
    rope_angles, rope_fwd, rope_bwd,
    silu, swiglu_fwd, swiglu_bwd,
    ACTS, act_value, act_deriv, glu_fwd, glu_bwd, act_fwd, act_bwd,
    xent_fwd_bwd, xent_rows, distill_fwd_bwd,
    flce_fwd_bwd,
    adamw_scalars, adamw_step,
)
