"""Python binding of libfo.so, the gfx950 library of fused per-token training ops.

Argument marshalling only: every step of every op runs in the library's HIP kernels.
PyTorch supplies device memory (outputs, workspaces) and the current HIP stream.
If the library is not built, or the current device is not gfx950, the calls raise;
there is no fallback of any kind.

The functions carry the names of the C entry points (see include/fo.h) and take
torch tensors; outputs not passed in are allocated on the input's device.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "load", "FoError", "FO_F32", "FO_BF16",
    "fo_rmsnorm_fwd", "fo_rmsnorm_bwd", "fo_rope_fwd", "fo_rope_bwd",
    "fo_swiglu_fwd", "fo_swiglu_bwd", "fo_xent_fwd_bwd", "fo_xent_fwd_bwd_noalloc",
    "fo_flce_fwd_bwd",
    "fo_rmsnorm_bwd_workspace", "fo_xent_workspace", "fo_flce_workspace", "fo_adamw_step",
    "fo_layernorm_fwd", "fo_layernorm_bwd", "fo_layernorm_bwd_workspace",
    "fo_glu_fwd", "fo_glu_bwd", "fo_act_fwd", "fo_act_bwd", "ACTS",
    "fo_distill_fwd_bwd", "fo_distill_workspace",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfo.so")
FO_F32, FO_BF16 = 0, 1

_lib = None
_checked_devices = set()

_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p

# name -> (restype, argtypes), exactly as declared in include/fo.h
SIGNATURES = {
    "fo_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "fo_abi_version": (ctypes.c_int, []),
    "fo_device_supported": (ctypes.c_int, [ctypes.c_int]),
    "fo_rmsnorm_fwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                      ctypes.c_float, _c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "fo_rmsnorm_bwd_workspace": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "fo_rmsnorm_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                      _c_i64, _c_ptr, _c_ptr, ctypes.c_float, _c_ptr, _c_i64,
                                      _c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]),
    "fo_layernorm_fwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                        _c_ptr, ctypes.c_float, _c_ptr, _c_i64, _c_ptr, _c_ptr,
                                        _c_ptr]),
    "fo_layernorm_bwd_workspace": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "fo_layernorm_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                        _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_ptr,
                                        _c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]),
    "fo_rope_fwd": (ctypes.c_int, [ctypes.c_int, _c_i64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                   ctypes.c_double, _c_ptr]),
    "fo_rope_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                   ctypes.c_double, _c_ptr]),
    "fo_swiglu_fwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                     _c_i64, _c_ptr, _c_i64, _c_ptr]),
    "fo_swiglu_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                     _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64,
                                     _c_ptr]),
    "fo_glu_fwd": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64,
                                  _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr]),
    "fo_glu_bwd": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64,
                                  _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                  _c_i64, _c_ptr]),
    "fo_act_fwd": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64,
                                  _c_ptr, _c_i64, _c_ptr]),
    "fo_act_bwd": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64,
                                  _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr]),
    "fo_xent_workspace": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "fo_xent_fwd_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                       _c_i64, ctypes.c_float, ctypes.c_float, _c_ptr, _c_i64,
                                       _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_size_t,
                                       _c_ptr]),
    "fo_xent_fwd_bwd_noalloc": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64,
                                               _c_ptr, _c_i64, ctypes.c_float, ctypes.c_float,
                                               _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                               _c_ptr]),
    "fo_distill_workspace": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "fo_distill_fwd_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                          _c_i64, _c_ptr, ctypes.c_float, _c_ptr, _c_i64, _c_ptr,
                                          _c_ptr, _c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]),
    "fo_flce_workspace": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int]),
    "fo_adamw_step": (ctypes.c_int, [ctypes.c_int32, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                     _c_ptr, _c_ptr, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_float, _c_ptr]),
    "fo_probe_copy": (ctypes.c_int, [_c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]),
    "fo_probe_mfma": (ctypes.c_int, [ctypes.c_int32, _c_i64, _c_ptr, _c_ptr]),
    "fo_flce_fwd_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr,
                                       _c_ptr, _c_i64, ctypes.c_float, ctypes.c_float, _c_ptr,
                                       _c_ptr, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                       _c_i64, _c_ptr, ctypes.c_size_t, _c_ptr]),
}


class FoError(RuntimeError):
    """A non-FO_OK status from the library."""

    def __init__(self, name, status, msg):
        super().__init__(f"{name}: {msg} (status {status})")
        self.status = status


def load_library():
    """Loads libfo.so and declares its signatures (no device needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m reduction_rmsnorm_fwd_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def load():
    """Loads the library and checks that the current torch device is gfx950."""
    import torch
    lib = load_library()
    dev = torch.cuda.current_device()
    if dev not in _checked_devices:
        st = lib.fo_device_supported(dev)
        if st != 0:
            raise RuntimeError(f"device {dev} is not supported by libfo.so: "
                               f"{lib.fo_status_str(st).decode()}")
        _checked_devices.add(dev)
    return lib


def _check(name, st):
    if st != 0:
        raise FoError(name, st, _lib.fo_status_str(st).decode())


def _dt(t):
    import torch
    if t.dtype == torch.float32:
        return FO_F32
    if t.dtype == torch.bfloat16:
        return FO_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows(t, name):
    """Row stride (elements) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: need a 2-D tensor with contiguous rows")
    return t.stride(0)


def _ws(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------- RMSNorm
def fo_rmsnorm_fwd(x, w, eps, y=None, rstd=None, want_rstd=True):
    import torch
    lib = load()
    T, d = x.shape
    if y is None:
        y = torch.empty_like(x)
    if rstd is None and want_rstd:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("fo_rmsnorm_fwd", lib.fo_rmsnorm_fwd(_dt(x), T, d, _ptr(x), _rows(x, "x"), _ptr(w),
                                                float(eps), _ptr(y), _rows(y, "y"), _ptr(rstd),
                                                _stream()))
    return y, rstd


def fo_rmsnorm_bwd_workspace(T, d):
    return load_library().fo_rmsnorm_bwd_workspace(T, d)


def fo_rmsnorm_bwd(dy, x, w, rstd, eps, dx=None, dw=None, ws=None):
    import torch
    lib = load()
    T, d = x.shape
    if dx is None:
        dx = torch.empty_like(x)
    if dw is None:
        dw = torch.empty(d, dtype=torch.float32, device=x.device)
    need = lib.fo_rmsnorm_bwd_workspace(T, d)
    if ws is None:
        ws = _ws(need, x.device)
    _check("fo_rmsnorm_bwd", lib.fo_rmsnorm_bwd(
        _dt(x), T, d, _ptr(dy), _rows(dy, "dy"), _ptr(x), _rows(x, "x"), _ptr(w), _ptr(rstd),
        float(eps), _ptr(dx), _rows(dx, "dx"), _ptr(dw), _ptr(ws), ws.numel(), _stream()))
    return dx, dw


# ----------------------------------------------------------------- LayerNorm
def fo_layernorm_fwd(x, w, b, eps, y=None, mean=None, rstd=None, want_stats=True):
    import torch
    lib = load()
    T, d = x.shape
    if y is None:
        y = torch.empty_like(x)
    if want_stats:
        if mean is None:
            mean = torch.empty(T, dtype=torch.float32, device=x.device)
        if rstd is None:
            rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("fo_layernorm_fwd", lib.fo_layernorm_fwd(
        _dt(x), T, d, _ptr(x), _rows(x, "x"), _ptr(w), _ptr(b), float(eps), _ptr(y),
        _rows(y, "y"), _ptr(mean), _ptr(rstd), _stream()))
    return y, mean, rstd


def fo_layernorm_bwd_workspace(T, d):
    return load_library().fo_layernorm_bwd_workspace(T, d)


def fo_layernorm_bwd(dy, x, w, mean, rstd, dx=None, dw=None, db=None, ws=None):
    import torch
    lib = load()
    T, d = x.shape
    if dx is None:
        dx = torch.empty_like(x)
    if dw is None:
        dw = torch.empty(d, dtype=torch.float32, device=x.device)
    if db is None:
        db = torch.empty(d, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = _ws(lib.fo_layernorm_bwd_workspace(T, d), x.device)
    _check("fo_layernorm_bwd", lib.fo_layernorm_bwd(
        _dt(x), T, d, _ptr(dy), _rows(dy, "dy"), _ptr(x), _rows(x, "x"), _ptr(w), _ptr(mean),
        _ptr(rstd), _ptr(dx), _rows(dx, "dx"), _ptr(dw), _ptr(db), _ptr(ws), ws.numel(),
        _stream()))
    return dx, dw, db


# ---------------------------------------------------------------------- RoPE
def _heads(t, name):
    if t.dim() != 3 or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{name}: need [T, heads, head_dim] with contiguous heads")
    return t.stride(0)


def _rope(fn, q, k, pos, theta):
    lib = load()
    T, hq, D = q.shape
    hk = k.shape[1]
    _check(fn, getattr(lib, fn)(_dt(q), T, hq, hk, D, _ptr(q), _heads(q, "q"), _ptr(k),
                                _heads(k, "k"), _ptr(pos), float(theta), _stream()))
    return q, k


def fo_rope_fwd(q, k, positions, theta):
    """In place on q [T,Hq,D] and k [T,Hkv,D]; positions [T] int64 on the device."""
    return _rope("fo_rope_fwd", q, k, positions, theta)


def fo_rope_bwd(dq, dk, positions, theta):
    return _rope("fo_rope_bwd", dq, dk, positions, theta)


# -------------------------------------------------------------------- SwiGLU
def fo_swiglu_fwd(gate, up, h=None):
    import torch
    lib = load()
    T, F = gate.shape
    if h is None:
        h = torch.empty((T, F), dtype=gate.dtype, device=gate.device)
    _check("fo_swiglu_fwd", lib.fo_swiglu_fwd(_dt(gate), T, F, _ptr(gate), _rows(gate, "gate"),
                                              _ptr(up), _rows(up, "up"), _ptr(h), _rows(h, "h"),
                                              _stream()))
    return h


def fo_swiglu_bwd(dh, gate, up, dgate=None, dup=None):
    import torch
    lib = load()
    T, F = gate.shape
    if dgate is None:
        dgate = torch.empty((T, F), dtype=gate.dtype, device=gate.device)
    if dup is None:
        dup = torch.empty((T, F), dtype=gate.dtype, device=gate.device)
    _check("fo_swiglu_bwd", lib.fo_swiglu_bwd(
        _dt(gate), T, F, _ptr(dh), _rows(dh, "dh"), _ptr(gate), _rows(gate, "gate"), _ptr(up),
        _rows(up, "up"), _ptr(dgate), _rows(dgate, "dgate"), _ptr(dup), _rows(dup, "dup"),
        _stream()))
    return dgate, dup


ACTS = {"silu": 0, "gelu": 1, "relu": 2}  # FO_ACT_SILU, FO_ACT_GELU, FO_ACT_RELU


def fo_glu_fwd(act, gate, up, h=None):
    """h = act(gate) * up, act in ACTS."""
    import torch
    lib = load()
    T, F = gate.shape
    if h is None:
        h = torch.empty((T, F), dtype=gate.dtype, device=gate.device)
    _check("fo_glu_fwd", lib.fo_glu_fwd(_dt(gate), ACTS[act], T, F, _ptr(gate), _rows(gate, "gate"),
                                        _ptr(up), _rows(up, "up"), _ptr(h), _rows(h, "h"),
                                        _stream()))
    return h


def fo_glu_bwd(act, dh, gate, up, dgate=None, dup=None):
    import torch
    lib = load()
    T, F = gate.shape
    if dgate is None:
        dgate = torch.empty((T, F), dtype=gate.dtype, device=gate.device)
    if dup is None:
        dup = torch.empty((T, F), dtype=gate.dtype, device=gate.device)
    _check("fo_glu_bwd", lib.fo_glu_bwd(
        _dt(gate), ACTS[act], T, F, _ptr(dh), _rows(dh, "dh"), _ptr(gate), _rows(gate, "gate"),
        _ptr(up), _rows(up, "up"), _ptr(dgate), _rows(dgate, "dgate"), _ptr(dup),
        _rows(dup, "dup"), _stream()))
    return dgate, dup


def fo_act_fwd(act, x, y=None):
    """y = act(x), act in ACTS."""
    import torch
    lib = load()
    T, F = x.shape
    if y is None:
        y = torch.empty((T, F), dtype=x.dtype, device=x.device)
    _check("fo_act_fwd", lib.fo_act_fwd(_dt(x), ACTS[act], T, F, _ptr(x), _rows(x, "x"), _ptr(y),
                                        _rows(y, "y"), _stream()))
    return y


def fo_act_bwd(act, dy, x, dx=None):
    import torch
    lib = load()
    T, F = x.shape
    if dx is None:
        dx = torch.empty((T, F), dtype=x.dtype, device=x.device)
    _check("fo_act_bwd", lib.fo_act_bwd(_dt(x), ACTS[act], T, F, _ptr(dy), _rows(dy, "dy"), _ptr(x),
                                        _rows(x, "x"), _ptr(dx), _rows(dx, "dx"), _stream()))
    return dx


# ------------------------------------------------------------- cross-entropy
def fo_xent_workspace(T, V):
    return load_library().fo_xent_workspace(T, V)


def _scalars(device):
    import torch
    return dict(loss=torch.empty(1, dtype=torch.float32, device=device),
                z_loss=torch.empty(1, dtype=torch.float32, device=device),
                n_valid=torch.empty(1, dtype=torch.int64, device=device),
                status=torch.empty(1, dtype=torch.int32, device=device))


def fo_xent_fwd_bwd(logits, targets, ignore_index=-100, z_loss=0.0, dloss=1.0, dlogits=None,
                    grad=True, ws=None, out=None):
    """dlogits: None (allocate), a tensor (may be `logits` itself for in place), or ignored
    when grad=False (forward only).  Returns dict of device tensors."""
    import torch
    lib = load()
    T, V = logits.shape
    if grad and dlogits is None:
        dlogits = torch.empty_like(logits)
    if not grad:
        dlogits = None
    o = out if out is not None else _scalars(logits.device)
    if ws is None:
        ws = _ws(lib.fo_xent_workspace(T, V), logits.device)
    _check("fo_xent_fwd_bwd", lib.fo_xent_fwd_bwd(
        _dt(logits), T, V, _ptr(logits), _rows(logits, "logits"), _ptr(targets),
        int(ignore_index), float(z_loss), float(dloss), _ptr(dlogits),
        _rows(dlogits, "dlogits") if dlogits is not None else V, _ptr(o["loss"]),
        _ptr(o["z_loss"]), _ptr(o["n_valid"]), _ptr(o["status"]), _ptr(ws), ws.numel(),
        _stream()))
    o["dlogits"] = dlogits
    return o


def fo_xent_fwd_bwd_noalloc(logits, targets, ignore_index=-100, z_loss=0.0, dloss=1.0,
                            dlogits=None, grad=True, out=None):
    """fo_xent_fwd_bwd on the library's own per-device workspace (no workspace tensor;
    the C call allocates nothing).  Outputs as fo_xent_fwd_bwd; pass dlogits and out to
    allocate nothing on this side either."""
    import torch
    lib = load()
    T, V = logits.shape
    if grad and dlogits is None:
        dlogits = torch.empty_like(logits)
    if not grad:
        dlogits = None
    o = out if out is not None else _scalars(logits.device)
    _check("fo_xent_fwd_bwd_noalloc", lib.fo_xent_fwd_bwd_noalloc(
        _dt(logits), T, V, _ptr(logits), _rows(logits, "logits"), _ptr(targets),
        int(ignore_index), float(z_loss), float(dloss), _ptr(dlogits),
        _rows(dlogits, "dlogits") if dlogits is not None else V, _ptr(o["loss"]),
        _ptr(o["z_loss"]), _ptr(o["n_valid"]), _ptr(o["status"]), _stream()))
    o["dlogits"] = dlogits
    return o


# ------------------------------------------------ soft-target cross-entropy
def fo_distill_workspace(T, V):
    return load_library().fo_distill_workspace(T, V)


def fo_distill_fwd_bwd(logits, teacher, row_mask=None, dloss=1.0, dlogits=None, want_grad=True,
                       ws=None, out=None):
    """Soft-target cross-entropy of logits against softmax(teacher); returns dict(loss,
    kl, n_valid, dlogits).  row_mask: optional uint8 device tensor [T]."""
    import torch
    lib = load()
    T, V = logits.shape
    if want_grad and dlogits is None:
        dlogits = torch.empty_like(logits)
    if out is None:
        out = dict(loss=torch.empty((), dtype=torch.float32, device=logits.device),
                   kl=torch.empty((), dtype=torch.float32, device=logits.device),
                   n_valid=torch.empty((), dtype=torch.int64, device=logits.device))
    if ws is None:
        ws = _ws(lib.fo_distill_workspace(T, V), logits.device)
    if row_mask is not None and row_mask.dtype != torch.uint8:
        raise ValueError("row_mask must be uint8")
    _check("fo_distill_fwd_bwd", lib.fo_distill_fwd_bwd(
        _dt(logits), T, V, _ptr(logits), _rows(logits, "logits"), _ptr(teacher),
        _rows(teacher, "teacher"), _ptr(row_mask), float(dloss), _ptr(dlogits),
        _rows(dlogits, "dlogits") if dlogits is not None else V, _ptr(out["loss"]),
        _ptr(out["kl"]), _ptr(out["n_valid"]), _ptr(ws), ws.numel(), _stream()))
    out["dlogits"] = dlogits
    return out


def fo_flce_workspace(T, H, V, chunk_tokens=0, dweight_dtype=FO_F32):
    return load_library().fo_flce_workspace(T, H, V, chunk_tokens, dweight_dtype)


def fo_flce_fwd_bwd(hidden, weight, targets, ignore_index=-100, z_loss=0.0, dloss=1.0,
                    dweight_dtype=None, chunk_tokens=0, dhidden=None, dweight=None,
                    grad=True, ws=None, out=None):
    import torch
    lib = load()
    T, H = hidden.shape
    V = weight.shape[0]
    if not (hidden.is_contiguous() and weight.is_contiguous()):
        raise ValueError("hidden and weight must be contiguous")
    dwt = torch.float32 if dweight_dtype is None else dweight_dtype
    dwcode = FO_F32 if dwt == torch.float32 else FO_BF16
    if grad:
        if dhidden is None:
            dhidden = torch.empty_like(hidden)
        if dweight is None:
            dweight = torch.empty((V, H), dtype=dwt, device=weight.device)
    else:
        dhidden = dweight = None
    o = out if out is not None else _scalars(hidden.device)
    if ws is None:
        ws = _ws(lib.fo_flce_workspace(T, H, V, chunk_tokens, dwcode), hidden.device)
    _check("fo_flce_fwd_bwd", lib.fo_flce_fwd_bwd(
        FO_BF16, T, H, V, _ptr(hidden), _ptr(weight), _ptr(targets), int(ignore_index),
        float(z_loss), float(dloss), _ptr(dhidden), _ptr(dweight), dwcode, _ptr(o["loss"]),
        _ptr(o["z_loss"]), _ptr(o["n_valid"]), _ptr(o["status"]), int(chunk_tokens), _ptr(ws),
        ws.numel(), _stream()))
    o["dhidden"] = dhidden
    o["dweight"] = dweight
    return o


def fo_adamw_step(params, grads, exp_avgs, exp_avg_sqs, step_size, beta1, beta2,
                  bias_correction, decay_factor, eps, noop_flag=None, grad_scale=None):
    """One fused AdamW step over lists of fp32 device tensors (updated in place).
    noop_flag: optional int32 device tensor of one element; grad_scale: optional fp32
    device tensor of one element."""
    import torch
    lib = load()
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs differ in length")
    for group in (params, grads, exp_avgs, exp_avg_sqs):
        for t in group:
            if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError("AdamW tensors must be contiguous fp32 device tensors")
    for a, b, c, d in zip(params, grads, exp_avgs, exp_avg_sqs):
        if not (a.numel() == b.numel() == c.numel() == d.numel()):
            raise ValueError("tensor sizes differ within one parameter")
    if noop_flag is not None and (noop_flag.dtype != torch.int32 or not noop_flag.is_cuda):
        raise ValueError("noop_flag must be an int32 device tensor")
    if grad_scale is not None and (grad_scale.dtype != torch.float32 or not grad_scale.is_cuda):
        raise ValueError("grad_scale must be an fp32 device tensor")
    arr = ctypes.c_void_p * max(n, 1)
    numel = (ctypes.c_int64 * max(n, 1))(*[t.numel() for t in params])
    ptrs = [arr(*[t.data_ptr() for t in g]) for g in (params, grads, exp_avgs, exp_avg_sqs)]
    _check("fo_adamw_step", lib.fo_adamw_step(
        n, ctypes.cast(numel, ctypes.c_void_p), *[ctypes.cast(p, ctypes.c_void_p) for p in ptrs],
        _ptr(noop_flag) if noop_flag is not None else None,
        _ptr(grad_scale) if grad_scale is not None else None,
        step_size, beta1, beta2, bias_correction, decay_factor, eps, _stream()))


def fo_probe_copy(src, dst):
    """dst.copy of src through the library's streaming copy probe (same byte count)."""
    lib = load()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check("fo_probe_copy", lib.fo_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream()))


def fo_probe_mfma(n_cu, iters, out):
    """Runs the MFMA probe; returns the flops it performs."""
    lib = load()
    _check("fo_probe_mfma", lib.fo_probe_mfma(int(n_cu), int(iters), _ptr(out), _stream()))
    return int(n_cu) * 8 * int(iters) * 4 * 32 * 32 * 16 * 2
