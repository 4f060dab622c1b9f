"""The C ABI library: it loads, exports every function include/fo.h declares, and its
host-side argument checks return the documented statuses before any launch.  No GPU:
only calls that must fail validation (or query sizes) are made."""
import ctypes
import os
import re

import pytest

import reduction_rmsnorm_fwd_amd as fo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fo.h")

OK, NULL, SHAPE, DTYPE, STRIDE, WS, DEVICE, HIP = range(8)
F32, BF16 = 0, 1
P = ctypes.c_void_p(0x1000)  # a non-NULL pointer that is never dereferenced
N = None


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fo_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fo.LIB_PATH):
        pytest.fail("libfo.so is not built (run python -m reduction_rmsnorm_fwd_amd.build)")
    return fo.load_library()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared()
    assert len(names) == 27, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in fo.SIGNATURES, f"binding lacks {n}"
    assert set(fo.SIGNATURES) == set(names)


def test_abi_version_and_status_strings(lib):
    assert lib.fo_abi_version() == 1
    for s in range(8):
        assert lib.fo_status_str(s).decode().startswith("FO_")
    assert b"unknown" in lib.fo_status_str(99)


def test_no_device_here(lib):
    # this container has no GPU: the device check must say so, not crash
    assert lib.fo_device_supported(0) == DEVICE
    assert lib.fo_device_supported(-1) == DEVICE


def test_rmsnorm_validation(lib):
    f = lib.fo_rmsnorm_fwd
    assert f(7, 4, 8, P, 8, P, 1e-5, P, 8, N, N) == DTYPE
    assert f(F32, -1, 8, P, 8, P, 1e-5, P, 8, N, N) == SHAPE
    assert f(F32, 4, 0, P, 8, P, 1e-5, P, 8, N, N) == SHAPE
    assert f(F32, 4, 8, P, 7, P, 1e-5, P, 8, N, N) == STRIDE
    assert f(F32, 4, 8, P, 8, P, 1e-5, P, 4, N, N) == STRIDE
    assert f(BF16, 4, 8, N, 8, P, 1e-5, P, 8, N, N) == NULL
    assert f(BF16, 4, 8, P, 8, N, 1e-5, P, 8, N, N) == NULL
    assert f(BF16, 0, 8, N, 8, N, 1e-5, N, 8, N, N) == OK  # empty: nothing to do
    b = lib.fo_rmsnorm_bwd
    ws = lib.fo_rmsnorm_bwd_workspace(100, 64)
    assert ws >= 64 * 4 * min(100, 256)
    assert lib.fo_rmsnorm_bwd_workspace(-1, 64) == 0
    assert b(BF16, 100, 64, P, 64, P, 64, P, N, 1e-5, P, 64, N, P, ws, N) == NULL  # dw
    assert b(BF16, 100, 64, P, 64, P, 64, P, N, 1e-5, P, 64, P, P, ws - 1, N) == WS
    assert b(BF16, 100, 64, P, 64, P, 64, P, N, 1e-5, P, 64, P, N, ws, N) == WS
    assert b(BF16, 100, 64, P, 63, P, 64, P, N, 1e-5, P, 64, P, P, ws, N) == STRIDE
    assert b(BF16, 100, 64, N, 64, P, 64, P, N, 1e-5, P, 64, P, P, ws, N) == NULL


def test_layernorm_validation(lib):
    f = lib.fo_layernorm_fwd
    assert f(BF16, 4, 8, P, 8, P, N, 1e-5, P, 8, N, N, N) == NULL       # bias required
    assert f(BF16, 4, 8, P, 7, P, P, 1e-5, P, 8, N, N, N) == STRIDE
    assert f(5, 4, 8, P, 8, P, P, 1e-5, P, 8, N, N, N) == DTYPE
    assert f(BF16, 0, 8, N, 8, N, N, 1e-5, N, 8, N, N, N) == OK         # empty
    b = lib.fo_layernorm_bwd
    ws = lib.fo_layernorm_bwd_workspace(100, 64)
    assert ws >= 2 * 64 * 100 * 4  # a dw and a db partial row per row group
    assert b(BF16, 100, 64, P, 64, P, 64, P, N, P, P, 64, P, P, P, ws, N) == NULL  # mean
    assert b(BF16, 100, 64, P, 64, P, 64, P, P, N, P, 64, P, P, P, ws, N) == NULL  # rstd
    assert b(BF16, 100, 64, P, 64, P, 64, P, P, P, P, 64, P, N, P, ws, N) == NULL  # db
    assert b(BF16, 100, 64, P, 64, P, 64, P, P, P, P, 64, P, P, P, ws - 1, N) == WS
    assert b(BF16, 100, 64, P, 63, P, 64, P, P, P, P, 64, P, P, P, ws, N) == STRIDE


def test_rope_validation(lib):
    f = lib.fo_rope_fwd
    assert f(BF16, 8, 4, 2, 7, P, 28, P, 14, P, 1e4, N) == SHAPE       # odd head_dim
    assert f(BF16, 8, 6, 4, 8, P, 48, P, 32, P, 1e4, N) == SHAPE       # 6 % 4 != 0
    assert f(BF16, 8, 4, 2, 1024, P, 4096, P, 2048, P, 1e4, N) == SHAPE  # head_dim > 512
    assert f(BF16, 8, 4, 2, 8, P, 32, P, 16, P, 0.0, N) == SHAPE       # theta <= 0
    assert f(BF16, 8, 4, 2, 8, P, 31, P, 16, P, 1e4, N) == STRIDE
    assert f(BF16, 8, 4, 2, 8, P, 32, P, 15, P, 1e4, N) == STRIDE
    assert f(BF16, 8, 4, 2, 8, P, 32, P, 16, N, 1e4, N) == NULL        # positions
    assert f(BF16, 8, 4, 0, 8, P, 32, P, 16, P, 1e4, N) == SHAPE
    assert lib.fo_rope_bwd(5, 8, 4, 2, 8, P, 32, P, 16, P, 1e4, N) == DTYPE


def test_swiglu_validation(lib):
    f = lib.fo_swiglu_fwd
    assert f(BF16, 4, 0, P, 8, P, 8, P, 8, N) == SHAPE
    assert f(BF16, 4, 8, P, 7, P, 8, P, 8, N) == STRIDE
    assert f(BF16, 4, 8, P, 8, N, 8, P, 8, N) == NULL
    assert f(BF16, 0, 8, N, 8, N, 8, N, 8, N) == OK
    b = lib.fo_swiglu_bwd
    assert b(BF16, 4, 8, P, 8, P, 8, P, 8, P, 8, P, 7, N) == STRIDE
    assert b(BF16, 4, 8, P, 8, P, 8, P, 8, N, 8, P, 8, N) == NULL
    assert b(2, 4, 8, P, 8, P, 8, P, 8, P, 8, P, 8, N) == DTYPE


def test_activation_validation(lib):
    g, a = lib.fo_glu_fwd, lib.fo_act_fwd
    assert g(BF16, 3, 4, 8, P, 8, P, 8, P, 8, N) == SHAPE      # unknown activation
    assert g(BF16, 1, 4, 8, P, 8, P, 7, P, 8, N) == STRIDE
    assert g(BF16, 2, 4, 8, P, 8, N, 8, P, 8, N) == NULL
    assert g(BF16, 1, 0, 8, N, 8, N, 8, N, 8, N) == OK         # empty
    assert a(BF16, -1, 4, 8, P, 8, P, 8, N) == SHAPE
    assert a(BF16, 1, 4, 8, P, 8, P, 7, N) == STRIDE
    assert a(BF16, 2, 4, 8, N, 8, P, 8, N) == NULL
    assert a(7, 1, 4, 8, P, 8, P, 8, N) == DTYPE
    gb, ab = lib.fo_glu_bwd, lib.fo_act_bwd
    assert gb(BF16, 1, 4, 8, P, 8, P, 8, P, 8, P, 8, N, 8, N) == NULL
    assert gb(BF16, 5, 4, 8, P, 8, P, 8, P, 8, P, 8, P, 8, N) == SHAPE
    assert ab(BF16, 1, 4, 8, P, 8, P, 8, N, 8, N) == NULL
    assert ab(BF16, 1, 4, 0, P, 8, P, 8, P, 8, N) == SHAPE


def test_xent_validation(lib):
    f = lib.fo_xent_fwd_bwd
    ws = lib.fo_xent_workspace(16, 100)
    assert ws >= 2 * 16 * 4
    assert f(BF16, 16, 100, P, 100, P, -100, 0.0, 1.0, P, 100, N, N, N, N, P, ws, N) == NULL
    assert f(BF16, 16, 100, P, 99, P, -100, 0.0, 1.0, P, 100, P, N, N, N, P, ws, N) == STRIDE
    assert f(BF16, 16, 100, P, 100, P, -100, 0.0, 1.0, P, 99, P, N, N, N, P, ws, N) == STRIDE
    assert f(BF16, 16, 100, P, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, P, ws - 1, N) == WS
    assert f(BF16, 16, 0, P, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, P, ws, N) == SHAPE
    assert f(BF16, 16, 100, N, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, P, ws, N) == NULL
    assert f(3, 16, 100, P, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, P, ws, N) == DTYPE


def test_xent_noalloc_validation(lib):
    # the same checks as fo_xent_fwd_bwd, all before the library's device array is
    # looked up; more tokens than that array holds are refused with FO_ERR_WORKSPACE
    f = lib.fo_xent_fwd_bwd_noalloc
    mx = 1048576
    assert "FO_XENT_NOALLOC_MAX_T %d" % mx in open(HEADER).read()
    assert f(BF16, 16, 100, P, 100, P, -100, 0.0, 1.0, P, 100, N, N, N, N, N) == NULL
    assert f(BF16, 16, 100, P, 99, P, -100, 0.0, 1.0, P, 100, P, N, N, N, N) == STRIDE
    assert f(BF16, 16, 100, P, 100, P, -100, 0.0, 1.0, P, 99, P, N, N, N, N) == STRIDE
    assert f(BF16, 16, 0, P, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, N) == SHAPE
    assert f(BF16, -1, 100, P, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, N) == SHAPE
    assert f(3, 16, 100, P, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, N) == DTYPE
    assert f(BF16, mx + 1, 100, P, 100, P, -100, 0.0, 1.0, P, 100, P, N, N, N, N) == WS
    # the array's size is the workspace query at the limit
    assert lib.fo_xent_workspace(mx, 100) == 256 + 2 * 4 * mx


def test_distill_validation(lib):
    f = lib.fo_distill_fwd_bwd
    ws = lib.fo_distill_workspace(16, 100)
    assert ws >= 2 * 16 * 4
    args = [BF16, 16, 100, P, 100, P, 100, N, 1.0, P, 100, P, N, N, P, ws, N]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)

    assert call(a0=4) == DTYPE
    assert call(a2=0) == SHAPE
    assert call(a4=99) == STRIDE                 # logits stride
    assert call(a6=99) == STRIDE                 # teacher stride
    assert call(a10=99) == STRIDE                # dlogits stride
    assert call(a11=N) == NULL                   # loss
    assert call(a5=N) == NULL                    # teacher
    assert call(a15=ws - 1) == WS
    assert call(a14=N) == WS


def test_flce_validation(lib):
    f = lib.fo_flce_fwd_bwd
    ws = lib.fo_flce_workspace(64, 32, 100, 0, F32)
    assert ws > 64 * 128 * 2  # at least the chunk's bf16 dZ rows (vocabulary padded to 64)
    assert lib.fo_flce_workspace(64, 32, 100, 0, BF16) >= ws + 100 * 32 * 4
    args = [BF16, 64, 32, 100, P, P, P, -100, 1e-4, 1.0, P, P, F32, P, N, N, N, 0, P, ws, N]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)

    assert call(a0=F32) == DTYPE                 # bf16 only
    assert call(a12=5) == DTYPE                  # dweight dtype
    assert call(a2=12) == SHAPE                  # H % 8
    assert call(a3=0) == SHAPE
    assert call(a13=N) == NULL                   # loss
    assert call(a5=N) == NULL                    # weight
    assert call(a4=ctypes.c_void_p(0x1002)) == STRIDE   # misaligned hidden
    assert call(a19=ws - 1) == WS
    assert call(a17=-1) == SHAPE


def test_flce_workspace_bounded_by_chunk(lib):
    # the fused linear cross-entropy exists so that the [T, V] logits never exist in
    # memory ("Kernels（自定义内核）", section Liger): at the lm-head workload (T 8192,
    # H 4096, V 128256) its whole workspace stays under half of the bf16 logits, and it
    # grows with the chunk, not with T * V
    T, H, V = 8192, 4096, 128256
    logits_bf16 = T * V * 2
    ws = lib.fo_flce_workspace(T, H, V, 0, F32)
    assert 0 < ws <= logits_bf16 // 2, (ws, logits_bf16)
    # doubling T adds per-token rows (hidden copies, statistics), not logits rows
    ws2 = lib.fo_flce_workspace(2 * T, H, V, 0, F32)
    assert ws2 - ws <= T * (2 * H * 2 + 64)
    # a smaller chunk needs less: the dZ rows scale with the chunk
    assert lib.fo_flce_workspace(T, H, V, 1024, F32) < ws - 1024 * V * 2
    # a bf16 dweight adds exactly its fp32 accumulator (V x H), nothing per token
    assert lib.fo_flce_workspace(T, H, V, 0, BF16) - ws <= V * H * 4 + 256


def test_adamw_validation(lib):
    f = lib.fo_adamw_step
    i64 = ctypes.c_int64
    ptrs = ctypes.c_void_p * 2
    numel = (i64 * 2)(5, 0)
    good = ptrs(P, P)
    half = ptrs(P, None)  # NULL allowed for the empty second tensor
    hyp = (1e-3, 0.9, 0.999, 0.5, 0.99, 1e-8, N)
    assert f(-1, N, N, N, N, N, N, N, *hyp) == SHAPE
    assert f(0, N, N, N, N, N, N, N, *hyp) == OK          # nothing to do
    assert f(2, N, good, good, good, good, N, N, *hyp) == NULL
    assert f(2, numel, good, N, good, good, N, N, *hyp) == NULL
    assert f(2, numel, ptrs(None, P), half, half, half, N, N, *hyp) == NULL
    assert f(2, (i64 * 2)(5, -1), good, good, good, good, N, N, *hyp) == SHAPE
    assert f(2, (i64 * 2)(0, 0), ptrs(None, None), ptrs(None, None), ptrs(None, None),
             ptrs(None, None), N, N, *hyp) == OK           # all empty: no launch


def test_probe_validation(lib):
    assert lib.fo_probe_copy(P, P, 0, N) == OK  # nothing to copy
    assert lib.fo_probe_copy(N, P, 16, N) == NULL
    assert lib.fo_probe_copy(P, P, 24, N) == STRIDE
    assert lib.fo_probe_copy(ctypes.c_void_p(0x1008), P, 16, N) == STRIDE
    assert lib.fo_probe_mfma(0, 10, P, N) == SHAPE
    assert lib.fo_probe_mfma(256, 0, P, N) == SHAPE
    assert lib.fo_probe_mfma(256, 10, N, N) == NULL
