"""fo_xent_fwd_bwd_noalloc (no workspace argument; the library's own per-device array)
against fo_xent_fwd_bwd on the same inputs: two calls in a row, the second with fewer
rows, so the second reuses an array that still holds the first call's contents."""
import pytest
import torch

from reduction_rmsnorm_fwd_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
IGN = synth.IGNORE_INDEX


def both(fo, z, t, zc):
    a = fo.fo_xent_fwd_bwd(z, t, IGN, zc, 1.0)
    b = fo.fo_xent_fwd_bwd_noalloc(z, t, IGN, zc, 1.0)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_call_twice(gpu, dtype):
    print(f"noalloc xent dtype={dtype}", flush=True)
    g = torch.Generator().manual_seed(77)
    td = synth.torch_dtype(dtype)
    for T, V, zc in ((300, 32000, 1e-4), (37, 4099, 0.0)):  # second call: fewer rows
        z = (2 * torch.randn(T, V, generator=g)).to(td).to(DEV)
        t = torch.randint(0, V, (T,), generator=g)
        t[::7] = IGN
        t[3] = V + 5  # a bad target
        a, b = both(gpu, z, t.to(DEV), zc)
        # the same kernels on the same inputs: the same bits
        for k in ("loss", "z_loss", "n_valid", "status", "dlogits"):
            assert torch.equal(a[k], b[k]), (T, k)
        assert b["status"].item() == 1


def test_noalloc_rejects_above_limit(gpu):
    # more rows than the library's array holds: refused on the host, nothing launched
    mx = 1048576
    z = torch.empty((mx + 1, 1), dtype=torch.bfloat16, device=DEV)
    t = torch.zeros(mx + 1, dtype=torch.int64, device=DEV)
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        gpu.fo_xent_fwd_bwd_noalloc(z, t)
