"""The measurement probes the bench states its ceilings with: the copy probe copies
exactly, and the MFMA probe runs and leaves finite wave sums."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_copy_probe_exact(gpu):
    g = torch.Generator(device="cpu").manual_seed(3)
    for n in (4, 1000, 1 << 20, (1 << 20) + 12):
        src = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, generator=g).cuda()
        dst = torch.zeros_like(src)
        gpu.fo_probe_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst, src), n


def test_mfma_probe_runs(gpu):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.full((n_cu * 8,), float("nan"), device="cuda")
    flops = gpu.fo_probe_mfma(n_cu, 100, out)
    torch.cuda.synchronize()
    assert flops == n_cu * 8 * 100 * 4 * 32768
    assert torch.isfinite(out).all()
