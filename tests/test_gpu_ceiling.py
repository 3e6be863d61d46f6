"""The ceiling probe (moe_ceiling_probe) on the GPU: every thread's observable result is the
value its kernel must produce, and the reported work and time are consistent."""
import pytest

torch = pytest.importorskip("torch")
from mixture_experts_layer_histogram_amd import moe  # noqa: E402

pytestmark = pytest.mark.gpu


def _scratch():
    n = moe.moe_ceiling_probe_bytes()
    assert n > 0
    return torch.zeros(n // 4, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("kind,per_rep,flop", [(0, 16.0, 32 * 32 * 16 * 2), (1, 64.0, 32 * 32 * 64 * 2)])
def test_mfma_probe_accumulates_exactly(kind, per_rep, flop):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    scr = _scratch()
    reps = 1000
    rc, work, ms = moe.moe_ceiling_probe(kind, reps, None, 0, scr)
    torch.cuda.synchronize()
    out = scr[:cus * 256].view(torch.float32)
    assert torch.all(out == per_rep * reps), out.unique()[:8]
    assert work == cus * 4 * reps * 8 * flop
    assert ms > 0


@pytest.mark.parametrize("kind", [2, 3])
def test_fill_probe_lands_the_predicted_words(kind):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    share_words = 4 * 65536 // 4                     # 4 rounds of 64 KiB per workgroup
    src = torch.arange(cus * share_words, dtype=torch.int32, device="cuda")
    scr = _scratch()
    rc, work, ms = moe.moe_ceiling_probe(kind, 1, src, src.numel() * 4, scr)
    torch.cuda.synchronize()
    out = scr.view(cus, 512).cpu()
    b = torch.arange(cus).view(-1, 1)
    t = torch.arange(512).view(1, -1)
    if kind == 2:           # last of the 4 rounds of its own share
        want = b * share_words + 3 * 16384 + t
        assert work == cus * 4 * 65536
    else:                   # its window, 16 rounds
        want = (b & 15) * 16384 + t
        assert work == cus * 16 * 65536
    assert torch.equal(out, want.to(torch.int32))
    assert ms > 0


def test_fill_probe_rejects_a_short_source():
    scr = _scratch()
    src = torch.zeros(1024, dtype=torch.int32, device="cuda")
    assert moe.moe_ceiling_probe(2, 1, src, src.numel() * 4, scr, check=False)[0] == -3
    assert moe.moe_ceiling_probe(3, 1, src, src.numel() * 4, scr, check=False)[0] == -3
