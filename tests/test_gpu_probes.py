"""The measurement probes run to completion and report sane counters."""
import pytest

torch = pytest.importorskip("torch")

from qlora_fine_tuning_amd import lora  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", range(8))
def test_mfma_issue_probe_modes(mode):
    blocks, iters = 4, 8
    out = lora.lora_probe_mfma_issue(mode, blocks, iters)
    torch.cuda.synchronize()
    o = out.cpu()
    assert o.shape == (blocks * 4, 3)
    cycles, ticks = o[:, 0], o[:, 1]
    assert bool((ticks > 0).all())
    # at least 8 cycles per 16x16x32 MFMA (the matrix core's own issue rate is about 16)
    assert bool((cycles >= 8 * 128 * iters).all())


def test_mfma_ceiling_probe():
    out = lora.lora_probe_mfma(4, 8)
    torch.cuda.synchronize()
    o = out.cpu()
    assert bool((o[:, 1] > 0).all()) and bool((o[:, 0] >= 8 * 64 * 8).all())
