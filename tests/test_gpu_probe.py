"""The matrix-core probe behind the measured-clock peak: its counters run
forward, and the rate it reports cannot exceed what the reported clock
allows (4096 bf16 / 8192 fp8 flop per clock per CU), which catches a wrong
flop count; nor can it fall far below it on an idle chip."""
import pytest

from tests import gpu_support as gs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4],
                         ids=["bf16", "fp8", "fp8-8waves", "fp8-exp", "fp8-beside-exp"])
def test_probe_rate_and_counters(kind):
    import torch
    from block_sparse_video_map_amd import vsa
    cu, clk_khz, wall_khz = vsa.vsa_device_clocks()
    assert cu > 0 and clk_khz > 0 and wall_khz > 0
    n_wg, iters = 2 * cu, 4000
    ticks = torch.zeros(4 * n_wg, dtype=torch.int64, device="cuda")
    vsa.vsa_mfma_probe(kind, iters, n_wg)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    f = vsa.vsa_mfma_probe(kind, iters, n_wg, ticks)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    rate = f / (ms * 1e-3)
    limit = cu * clk_khz * 1e3 * (4096 if kind == 0 else 8192)
    gs.log(f"[probe] kind={kind}: {rate / 1e12:.1f} TFLOP/s, limit {limit / 1e12:.1f}, "
           f"{ms:.3f} ms")
    assert rate <= 1.02 * limit
    assert rate >= 0.25 * limit
    tk = ticks.view(n_wg, 4).cpu()
    assert bool((tk[:, 1] > tk[:, 0]).all()) and bool((tk[:, 3] > tk[:, 2]).all())


def test_probe_null_ticks_and_errors():
    from block_sparse_video_map_amd import vsa
    import torch
    vsa.vsa_mfma_probe(0, 1, 1)
    torch.cuda.synchronize()
    with pytest.raises(vsa.VSAError):
        vsa.vsa_mfma_probe(5, 1, 1)
