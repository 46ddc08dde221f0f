"""The shader-clock probe (fa_clock_probe, a measurement utility): its
counters advance and give a clock within the part's range."""
import pytest

pytestmark = pytest.mark.gpu


def test_clock_probe_gives_a_plausible_shader_clock():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    print("fa_clock_probe: 256 samples, sleep_units 1", flush=True)
    samples = torch.zeros((256, 2), dtype=torch.int64, device="cuda")
    fa.fa_clock_probe(samples, sleep_units=1)
    torch.cuda.synchronize()
    x = samples.cpu()
    assert bool((x[1:, 0] > x[:-1, 0]).all()) and bool((x[1:, 1] >= x[:-1, 1]).all())
    dt = int(x[-1, 0] - x[0, 0])
    dr = int(x[-1, 1] - x[0, 1])
    assert dr > 0
    mhz = dt / dr * 100.0
    print(f"  shader clock {mhz:.0f} MHz over {dr / 100.0:.0f} us", flush=True)
    assert 100.0 <= mhz <= 3000.0
    with pytest.raises(ValueError):
        fa.fa_clock_probe(torch.zeros((4, 3), dtype=torch.int64, device="cuda"))
