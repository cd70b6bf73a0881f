"""pa_clock_probe (a measurement aid beside the attention path): every wave
reports a shader clock in the range a gfx950 part runs at, and the host checks
reject bad arguments before launching."""

import pytest
import torch

import paged_kv_cache_amd as pa


@pytest.mark.gpu
def test_clock_probe_reports_a_plausible_clock():
    ghz = pa.clock_probe(4096, 5000)
    torch.cuda.synchronize()
    assert bool((ghz > 0.3).all()) and bool((ghz < 3.0).all()), ghz.min().item()
    med = float(ghz.median())
    assert 0.8 < med < 2.6, med


def test_clock_probe_host_checks():
    lib = pa.load()
    assert lib.pa_clock_probe(None, 0, 10, None) == 0
    assert lib.pa_clock_probe(None, 4, 10, None) == -1
    assert lib.pa_clock_probe(None, -1, 10, None) == -2
    assert lib.pa_clock_probe(None, 4, -1, None) == -2
