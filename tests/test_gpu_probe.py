"""moe_lds_probe: every kind alone and the direct-to-LDS loads beside each
kind of read run to completion with plausible rates (benchmark support; it
computes nothing that is checked)."""
import math

import pytest

from mixture_experts_layer_permute_amd import lds_probe

pytestmark = pytest.mark.gpu


def test_lds_probe_runs_every_kind():
    print("lds_probe", flush=True)
    res = lds_probe.run(iters=200, reps=3, src_kb=256)
    assert set(res) == set(lds_probe.MODES)
    for mode, (rates, ratio) in res.items():
        # side by side the kinds take about the longer one's time alone or
        # more, at most about the sum of both (short runs: loose bounds)
        assert ratio is None or 0.5 < ratio < 3.0, (mode, ratio)
        assert len(rates) == bin(mode & 7).count("1")
        for kind, r in rates.items():
            # per compute unit: above 1 byte per ns, below 512 B per cycle at 4 GHz
            assert math.isfinite(r) and 1.0 < r < 2048.0, (mode, kind, r)
