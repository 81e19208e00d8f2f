"""Pin of the oracle's loss-scale rule against an independent implementation:
torch's dynamic loss-scale update (the operator behind torch.amp.GradScaler),
run on the CPU.

The tutorial (§4.3) only says fp16 training may need loss scaling; the oracle
reads it as the usual dynamic rule: halve the scale on a step with inf/NaN
(and skip it), double it after `growth_interval` clean steps in a row.  torch
keeps the same two numbers (scale and the clean-step counter), so random
sequences of skipped and applied steps must give equal scales and counters
after every step.  The oracle's floor (the scale never drops below
`min_scale`) has no torch counterpart; it is a stated reading, checked on its
own at the end.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _torch_rule(scale: float, good: int, skipped: bool, interval: int):
    s = torch.tensor([scale], dtype=torch.float32)
    g = torch.tensor([good], dtype=torch.int32)
    inf = torch.tensor([1.0 if skipped else 0.0], dtype=torch.float32)
    torch._amp_update_scale_(s, g, inf, 2.0, 0.5, interval)
    return float(s[0]), int(g[0])


@pytest.mark.parametrize("interval", [1, 2, 7, 1000])
def test_scaler_rule_equals_torch(interval):
    rng = np.random.default_rng(interval)
    for p_skip in (0.0, 0.01, 0.2, 0.5):
        scale, good = 65536.0, 0
        ts, tg = scale, good
        for _ in range(3000):
            skipped = bool(rng.random() < p_skip)
            scale, good = oracle.scaler_update(scale, good, skipped, growth_interval=interval)
            ts, tg = _torch_rule(ts, tg, skipped, interval)
            if scale <= 1.0 or scale >= 2.0**100:
                break  # the oracle's floor, or beyond fp32's comfortable range
            assert (scale, good) == (ts, tg), (interval, p_skip)


def test_scaler_floor_reading():
    # not pinned by torch: the scale stops halving at min_scale
    scale, good = 4.0, 0
    for _ in range(5):
        scale, good = oracle.scaler_update(scale, good, True)
    assert scale == 1.0 and good == 0
