"""The calibration loops behind the bench's attainable-rate figures run through the C ABI
and leave finite, deterministic outputs (their rates are measured by bench.py, not here)."""

import pytest
import torch

from exact_attention_78_amd import _binding, attn_calibrate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", list(_binding.CALIBRATION_KINDS))
def test_calibration_loop_runs(kind):
    out, ops = attn_calibrate(kind, 16, 4)
    first = out.clone()
    attn_calibrate(kind, 16, 4, out=out)
    torch.cuda.synchronize()
    assert ops > 0
    assert bool(torch.isfinite(out).all())
    assert torch.equal(first, out)
