"""The micro-benchmark export runs and reports rates of the right magnitude:
each within a factor of two of what the part's published figures allow (dense
INT8 5.0 POPS, FP8 5.0 PFLOP/s, FP32 vector 157.3 TFLOP/s at 2.4 GHz).  AMD
publishes no v_exp_f32 rate; the reference here is half the FP32 lane rate,
256 CUs x 4 SIMDs x 8 results per clock, which a single wave's issue interval
of this instruction (8 to 9 clocks per 64 results, measured) implies."""
import pytest

import quantized_attention_03_amd as qa

pytestmark = pytest.mark.gpu

SPEC = {"i8": 5.0e15, "f8": 5.0e15, "fma": 157.3e12, "exp": 256 * 4 * 8 * 2.4e9}


@pytest.mark.parametrize("op", sorted(SPEC))
def test_micro_rate_is_near_the_published_rate(op):
    r = qa.sage_micro_rate(op, 1024)
    print(f"{op}: {r:.4g} per s ({r / SPEC[op]:.3f} of the published rate)")
    assert SPEC[op] / 2 < r < SPEC[op] * 2
