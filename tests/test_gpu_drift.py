"""Long-decode precision of the linear state (P2 §2.3, §4.1: a 16-bit state
drifts over long sequences, an fp32 one does not).

The library keeps states in fp32: over 4096 decode steps its outputs meet
the bf16 rule and its state the fp32 rule against the oracle's fp64
recurrence at every checkpoint. The same run with the state rounded to bf16
after every step (the storage the pages warn about) must come out far less
accurate, which confirms that the comparison can see the difference.
"""
import pytest

from tests import drift_study
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gated", [False, True])
def test_fp32_state_does_not_drift_over_long_decodes(gated):
    res = drift_study.run(T=4096, B=2, H=2, D=128, seed=7, gated=gated, arms=("fp32", "bf16"))
    for t, om, oa, sm, sf in res["fp32"]:
        assert om <= gu.TOL_BF16_MAX and oa <= gu.TOL_BF16_MEAN, (t, om, oa)
        assert sm <= gu.TOL_F32, (t, sm)
    t, _, _, sm32, sf32 = res["fp32"][-1]
    _, _, _, sm16, sf16 = res["bf16"][-1]
    assert sf16 > 20 * sf32, (sf16, sf32)
