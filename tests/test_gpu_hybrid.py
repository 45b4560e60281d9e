"""GPU parity of the whole per-layer hybrid step (hyattn_hybrid_step) against
the oracle's composition of the same layer operations.

Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2) §2.2
(layer types, split memory pools, per-forward metadata), §2.3 and §2.4.
"""
import numpy as np
import pytest

from synth import hybrid
from tests import hybrid_run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kw", [
    dict(),                                                        # bf16, [lin,lin,lin,full]
    dict(n_layers=8, prefill_lens=(1, 130, 16), decode_ctx=(2, 600, 33, 1), chunk=64),
    dict(dtype="f32", D=64, H=4, Hkv=4, prefill_lens=(256,), decode_ctx=(257,), chunk=64,
         n_layers=2, pattern=("linear", "full")),                  # the tiny fp32 case
    dict(prefill_lens=(), decode_ctx=(5, 900)),                    # decode only
    dict(prefill_lens=(33, 8), decode_ctx=()),
])
def test_hybrid_step_matches_oracle(kw):
    case = hybrid.small_case(seed=len(str(kw)), **kw)
    got = hybrid_run.run_gpu(case)
    want = hybrid_run.run_oracle(case)
    hybrid_run.compare(case, got, want)


def test_hybrid_step_slot_assignment_does_not_matter():
    case = hybrid.small_case(seed=5)
    B = case["n_prefill"] + case["n_decode"]
    a = hybrid_run.run_gpu(case)
    b = hybrid_run.run_gpu(case, slot_perm=list(reversed(range(B))))
    for x, y in zip(a[0], b[0]):
        assert np.array_equal(x, y)
