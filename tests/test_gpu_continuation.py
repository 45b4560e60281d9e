"""A request's tokens served over two hybrid steps against the oracle's one
step over all of them: chunked prefill with earlier context, and decode that
carries on from it.

Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2) §2.4
(chunked prefill: full layers keep K/V between chunks, linear layers keep
their state, and every layer of a request cuts at the same boundary).
The first step of each prompt ends at split[r]; the second step brings the
rest with context_len = all tokens so far. Outputs, final linear states and
pools must match the oracle's single step over the whole prompt.
"""
import pytest

from synth import hybrid
from tests import hybrid_run

pytestmark = pytest.mark.gpu

CASES = [
    dict(),                                                   # bf16, [lin,lin,lin,full], D=128
    dict(prompts=((50, 49), (33, 1), (300, 128), (48, 16)),   # 1-token steps, block/chunk edges
         decode_prior=(1, 600), n_layers=8, H=8, Hkv=2, chunk=64),
    dict(prompts=((400, 150),), decode_prior=(), D=64, chunk=16),
    dict(dtype="f32", D=64, H=4, Hkv=4, prompts=((100, 37),), decode_prior=(5,), chunk=40,
         n_layers=2, pattern=("linear", "full")),
]


@pytest.mark.parametrize("kw", CASES)
def test_two_steps_match_one_step_of_the_oracle(kw):
    case = hybrid.continuation_case(seed=11 + len(str(kw)), **kw)
    got = hybrid_run.run_gpu_steps(case)
    want = hybrid_run.run_oracle_whole(case)
    hybrid_run.compare(case, got, want)
