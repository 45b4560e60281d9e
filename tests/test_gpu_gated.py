"""GPU parity of the gated (decayed) linear layer against the fp64 oracle,
through the C ABI: S <- exp(g) S + k (x) v per token, chunked prefill with
per-chunk cumulative gates, decode, and the hybrid step with gated layers.

Pages cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2) §1.3
(Mamba- and RWKV-style state layers) and §2.4 (chunked prefill carries the
state); "Hybrid Model推理适配：vLLM与SGLang的工程实践指南" (P1) §2.1 (a state
carried as h_t = f(h_{t-1}, x_t)).
"""
import numpy as np
import pytest

import synth
from oracle import ref
from synth import hybrid
from tests import gpu_util as gu
from tests import hybrid_run
from tests.test_gpu_linear import Pool
from tests.test_gpu_linear import _prefill as _plain_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hy():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from linear_attention_attn_amd import hyattn
    hyattn.load()
    return hyattn


def _dt(hy, dtype):
    return hy.BF16 if dtype == "bf16" else hy.F32


def _gated_prefill(hy, pool, layer, q, k, v, g, cu, slots, chunk, dtype):
    import torch
    dq, dk, dv = gu.dev(q), gu.dev(k), gu.dev(v)
    do = torch.full_like(dq, float("nan"))
    hy.hyattn_linear_prefill_chunked_gated(pool.handle, layer, dq, dk, dv, gu.dev(g), do,
                                           gu.i32(cu), gu.i32(slots), len(slots), chunk,
                                           _dt(hy, dtype))
    torch.cuda.synchronize()
    return do


@pytest.mark.parametrize("dtype,D,chunk", [
    ("bf16", 128, 64), ("bf16", 128, 16), ("bf16", 128, 128), ("bf16", 128, 256),
    ("bf16", 128, 48), ("bf16", 64, 64), ("bf16", 64, 256), ("f32", 64, 40), ("f32", 128, 128),
    ("f32", 64, 1),
])
def test_gated_prefill_matches_oracle(hy, dtype, D, chunk):
    """Ragged requests (empty and single-token ones included) from non-zero prior
    states, with heads that forget fast and heads that forget slowly."""
    import torch
    rng = np.random.default_rng(300 + chunk + D)
    H = 8
    lens = [1, 77, 0, 300, 16]
    cu = synth.cu_lens(lens)
    N = int(cu[-1])
    q, k, v = (synth.normal(rng, (N, H, D), D ** -0.5, dtype) for _ in range(3))
    g = synth.log_forget(rng, (N, H))
    pool = Pool(hy, 1, 8, H, D)
    slots = pool.alloc(len(lens))
    slots = [slots[i] for i in (3, 0, 4, 1, 2)]
    S0 = (rng.standard_normal((len(lens), H, D, D)) * 0.1).astype(np.float32)
    for r, s in enumerate(slots):
        pool.view[0, s] = torch.from_numpy(S0[r]).cuda()
    do = _gated_prefill(hy, pool, 0, q, k, v, g, cu, slots, chunk, dtype)
    st = S0.astype(np.float64)
    want = ref.linear_prefill(q, k, v, cu, st, chunk=chunk, log_gamma=g)
    gu.assert_io(gu.host(do), want, dtype, f"gated prefill out C={chunk}")
    got_S = np.stack([gu.host(pool.view[0, s]) for s in slots])
    gu.assert_f32(got_S, st, f"gated prefill states C={chunk}")
    pool.close()


@pytest.mark.parametrize("D,chunk", [(128, 64), (64, 256)])
def test_gated_prefill_strong_forgetting(hy, D, chunk):
    """Forget factors down to 0.01 (the decay across one chunk spans far more
    than fp32's range) on half the heads, mixed with slow heads: the kernel's
    per-score path for such chunks, and exact zeros of exp where the oracle
    underflows too."""
    import torch
    rng = np.random.default_rng(500 + D)
    H = 4
    lens = [200, 33]
    cu = synth.cu_lens(lens)
    N = int(cu[-1])
    q, k, v = (synth.normal(rng, (N, H, D), D ** -0.5, "bf16") for _ in range(3))
    g = synth.log_forget(rng, (N, H))
    g[:, ::2] = np.log(rng.uniform(0.01, 1.0, (N, (H + 1) // 2))).astype(np.float32)
    pool = Pool(hy, 1, 2, H, D)
    slots = pool.alloc(2)
    pool.zero(slots)
    do = _gated_prefill(hy, pool, 0, q, k, v, g, cu, slots, chunk, "bf16")
    st = np.zeros((2, H, D, D))
    want = ref.linear_prefill(q, k, v, cu, st, chunk=chunk, log_gamma=g)
    gu.assert_io(gu.host(do), want, "bf16", f"strong gates C={chunk}")
    gu.assert_f32(np.stack([gu.host(pool.view[0, s]) for s in slots]), st, "strong gates states")
    pool.close()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_gated_decode_matches_oracle(hy, dtype, D):
    import torch
    rng = np.random.default_rng(400 + D)
    B, H, steps = 5, 8, 3
    pool = Pool(hy, 1, 8, H, D)
    slots = pool.alloc(B)[::-1]
    S0 = (rng.standard_normal((B, H, D, D)) * 0.1).astype(np.float32)
    for r, s in enumerate(slots):
        pool.view[0, s] = torch.from_numpy(S0[r]).cuda()
    st = S0.astype(np.float64)
    for step in range(steps):
        q, k, v = (synth.normal(rng, (B, H, D), D ** -0.5, dtype) for _ in range(3))
        g = synth.log_forget(rng, (B, H))
        dq = gu.dev(q)
        do = torch.full_like(dq, float("nan"))
        hy.hyattn_linear_decode_gated(pool.handle, 0, dq, gu.dev(k), gu.dev(v), gu.dev(g), do,
                                      gu.i32(slots), B, _dt(hy, dtype))
        torch.cuda.synchronize()
        want = ref.linear_decode(q, k, v, st, log_gamma=g)
        gu.assert_io(gu.host(do), want, dtype, f"gated decode step {step}")
    gu.assert_f32(np.stack([gu.host(pool.view[0, s]) for s in slots]), st, "gated decode states")
    pool.close()


@pytest.mark.parametrize("gated,dtype,D", [(False, "bf16", 128), (True, "bf16", 128),
                                           (True, "f32", 64)])
def test_decode_large_batch(hy, gated, dtype, D):
    """B x H = 4352 (request, head) units: the decode splits each state over 4 workgroups
    (column slices) from 4096 units on. Sampled units against the oracle, outputs and
    states."""
    import torch
    rng = np.random.default_rng(410 + D + int(gated))
    B, H = 136, 32
    pool = Pool(hy, 1, B, H, D)
    slots = pool.alloc(B)[::-1]
    g0 = torch.Generator(device="cuda")
    g0.manual_seed(411)
    pool.view.normal_(0.0, 0.1, generator=g0)
    units = [(int(r), int(h)) for r, h in zip(rng.integers(0, B, 24), rng.integers(0, H, 24))]
    units = sorted(set(units))
    st = np.zeros((B, H, D, D))
    for r, h in units:
        st[r, h] = gu.host(pool.view[0, slots[r], h]).astype(np.float64)
    q, k, v = (synth.normal(rng, (B, H, D), D ** -0.5, dtype) for _ in range(3))
    g = synth.log_forget(rng, (B, H)) if gated else None
    dq = gu.dev(q)
    do = torch.full_like(dq, float("nan"))
    if gated:
        hy.hyattn_linear_decode_gated(pool.handle, 0, dq, gu.dev(k), gu.dev(v), gu.dev(g), do,
                                      gu.i32(slots), B, _dt(hy, dtype))
    else:
        hy.hyattn_linear_decode(pool.handle, 0, dq, gu.dev(k), gu.dev(v), do, gu.i32(slots), B,
                                _dt(hy, dtype))
    torch.cuda.synchronize()
    want = ref.linear_decode(q, k, v, st, units=units, log_gamma=g)
    got = gu.host(do)
    idx = tuple(np.array(units).T)
    gu.assert_io(got[idx], want[idx], dtype, "large-batch decode outputs")
    gu.assert_f32(np.stack([gu.host(pool.view[0, slots[r], h]) for r, h in units]),
                  np.stack([st[r, h] for r, h in units]), "large-batch decode states")
    pool.close()


def test_zero_gates_reproduce_the_plain_layer_bit_for_bit(hy):
    """g = 0 multiplies by exactly 1 and adds exact zeros (the lo half of the
    weighted values), so the gated kernels must give the plain ones' bits."""
    import torch
    rng = np.random.default_rng(17)
    for dtype, D, chunk in (("bf16", 128, 128), ("bf16", 64, 32), ("f32", 64, 24)):
        H, lens = 4, [5, 130, 64]
        cu = synth.cu_lens(lens)
        N = int(cu[-1])
        q, k, v = (synth.normal(rng, (N, H, D), D ** -0.5, dtype) for _ in range(3))
        g = np.zeros((N, H), np.float32)
        pool = Pool(hy, 2, 4, H, D)
        slots = pool.alloc(3)
        S0 = torch.from_numpy((rng.standard_normal((3, H, D, D)) * 0.1).astype(np.float32)).cuda()
        for li in range(2):
            for r, s in enumerate(slots):
                pool.view[li, s] = S0[r]
        rows = cu[:-1]  # one decode token per request: the first of each prompt
        a = gu.host(_gated_prefill(hy, pool, 0, q, k, v, g, cu, slots, chunk, dtype))
        b = gu.host(_plain_prefill(hy, pool, 1, q, k, v, cu, slots, chunk, dtype))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (dtype, D, chunk)
        assert torch.equal(pool.view[0], pool.view[1])
        dq, dk, dv = (gu.dev(x[rows]) for x in (q, k, v))
        oa, ob = torch.empty_like(dq), torch.empty_like(dq)
        hy.hyattn_linear_decode_gated(pool.handle, 0, dq, dk, dv, gu.dev(g[rows]), oa,
                                      gu.i32(slots), 3, _dt(hy, dtype))
        hy.hyattn_linear_decode(pool.handle, 1, dq, dk, dv, ob, gu.i32(slots), 3, _dt(hy, dtype))
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int16) if dtype == "bf16" else oa,
                           ob.view(torch.int16) if dtype == "bf16" else ob)
        assert torch.equal(pool.view[0], pool.view[1])
        pool.close()


def test_gated_hybrid_step_matches_oracle():
    case = hybrid.small_case(seed=41, gated=True, n_layers=8, prefill_lens=(1, 130, 16),
                             decode_ctx=(2, 600, 33, 1), chunk=64)
    got = hybrid_run.run_gpu(case)
    want = hybrid_run.run_oracle(case)
    hybrid_run.compare(case, got, want)


def test_gated_two_steps_match_one_step_of_the_oracle():
    case = hybrid.continuation_case(seed=43, gated=True, prompts=((50, 49), (33, 1), (300, 128)),
                                    decode_prior=(1, 600), chunk=64)
    got = hybrid_run.run_gpu_steps(case)
    want = hybrid_run.run_oracle_whole(case)
    hybrid_run.compare(case, got, want)
