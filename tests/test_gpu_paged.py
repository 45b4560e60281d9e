"""GPU parity of the full-layer path (paged KV append, decode, causal prefill)
against the fp64 oracle, through the C ABI.

Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2):
§2.1 16-token blocks behind a page table, §2.3 PagedAttention decode and
FlashAttention-class prefill, §2.4 KV kept across prefill chunks.
Spare blocks and the unused tail of each request's last block are filled with
NaN, so any read of a token outside the context poisons the result.
"""
import numpy as np
import pytest

import synth
from oracle import ref
from tests import gpu_util as gu

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


def _poisoned_pools(rng, lay, Hkv, D, dtype, fill_ctx=None):
    """Pools with NaN everywhere except the first fill_ctx[r] logical tokens."""
    shape = (lay.n_blocks, Hkv, 16, D)
    nan = synth.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    kp = np.full(shape, nan, dtype=np.uint16 if dtype == "bf16" else np.float32)
    vp = kp.copy()
    fill = lay.context_lens if fill_ctx is None else fill_ctx
    for r, n in enumerate(fill):
        for j in range((int(n) + 15) // 16):
            b = lay.block_tables[r, j]
            m = min(16, int(n) - 16 * j)
            kp[b, :, :m] = synth.normal(rng, (Hkv, m, D), 1.0, dtype)
            vp[b, :, :m] = synth.normal(rng, (Hkv, m, D), 1.0, dtype)
    return kp, vp


def _decode(hy, q, kp, vp, lay, Hq, Hkv, D, scale, dtype, max_context=None):
    import torch
    B = q.shape[0]
    maxc = int(lay.context_lens.max()) if max_context is None else max_context
    wsb = hy.hyattn_paged_decode_workspace_bytes(B, Hq, D, maxc)
    ws = torch.empty(max(wsb, 4) // 4, dtype=torch.float32, device="cuda")
    ws.fill_(float("nan"))
    dq = gu.dev(q)
    do = torch.full_like(dq, float("nan"))
    hy.hyattn_paged_decode(dq, do, gu.dev(kp), gu.dev(vp), lay.n_blocks, gu.i32(lay.block_tables),
                           lay.max_blocks, gu.i32(lay.context_lens), maxc, B, Hq, Hkv, D, scale,
                           ws, wsb, _dt(hy, dtype))
    torch.cuda.synchronize()
    return gu.host(do)


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [
    ("bf16", 128, 8, 2), ("bf16", 128, 4, 4), ("bf16", 64, 8, 1), ("bf16", 128, 16, 2),
    ("f32", 64, 4, 4), ("f32", 128, 4, 2),
])
def test_decode_matches_oracle(hy, dtype, D, Hq, Hkv):
    rng = np.random.default_rng(300 + D + Hq)
    ctx = np.array([0, 1, 15, 16, 17, 513, 1500, 2049], np.int32)
    lay = synth.paged_layout(rng, ctx, n_spare=5)
    kp, vp = _poisoned_pools(rng, lay, Hkv, D, dtype)
    q = synth.normal(rng, (len(ctx), Hq, D), 1.0, dtype)
    scale = D ** -0.5
    got = _decode(hy, q, kp, vp, lay, Hq, Hkv, D, scale, dtype)
    cu = np.arange(len(ctx) + 1)
    want = ref.paged_attention(q, kp, vp, lay.block_tables, ctx, cu, scale)
    assert not gu.as_f64(got[0]).any(), "empty context gives zeros"
    delta = gu.attention_delta(q, kp, vp, lay.block_tables, ctx, cu, scale, want)
    gu.assert_io(got, want, dtype, "paged decode", delta)


def test_decode_many_partitions(hy):
    """A long context (many partitions) next to short ones; partition size grows with max_context."""
    rng = np.random.default_rng(301)
    D, Hq, Hkv = 128, 8, 2
    ctx = np.array([40000, 700, 33, 12345], np.int32)
    lay = synth.paged_layout(rng, ctx, n_spare=3)
    kp, vp = _poisoned_pools(rng, lay, Hkv, D, "bf16")
    q = synth.normal(rng, (len(ctx), Hq, D), 1.0, "bf16")
    got = _decode(hy, q, kp, vp, lay, Hq, Hkv, D, D ** -0.5, "bf16")
    cu = np.arange(len(ctx) + 1)
    want = ref.paged_attention(q, kp, vp, lay.block_tables, ctx, cu, D ** -0.5)
    delta = gu.attention_delta(q, kp, vp, lay.block_tables, ctx, cu, D ** -0.5, want)
    gu.assert_bf16(got, want, "paged decode, long contexts", delta)


def test_decode_work_scaled_partitions(hy):
    """A batch whose partition size comes from the work bound rather than from the longest
    context alone: B = 24 x H_kv = 8 pairs x 2000 blocks leaves 48-block partitions (the
    longest context alone would give 32, the floor's cap is 256). Sampled requests against
    the oracle."""
    rng = np.random.default_rng(302)
    D, Hq, Hkv = 128, 32, 8
    ctx = synth.uniform_contexts(rng, 24, 512, 32000)
    ctx[int(np.argmax(ctx))] = 32000
    lay = synth.paged_layout(rng, ctx, n_spare=2)
    kp, vp = _poisoned_pools(rng, lay, Hkv, D, "bf16")
    q = synth.normal(rng, (len(ctx), Hq, D), 1.0, "bf16")
    got = _decode(hy, q, kp, vp, lay, Hq, Hkv, D, D ** -0.5, "bf16")
    samp = sorted({int(np.argmax(ctx)), int(np.argmin(ctx)), 3, 17})
    cu = np.arange(len(samp) + 1)
    want = ref.paged_attention(q[samp], kp, vp, lay.block_tables[samp], ctx[samp], cu, D ** -0.5)
    delta = gu.attention_delta(q[samp], kp, vp, lay.block_tables[samp], ctx[samp], cu, D ** -0.5,
                               want)
    gu.assert_bf16(got[samp], want, "paged decode, work-scaled partitions", delta)


def test_decode_onehot_probe_bit_exact(hy):
    """q = 64 e0 against one key 64 e0 (others 0): the output is that token's value, exactly.

    Values encode the logical position; sweeping the target over positions pins the
    block-table address arithmetic bit for bit."""
    rng = np.random.default_rng(302)
    D, Hq, Hkv, n = 128, 4, 1, 1100
    lay = synth.paged_layout(rng, [n], n_spare=4)
    base_k = np.zeros((lay.n_blocks, Hkv, 16, D), np.float32)
    vp = np.zeros_like(base_k)
    for p in range(n):
        vp[lay.block_tables[0, p // 16], 0, p % 16, :] = p % 200 + 1
        vp[lay.block_tables[0, p // 16], 0, p % 16, 1] = p // 200
    q = np.zeros((1, Hq, D), np.float32)
    q[0, :, 0] = 64.0
    qb = synth.f32_to_bf16_bits(q)
    vb = synth.f32_to_bf16_bits(vp)
    for target in (0, 15, 16, 511, 512, 1023, 1099):
        kp = base_k.copy()
        kp[lay.block_tables[0, target // 16], 0, target % 16, 0] = 64.0
        got = _decode(hy, qb, synth.f32_to_bf16_bits(kp), vb, lay, Hq, Hkv, D, 1.0, "bf16")
        expect = np.full((Hq, D), target % 200 + 1, np.float32)
        expect[:, 1] = target // 200
        assert np.array_equal(got[0], synth.f32_to_bf16_bits(expect)), target


def test_decode_permutation_invariance(hy):
    """The same logical KV in two physical layouts gives bit-identical outputs."""
    rng = np.random.default_rng(303)
    D, Hq, Hkv = 128, 8, 2
    ctx = np.array([600, 37, 2000], np.int32)
    logical_k = synth.normal(rng, (3, 2000, Hkv, D), 1.0, "bf16")
    logical_v = synth.normal(rng, (3, 2000, Hkv, D), 1.0, "bf16")
    q = synth.normal(rng, (3, Hq, D), 1.0, "bf16")
    outs = []
    for seed in (1, 2):
        lay = synth.paged_layout(np.random.default_rng(seed), ctx, n_spare=2)
        kp = np.full((lay.n_blocks, Hkv, 16, D), synth.BF16_NAN, np.uint16)
        vp = kp.copy()
        for r in range(3):
            for p in range(int(ctx[r])):
                b = lay.block_tables[r, p // 16]
                kp[b, :, p % 16] = logical_k[r, p]
                vp[b, :, p % 16] = logical_v[r, p]
        outs.append(_decode(hy, q, kp, vp, lay, Hq, Hkv, D, D ** -0.5, "bf16"))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_bit_exact(hy, dtype):
    import torch
    rng = np.random.default_rng(304)
    D, Hkv = 128, 2
    ctx = np.array([5, 40, 16, 100], np.int32)
    qlen = [5, 3, 1, 60]
    cu = synth.cu_lens(qlen)
    lay = synth.paged_layout(rng, ctx, n_spare=3)
    kp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, dtype)
    vp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, dtype)
    kn = synth.normal(rng, (int(cu[-1]), Hkv, D), 1.0, dtype)
    vn = synth.normal(rng, (int(cu[-1]), Hkv, D), 1.0, dtype)
    dk, dv = gu.dev(kp), gu.dev(vp)
    hy.hyattn_paged_append(gu.dev(kn), gu.dev(vn), dk, dv, lay.n_blocks, gu.i32(lay.block_tables),
                           lay.max_blocks, gu.i32(ctx), gu.i32(cu), len(ctx), max(qlen), Hkv, D,
                           _dt(hy, dtype))
    torch.cuda.synchronize()
    assert np.array_equal(gu.host(dk), ref.append_kv(kp, kn, lay.block_tables, ctx, cu))
    assert np.array_equal(gu.host(dv), ref.append_kv(vp, vn, lay.block_tables, ctx, cu))


CHUNK_CASES = {  # (total context, first chunk) per request
    "short": ([150, 33, 64], [100, 16, 1]),
    "long": ([700, 33, 64], [300, 16, 1]),
    "empty": ([150, 40, 64], [100, 40, 1]),  # request 1 has no new token in the second chunk
}


@pytest.mark.parametrize("dtype,D,Hq,Hkv,case", [
    ("bf16", 128, 8, 2, "short"), ("f32", 64, 4, 4, "short"), ("bf16", 64, 4, 1, "short"),
    ("bf16", 128, 4, 4, "short"), ("bf16", 128, 16, 2, "short"), ("bf16", 64, 4, 2, "short"),
    ("bf16", 128, 8, 2, "long"), ("bf16", 128, 8, 2, "empty"), ("f32", 64, 4, 2, "empty")])
def test_prefill_two_chunks_matches_oracle(hy, dtype, D, Hq, Hkv, case):
    """Causal prefill in two chunks: the second attends to the first through the table.
    In the "empty" case one request brings no new token to the second chunk: its rows of
    the packed batch are absent and nothing of it may be written."""
    import torch
    rng = np.random.default_rng(305 + D + Hq)
    total = np.array(CHUNK_CASES[case][0], np.int32)
    first = np.array(CHUNK_CASES[case][1], np.int32)
    lay = synth.paged_layout(rng, total, n_spare=2)
    kp, vp = _poisoned_pools(rng, lay, Hkv, D, dtype, fill_ctx=np.zeros(3, np.int32))
    dkp, dvp = gu.dev(kp), gu.dev(vp)
    bt = gu.i32(lay.block_tables)
    scale = D ** -0.5
    kp_ref, vp_ref = kp.copy(), vp.copy()
    for stage, ctx in ((0, first), (1, total)):
        qlen = ctx - (first if stage else 0)
        cu = synth.cu_lens(qlen)
        N = int(cu[-1])
        q = synth.normal(rng, (N, Hq, D), 1.0, dtype)
        kn = synth.normal(rng, (N, Hkv, D), 1.0, dtype)
        vn = synth.normal(rng, (N, Hkv, D), 1.0, dtype)
        hy.hyattn_paged_append(gu.dev(kn), gu.dev(vn), dkp, dvp, lay.n_blocks, bt, lay.max_blocks,
                               gu.i32(ctx), gu.i32(cu), 3, int(qlen.max()), Hkv, D, _dt(hy, dtype))
        dq = gu.dev(q)
        do = torch.full_like(dq, float("nan"))
        hy.hyattn_paged_prefill(dq, do, dkp, dvp, lay.n_blocks, bt, lay.max_blocks, gu.i32(ctx),
                                gu.i32(cu), int(qlen.max()), 3, Hq, Hkv, D, scale, _dt(hy, dtype))
        torch.cuda.synchronize()
        kp_ref = ref.append_kv(kp_ref, kn, lay.block_tables, ctx, cu)
        vp_ref = ref.append_kv(vp_ref, vn, lay.block_tables, ctx, cu)
        want = ref.paged_attention(q, kp_ref, vp_ref, lay.block_tables, ctx, cu, scale)
        delta = gu.attention_delta(q, kp_ref, vp_ref, lay.block_tables, ctx, cu, scale, want)
        gu.assert_io(gu.host(do), want, dtype, f"paged prefill stage {stage}", delta)


def test_checked_mode_rejects_bad_block_ids(hy, monkeypatch):
    import torch
    monkeypatch.setenv("HYATTN_CHECK", "1")
    rng = np.random.default_rng(306)
    D, Hq, Hkv = 64, 2, 1
    lay = synth.paged_layout(rng, [40], n_spare=0)
    bt = lay.block_tables.copy()
    bt[0, 2] = lay.n_blocks  # out of range
    kp = torch.zeros(lay.n_blocks, Hkv, 16, D, device="cuda")
    q = torch.zeros(1, Hq, D, device="cuda")
    with pytest.raises(hy.HyattnError) as e:
        hy.hyattn_paged_decode(q, q, kp, kp, lay.n_blocks, gu.i32(bt), lay.max_blocks,
                               gu.i32([40]), 40, 1, Hq, Hkv, D, 1.0, None, 0, hy.F32)
    assert e.value.status == hy.ERR_INVALID_ARG
    torch.cuda.synchronize()
