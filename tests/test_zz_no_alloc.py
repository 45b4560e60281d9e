"""The allocation-free decode entry point (hyattn_paged_decode_noalloc) against
hyattn_paged_decode with a caller workspace: the same kernels and partition
plan, so the outputs must agree bit for bit. Two calls in a row, the second
with a smaller batch and shorter contexts (the scratch array keeps the first
call's contents), plus the oracle on sampled requests, and a call that needs
more scratch than the array holds, refused before any launch.

Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2) §2.1
(16-token blocks behind a block table) and §2.3 (PagedAttention decode).
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


def _case(seed, B, lo, hi, Hq, Hkv, D):
    import torch
    rng = np.random.default_rng(seed)
    ctx = synth.uniform_contexts(rng, B, lo, hi)
    lay = synth.paged_layout(rng, ctx, n_spare=3)
    kp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "bf16")
    vp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "bf16")
    for b in lay.spare:  # blocks no request uses hold NaN
        kp[b] = synth.BF16_NAN
        vp[b] = synth.BF16_NAN
    q = synth.normal(rng, (B, Hq, D), 1.0, "bf16")
    return dict(ctx=ctx, lay=lay, kp=kp, vp=vp, q=q, dkp=gu.dev(kp), dvp=gu.dev(vp), dq=gu.dev(q),
                bt=gu.i32(lay.block_tables), dctx=gu.i32(ctx))


def _both(hy, c, Hq, Hkv, D):
    import torch
    B, lay, maxc = len(c["ctx"]), c["lay"], int(c["ctx"].max())
    scale = D ** -0.5
    wsb = hy.hyattn_paged_decode_workspace_bytes(B, Hq, D, maxc)
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device="cuda")
    o_ws = torch.full_like(c["dq"], float("nan"))
    o_na = torch.full_like(c["dq"], float("nan"))
    hy.hyattn_paged_decode(c["dq"], o_ws, c["dkp"], c["dvp"], lay.n_blocks, c["bt"],
                           lay.max_blocks, c["dctx"], maxc, B, Hq, Hkv, D, scale, ws, wsb, hy.BF16)
    hy.hyattn_paged_decode_noalloc(c["dq"], o_na, c["dkp"], c["dvp"], lay.n_blocks, c["bt"],
                                   lay.max_blocks, c["dctx"], maxc, B, Hq, Hkv, D, scale, hy.BF16)
    torch.cuda.synchronize()
    return gu.host(o_ws), gu.host(o_na)


def test_noalloc_decode_matches_the_workspace_entry_point(hy):
    Hq, Hkv, D = 32, 8, 128
    # first call: long contexts, many partitions per request
    c1 = _case(61, 24, 3000, 40000, Hq, Hkv, D)
    a1, b1 = _both(hy, c1, Hq, Hkv, D)
    assert np.array_equal(a1, b1), "first call: outputs differ from the workspace entry point"
    # second call: fewer requests, short contexts (one partition each); the scratch
    # still holds the first call's partials
    c2 = _case(62, 7, 1, 900, Hq, Hkv, D)
    a2, b2 = _both(hy, c2, Hq, Hkv, D)
    assert np.array_equal(a2, b2), "second call: outputs differ from the workspace entry point"
    # and both against the oracle on sampled requests (the bf16 rule and rounding floor)
    for c, got in ((c1, b1), (c2, b2)):
        samp = [0, len(c["ctx"]) - 1]
        cu = np.arange(len(samp) + 1)
        want = ref.paged_attention(c["q"][samp], c["kp"], c["vp"], c["lay"].block_tables[samp],
                                   c["ctx"][samp], cu, D ** -0.5)
        delta = gu.attention_delta(c["q"][samp], c["kp"], c["vp"], c["lay"].block_tables[samp],
                                   c["ctx"][samp], cu, D ** -0.5, want)
        gu.assert_bf16(got[samp], want, "allocation-free decode", delta)


def test_noalloc_decode_refuses_more_than_its_scratch(hy):
    """A batch whose partials exceed the scratch array is refused before launching
    (outputs untouched)."""
    import torch
    Hq, Hkv, D = 32, 8, 128
    B, maxc = 512, 131072  # 512 x 32 x 32 partitions x 130 x 4 B = 272 MB > 64 MiB
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    pool = torch.zeros(1, Hkv, 16, D, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, maxc // 16, dtype=torch.int32, device="cuda")
    ctx = torch.full((B,), 16, dtype=torch.int32, device="cuda")
    with pytest.raises(hy.HyattnError) as e:
        hy.hyattn_paged_decode_noalloc(q, o, pool, pool, 1, bt, maxc // 16, ctx, maxc, B, Hq,
                                       Hkv, D, D ** -0.5, hy.BF16)
    assert e.value.status == hy.ERR_INVALID_ARG and "scratch" in e.value.message
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
