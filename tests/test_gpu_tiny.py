"""The tiny workload end to end, fp32, seed 0: one request's 256-token prompt,
prefilled in 64-token chunks, then 16 decode steps of that same request, on one
linear layer (H = 4, D = 64) and one full layer of the same H and D whose KV
lives in a shuffled 32-block pool (17 blocks used, 15 spare blocks NaN).

Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2):
§2.1 (the linear recurrence, 16-token pages behind a block table), §2.3 (the
state is zeroed once at request start, accumulated by prefill and then read
and updated by decode; decode attention over the cached KV), §2.4 (chunked
prefill carries the state), §3.5 (the same prompt at growing length stays
consistent) and §4.1 (decode must carry on from the prefilled state, not
re-zero it). Every output, the state after the prefill and after each
decode, and the pools after every append are checked against the oracle
(fp32 rule, 1e-4; pools bit for bit).
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


def test_tiny_linear_layer_prefill_then_16_decodes(hy):
    import torch
    t = synth.tiny_inputs()
    cfg = t["cfg"]
    H, D, T, C, nd = cfg["H"], cfg["D"], cfg["T"], cfg["chunk"], cfg["n_decode"]
    q, k, v = (t["linear"][x] for x in ("q", "k", "v"))
    nbytes = hy.hyattn_state_pool_bytes(1, 1, H, D)
    buf = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    pool = hy.hyattn_state_pool_create(buf, nbytes, 1, 1, H, D)
    slots = hy.hyattn_state_pool_alloc(pool, 1)
    sl = gu.i32(slots)
    hy.hyattn_state_pool_zero(pool, sl, 1)  # request start, the only zeroing
    view = buf.view(H, D, D)
    dq, dk, dv = gu.dev(q), gu.dev(k), gu.dev(v)
    do = torch.full_like(dq, float("nan"))
    hy.hyattn_linear_prefill_chunked(pool, 0, dq[:T], dk[:T], dv[:T], do[:T], gu.i32([0, T]), sl,
                                     1, C, hy.F32)
    torch.cuda.synchronize()
    S = np.zeros((1, H, D, D))
    want = np.zeros((T + nd, H, D))
    want[:T] = ref.linear_prefill(q[:T], k[:T], v[:T], [0, T], S, chunk=C)
    gu.assert_f32(gu.host(view)[None], S, "state after the 256-token prefill")
    for step in range(nd):
        row = slice(T + step, T + step + 1)
        hy.hyattn_linear_decode(pool, 0, dq[row], dk[row], dv[row], do[row], sl, 1, hy.F32)
        torch.cuda.synchronize()
        want[row] = ref.linear_decode(q[row], k[row], v[row], S)
        gu.assert_f32(gu.host(do[row]), want[row], f"decode step {step} output")
        gu.assert_f32(gu.host(view)[None], S, f"state after decode step {step}")
    got = gu.host(do)
    gu.assert_f32(got, want, "all 272 outputs")
    # the same outputs as the token recurrence over the whole sequence (P2 §3.5)
    S_rec = np.zeros((1, H, D, D))
    rec = ref.linear_prefill(q, k, v, [0, T + nd], S_rec, form="recurrent")
    gu.assert_f32(got, rec, "against the recurrence over all 272 tokens")
    hy.hyattn_state_pool_destroy(pool)


def test_tiny_full_layer_prefill_then_16_decodes(hy):
    import torch
    t = synth.tiny_inputs()
    cfg = t["cfg"]
    H, D, T, nd = cfg["H"], cfg["D"], cfg["T"], cfg["n_decode"]
    q, k, v = (t["full"][x] for x in ("q", "k", "v"))
    lay = t["layout"]
    bt = lay.block_tables
    scale = D ** -0.5
    kp_ref, vp_ref = t["k_pool"].copy(), t["v_pool"].copy()
    dkp, dvp = gu.dev(kp_ref), gu.dev(vp_ref)
    dbt = gu.i32(bt)
    dq = gu.dev(q)
    do = torch.full_like(dq, float("nan"))
    # prefill: append the prompt's K/V, causal attention of its 256 queries
    ctx, cu = np.array([T], np.int32), np.array([0, T], np.int32)
    hy.hyattn_paged_append(gu.dev(k[:T]), gu.dev(v[:T]), dkp, dvp, lay.n_blocks, dbt,
                           lay.max_blocks, gu.i32(ctx), gu.i32(cu), 1, T, H, D, hy.F32)
    hy.hyattn_paged_prefill(dq[:T], do[:T], dkp, dvp, lay.n_blocks, dbt, lay.max_blocks,
                            gu.i32(ctx), gu.i32(cu), T, 1, H, H, D, scale, hy.F32)
    torch.cuda.synchronize()
    kp_ref = ref.append_kv(kp_ref, k[:T], bt, ctx, cu)
    vp_ref = ref.append_kv(vp_ref, v[:T], bt, ctx, cu)
    assert np.array_equal(gu.host(dkp).view(np.uint32), kp_ref.view(np.uint32)), "K pool after prefill"
    assert np.array_equal(gu.host(dvp).view(np.uint32), vp_ref.view(np.uint32)), "V pool after prefill"
    want = np.zeros((T + nd, H, D))
    want[:T] = ref.paged_attention(q[:T], kp_ref, vp_ref, bt, ctx, cu, scale)
    gu.assert_f32(gu.host(do[:T]), want[:T], "prefill outputs")
    # 16 decode steps: append the new token, attend over ctx = 257 .. 272 keys
    ws_bytes = hy.hyattn_paged_decode_workspace_bytes(1, H, D, T + nd)
    ws = torch.full((max(ws_bytes, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    one = np.array([0, 1], np.int32)
    for step in range(nd):
        row = slice(T + step, T + step + 1)
        ctx = np.array([T + step + 1], np.int32)
        hy.hyattn_paged_append(gu.dev(k[row]), gu.dev(v[row]), dkp, dvp, lay.n_blocks, dbt,
                               lay.max_blocks, gu.i32(ctx), gu.i32(one), 1, 1, H, D, hy.F32)
        hy.hyattn_paged_decode(dq[row], do[row], dkp, dvp, lay.n_blocks, dbt, lay.max_blocks,
                               gu.i32(ctx), int(ctx[0]), 1, H, H, D, scale, ws, ws_bytes, hy.F32)
        torch.cuda.synchronize()
        kp_ref = ref.append_kv(kp_ref, k[row], bt, ctx, one)
        vp_ref = ref.append_kv(vp_ref, v[row], bt, ctx, one)
        want[row] = ref.paged_attention(q[row], kp_ref, vp_ref, bt, ctx, one, scale)
        gu.assert_f32(gu.host(do[row]), want[row], f"decode step {step} (ctx {int(ctx[0])})")
    assert np.array_equal(gu.host(dkp).view(np.uint32), kp_ref.view(np.uint32)), "K pool at the end"
    assert np.array_equal(gu.host(dvp).view(np.uint32), vp_ref.view(np.uint32)), "V pool at the end"
    spare = lay.spare.astype(np.int64)
    assert np.isnan(gu.host(dkp)[spare]).all() and np.isnan(gu.host(dvp)[spare]).all(), \
        "spare blocks untouched"
    gu.assert_f32(gu.host(do), want, "all 272 outputs")
    # each query attends to every earlier token of the request, whether it came in
    # the prompt or in a decode step: one causal pass over all 272 tokens agrees
    whole = ref.paged_attention(q, kp_ref, vp_ref, bt, [T + nd], [0, T + nd], scale)
    gu.assert_f32(gu.host(do), whole, "against one causal pass over all 272 tokens")


def test_tiny_through_the_hybrid_step(hy):
    """The same two layers as one [linear, full] model through hyattn_hybrid_step: a
    prefill step of the prompt, then 16 decode steps of the same request."""
    import torch
    from linear_attention_attn_amd import layer_types
    t = synth.tiny_inputs()
    cfg = t["cfg"]
    H, D, T, C, nd = cfg["H"], cfg["D"], cfg["T"], cfg["chunk"], cfg["n_decode"]
    lay = t["layout"]
    bt = lay.block_tables
    scale = D ** -0.5
    types = layer_types.parse(["linear", "full"])
    nbytes = hy.hyattn_state_pool_bytes(1, 1, H, D)
    buf = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    pool = hy.hyattn_state_pool_create(buf, nbytes, 1, 1, H, D)
    slots = hy.hyattn_state_pool_alloc(pool, 1)
    sl = gu.i32(slots)
    hy.hyattn_state_pool_zero(pool, sl, 1)
    lin = {x: gu.dev(t["linear"][x]) for x in ("q", "k", "v")}
    lin["o"] = torch.full_like(lin["q"], float("nan"))
    full = {x: gu.dev(t["full"][x]) for x in ("q", "k", "v")}
    full["o"] = torch.full_like(full["q"], float("nan"))
    dkp, dvp = gu.dev(t["k_pool"]), gu.dev(t["v_pool"])
    ws_bytes = hy.hyattn_paged_decode_workspace_bytes(1, H, D, T + nd)
    ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device="cuda")
    dbt = gu.i32(bt)

    def step(rows, n_prefill, ctx):
        io = [{x: lin[x][rows] for x in ("q", "k", "v", "o")},
              dict({x: full[x][rows] for x in ("q", "k", "v", "o")}, k_pool=dkp, v_pool=dvp)]
        n = rows.stop - rows.start
        cu = gu.i32([0, n])
        batch = hy.make_batch(
            n_prefill=n_prefill, n_decode=1 - n_prefill, cu_seqlens=cu if n_prefill else None,
            n_prefill_tokens=n if n_prefill else 0, max_prefill_len=n if n_prefill else 0,
            prefill_slots=sl if n_prefill else None, decode_slots=None if n_prefill else sl,
            block_tables=dbt, max_blocks_per_seq=lay.max_blocks, context_lens=gu.i32([ctx]),
            cu_q_lens=cu, max_context=ctx, n_blocks=lay.n_blocks, H=H, H_kv=H, D=D,
            chunk_size=C, scale=scale, dtype=hy.F32, workspace=ws, workspace_bytes=ws_bytes)
        hy.hyattn_hybrid_step(types, 2, io, batch, pool)

    step(slice(0, T), 1, T)
    for s in range(nd):
        step(slice(T + s, T + s + 1), 0, T + s + 1)
    torch.cuda.synchronize()
    S = np.zeros((1, H, D, D))
    q, k, v = (t["linear"][x] for x in ("q", "k", "v"))
    want_lin = ref.linear_prefill(q, k, v, [0, T + nd], S, form="recurrent")
    gu.assert_f32(gu.host(lin["o"]), want_lin, "linear layer, 272 outputs")
    gu.assert_f32(gu.host(buf.view(H, D, D))[None], S, "linear state after 16 decodes")
    kp_ref = ref.append_kv(t["k_pool"], t["full"]["k"], bt, [T + nd], [0, T + nd])
    vp_ref = ref.append_kv(t["v_pool"], t["full"]["v"], bt, [T + nd], [0, T + nd])
    assert np.array_equal(gu.host(dkp).view(np.uint32), kp_ref.view(np.uint32)), "K pool"
    assert np.array_equal(gu.host(dvp).view(np.uint32), vp_ref.view(np.uint32)), "V pool"
    want_full = ref.paged_attention(t["full"]["q"], kp_ref, vp_ref, bt, [T + nd], [0, T + nd], scale)
    gu.assert_f32(gu.host(full["o"]), want_full, "full layer, 272 outputs")
    hy.hyattn_state_pool_destroy(pool)
