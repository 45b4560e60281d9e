"""GPU parity at full workload sizes, on sampled outputs the oracle computes unit
by unit, plus properties that hold at any size.

Workloads (seeded, synthetic; recipes in synth.WORKLOADS):
  * linear decode batch: B=64, H=32, D=128, 256 decode steps from prior states
    ~ N(0,1)*0.1, bf16 q/k/v;
  * linear chunked prefill: B=8, H=32, D=128, T=8192, chunk sizes 64/128/256,
    from a zeroed state; each chunk size against the oracle's sums at that size,
    and the kernel's outputs the same bits at every chunk size;
  * paged decode: B=128, H_q=32, H_kv=8, D=128, contexts uniform in
    [512, 32768], 16-token blocks in a randomly permuted pool with 1024
    NaN-poisoned spare blocks;
  * the hybrid 32-layer step exactly as bench.py times it.
Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" §2.1-§2.4.
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


def _host_bf16(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _pool(hy, L, n, H, D):
    import torch
    nbytes = hy.hyattn_state_pool_bytes(L, n, H, D)
    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    return buf, hy.hyattn_state_pool_create(buf, nbytes, L, n, H, D)


def test_linear_decode_batch_256_steps(hy):
    import torch
    cfg = synth.WORKLOADS["linear_decode"]
    B, H, D, steps = cfg["B"], cfg["H"], cfg["D"], cfg["steps"]
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg["seed"])
    buf, pool = _pool(hy, 1, B, H, D)
    slots = hy.hyattn_state_pool_alloc(pool, B)
    view = buf.view(B, H, D, D)
    view.normal_(0.0, cfg["state_scale"], generator=g)
    S0 = view.cpu().numpy().astype(np.float64)
    qkv = synth.device_normal_bf16((steps, 3, B, H, D), D ** -0.5, cfg["seed"] * 1000 + 1)
    out = torch.empty(steps, B, H, D, dtype=torch.bfloat16, device="cuda")
    sl = gu.i32(slots)
    for t in range(steps):
        hy.hyattn_linear_decode(pool, 0, qkv[t, 0], qkv[t, 1], qkv[t, 2], out[t], sl, B, hy.BF16)
    torch.cuda.synchronize()
    # oracle on one sampled head per request, all 256 steps
    rng = np.random.default_rng(5)
    units = [(r, int(rng.integers(H))) for r in range(B)]
    qh = _host_bf16(qkv)
    got = _host_bf16(out)
    got_S = view.cpu().numpy()
    want_o, g_o, want_S, g_S = [], [], [], []
    for r, h in units:
        S = S0[slots[r], h].copy()
        rows = np.arange(steps)
        q = np.ascontiguousarray(qh[rows, 0, r, h][:, None])
        k = np.ascontiguousarray(qh[rows, 1, r, h][:, None])
        v = np.ascontiguousarray(qh[rows, 2, r, h][:, None])
        want_o.append(ref.linear_unit("recurrent", q, k, v, S, 0, steps, 0))
        g_o.append(got[:, r, h])
        want_S.append(S)
        g_S.append(got_S[slots[r], h])
    gu.assert_bf16(np.stack(g_o), np.stack(want_o), "256-step decode outputs")
    gu.assert_f32(np.stack(g_S), np.stack(want_S), "states after 256 steps")
    hy.hyattn_state_pool_destroy(pool)


def test_linear_prefill_8x8192_all_chunk_sizes(hy):
    import torch
    cfg = synth.WORKLOADS["linear_prefill"]
    B, H, D, T = cfg["B"], cfg["H"], cfg["D"], cfg["T"]
    N = B * T
    q, k, v = (synth.device_normal_bf16((N, H, D), D ** -0.5, cfg["seed"] * 1000 + i)
               for i in range(3))
    cu = gu.i32(synth.cu_lens([T] * B))
    rng = np.random.default_rng(6)
    units = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(6)]
    qh, kh, vh = (_host_bf16(x) for x in (q, k, v))
    outs = {}
    for C in cfg["chunks"]:
        buf, pool = _pool(hy, 1, B, H, D)
        slots = hy.hyattn_state_pool_alloc(pool, B)
        sl = gu.i32(slots)
        hy.hyattn_state_pool_zero(pool, sl, B)
        o = torch.empty_like(q)
        hy.hyattn_linear_prefill_chunked(pool, 0, q, k, v, o, cu, sl, B, C, hy.BF16)
        torch.cuda.synchronize()
        oh = _host_bf16(o)
        Sv = buf.view(B, H, D, D).cpu().numpy()
        want_o, g_o, want_S, g_S = [], [], [], []
        for r, h in units:
            S = np.zeros((D, D))
            want_o.append(ref.linear_unit("chunked", qh, kh, vh, S, r * T, T, h, C))
            g_o.append(oh[r * T:(r + 1) * T, h])
            want_S.append(S)
            g_S.append(Sv[slots[r], h])
        gu.assert_bf16(np.stack(g_o), np.stack(want_o), f"prefill outputs C={C}")
        gu.assert_f32(np.stack(g_S), np.stack(want_S), f"prefill states C={C}")
        outs[C] = oh
        hy.hyattn_state_pool_destroy(pool)
        del buf
    # Chunk size only regroups the sums (P2 §2.4). The bf16 kernel streams the
    # tokens in 32-token blocks whatever C is, so its outputs are the same bits
    # at every C, while each C was checked above against the oracle's own
    # C-chunked sums.
    for C in cfg["chunks"][1:]:
        assert np.array_equal(outs[C], outs[cfg["chunks"][0]]), f"C={C}: output depends on C"


def test_paged_decode_b128_contexts_to_32k(hy):
    import torch
    cfg = synth.WORKLOADS["paged_decode"]
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    rng = np.random.default_rng(cfg["seed"])
    ctx = synth.uniform_contexts(rng, B, cfg["ctx_lo"], cfg["ctx_hi"])
    lay = synth.paged_layout(rng, ctx, n_spare=cfg["n_spare"])
    kp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, cfg["seed"] * 1000 + 1)
    vp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, cfg["seed"] * 1000 + 2)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device="cuda")
    spare = torch.as_tensor(lay.spare.astype(np.int64)).cuda()
    kp[spare] = nan
    vp[spare] = nan
    for r in range(B):  # poison the unused tail of each last block
        c = int(ctx[r])
        if c % 16:
            blk = int(lay.block_tables[r, c // 16])
            kp[blk, :, c % 16:] = nan
            vp[blk, :, c % 16:] = nan
    q = synth.device_normal_bf16((B, Hq, D), 1.0, cfg["seed"] * 1000 + 3)
    maxc = int(ctx.max())
    wsb = hy.hyattn_paged_decode_workspace_bytes(B, Hq, D, maxc)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    hy.hyattn_paged_decode(q, o, kp, vp, lay.n_blocks, gu.i32(lay.block_tables), lay.max_blocks,
                           gu.i32(ctx), maxc, B, Hq, Hkv, D, D ** -0.5, ws, wsb, hy.BF16)
    torch.cuda.synchronize()
    got = _host_bf16(o)
    assert np.isfinite(gu.as_f64(got)).all()
    samp = np.random.default_rng(7).choice(B, size=12, replace=False)
    g_all, w_all, d_all = [], [], []
    for r in samp:
        nb = (int(ctx[r]) + 15) // 16
        idx = torch.as_tensor(lay.block_tables[r, :nb].astype(np.int64)).cuda()
        kk, vv = _host_bf16(kp[idx]), _host_bf16(vp[idx])
        qq = _host_bf16(q[int(r):int(r) + 1])
        want = ref.paged_attention(qq, kk, vv, np.arange(nb, dtype=np.int32)[None], [int(ctx[r])],
                                   [0, 1], D ** -0.5)
        g_all.append(got[r])
        w_all.append(want[0])
        d_all.append(gu.attention_delta(qq, kk, vv, np.arange(nb, dtype=np.int32)[None],
                                        [int(ctx[r])], [0, 1], D ** -0.5, want)[0])
    gu.assert_bf16(np.stack(g_all), np.stack(w_all), "paged decode, sampled requests",
                   np.stack(d_all))


def test_hybrid_step_full_workload_sampled(hy):
    """The hybrid step exactly as bench.py times it: one step, sampled units of every op."""
    import torch
    import bench
    torch.cuda.empty_cache()
    wl = bench.Workload()
    W = bench.W
    P, n_p, n_d = W["prefill_len"], wl.n_p, wl.n_d
    H, Hkv, D = wl.H, wl.Hkv, wl.D
    # states before the step (decode requests hold a prior state; prefill slots get zeroed)
    sv = wl.state_buf.view(wl.n_lin, n_p + n_d, H, D, D)
    rng = np.random.default_rng(8)
    lin_units = [(int(rng.integers(n_p)), int(rng.integers(H))) for _ in range(2)] + \
                [(n_p + int(rng.integers(n_d)), int(rng.integers(H))) for _ in range(6)]
    slots_all = np.concatenate([wl.slots_p.cpu().numpy(), wl.slots_d.cpu().numpy()])
    S_before = {(r, h): sv[-1, slots_all[r], h].double().cpu().numpy() for r, h in lin_units}
    dec_req = rng.choice(np.arange(n_p, n_p + n_d), size=3, replace=False)
    pre_units = [(int(rng.integers(n_p)), int(rng.integers(H)))]
    kp_last, vp_last = wl.pools[-1]
    wl.step()
    torch.cuda.synchronize()
    lin_o = _host_bf16(wl.lin["o"])     # the last linear layer wrote it
    full_o = _host_bf16(wl.full["o"])   # the last full layer wrote it
    qh, kh, vh = (_host_bf16(wl.lin[n]) for n in ("q", "k", "v"))
    # linear layer (the last one): prefill units and decode units
    g_l, w_l = [], []
    for r, h in lin_units:
        S = S_before[(r, h)].copy()
        if r < n_p:
            S[:] = 0.0  # request start
            o = ref.linear_unit("chunked", qh, kh, vh, S, r * P, P, h, W["chunk"])
            g_l.append(lin_o[r * P:(r + 1) * P, h]); w_l.append(o)
        else:
            row = n_p * P + (r - n_p)
            o = ref.linear_unit("recurrent", qh, kh, vh, S, row, 1, h)
            g_l.append(lin_o[row:row + 1, h]); w_l.append(o)
    gu.assert_bf16(np.concatenate(g_l), np.concatenate(w_l), "hybrid step: linear layer")
    # full layer (the last one): decode requests over their whole context, all heads
    fq = _host_bf16(wl.full["q"])
    g_f, w_f, d_f = [], [], []
    for r in dec_req:
        c = int(wl.ctx[r]); nb = (c + 15) // 16
        idx = torch.as_tensor(wl.lay.block_tables[r, :nb].astype(np.int64)).cuda()
        kk, vv = _host_bf16(kp_last[idx]), _host_bf16(vp_last[idx])
        row = n_p * P + (r - n_p)
        want = ref.paged_attention(fq[row:row + 1], kk, vv, np.arange(nb, dtype=np.int32)[None],
                                   [c], [0, 1], D ** -0.5)
        g_f.append(full_o[row]); w_f.append(want[0])
        d_f.append(gu.attention_delta(fq[row:row + 1], kk, vv, np.arange(nb, dtype=np.int32)[None],
                                      [c], [0, 1], D ** -0.5, want)[0])
    # a causal-prefill unit: 64 sampled query rows of one (request, head)
    for r, h in pre_units:
        nb = P // 16
        idx = torch.as_tensor(wl.lay.block_tables[r, :nb].astype(np.int64)).cuda()
        kk, vv = _host_bf16(kp_last[idx]), _host_bf16(vp_last[idx])
        rows = np.sort(np.random.default_rng(9).choice(P, size=64, replace=False))
        for i in rows:
            qq = np.ascontiguousarray(fq[r * P + i:r * P + i + 1])
            want = ref.paged_attention(qq, kk, vv, np.arange(nb, dtype=np.int32)[None], [int(i) + 1],
                                       [0, 1], D ** -0.5, units=[(0, h)])
            g_f.append(full_o[r * P + i, h][None]); w_f.append(want[0, h][None])
            d_f.append(gu.attention_delta(qq, kk, vv, np.arange(nb, dtype=np.int32)[None],
                                          [int(i) + 1], [0, 1], D ** -0.5, want,
                                          units=[(0, h)])[0, h][None])
    gu.assert_bf16(np.concatenate([x.reshape(-1, D) for x in g_f]),
                   np.concatenate([x.reshape(-1, D) for x in w_f]), "hybrid step: full layer",
                   np.concatenate([x.reshape(-1, D) for x in d_f]))
