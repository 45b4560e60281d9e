"""Run a synth.hybrid case through hyattn_hybrid_step and through the oracle.

Shared by the GPU hybrid tests and the smoke check. The HIP side sees only
device copies of the case's arrays; the oracle side sees only the host arrays.
"""
from __future__ import annotations

import numpy as np

from oracle import ref
from tests import gpu_util as gu


def setup_gpu(case, slot_perm=None):
    """Device copies of a synth.hybrid case, a state pool with the case's prior
    states in its slots, and the hyattn_batch of the step. Returns a dict."""
    import torch
    from linear_attention_attn_amd import hyattn as hy
    from linear_attention_attn_amd import layer_types
    types = layer_types.parse(case["types"])
    H, Hkv, D = case["H"], case["Hkv"], case["D"]
    n_p, n_d = case["n_prefill"], case["n_decode"]
    B = n_p + n_d
    n_lin = sum(t == 0 for t in types)
    lay = case["layout"]
    n_slots = B + 3
    nbytes = hy.hyattn_state_pool_bytes(max(n_lin, 1), n_slots, H, D)
    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    view = buf.view(max(n_lin, 1), n_slots, H, D, D)
    pool = hy.hyattn_state_pool_create(buf, nbytes, max(n_lin, 1), n_slots, H, D)
    slots = hy.hyattn_state_pool_alloc(pool, n_slots)[:B]
    if slot_perm is not None:
        slots = [slots[i] for i in slot_perm]
    hy.hyattn_state_pool_zero(pool, gu.i32(slots), B)  # request start
    for li in range(n_lin):
        for r in range(B):
            view[li, slots[r]] = torch.from_numpy(case["states"][li, r]).cuda()
    dev_layers = []
    fi = 0
    for t, io in zip(types, case["layers"]):
        d = {n: gu.dev(io[n]) for n in ("q", "k", "v")}
        d["o"] = torch.full_like(d["q"], float("nan"))
        if "g" in io:  # gated linear layer
            d["log_gamma"] = gu.dev(io["g"])
        if t == 1:
            d["k_pool"], d["v_pool"] = (gu.dev(x) for x in case["pools"][fi])
            fi += 1
        dev_layers.append(d)
    ws_bytes = hy.hyattn_paged_decode_workspace_bytes(n_d, H, D, int(case["ctx"].max()))
    ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device="cuda")
    tensors = dict(cu_seqlens=gu.i32(case["prefill_cu"]), prefill_slots=gu.i32(slots[:n_p]),
                   decode_slots=gu.i32(slots[n_p:]), block_tables=gu.i32(lay.block_tables),
                   context_lens=gu.i32(case["ctx"]), cu_q_lens=gu.i32(case["cu_q"]), workspace=ws)
    kw = dict(n_prefill=n_p, n_decode=n_d, n_prefill_tokens=int(case["prefill_cu"][-1]),
              max_prefill_len=case["max_prefill_len"], max_blocks_per_seq=lay.max_blocks,
              max_context=int(case["ctx"].max()), n_blocks=lay.n_blocks, H=H, H_kv=Hkv, D=D,
              chunk_size=case["chunk"], scale=case["scale"],
              dtype=hy.BF16 if case["dtype"] == "bf16" else hy.F32, workspace_bytes=ws_bytes)
    return dict(hy=hy, types=types, n_lin=n_lin, B=B, buf=buf, view=view, pool=pool, slots=slots,
                layers=dev_layers, tensors=tensors, batch_kw=kw,
                batch=hy.make_batch(**kw, **tensors))


def run_gpu(case, slot_perm=None):
    import torch
    g = setup_gpu(case, slot_perm)
    hy, types, view, slots, B, n_lin = g["hy"], g["types"], g["view"], g["slots"], g["B"], g["n_lin"]
    hy.hyattn_hybrid_step(types, len(types), g["layers"], g["batch"], g["pool"])
    torch.cuda.synchronize()
    outs = [gu.host(d["o"]) for d in g["layers"]]
    states = np.stack([np.stack([gu.host(view[li, slots[r]]) for r in range(B)])
                       for li in range(n_lin)]) if n_lin else None
    pools = [(gu.host(d["k_pool"]), gu.host(d["v_pool"])) for t, d in zip(types, g["layers"])
             if t == 1]
    hy.hyattn_state_pool_destroy(g["pool"])
    return outs, states, pools


def run_oracle(case, units_linear=None, units_full=None):
    types = ref.parse_layer_types(case["types"])
    states = case["states"].astype(np.float64)
    pools = [(kp.copy(), vp.copy()) for kp, vp in case["pools"]]
    batch = dict(prefill_cu=case["prefill_cu"], n_decode=case["n_decode"],
                 block_tables=case["layout"].block_tables, context_lens=case["ctx"],
                 chunk=case["chunk"], scale=case["scale"])
    outs = ref.hybrid_step(types, case["layers"], batch, states, pools,
                           units_linear=units_linear, units_full=units_full)
    return outs, states, pools


def compare(case, got, want, check_pools=True):
    """Outputs against the oracle's (full layers with the softmax-weight rounding term
    in the bf16 bound, computed over the oracle's pools after append), final states
    at the fp32 rule, pools bit for bit. A one-step case gives its query offsets as
    cu_q; a multi-step case is compared with the oracle's single step over all new
    tokens, whose offsets are its cu."""
    g_outs, g_states, g_pools = got
    w_outs, w_states, w_pools = want
    lay = case["layout"]
    ctx = case["ctx"]
    cu = case["cu_q"] if "cu_q" in case else case["cu"]
    report = []
    fi = 0
    for i, (g, w) in enumerate(zip(g_outs, w_outs)):
        delta = None
        if case["types"][i] == "full":
            if case["dtype"] == "bf16":
                q = case["layers"][i]["q"]
                kp, vp = w_pools[fi]
                delta = gu.attention_delta(q, kp, vp, lay.block_tables, ctx, cu, case["scale"], w)
            fi += 1
        report.append((i, case["types"][i],
                       gu.assert_io(g, w, case["dtype"], f"layer {i} output", delta)))
    if g_states is not None:
        gu.assert_f32(g_states, w_states, "linear states")
    if check_pools:
        for (gk, gv), (wk, wv) in zip(g_pools, w_pools):
            assert np.array_equal(gk.view(np.uint8), wk.view(np.uint8)), "K pool after append"
            assert np.array_equal(gv.view(np.uint8), wv.view(np.uint8)), "V pool after append"
    return report


def _step_plan(case, step):
    """Rows (in the case's packed order), context lengths and offsets of one
    step of a continuation_case: step 0 serves the first split[r] tokens of
    request r, step 1 the rest; prompts are prefill requests, the others
    decode requests (one token per step)."""
    cu, split, new = case["cu"], case["split"], case["new"]
    n_p = case["n_prompts"]
    rows = []
    for r in range(len(new)):
        lo = int(cu[r]) + (0 if step == 0 else int(split[r]))
        hi = int(cu[r]) + (int(split[r]) if step == 0 else int(new[r]))
        rows.append(np.arange(lo, hi))
    lens = np.array([len(x) for x in rows], np.int64)
    assert np.all(lens[n_p:] == 1), "decode requests bring one token per step"
    cu_p = np.concatenate([[0], np.cumsum(lens[:n_p])]).astype(np.int32)
    Np = int(cu_p[-1])
    return dict(order=np.concatenate(rows), lens=lens, n_p=n_p, n_d=len(new) - n_p,
                ctx=(case["prior"] + (split if step == 0 else new)).astype(np.int32), cu_p=cu_p,
                cu_q=np.concatenate([cu_p, Np + np.arange(1, len(new) - n_p + 1)]).astype(np.int32))


def run_gpu_steps(case):
    """Serve a continuation_case over two hyattn_hybrid_step calls.

    Step 0 brings the first split[r] tokens of every request, step 1 the rest;
    prompts are prefill requests in both steps, the others decode requests.
    Pools and linear states carry over between the steps on the device.
    Returns the outputs in the case's packed order, the final states and pools.
    """
    import torch
    from linear_attention_attn_amd import hyattn as hy
    from linear_attention_attn_amd import layer_types
    types = layer_types.parse(case["types"])
    H, Hkv, D = case["H"], case["Hkv"], case["D"]
    n_p = case["n_prompts"]
    B = len(case["new"])
    n_d = B - n_p
    n_lin = sum(t == 0 for t in types)
    lay = case["layout"]
    nbytes = hy.hyattn_state_pool_bytes(max(n_lin, 1), B + 1, H, D)
    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    view = buf.view(max(n_lin, 1), B + 1, H, D, D)
    pool = hy.hyattn_state_pool_create(buf, nbytes, max(n_lin, 1), B + 1, H, D)
    slots = hy.hyattn_state_pool_alloc(pool, B)
    hy.hyattn_state_pool_zero(pool, gu.i32(slots), B)
    for li in range(n_lin):
        for r in range(n_p, B):
            view[li, slots[r]] = torch.from_numpy(case["states"][li, r]).cuda()
    dev_pools = [tuple(gu.dev(x) for x in p) for p in case["pools"]]
    outs = [np.zeros_like(io["q"]) for io in case["layers"]]
    for step in (0, 1):
        sp = _step_plan(case, step)
        order, lens, ctx, cu_p, cu_q = sp["order"], sp["lens"], sp["ctx"], sp["cu_p"], sp["cu_q"]
        Np = int(cu_p[-1])
        dev_layers, fi = [], 0
        for t, io in zip(types, case["layers"]):
            d = {n: gu.dev(io[n][order]) for n in ("q", "k", "v")}
            d["o"] = torch.full_like(d["q"], float("nan"))
            if "g" in io:  # gated linear layer
                d["log_gamma"] = gu.dev(io["g"][order])
            if t == 1:
                d["k_pool"], d["v_pool"] = dev_pools[fi]
                fi += 1
            dev_layers.append(d)
        ws_bytes = hy.hyattn_paged_decode_workspace_bytes(n_d, H, D, int(ctx.max()))
        ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device="cuda")
        tensors = dict(cu_seqlens=gu.i32(cu_p), prefill_slots=gu.i32(slots[:n_p]),
                       decode_slots=gu.i32(slots[n_p:]), block_tables=gu.i32(lay.block_tables),
                       context_lens=gu.i32(ctx), cu_q_lens=gu.i32(cu_q), workspace=ws)
        batch = hy.make_batch(n_prefill=n_p, n_decode=n_d, n_prefill_tokens=Np,
                              max_prefill_len=int(lens[:n_p].max()) if n_p else 0,
                              max_blocks_per_seq=lay.max_blocks, max_context=int(ctx.max()),
                              n_blocks=lay.n_blocks, H=H, H_kv=Hkv, D=D, chunk_size=case["chunk"],
                              scale=case["scale"], dtype=hy.BF16 if case["dtype"] == "bf16" else hy.F32,
                              workspace_bytes=ws_bytes, **tensors)
        hy.hyattn_hybrid_step(types, len(types), dev_layers, batch, pool)
        torch.cuda.synchronize()
        for i, d in enumerate(dev_layers):
            outs[i][order] = gu.host(d["o"])
    states = np.stack([np.stack([gu.host(view[li, slots[r]]) for r in range(B)])
                       for li in range(n_lin)]) if n_lin else None
    pools = [(gu.host(k), gu.host(v)) for k, v in dev_pools]
    hy.hyattn_state_pool_destroy(pool)
    return outs, states, pools


def run_oracle_whole(case):
    """The oracle's single step over every request's new tokens at once."""
    types = ref.parse_layer_types(case["types"])
    states = case["states"].astype(np.float64)
    pools = [(kp.copy(), vp.copy()) for kp, vp in case["pools"]]
    batch = dict(prefill_cu=case["cu"], n_decode=0, block_tables=case["layout"].block_tables,
                 context_lens=case["ctx"], chunk=case["chunk"], scale=case["scale"])
    outs = ref.hybrid_step(types, case["layers"], batch, states, pools)
    return outs, states, pools


def run_oracle_steps(case):
    """The oracle over the same two steps as run_gpu_steps."""
    types = ref.parse_layer_types(case["types"])
    states = case["states"].astype(np.float64)
    pools = [(kp.copy(), vp.copy()) for kp, vp in case["pools"]]
    outs = [np.zeros(io["q"].shape) for io in case["layers"]]
    for step in (0, 1):
        sp = _step_plan(case, step)
        layers = [{n: io[n][sp["order"]] for n in ("q", "k", "v")} for io in case["layers"]]
        batch = dict(prefill_cu=sp["cu_p"], n_decode=sp["n_d"],
                     block_tables=case["layout"].block_tables, context_lens=sp["ctx"],
                     chunk=case["chunk"], scale=case["scale"])
        for li, io in zip(layers, case["layers"]):
            if "g" in io:
                li["g"] = io["g"][sp["order"]]
        for i, o in enumerate(ref.hybrid_step(types, layers, batch, states, pools)):
            outs[i][sp["order"]] = o
    return outs, states, pools
