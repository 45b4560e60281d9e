"""GPU parity of the whole per-layer hybrid step (hyattn_hybrid_step) against
the oracle's composition of the same layer operations.

Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2) §2.2
(layer types, split memory pools, per-forward metadata), §2.3 and §2.4.
"""
import numpy as np
import pytest

from synth import hybrid
from tests import gpu_util as gu
from tests import hybrid_run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kw", [
    dict(),                                                        # bf16, [lin,lin,lin,full]
    dict(n_layers=8, prefill_lens=(1, 130, 16), decode_ctx=(2, 600, 33, 1), chunk=64),
    dict(dtype="f32", D=64, H=4, Hkv=4, prefill_lens=(256,), decode_ctx=(257,), chunk=64,
         n_layers=2, pattern=("linear", "full")),                  # fp32, [linear, full]
    dict(prefill_lens=(), decode_ctx=(5, 900)),                    # decode only
    dict(prefill_lens=(33, 8), decode_ctx=()),
])
def test_hybrid_step_matches_oracle(kw):
    case = hybrid.small_case(seed=len(str(kw)), **kw)
    got = hybrid_run.run_gpu(case)
    want = hybrid_run.run_oracle(case)
    hybrid_run.compare(case, got, want)


@pytest.mark.parametrize("H,Hkv,D", [(4, 2, 128), (8, 2, 64)])
def test_hybrid_step_prefill_beside_decode_walks_several_tiles_per_workgroup(H, Hkv, D):
    """A full layer whose prefill has more query-tile work items than the device has
    CUs, with decode requests beside it: the step then runs the prefill as one
    persistent workgroup per CU (each walking several tiles) next to the decode on
    the second stream. Outputs, states and pools against the oracle."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    qt = 64 * 3 // (H // Hkv)           # query positions per work item
    n_len = (cus // 8 + 2) * qt         # query tiles x 8 XCD slots > CUs
    case = hybrid.small_case(seed=21 + D, n_layers=4, H=H, Hkv=Hkv, D=D, prefill_lens=(n_len, 50),
                             decode_ctx=(7, 700, 33), chunk=64)
    n_qt = -(-n_len // qt)
    assert n_qt * 8 * -(-(Hkv * 5) // 8) > cus
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


def test_hybrid_step_replays_from_a_captured_graph():
    """The step (prefill and decode requests, so each full layer forks its decode onto
    the library's second stream and joins it back) captured into a graph and replayed
    three times, with the states and pools restored by eager copies and a device
    synchronisation before each replay: every replay gives the eager step's outputs,
    states and pools bit for bit."""
    import torch
    case = hybrid.small_case(seed=7, n_layers=8)
    assert case["n_prefill"] > 0 and case["n_decode"] > 0
    g = hybrid_run.setup_gpu(case)
    hy, types, layers = g["hy"], g["types"], g["layers"]
    live = [g["buf"]] + [d[x] for t, d in zip(types, layers) if t == 1 for x in ("k_pool", "v_pool")]
    saved = [x.clone() for x in live]

    def restore():
        for a, b in zip(live, saved):
            a.copy_(b)
        for d in layers:
            d["o"].fill_(float("nan"))
        torch.cuda.synchronize()

    def snapshot():
        return [d["o"].clone() for d in layers] + [x.clone() for x in live]

    hy.hyattn_hybrid_step(types, len(types), layers, g["batch"], g["pool"])
    torch.cuda.synchronize()
    want = snapshot()
    restore()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hy.hyattn_hybrid_step(types, len(types), layers, g["batch"], g["pool"])
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}, tensor {i}"
    hy.hyattn_state_pool_destroy(g["pool"])


@pytest.mark.parametrize("fault", ["block id out of range", "slot never zeroed",
                                   "context beyond max_context", "q lengths inconsistent"])
def test_hybrid_step_checked_mode_rejects_before_any_launch(monkeypatch, fault):
    """In checked mode the step reads and validates every index array before its
    first launch: a bad entry anywhere (here in the last request, which only the last
    layer's kernels would reach) gives INVALID_ARG or BAD_SLOT, and every linear state
    and KV pool is left bit for bit as it was."""
    import torch
    monkeypatch.setenv("HYATTN_CHECK", "1")
    case = hybrid.small_case(seed=12, n_layers=8)
    g = hybrid_run.setup_gpu(case)
    hy, t = g["hy"], dict(g["tensors"])
    kw = dict(g["batch_kw"])
    lay = case["layout"]
    B = g["B"]
    if fault == "block id out of range":
        bt = lay.block_tables.copy()
        bt[B - 1, (int(case["ctx"][B - 1]) - 1) // 16] = lay.n_blocks
        t["block_tables"] = gu.i32(bt)
        want = hy.ERR_INVALID_ARG
    elif fault == "slot never zeroed":
        spare = [i for i in range(B + 3) if i not in g["slots"]][:1]
        hy.hyattn_state_pool_free(g["pool"], spare)
        extra = hy.hyattn_state_pool_alloc(g["pool"], 1)  # allocated again, not zeroed
        t["decode_slots"] = gu.i32(g["slots"][case["n_prefill"]:-1] + extra)
        want = hy.ERR_BAD_SLOT
    elif fault == "context beyond max_context":
        kw["max_context"] = int(case["ctx"].max()) - 1
        ws_bytes = hy.hyattn_paged_decode_workspace_bytes(case["n_decode"], case["H"], case["D"],
                                                          int(case["ctx"].max()))
        kw["workspace_bytes"] = ws_bytes
        want = hy.ERR_INVALID_ARG
    else:
        cu = case["cu_q"].copy()
        cu[-1] += 1
        t["cu_q_lens"] = gu.i32(cu)
        want = hy.ERR_INVALID_ARG
    batch = hy.make_batch(**kw, **t)
    torch.cuda.synchronize()
    states0 = g["buf"].clone()
    pools0 = [(d["k_pool"].clone(), d["v_pool"].clone()) for d in g["layers"] if "k_pool" in d]
    outs0 = [d["o"].clone() for d in g["layers"]]
    with pytest.raises(hy.HyattnError) as e:
        hy.hyattn_hybrid_step(g["types"], len(g["types"]), g["layers"], batch, g["pool"])
    assert e.value.status == want, str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(g["buf"].view(torch.int32), states0.view(torch.int32)), "a state changed"
    for (k0, v0), d in zip(pools0, [d for d in g["layers"] if "k_pool" in d]):
        assert torch.equal(d["k_pool"].view(torch.int16), k0.view(torch.int16)), "a K pool changed"
        assert torch.equal(d["v_pool"].view(torch.int16), v0.view(torch.int16)), "a V pool changed"
    for o0, d in zip(outs0, g["layers"]):
        assert torch.equal(d["o"].view(torch.int16), o0.view(torch.int16)), "an output was written"
    hy.hyattn_state_pool_destroy(g["pool"])
