"""GPU parity of the linear-layer path (state pool, chunked prefill, decode)
against the fp64 oracle, through the C ABI.

Page cited: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2):
§2.1 recurrence, §2.3 state lifecycle, §2.4 chunked prefill, §3.5 batch
consistency, §4.1 decode must not re-zero the state.
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


class Pool:
    def __init__(self, hy, L, n_slots, H, D):
        import torch
        self.hy, self.L, self.n, self.H, self.D = hy, L, n_slots, H, D
        nbytes = hy.hyattn_state_pool_bytes(L, n_slots, H, D)
        self.buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
        self.handle = hy.hyattn_state_pool_create(self.buf, nbytes, L, n_slots, H, D)
        self.view = self.buf.view(L, n_slots, H, D, D)

    def alloc(self, n):
        return self.hy.hyattn_state_pool_alloc(self.handle, n)

    def zero(self, slots):
        self.hy.hyattn_state_pool_zero(self.handle, gu.i32(slots), len(slots))

    def close(self):
        self.hy.hyattn_state_pool_destroy(self.handle)


def _prefill(hy, pool, layer, q, k, v, cu, slots, chunk, dtype):
    import torch
    dq, dk, dv = gu.dev(q), gu.dev(k), gu.dev(v)
    do = torch.empty_like(dq)
    do.fill_(float("nan"))
    hy.hyattn_linear_prefill_chunked(pool.handle, layer, dq, dk, dv, do, gu.i32(cu),
                                     gu.i32(slots), len(slots), chunk,
                                     hy.BF16 if dtype == "bf16" else hy.F32)
    torch.cuda.synchronize()
    return do


# ----------------------------------------------------------------- decode --
@pytest.mark.parametrize("B,D", [(37, 128), (53, 64)])
def test_decode_batch_with_several_states_per_workgroup(hy, B, D):
    """A batch between one and the split threshold's worth of (request, head) units: the
    persistent decode walks 2-3 states per workgroup, in an order unrelated to the slots
    (slots reversed and gapped). Every unit against the oracle, two steps in a row, and
    the slots outside the batch untouched."""
    import torch
    rng = np.random.default_rng(140 + B)
    H = 32
    pool = Pool(hy, 1, 2 * B + 1, H, D)
    all_slots = pool.alloc(2 * B + 1)
    slots = all_slots[::-2][:B]  # every other slot, descending
    others = sorted(set(all_slots) - set(slots))
    pool.view[...] = 5.0
    S0 = (rng.standard_normal((B, H, D, D)) * 0.1).astype(np.float32)
    for r, s in enumerate(slots):
        pool.view[0, s] = torch.from_numpy(S0[r]).cuda()
    st = S0.astype(np.float64)
    for step in range(2):
        q, k, v = (synth.normal(rng, (B, H, D), D ** -0.5, "bf16") for _ in range(3))
        do = torch.full_like(gu.dev(q), float("nan"))
        hy.hyattn_linear_decode(pool.handle, 0, gu.dev(q), gu.dev(k), gu.dev(v), do,
                                gu.i32(slots), B, hy.BF16)
        torch.cuda.synchronize()
        want = ref.linear_decode(q, k, v, st)
        gu.assert_bf16(gu.host(do), want, f"decode step {step}, B={B}")
    got_S = np.stack([gu.host(pool.view[0, s]) for s in slots])
    gu.assert_f32(got_S, st, "final states")
    assert bool((pool.view[0, others] == 5.0).all()), "slots outside the batch changed"
    pool.close()


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_decode_matches_oracle(hy, dtype, D):
    """Several decode steps from random prior states (mid-request decode)."""
    import torch
    rng = np.random.default_rng(100 + D)
    B, H, steps = 5, 4, 3
    pool = Pool(hy, 2, 8, H, D)
    slots = pool.alloc(B)
    slots = slots[::-1]  # non-identity slot order
    S0 = (rng.standard_normal((B, H, D, D)) * 0.1).astype(np.float32)
    for r, s in enumerate(slots):
        pool.view[1, s] = torch.from_numpy(S0[r]).cuda()
    st = S0.astype(np.float64)
    for step in range(steps):
        q, k, v = (synth.normal(rng, (B, H, D), D ** -0.5, dtype) for _ in range(3))
        dq, dk, dv = gu.dev(q), gu.dev(k), gu.dev(v)
        do = torch.full_like(dq, float("nan"))
        hy.hyattn_linear_decode(pool.handle, 1, dq, dk, dv, do, gu.i32(slots), B,
                                hy.BF16 if dtype == "bf16" else hy.F32)
        torch.cuda.synchronize()
        want = ref.linear_decode(q, k, v, st)
        gu.assert_io(gu.host(do), want, dtype, f"decode step {step}")
    got_S = np.stack([gu.host(pool.view[1, s]) for s in slots])
    gu.assert_f32(got_S, st, "decode final states")
    assert not pool.view[0].any(), "layer 0 must be untouched"
    pool.close()


def test_decode_integer_inputs_bit_exact(hy):
    """Small-integer inputs keep every partial sum exact in fp32: results must be exact."""
    import torch
    rng = np.random.default_rng(7)
    B, H, D = 3, 2, 128
    pool = Pool(hy, 1, 4, H, D)
    slots = pool.alloc(B)
    S0 = rng.integers(-4, 5, size=(B, H, D, D)).astype(np.float32)
    for r, s in enumerate(slots):
        pool.view[0, s] = torch.from_numpy(S0[r]).cuda()
    q, k, v = (synth.small_ints(rng, (B, H, D), -2, 2, "f32") for _ in range(3))
    do = torch.empty(B, H, D, device="cuda")
    hy.hyattn_linear_decode(pool.handle, 0, gu.dev(q), gu.dev(k), gu.dev(v), do, gu.i32(slots),
                            B, hy.F32)
    torch.cuda.synchronize()
    st = S0.astype(np.float64)
    want = ref.linear_decode(q, k, v, st)
    assert np.array_equal(gu.host(do).astype(np.float64), want)
    assert np.array_equal(np.stack([gu.host(pool.view[0, s]) for s in slots]).astype(np.float64), st)
    pool.close()


# ---------------------------------------------------------------- prefill --
@pytest.mark.parametrize("dtype,D,chunk", [
    ("bf16", 128, 64), ("bf16", 128, 16), ("bf16", 128, 32), ("bf16", 128, 128),
    ("bf16", 128, 48), ("bf16", 64, 64), ("bf16", 64, 256), ("f32", 64, 64), ("f32", 128, 7),
])
def test_prefill_matches_oracle(hy, dtype, D, chunk):
    """Ragged requests (including empty and single-token ones) from non-zero prior states."""
    import torch
    rng = np.random.default_rng(200 + chunk + D)
    H = 3
    lens = [1, 77, 0, 300, 16]
    cu = synth.cu_lens(lens)
    N = int(cu[-1])
    q, k, v = (synth.normal(rng, (N, H, D), D ** -0.5, dtype) for _ in range(3))
    pool = Pool(hy, 1, 8, H, D)
    slots = pool.alloc(len(lens))
    slots = [slots[i] for i in (3, 0, 4, 1, 2)]
    S0 = (rng.standard_normal((len(lens), H, D, D)) * 0.1).astype(np.float32)
    for r, s in enumerate(slots):
        pool.view[0, s] = torch.from_numpy(S0[r]).cuda()
    do = _prefill(hy, pool, 0, q, k, v, cu, slots, chunk, dtype)
    st = S0.astype(np.float64)
    want = ref.linear_prefill(q, k, v, cu, st, chunk=chunk)
    gu.assert_io(gu.host(do), want, dtype, f"prefill out C={chunk}")
    got_S = np.stack([gu.host(pool.view[0, s]) for s in slots])
    gu.assert_f32(got_S, st, f"prefill states C={chunk}")
    pool.close()


@pytest.mark.parametrize("gated", [False, True])
def test_prefill_with_more_units_than_compute_units(hy, gated):
    """bf16, D = 128, with more (request, head) units than the device has compute
    units, so that workgroups share CUs and the launcher takes the 16x16-tile
    kernel (the other tests' batches give each unit a CU of its own and run the
    32x32-tile kernel): ragged requests, empty and single-token ones included,
    from non-zero prior states."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(450 + gated)
    H, D = 8, 128
    B = cus // H + 9
    lens = [(1, 77, 0, 33, 64, 5, 31, 32)[r % 8] for r in range(B)]
    assert B * H > cus
    cu = synth.cu_lens(lens)
    N = int(cu[-1])
    q, k, v = (synth.normal(rng, (N, H, D), D ** -0.5, "bf16") for _ in range(3))
    g = synth.log_forget(rng, (N, H)) if gated else None
    pool = Pool(hy, 1, B, H, D)
    slots = list(rng.permutation(pool.alloc(B)))
    S0 = (rng.standard_normal((B, H, D, D)) * 0.1).astype(np.float32)
    for r, sl in enumerate(slots):
        pool.view[0, sl] = torch.from_numpy(S0[r]).cuda()
    dq, dk, dv = gu.dev(q), gu.dev(k), gu.dev(v)
    do = torch.full_like(dq, float("nan"))
    if gated:
        hy.hyattn_linear_prefill_chunked_gated(pool.handle, 0, dq, dk, dv, gu.dev(g), do, gu.i32(cu),
                                               gu.i32(slots), B, 64, hy.BF16)
    else:
        hy.hyattn_linear_prefill_chunked(pool.handle, 0, dq, dk, dv, do, gu.i32(cu), gu.i32(slots),
                                         B, 64, hy.BF16)
    torch.cuda.synchronize()
    st = S0.astype(np.float64)
    want = ref.linear_prefill(q, k, v, cu, st, chunk=64, log_gamma=g)
    gu.assert_io(gu.host(do), want, "bf16", f"{B * H} units")
    got_S = np.stack([gu.host(pool.view[0, sl]) for sl in slots])
    gu.assert_f32(got_S, st, f"{B * H} units, states")
    pool.close()


def test_prefill_integer_inputs_bit_exact(hy):
    """bf16 MFMA path with small-integer inputs: exact results (all sums < 2^24)."""
    rng = np.random.default_rng(8)
    H, D, T = 2, 128, 96
    q, k, v = (synth.small_ints(rng, (T, H, D), -1, 1, "bf16") for _ in range(3))
    pool = Pool(hy, 1, 2, H, D)
    slots = pool.alloc(1)
    pool.zero(slots)
    do = _prefill(hy, pool, 0, q, k, v, [0, T], slots, 32, "bf16")
    st = np.zeros((1, H, D, D))
    want = ref.linear_prefill(q, k, v, [0, T], st, chunk=32)
    assert np.abs(want).max() < 2 ** 24  # exact in fp32, so the output is RNE(exact)
    assert np.array_equal(gu.host(do), synth.f32_to_bf16_bits(want.astype(np.float32)))
    assert np.array_equal(gu.host(pool.view[0, slots[0]]).astype(np.float64), st[0])
    pool.close()


def test_chunk_size_invariance_and_continuation(hy):
    """Every chunk size against the oracle; prefill(T) + decodes == prefill(T + n) (P2 §2.4, §4.1)."""
    import torch
    rng = np.random.default_rng(9)
    H, D, T, extra = 2, 128, 200, 5
    q, k, v = (synth.normal(rng, (T + extra, H, D), D ** -0.5, "bf16") for _ in range(3))
    st = np.zeros((1, H, D, D))
    want = ref.linear_prefill(q, k, v, [0, T + extra], st, chunk=64)
    outs = {}
    for chunk in (16, 64, 128):
        pool = Pool(hy, 1, 1, H, D)
        slots = pool.alloc(1)
        pool.zero(slots)
        o1 = _prefill(hy, pool, 0, q[:T], k[:T], v[:T], [0, T], slots, chunk, "bf16")
        rows = [gu.host(o1)]
        for t in range(T, T + extra):
            do = torch.empty(1, H, D, dtype=torch.bfloat16, device="cuda")
            hy.hyattn_linear_decode(pool.handle, 0, gu.dev(q[t:t + 1]), gu.dev(k[t:t + 1]),
                                    gu.dev(v[t:t + 1]), do, gu.i32(slots), 1, hy.BF16)
            rows.append(gu.host(do))
        torch.cuda.synchronize()
        got = np.concatenate(rows)
        gu.assert_bf16(got, want, f"C={chunk} + decode")
        gu.assert_f32(gu.host(pool.view[0, 0])[None], st, f"C={chunk} state")
        outs[chunk] = got
        pool.close()
    # the bf16 kernel streams 32-token blocks whatever the chunk size (each size
    # was checked above against the oracle), so its outputs are the same bits
    for c in (16, 128):
        assert np.array_equal(outs[c], outs[64]), f"C={c}: output depends on the chunk size"


def test_batch_consistency_and_slot_isolation(hy):
    """A request alone == inside a batch, bit for bit; other slots/layers untouched (P2 §3.5)."""
    import torch
    rng = np.random.default_rng(10)
    H, D = 2, 128
    lens = [40, 130, 7]
    cu = synth.cu_lens(lens)
    q, k, v = (synth.normal(rng, (int(cu[-1]), H, D), D ** -0.5, "bf16") for _ in range(3))
    pool = Pool(hy, 2, 6, H, D)
    slots = pool.alloc(6)
    pool.view[...] = 3.0  # canary in every slot and layer
    batch_slots = [slots[4], slots[1], slots[2]]
    pool.zero(batch_slots)
    do = _prefill(hy, pool, 1, q, k, v, cu, batch_slots, 64, "bf16")
    ob = gu.host(do)
    v_all = gu.host(pool.view)
    for s in (slots[0], slots[3], slots[5]):
        assert (v_all[:, s] == 3.0).all()
    assert (v_all[0][batch_slots] == 0.0).all(), "zeroing clears every linear layer"
    for r in range(3):
        p2 = Pool(hy, 2, 6, H, D)
        s2 = p2.alloc(1)
        p2.zero(s2)
        sl = slice(int(cu[r]), int(cu[r + 1]))
        o1 = _prefill(hy, p2, 1, q[sl], k[sl], v[sl], [0, lens[r]], s2, 64, "bf16")
        assert np.array_equal(gu.host(o1), ob[sl])
        assert np.array_equal(gu.host(p2.view[1, s2[0]]), v_all[1, batch_slots[r]])
        p2.close()
    # determinism: run again from zero, identical bits
    pool.zero(batch_slots)
    do2 = _prefill(hy, pool, 1, q, k, v, cu, batch_slots, 64, "bf16")
    assert np.array_equal(gu.host(do2), ob)
    pool.close()


def test_reused_slot_starts_clean(hy):
    """A freed-then-reallocated slot, once zeroed, gives a fresh request's result (P2 §3.5)."""
    rng = np.random.default_rng(11)
    H, D, T = 2, 64, 50
    q, k, v = (synth.normal(rng, (T, H, D), D ** -0.5, "bf16") for _ in range(3))
    pool = Pool(hy, 1, 2, H, D)
    s = pool.alloc(1)
    pool.zero(s)
    first = gu.host(_prefill(hy, pool, 0, q, k, v, [0, T], s, 32, "bf16"))
    hy.hyattn_state_pool_free(pool.handle, s)
    s2 = pool.alloc(1)
    assert s2 == s
    pool.zero(s2)
    again = gu.host(_prefill(hy, pool, 0, q, k, v, [0, T], s2, 32, "bf16"))
    assert np.array_equal(first, again)
    pool.close()


def test_checked_mode_rejects_unzeroed_and_foreign_slots(hy, monkeypatch):
    import torch
    monkeypatch.setenv("HYATTN_CHECK", "1")
    H, D = 2, 64
    pool = Pool(hy, 1, 4, H, D)
    s = pool.alloc(2)
    x = torch.zeros(2, H, D, device="cuda")
    with pytest.raises(hy.HyattnError) as e:
        hy.hyattn_linear_decode(pool.handle, 0, x, x, x, x, gu.i32(s), 2, hy.F32)
    assert e.value.status == hy.ERR_BAD_SLOT
    pool.zero(s)
    hy.hyattn_linear_decode(pool.handle, 0, x, x, x, x, gu.i32(s), 2, hy.F32)
    with pytest.raises(hy.HyattnError) as e:
        hy.hyattn_linear_decode(pool.handle, 0, x, x, x, x, gu.i32([s[0], 3]), 2, hy.F32)
    assert e.value.status == hy.ERR_BAD_SLOT
    torch.cuda.synchronize()
    pool.close()
