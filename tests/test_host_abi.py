"""CPU tests of the hyattn C ABI: the library loads, exports every entry point
the header declares, and its host logic (slot free list, argument validation,
layer-type rejection) behaves as documented. Nothing here launches a kernel:
every call below returns before touching the device.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from linear_attention_attn_amd import hyattn as hy
from oracle import ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # a non-NULL, aligned address; never dereferenced on these paths


def header_functions():
    text = open(os.path.join(ROOT, "include", "hyattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hyattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = hy.load()
    names = header_functions()
    assert len(names) >= 18
    assert set(names) == set(hy.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert hy.hyattn_abi_version() == hy.ABI_VERSION == 2


def test_library_is_gfx950_code_object():
    blob = open(hy.lib_path(), "rb").read()
    assert b"gfx950" in blob


def test_state_pool_bytes_is_independent_of_sequence_length():
    # the formula has no sequence-length argument at all (P2 §2.1 constant-size state)
    assert hy.hyattn_state_pool_bytes(24, 256, 32, 128) == 24 * 256 * 32 * 128 * 128 * 4
    assert hy.hyattn_state_pool_bytes(-1, 1, 1, 1) == 0


def test_slot_pool_matches_reference_simulation():
    h = hy.hyattn_state_pool_create(FAKE, 1 << 40, 3, 6, 2, 64)
    sim = ref.SlotAllocator(6)
    rng = np.random.default_rng(0)
    held = []
    for _ in range(300):
        if rng.random() < 0.55:
            n = int(rng.integers(0, 4))
            want = sim.alloc(n)
            if want is None:
                with pytest.raises(hy.HyattnError) as e:
                    hy.hyattn_state_pool_alloc(h, n)
                assert e.value.status == hy.ERR_OUT_OF_SLOTS
            else:
                got = hy.hyattn_state_pool_alloc(h, n)
                assert got == want
                held += got
        elif held:
            k = int(rng.integers(1, len(held) + 1))
            idx = rng.choice(len(held), size=k, replace=False)
            ids = [held[i] for i in idx]
            assert sim.free(ids)
            hy.hyattn_state_pool_free(h, ids)
            held = [x for x in held if x not in ids]
        assert hy.hyattn_state_pool_in_use(h) == sim.in_use()
    hy.hyattn_state_pool_destroy(h)


def test_slot_free_errors_change_nothing():
    h = hy.hyattn_state_pool_create(FAKE, 1 << 40, 1, 4, 1, 64)
    assert hy.hyattn_state_pool_alloc(h, 2) == [0, 1]
    for bad in ([2], [0, 0], [7], [-1], [0, 3]):
        with pytest.raises(hy.HyattnError) as e:
            hy.hyattn_state_pool_free(h, bad)
        assert e.value.status == hy.ERR_BAD_SLOT
        assert hy.hyattn_state_pool_in_use(h) == 2
    hy.hyattn_state_pool_free(h, [1, 0])
    assert hy.hyattn_state_pool_in_use(h) == 0
    hy.hyattn_state_pool_destroy(h)


def test_state_ptr_layout():
    h = hy.hyattn_state_pool_create(FAKE, 1 << 40, 3, 5, 2, 128)
    slot_bytes = 2 * 128 * 128 * 4
    assert hy.hyattn_state_pool_state_ptr(h, 0, 0) == FAKE
    assert hy.hyattn_state_pool_state_ptr(h, 2, 3) == FAKE + (2 * 5 + 3) * slot_bytes
    assert hy.hyattn_state_pool_state_ptr(h, 3, 0) is None
    hy.hyattn_state_pool_destroy(h)


def test_pool_create_validation():
    for args, st in (((None, 1 << 30, 1, 1, 1, 64), hy.ERR_INVALID_ARG),
                     ((FAKE, 100, 1, 1, 1, 64), hy.ERR_INVALID_ARG),
                     ((FAKE + 4, 1 << 30, 1, 1, 1, 64), hy.ERR_INVALID_ARG),
                     ((FAKE, 1 << 30, 1, 1, 1, 96), hy.ERR_UNSUPPORTED),
                     ((FAKE, 1 << 30, 0, 1, 1, 64), hy.ERR_INVALID_ARG),
                     ((FAKE, 1 << 40, 1, 1, 65536, 128), hy.ERR_UNSUPPORTED)):  # H D = 2^23
        with pytest.raises(hy.HyattnError) as e:
            hy.hyattn_state_pool_create(*args)
        assert e.value.status == st, args


def test_argument_validation_before_launch():
    h = hy.hyattn_state_pool_create(FAKE, 1 << 40, 2, 4, 2, 128)
    P = FAKE
    cases = [
        (lambda: hy.hyattn_linear_decode(h, 2, P, P, P, P, P, 1, hy.BF16, 0), hy.ERR_INVALID_ARG),
        (lambda: hy.hyattn_linear_decode(h, 0, None, P, P, P, P, 1, hy.BF16, 0), hy.ERR_INVALID_ARG),
        (lambda: hy.hyattn_linear_decode(h, 0, P, P, P, P, P, 1, 7, 0), hy.ERR_UNSUPPORTED),
        (lambda: hy.hyattn_linear_prefill_chunked(h, 0, P, P, P, P, P, P, 1, 17, hy.BF16, 0),
         hy.ERR_UNSUPPORTED),
        (lambda: hy.hyattn_linear_prefill_chunked(h, 0, P, P, P, P, P, P, 1, 512, hy.BF16, 0),
         hy.ERR_UNSUPPORTED),
        (lambda: hy.hyattn_linear_prefill_chunked(h, 0, P, P, P, P, P, P, 1, 256, hy.F32, 0),
         hy.ERR_UNSUPPORTED),
        (lambda: hy.hyattn_paged_decode(P, P, P, P, 10, P, 4, P, 64, 1, 6, 4, 128, 1.0, P, 1 << 20,
                                        hy.BF16, 0), hy.ERR_INVALID_ARG),   # 6 % 4 != 0
        (lambda: hy.hyattn_paged_decode(P, P, P, P, 10, P, 4, P, 65, 1, 8, 4, 128, 1.0, P, 1 << 20,
                                        hy.BF16, 0), hy.ERR_INVALID_ARG),   # ctx > 16 * max_blocks
        (lambda: hy.hyattn_paged_decode(P, P, P, P, 10, P, 4, P, 64, 1, 8, 4, 128, 1.0, P, 16,
                                        hy.BF16, 0), hy.ERR_INVALID_ARG),   # workspace too small
        (lambda: hy.hyattn_paged_decode(P, P, P, P, 10, P, 4, P, 64, 1, 32, 2, 128, 1.0, P, 1 << 30,
                                        hy.BF16, 0), hy.ERR_UNSUPPORTED),   # 16 q heads per KV head
        (lambda: hy.hyattn_paged_prefill(P, P, P, P, 10, P, 4, P, P, 8, 1, 8, 4, 80, 1.0, hy.BF16, 0),
         hy.ERR_UNSUPPORTED),                                               # D = 80
        (lambda: hy.hyattn_paged_append(P, P, P, P, 0, P, 4, P, P, 1, 1, 4, 128, hy.BF16, 0),
         hy.ERR_INVALID_ARG),                                               # no blocks
    ]
    for i, (fn, st) in enumerate(cases):
        with pytest.raises(hy.HyattnError) as e:
            fn()
        assert e.value.status == st, (i, e.value)
    # zero-sized calls are no-ops that succeed without a device
    hy.hyattn_linear_decode(h, 0, None, None, None, None, None, 0, hy.BF16, 0)
    hy.hyattn_linear_prefill_chunked(h, 0, None, None, None, None, None, None, 0, 64, hy.BF16, 0)
    hy.hyattn_state_pool_destroy(h)


def test_gated_argument_validation_before_launch():
    """Gated state update (the Mamba/RWKV-style layers of P2 §1.3, read as one
    scalar forget factor per token and head): the factors are a required
    input of the gated calls and belong to linear layers only; both mistakes
    are refused on the host before any launch."""
    h = hy.hyattn_state_pool_create(FAKE, 1 << 40, 2, 4, 2, 128)
    P = FAKE
    cases = [
        (lambda: hy.hyattn_linear_decode_gated(h, 0, P, P, P, None, P, P, 1, hy.BF16, 0),
         hy.ERR_INVALID_ARG),                                               # no log_gamma
        (lambda: hy.hyattn_linear_prefill_chunked_gated(h, 0, P, P, P, None, P, P, P, 1, 64,
                                                        hy.BF16, 0), hy.ERR_INVALID_ARG),
        (lambda: hy.hyattn_linear_decode_gated(h, 2, P, P, P, P, P, P, 1, hy.BF16, 0),
         hy.ERR_INVALID_ARG),                                               # layer out of range
        (lambda: hy.hyattn_linear_prefill_chunked_gated(h, 0, P, P, P, P, P, P, P, 1, 17,
                                                        hy.BF16, 0), hy.ERR_UNSUPPORTED),
        (lambda: hy.hyattn_linear_decode_gated(h, 0, P, P, P, P, P, P, -1, hy.BF16, 0),
         hy.ERR_INVALID_ARG),
    ]
    for i, (fn, st) in enumerate(cases):
        with pytest.raises(hy.HyattnError) as e:
            fn()
        assert e.value.status == st, (i, e.value)
    # zero-sized gated calls succeed without touching the device, log_gamma or not
    hy.hyattn_linear_decode_gated(h, 0, None, None, None, None, None, None, 0, hy.BF16, 0)
    hy.hyattn_linear_prefill_chunked_gated(h, 0, None, None, None, None, None, None, None, 0, 64,
                                           hy.BF16, 0)
    # a full layer that carries forget factors is a caller mistake
    b = hy.make_batch(n_prefill=0, n_decode=1, decode_slots=FAKE, H=2, H_kv=2, D=128,
                      chunk_size=64, dtype=hy.BF16, block_tables=FAKE, context_lens=FAKE,
                      cu_q_lens=FAKE, max_blocks_per_seq=4, n_blocks=8, max_context=64,
                      workspace=FAKE, workspace_bytes=1 << 20, scale=1.0)
    lin = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, log_gamma=FAKE)
    full = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, k_pool=FAKE, v_pool=FAKE, log_gamma=FAKE)
    with pytest.raises(hy.HyattnError) as e:
        hy.hyattn_hybrid_step([hy.LAYER_LINEAR, hy.LAYER_FULL], 2, [lin, full], b, h, 0)
    assert e.value.status == hy.ERR_INVALID_ARG
    assert "log_gamma" in e.value.message
    hy.hyattn_state_pool_destroy(h)


def test_unknown_layer_type_rejected_before_any_launch():
    """P1 §4.3: an unsupported attention type is refused; nothing is launched."""
    h = hy.hyattn_state_pool_create(FAKE, 1 << 40, 2, 4, 2, 128)
    b = hy.make_batch(n_prefill=0, n_decode=1, decode_slots=FAKE, H=2, H_kv=2, D=128,
                      chunk_size=64, dtype=hy.BF16, block_tables=FAKE, context_lens=FAKE,
                      cu_q_lens=FAKE, max_blocks_per_seq=4, n_blocks=8, max_context=64,
                      workspace=FAKE, workspace_bytes=1 << 20, scale=1.0)
    layers = [dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, k_pool=FAKE, v_pool=FAKE)] * 3
    for types in ([0, 2, 1], [1, 0, -1], [5, 5, 5]):
        with pytest.raises(hy.HyattnError) as e:
            hy.hyattn_hybrid_step(types, 3, layers, b, h, 0)
        assert e.value.status == hy.ERR_UNSUPPORTED_LAYER
        assert "layer" in e.value.message
    # missing KV pool on a full layer is caught before launches too
    bad = [dict(layers[0]), dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE)]
    with pytest.raises(hy.HyattnError) as e:
        hy.hyattn_hybrid_step([0, 1], 2, bad, b, h, 0)
    assert e.value.status == hy.ERR_INVALID_ARG
    hy.hyattn_state_pool_destroy(h)


def test_layer_type_spellings_map_like_the_oracle():
    from linear_attention_attn_amd import layer_types
    assert layer_types.parse(["linear", "full_attn", "linear_attn", "full"]) == [0, 1, 0, 1]
    assert layer_types.parse(["linear", "full"]) == ref.parse_layer_types(["linear", "full"])
    with pytest.raises(ValueError):
        layer_types.parse(["mamba"])


def test_memory_estimate_matches_the_oracle_exactly():
    """hyattn_estimate_memory (host) == the oracle's integer formula (P2 §3.3)."""
    rng = np.random.default_rng(31)
    names = {0: "linear", 1: "full"}
    for trial in range(25):
        n = int(rng.integers(0, 40))
        codes = rng.integers(0, 2, size=n).tolist()
        ctx = rng.integers(0, 200000, size=int(rng.integers(0, 300))).tolist()
        H, H_kv, D = int(rng.choice([8, 32, 64])), int(rng.choice([1, 8, 32])), int(rng.choice([64, 128]))
        kvb, stb = int(rng.choice([2, 4])), int(rng.choice([2, 4]))
        got = hy.hyattn_estimate_memory(codes, H, H_kv, D, ctx, kvb, stb)
        want = ref.memory_estimate([names[c] for c in codes], H, H_kv, D, ctx, kvb, stb)
        assert got == want, (trial, got, want)
    # the state pool of this library is the fp32 figure
    e = hy.hyattn_estimate_memory([0] * 24 + [1] * 8, 32, 8, 128, [5] * 256, 2, 4)
    assert e["state_bytes"] == hy.hyattn_state_pool_bytes(24, 256, 32, 128)


def test_memory_estimate_errors():
    with pytest.raises(hy.HyattnError) as ex:
        hy.hyattn_estimate_memory([0, 7], 32, 8, 128, [1], 2, 4)
    assert ex.value.status == hy.ERR_UNSUPPORTED_LAYER
    with pytest.raises(hy.HyattnError) as ex:
        hy.hyattn_estimate_memory([0, 1], 32, 8, 128, [1, -1], 2, 4)
    assert ex.value.status == hy.ERR_INVALID_ARG
    with pytest.raises(hy.HyattnError) as ex:  # beyond 2^64 - 1 bytes
        hy.hyattn_estimate_memory([1] * 100000, 2**31 - 1, 2**31 - 1, 2**31 - 1, [2**31 - 1] * 4, 4, 4)
    assert ex.value.status == hy.ERR_INVALID_ARG



def test_bucket_by_length_matches_the_oracle_exactly():
    rng = np.random.default_rng(12)
    for trial in range(40):
        n = int(rng.integers(0, 300))
        mix = rng.integers(0, 3, n)  # short, medium and long requests
        lengths = np.where(mix == 0, rng.integers(0, 64, n),
                           np.where(mix == 1, rng.integers(64, 2048, n), rng.integers(2048, 32768, n)))
        T = int(rng.integers(max(int(lengths.max(initial=0)), 1), 200000))
        R = int(rng.integers(1, 64))
        assert hy.hyattn_bucket_by_length(lengths, T, R) == ref.bucket_by_length(lengths, T, R)


def test_bucket_by_length_errors_leave_outputs_untouched():
    L = hy.load()
    ln = np.array([3, 11], np.int32)
    order = np.full(2, -7, np.int32)
    offs = np.full(3, -7, np.int32)
    nb = C.c_int(-7)
    for T, R, lens in ((10, 4, ln), (0, 4, ln[:1]), (10, 0, ln[:1]),
                       (10, 4, np.array([2, -1], np.int32))):
        st = L.hyattn_bucket_by_length(lens.ctypes.data, int(lens.size), T, R, order.ctypes.data,
                                       offs.ctypes.data, C.byref(nb))
        assert st == hy.ERR_INVALID_ARG
        assert (order == -7).all() and (offs == -7).all() and nb.value == -7
    assert L.hyattn_bucket_by_length(None, 0, 5, 5, None, offs.ctypes.data, C.byref(nb)) == 0
    assert nb.value == 0 and offs[0] == 0
    assert L.hyattn_bucket_by_length(None, -1, 5, 5, None, offs.ctypes.data, C.byref(nb)) != 0
