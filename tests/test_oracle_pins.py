"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against what the pages and the mathematics fix:
closed forms evaluated with library primitives, exact rational brute force on
tiny integer inputs, hand-worked special cases, textbook softmax attention on
a densely gathered KV, and invariants (chunk-size invariance, permutation
invariance of the physical block layout, GQA head mapping). The inputs are
deliberately asymmetric so that a transposed operand, a swapped index or a
dropped term changes the result.

Pages: "P2" = "推理框架适配Hybrid Model：KV Cache管理与算子调度实战".
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import synth
from oracle import ref

RTOL = 1e-12


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / scale)


def _packed(rng, N, H, D, dtype="f32", scale=None):
    s = D ** -0.5 if scale is None else scale
    return [synth.normal(rng, (N, H, D), s, dtype) for _ in range(3)]


# ------------------------------------------------------- linear attention --
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linear_forms_agree_for_every_chunk_size(dtype):
    """P2 §2.1 recurrence == §2.4 chunked form (any C) == closed form."""
    rng = np.random.default_rng(11)
    N, H, D = 37, 2, 8
    q, k, v = _packed(rng, N, H, D, dtype)
    S0 = rng.standard_normal((D, D)) * 0.3
    for h in range(H):
        Sr = S0.copy()
        o_rec = ref.linear_unit("recurrent", q, k, v, Sr, 0, N, h)
        Sc = S0.copy()
        o_cls = ref.linear_unit("closed", q, k, v, Sc, 0, N, h)
        assert _rel(o_cls, o_rec) < RTOL and _rel(Sc, Sr) < RTOL
        for C in (1, 2, 3, 5, 7, 16, 36, 37, 64, 1000):
            Sk = S0.copy()
            o_chk = ref.linear_unit("chunked", q, k, v, Sk, 0, N, h, C)
            assert _rel(o_chk, o_rec) < RTOL, C
            assert _rel(Sk, Sr) < RTOL, C


def test_linear_matches_matrix_closed_form():
    """O = Q S0 + tril(Q K^T) V and S_T = S0 + K^T V, by numpy matmul."""
    rng = np.random.default_rng(12)
    N, H, D = 29, 3, 6
    q, k, v = _packed(rng, N, H, D, "f32")
    for h in range(H):
        Q, K, V = (x[:, h].astype(np.float64) for x in (q, k, v))
        S0 = rng.standard_normal((D, D))
        expect_o = Q @ S0 + np.tril(Q @ K.T) @ V
        expect_S = S0 + K.T @ V
        for form, C in (("recurrent", 0), ("chunked", 4), ("closed", 0)):
            S = S0.copy()
            o = ref.linear_unit(form, q, k, v, S, 0, N, h, C)
            assert _rel(o, expect_o) < RTOL, form
            assert _rel(S, expect_S) < RTOL, form


# ------------------------------------------- gated (decayed) linear attention --
def test_gated_with_zero_gates_is_the_plain_layer():
    """g = 0 (gamma = 1) everywhere: the gated recurrence and chunked form give
    the plain layer's results bit for bit."""
    rng = np.random.default_rng(21)
    N, H, D = 41, 2, 8
    for dtype in ("f32", "bf16"):
        q, k, v = _packed(rng, N, H, D, dtype)
        g = np.zeros((N, H), np.float32)
        S0 = rng.standard_normal((D, D)) * 0.3
        for h in range(H):
            for form, C in (("recurrent", 0), ("chunked", 1), ("chunked", 6), ("chunked", 64)):
                Sa, Sb = S0.copy(), S0.copy()
                a = ref.linear_unit(form, q, k, v, Sa, 0, N, h, C)
                b = ref.linear_unit(form, q, k, v, Sb, 0, N, h, C, log_gamma=g)
                assert np.array_equal(a, b) and np.array_equal(Sa, Sb), (dtype, form, C)


def test_gated_matches_decay_masked_matrix_form():
    """With L = cumsum(g): O = (tril(Q K^T) * exp(L_t - L_u)) V + exp(L_t) Q S0 and
    S_T = exp(L_T) S0 + K^T diag(exp(L_T - L_u)) V, by numpy matmul; the
    recurrence and the chunked form for every chunk size agree with it."""
    rng = np.random.default_rng(22)
    N, H, D = 45, 8, 6
    q, k, v = _packed(rng, N, H, D, "f32")
    g = synth.log_forget(rng, (N, H), p_one=0.2)
    for h in range(H):
        Q, K, V = (x[:, h].astype(np.float64) for x in (q, k, v))
        L = np.cumsum(g[:, h].astype(np.float64))
        M = np.tril(np.exp(L[:, None] - L[None, :]))
        S0 = rng.standard_normal((D, D))
        expect_o = ((Q @ K.T) * M) @ V + np.exp(L)[:, None] * (Q @ S0)
        expect_S = np.exp(L[-1]) * S0 + K.T @ (np.exp(L[-1] - L)[:, None] * V)
        for form, C in [("recurrent", 0)] + [("chunked", c) for c in (1, 2, 5, 16, 44, 45, 100)]:
            S = S0.copy()
            o = ref.linear_unit(form, q, k, v, S, 0, N, h, C, log_gamma=g)
            assert _rel(o, expect_o) < RTOL, (form, C)
            assert _rel(S, expect_S) < RTOL, (form, C)


def test_gated_handworked():
    """D = 2, S0 = I, gammas 1/2 then 1/4, worked by hand:
    S1 = I/2 + k1 v1^T = [[2.5, 0], [2, 0.5]], o1 = row 0 of S1 = (2.5, 0);
    S2 = S1/4 + k2 v2^T = [[0.625, 0], [1.5, 1.125]], o2 = row 1 of S2 = (1.5, 1.125)."""
    q = np.array([[[1, 0]], [[0, 1]]], np.float64)
    k = np.array([[[1, 1]], [[0, 1]]], np.float64)
    v = np.array([[[2, 0]], [[1, 1]]], np.float64)
    g = np.log(np.array([[0.5], [0.25]]))
    for form, C in (("recurrent", 0), ("chunked", 1), ("chunked", 2)):
        S = np.eye(2)
        o = ref.linear_unit(form, q, k, v, S, 0, 2, 0, C, log_gamma=g)
        assert np.allclose(o, [[2.5, 0], [1.5, 1.125]], rtol=0, atol=1e-14), form
        assert np.allclose(S, [[0.625, 0], [1.5, 1.125]], rtol=0, atol=1e-14), form


def test_gated_full_forgetting():
    """gamma = 0 (g = -1000 underflows exp to 0): each token sees only itself,
    o_t = (q_t . k_t) v_t, and the state ends as k_T (x) v_T."""
    rng = np.random.default_rng(23)
    N, H, D = 20, 1, 5
    q, k, v = _packed(rng, N, H, D, "f32")
    g = np.full((N, H), -1000.0)
    Q, K, V = (x[:, 0].astype(np.float64) for x in (q, k, v))
    for form, C in (("recurrent", 0), ("chunked", 7)):
        S = rng.standard_normal((D, D))
        o = ref.linear_unit(form, q, k, v, S, 0, N, 0, C, log_gamma=g)
        assert _rel(o, np.sum(Q * K, axis=1)[:, None] * V) < RTOL
        assert _rel(S, np.outer(K[-1], V[-1])) < RTOL


def test_linear_exact_rational_bruteforce():
    """Tiny integer case, exact: o_t[j] = sum_i q_t[i] S0[i][j] + sum_{u<=t} (q_t.k_u) v_u[j]."""
    rng = np.random.default_rng(13)
    T, D = 6, 3
    q = rng.integers(-3, 4, size=(T, 1, D)).astype(np.float32)
    k = rng.integers(-3, 4, size=(T, 1, D)).astype(np.float32)
    v = rng.integers(-3, 4, size=(T, 1, D)).astype(np.float32)
    S0 = rng.integers(-2, 3, size=(D, D)).astype(np.float64)
    Fq = [[Fraction(int(x)) for x in q[t, 0]] for t in range(T)]
    Fk = [[Fraction(int(x)) for x in k[t, 0]] for t in range(T)]
    Fv = [[Fraction(int(x)) for x in v[t, 0]] for t in range(T)]
    FS = [[Fraction(int(S0[i, j])) for j in range(D)] for i in range(D)]
    expect = []
    for t in range(T):
        row = []
        for j in range(D):
            acc = sum(Fq[t][i] * FS[i][j] for i in range(D))
            for u in range(t + 1):
                acc += sum(Fq[t][i] * Fk[u][i] for i in range(D)) * Fv[u][j]
            row.append(acc)
        expect.append(row)
    S_T = [[FS[i][j] + sum(Fk[u][i] * Fv[u][j] for u in range(T)) for j in range(D)]
           for i in range(D)]
    for form, C in (("recurrent", 0), ("chunked", 4), ("chunked", 1), ("closed", 0)):
        S = S0.copy()
        o = ref.linear_unit(form, q, k, v, S, 0, T, 0, C)
        assert all(o[t, j] == float(expect[t][j]) for t in range(T) for j in range(D)), form
        assert all(S[i, j] == float(S_T[i][j]) for i in range(D) for j in range(D)), form


def test_linear_handworked_orientation():
    """D=2 hand-worked case that separates S from S^T and inclusive from exclusive.

    One token from a zero state: S = k v^T = [[1*3, 1*5], [2*3, 2*5]] = [[3,5],[6,10]];
    o = q S with q = (1, 0) -> (3, 5) (the transpose would give (3, 6); an
    exclusive read, using the state before the token, would give (0, 0)).
    A second token k=(0,1), v=(1,0): S = [[3,5],[7,10]]; with q=(0,1): o = (7, 10).
    """
    q = np.array([[[1, 0]], [[0, 1]]], np.float32)
    k = np.array([[[1, 2]], [[0, 1]]], np.float32)
    v = np.array([[[3, 5]], [[1, 0]]], np.float32)
    for form in ("recurrent", "chunked", "closed"):
        S = np.zeros((2, 2))
        o = ref.linear_unit(form, q, k, v, S, 0, 2, 0, 2)
        assert o.tolist() == [[3.0, 5.0], [7.0, 10.0]], form
        assert S.tolist() == [[3.0, 5.0], [7.0, 10.0]], form


def test_prefill_then_decode_equals_longer_prefill():
    """P2 §4.1: decode continues from the prefill state (no re-zeroing)."""
    rng = np.random.default_rng(14)
    N, H, D = 40, 2, 8
    q, k, v = _packed(rng, N, H, D, "bf16")
    st = np.zeros((1, H, D, D))
    o_full = ref.linear_prefill(q, k, v, [0, N], st, chunk=16)
    st2 = np.zeros((1, H, D, D))
    o_a = ref.linear_prefill(q[:33], k[:33], v[:33], [0, 33], st2, chunk=16)
    outs = [o_a]
    for t in range(33, N):
        outs.append(ref.linear_decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], st2))
    assert _rel(np.concatenate(outs), o_full) < RTOL
    assert _rel(st2, st) < RTOL


def test_batch_and_slot_invariance():
    """P2 §3.5: a request alone == the same request inside a batch."""
    rng = np.random.default_rng(15)
    H, D = 2, 8
    lens = [5, 17, 0, 9]
    cu = synth.cu_lens(lens)
    q, k, v = _packed(rng, int(cu[-1]), H, D, "f32")
    st = np.zeros((4, H, D, D))
    o = ref.linear_prefill(q, k, v, cu, st, chunk=4)
    for r, L in enumerate(lens):
        s1 = np.zeros((1, H, D, D))
        sl = slice(int(cu[r]), int(cu[r + 1]))
        o1 = ref.linear_prefill(q[sl], k[sl], v[sl], [0, L], s1, chunk=4)
        assert np.array_equal(o1, o[sl]) and np.array_equal(s1[0], st[r])


# --------------------------------------------------------- paged attention --
def _dense_attention(q, K, V, scale):
    """Textbook softmax attention on a plain array (scipy softmax)."""
    s = scale * (K.astype(np.float64) @ q.astype(np.float64))
    return softmax(s) @ V.astype(np.float64)


def _gather(pool, bt_row, n, g):
    """Logical K (or V) rows 0..n-1 of KV head g, by walking blocks in order."""
    rows = []
    for blk_idx in range((n + 15) // 16):
        blk = int(bt_row[blk_idx])
        take = min(16, n - 16 * blk_idx)
        rows.append(synth.to_f32(pool[blk, g, :take]))
    return np.concatenate(rows, axis=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_decode_matches_dense_softmax(dtype):
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D = 5, 4, 2, 16
    ctx = np.array([1, 16, 17, 50, 33], np.int32)
    lay = synth.paged_layout(rng, ctx, n_spare=3)
    kp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, dtype)
    vp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, dtype)
    q = synth.normal(rng, (B, Hq, D), 1.0, dtype)
    scale = D ** -0.5
    o = ref.paged_attention(q, kp, vp, lay.block_tables, ctx, np.arange(B + 1), scale)
    for r in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            K = _gather(kp, lay.block_tables[r], int(ctx[r]), g)
            V = _gather(vp, lay.block_tables[r], int(ctx[r]), g)
            e = _dense_attention(synth.to_f32(q[r, h]), K, V, scale)
            assert _rel(o[r, h], e) < 1e-12


def test_paged_prefill_is_causal_dense_softmax():
    """Query i of a q_len-token chunk sees keys 0 .. ctx - q_len + i."""
    rng = np.random.default_rng(22)
    Hq, Hkv, D = 2, 1, 8
    ctx = np.array([40, 7], np.int32)
    qlen = [12, 7]
    cu = synth.cu_lens(qlen)
    lay = synth.paged_layout(rng, ctx)
    kp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "f32")
    vp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "f32")
    q = synth.normal(rng, (int(cu[-1]), Hq, D), 1.0, "f32")
    o = ref.paged_attention(q, kp, vp, lay.block_tables, ctx, cu, 0.3)
    for r in range(2):
        K = _gather(kp, lay.block_tables[r], int(ctx[r]), 0)
        V = _gather(vp, lay.block_tables[r], int(ctx[r]), 0)
        for i in range(qlen[r]):
            n = int(ctx[r]) - qlen[r] + i + 1
            for h in range(Hq):
                e = _dense_attention(q[cu[r] + i, h], K[:n], V[:n], 0.3)
                assert _rel(o[cu[r] + i, h], e) < 1e-12


def test_paged_special_cases():
    rng = np.random.default_rng(23)
    D, Hkv = 8, 1
    lay = synth.paged_layout(rng, [1, 35])
    kp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "f32")
    vp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "f32")
    q = synth.normal(rng, (2, 1, D), 1.0, "f32")
    # one key: softmax of a single score is 1, the output is that value row
    o = ref.paged_attention(q[:1], kp, vp, lay.block_tables[:1], [1], [0, 1], 0.7)
    assert np.array_equal(o[0, 0], vp[lay.block_tables[0, 0], 0, 0].astype(np.float64))
    # all keys equal: uniform weights, the output is the mean of the values
    kp2 = kp.copy()
    kp2[...] = kp[0, 0, 0]
    o = ref.paged_attention(q[1:], kp2, vp, lay.block_tables[1:], [35], [0, 1], 0.7)
    V = _gather(vp, lay.block_tables[1], 35, 0).astype(np.float64)
    assert _rel(o[0, 0], V.mean(axis=0)) < 1e-13
    # no keys: zero output (padded batch entry)
    o = ref.paged_attention(q[:1], kp, vp, lay.block_tables[:1], [0], [0, 1], 0.7)
    assert not o.any()


def test_paged_onehot_probe_is_exact():
    """A key of 64*e0 against q = 64*e0 makes every other weight underflow to 0."""
    rng = np.random.default_rng(24)
    D, Hkv, n = 8, 1, 45
    lay = synth.paged_layout(rng, [n], n_spare=2)
    kp = np.zeros((lay.n_blocks, Hkv, 16, D), np.float32)
    vp = np.zeros_like(kp)
    for p in range(n):  # v encodes the logical position
        vp[lay.block_tables[0, p // 16], 0, p % 16, :] = p
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 64.0
    for target in (0, 15, 16, 31, 44):
        k2 = kp.copy()
        k2[lay.block_tables[0, target // 16], 0, target % 16, 0] = 64.0
        o = ref.paged_attention(q, k2, vp, lay.block_tables, [n], [0, 1], 1.0)
        assert o[0, 0].tolist() == [float(target)] * D


def test_paged_permutation_invariance_and_gqa():
    """Same logical KV in two physical layouts -> identical outputs; head h reads h // group."""
    rng = np.random.default_rng(25)
    Hq, Hkv, D = 6, 3, 8
    ctx = np.array([20, 33], np.int32)
    lay1 = synth.paged_layout(np.random.default_rng(1), ctx, n_spare=4)
    lay2 = synth.paged_layout(np.random.default_rng(2), ctx, n_spare=4)
    assert not np.array_equal(lay1.block_tables, lay2.block_tables)
    logical_k = synth.normal(rng, (2, 48, Hkv, D), 1.0, "f32")
    logical_v = synth.normal(rng, (2, 48, Hkv, D), 1.0, "f32")
    pools = []
    for lay in (lay1, lay2):
        kp = np.full((lay.n_blocks, Hkv, 16, D), np.nan, np.float32)
        vp = np.full_like(kp, np.nan)
        for r in range(2):
            for p in range(int(ctx[r])):
                b = lay.block_tables[r, p // 16]
                kp[b, :, p % 16] = logical_k[r, p]
                vp[b, :, p % 16] = logical_v[r, p]
        pools.append((lay, kp, vp))
    q = synth.normal(rng, (2, Hq, D), 1.0, "f32")
    o1, o2 = (ref.paged_attention(q, kp, vp, lay.block_tables, ctx, [0, 1, 2], 0.5)
              for lay, kp, vp in pools)
    assert np.array_equal(o1, o2) and np.isfinite(o1).all()
    for r in range(2):
        for h in range(Hq):
            g = h // 2
            e = _dense_attention(q[r, h], logical_k[r, :ctx[r], g], logical_v[r, :ctx[r], g], 0.5)
            assert _rel(o1[r, h], e) < 1e-12


def test_kv_offset_handworked():
    """Pool [n_blocks][H_kv][16][D]: token p of KV head g at ((bt[p//16]*H_kv+g)*16 + p%16)*D."""
    bt = np.array([5, 2, 7, -1], np.int32)
    assert ref.kv_offset(bt, 0, 2, 0, 4) == ((5 * 2 + 0) * 16 + 0) * 4
    assert ref.kv_offset(bt, 17, 2, 1, 4) == ((2 * 2 + 1) * 16 + 1) * 4 == 324
    assert ref.kv_offset(bt, 47, 3, 2, 8) == ((7 * 3 + 2) * 16 + 15) * 8 == 3064
    assert ref.kv_offset(bt, 48, 3, 2, 8) == -1


def test_append_kv_handworked():
    pool = np.zeros((3, 1, 16, 2), np.float32)
    bt = np.array([[2, 0]], np.int32)
    new = np.array([[[1, 2]], [[3, 4]]], np.float32)
    out = ref.append_kv(pool, new, bt, [17], [0, 2])  # positions 15 and 16
    expect = np.zeros_like(pool)
    expect[2, 0, 15] = [1, 2]
    expect[0, 0, 0] = [3, 4]
    assert np.array_equal(out, expect)


# ------------------------------------------------------------ slots/types --
def test_slot_allocator_reading():
    a = ref.SlotAllocator(5)
    assert a.alloc(2) == [0, 1] and a.alloc(2) == [2, 3]
    assert a.alloc(2) is None and a.in_use() == 4  # all-or-nothing
    assert a.free([1]) and a.alloc(1) == [1]       # lowest free id first
    assert not a.free([4]) and not a.free([0, 0])  # not in use / duplicate
    assert a.free([0, 2, 3, 1]) and a.in_use() == 0
    assert a.alloc(5) == [0, 1, 2, 3, 4]


def test_layer_type_names():
    assert ref.parse_layer_types(["linear", "full", "linear_attn", "full_attn"]) == [0, 1, 0, 1]
    with pytest.raises(ValueError):
        ref.parse_layer_types(["linear", "ssm"])


def test_hybrid_step_composes_the_layer_ops():
    rng = np.random.default_rng(31)
    H, Hkv, D = 2, 1, 8
    pre = [9, 20]
    cu_p = synth.cu_lens(pre)
    n_d = 3
    ctx = np.array([9, 20, 30, 5, 17], np.int32)
    lay = synth.paged_layout(rng, ctx, n_spare=2)
    N = int(cu_p[-1]) + n_d
    types = ref.parse_layer_types(["linear", "full", "linear"])
    layers = []
    for t in types:
        if t == 0:
            q, k, v = _packed(rng, N, H, D, "f32")
        else:
            q = synth.normal(rng, (N, H, D), 1.0, "f32")
            k = synth.normal(rng, (N, Hkv, D), 1.0, "f32")
            v = synth.normal(rng, (N, Hkv, D), 1.0, "f32")
        layers.append(dict(q=q, k=k, v=v))
    states = rng.standard_normal((2, 5, H, D, D)) * 0.1
    states[:, :2] = 0.0  # prefill requests start from zero
    kp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "f32")
    vp = synth.normal(rng, (lay.n_blocks, Hkv, 16, D), 1.0, "f32")
    batch = dict(prefill_cu=cu_p, n_decode=n_d, block_tables=lay.block_tables,
                 context_lens=ctx, chunk=4, scale=0.35)
    st0 = states.copy()
    kp0, vp0 = kp.copy(), vp.copy()
    outs = ref.hybrid_step(types, layers, batch, states, [(kp, vp)])
    # layer 0 / 2: linear, recurrent reference per request
    for li, l in ((0, 0), (1, 2)):
        io = layers[l]
        for r in range(5):
            if r < 2:
                sl = slice(int(cu_p[r]), int(cu_p[r + 1]))
            else:
                sl = slice(int(cu_p[-1]) + r - 2, int(cu_p[-1]) + r - 1)
            for h in range(H):
                S = st0[li, r, h].copy()
                o = ref.linear_unit("recurrent", io["q"][sl], io["k"][sl], io["v"][sl], S, 0,
                                    sl.stop - sl.start, h)
                assert _rel(outs[l][sl, h], o) < 1e-12 and _rel(states[li, r, h], S) < 1e-12
    # layer 1: full, dense attention over the appended logical KV
    cu_all = np.concatenate([cu_p, cu_p[-1] + np.arange(1, n_d + 1)])
    kpa = ref.append_kv(kp0, layers[1]["k"], lay.block_tables, ctx, cu_all)
    vpa = ref.append_kv(vp0, layers[1]["v"], lay.block_tables, ctx, cu_all)
    assert np.array_equal(kp, kpa) and np.array_equal(vp, vpa)
    for r in range(5):
        K = _gather(kpa, lay.block_tables[r], int(ctx[r]), 0)
        V = _gather(vpa, lay.block_tables[r], int(ctx[r]), 0)
        ql = int(cu_all[r + 1] - cu_all[r])
        for i in range(ql):
            n = int(ctx[r]) - ql + i + 1
            for h in range(H):
                e = _dense_attention(layers[1]["q"][cu_all[r] + i, h], K[:n], V[:n], 0.35)
                assert _rel(outs[1][cu_all[r] + i, h], e) < 1e-12


@pytest.mark.parametrize("gated", [False, True])
def test_hybrid_step_two_steps_equal_one_step(gated):
    """P2 §2.4: a prompt cut into two chunks, with K/V kept in the pools and the
    linear state carried between them (same cut for every layer), gives what
    one step over the whole prompt gives; a decode request's two tokens over
    two steps equal a two-token chunk with its earlier context."""
    from synth import hybrid
    from tests import hybrid_run
    case = hybrid.continuation_case(seed=3, n_layers=4, H=2, Hkv=1, D=16,
                                    prompts=((40, 17), (9, 1), (33, 32)), decode_prior=(1, 45),
                                    chunk=8, dtype="f32", gated=gated)
    a_outs, a_states, a_pools = hybrid_run.run_oracle_steps(case)
    b_outs, b_states, b_pools = hybrid_run.run_oracle_whole(case)
    for a, b in zip(a_outs, b_outs):
        assert _rel(a, b) < 1e-12
    assert _rel(a_states, b_states) < 1e-12
    for (ka, va), (kb, vb) in zip(a_pools, b_pools):
        assert np.array_equal(ka.view(np.uint8), kb.view(np.uint8))  # unwritten rows are NaN
        assert np.array_equal(va.view(np.uint8), vb.view(np.uint8))
        assert not np.isnan(ka[case["layout"].block_tables[0, :2]]).any()


# ------------------------------------------------------- memory estimate --
def _golden(name):
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    vals = {}
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = (x.strip() for x in line.split("="))
            vals[k] = int(v)
    return vals


def test_memory_estimate_reproduces_the_pages_worked_example():
    """P2 §3.3 prints ~103 GB of full-layer KV and ~67 MB of linear state for
    32 layers (24 full, 8 linear), H = 32, D = 128, S = 32768, batch 8, bf16."""
    g = _golden("p2_s3_3_memory_example.txt")
    types = ["full"] * g["n_full_layers"] + ["linear"] * g["n_linear_layers"]
    assert len(types) == g["n_layers"]
    est = ref.memory_estimate(types, g["heads"], g["heads"], g["head_dim"],
                              [g["seq_len"]] * g["batch"], g["dtype_bytes"], g["dtype_bytes"])
    assert round(est["kv_bytes"] / 1e9) == g["printed_full_kv_gb"]
    assert round(est["state_bytes"] / 1e6) == g["printed_linear_state_mb"]
    assert est["kv_paged_bytes"] == est["kv_bytes"]  # 32768 is a whole number of blocks
    assert est["kv_blocks"] == g["batch"] * g["seq_len"] // 16


def test_memory_estimate_invariants():
    """Block rounding, independence of the state from the length, linearity."""
    types = ["linear", "full", "linear", "linear"]
    per_tok = 2 * 1 * 8 * 128 * 2
    e = ref.memory_estimate(types, 32, 8, 128, [1], 2, 4)
    assert e["kv_bytes"] == per_tok and e["kv_paged_bytes"] == 16 * per_tok and e["kv_blocks"] == 1
    e2 = ref.memory_estimate(types, 32, 8, 128, [100000], 2, 4)
    assert e2["state_bytes"] == e["state_bytes"] == 3 * 32 * 128 * 128 * 4
    e3 = ref.memory_estimate(types, 32, 8, 128, [17, 32, 0], 2, 4)
    assert e3["kv_blocks"] == 2 + 2 + 0 and e3["kv_bytes"] == 49 * per_tok
    assert e3["state_bytes"] == 3 * e["state_bytes"]
    assert ref.memory_estimate(["linear"], 32, 8, 128, [4096], 2, 4)["kv_bytes"] == 0
    with pytest.raises(ValueError):
        ref.memory_estimate(["sliding"], 32, 8, 128, [1], 2, 4)



# ------------------------------------------------- length-bucketed batches --
def _set_partitions(items):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in _set_partitions(rest):
        yield [[first]] + part
        for i in range(len(part)):
            yield part[:i] + [[first] + part[i]] + part[i + 1:]


def _feasible(batch, lengths, T, R):
    return len(batch) <= R and len(batch) * max(lengths[r] for r in batch) <= T


def test_bucket_by_length_handworked():
    # sorted: 1 (r1), 3 (r2), 3 (r3), 5 (r0), 8 (r4); budget 9:
    # 1,3,3 -> 3 x 3 = 9 fits; adding 5 gives 4 x 5 = 20; 5 then 8 gives 2 x 8 = 16
    assert ref.bucket_by_length([5, 1, 3, 3, 8], 9, 4) == [[1, 2, 3], [0], [4]]
    assert ref.bucket_by_length([5, 1, 3, 3, 8], 9, 2) == [[1, 2], [3], [0], [4]]
    assert ref.bucket_by_length([4, 4, 4], 100, 1) == [[0], [1], [2]]
    assert ref.bucket_by_length([7, 2, 9, 2], 10 ** 6, 8) == [[1, 3, 0, 2]]
    assert ref.bucket_by_length([], 5, 5) == []
    assert ref.bucket_by_length([0, 0, 0], 1, 2) == [[0, 1], [2]]
    with pytest.raises(ValueError):
        ref.bucket_by_length([3, 11], 10, 4)


def test_bucket_by_length_fewest_batches_by_brute_force():
    """Against every grouping of small request sets: the batches are valid,
    cover each request once, and no valid grouping has fewer batches."""
    rng = np.random.default_rng(8)
    for trial in range(60):
        n = int(rng.integers(1, 8))
        lengths = [int(x) for x in rng.integers(0, 20, n)]
        T = int(rng.integers(max(lengths + [1]), 60))
        R = int(rng.integers(1, 5))
        got = ref.bucket_by_length(lengths, T, R)
        assert sorted(r for b in got for r in b) == list(range(n))
        assert all(_feasible(b, lengths, T, R) for b in got)
        best = min(len(p) for p in _set_partitions(list(range(n)))
                   if all(_feasible(b, lengths, T, R) for b in p))
        assert len(got) == best, (lengths, T, R, got)
        # similar lengths together: batches are consecutive runs of the sorted order
        flat = [r for b in got for r in b]
        assert flat == sorted(range(n), key=lambda r: (lengths[r], r))
