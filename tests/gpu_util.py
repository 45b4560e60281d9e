"""Helpers shared by the GPU parity tests: host<->device copies of stored
tensors and the tolerance rules.

Tolerances (the fp32 and bf16 rules applied to every parity comparison):
  * fp32 I/O: max_i |g_i - r_i| / max(|r_i|, RMS(r)) <= 1e-4.
  * bf16 I/O: max_i |g_i - r_i| / RMS(r_v) <= 2e-2 and mean_i |g_i - r_i| / RMS(r_v)
    <= 5e-3, where r_v is the output vector (the D values of one token and head)
    that element i belongs to; a vector whose reference is exactly zero must be
    exactly zero. Normalising by the RMS of the whole tensor instead makes the
    bound unattainable even for the correctly rounded fp64 result whenever row
    magnitudes differ (the first rows of a causal prefill average over a few
    keys): rounding alone scores ~2.1e-2 there. ``rounding_floor`` reports what
    the correctly rounded oracle scores under the same rule.
  * fp32 states in bf16 runs use the fp32 rule.

Every bf16 comparison also bounds the error element by element against the
rounding floor, the error |RNE(r_i) - r_i| that the correctly rounded exact
result itself carries. If a kernel's value before its final rounding, y_i, is
within delta_i of r_i, then its bf16 output satisfies
    |RNE(y_i) - r_i| <= |RNE(r_i) - r_i| + 2 delta_i
(when RNE(y_i) != RNE(r_i), a rounding midpoint m lies between r_i and y_i;
the nearer neighbour of r_i is then h - |r_i - m| away and RNE(y_i) at most
h + |r_i - m|, h being half the bf16 spacing at m, with |r_i - m| <= delta_i).
delta_i comes from each kernel's arithmetic, not from measured errors:
  * fp32-faithful kernels (the linear layers: fp32 accumulation, bf16 operands
    that are exact inputs or hi + lo splits of fp32 values, which carry a
    value to 2^-16 relative): delta_i = 1e-4 * max(|r_i|, RMS(r_v)), the fp32
    rule the same kernels meet with fp32 I/O;
  * softmax attention kernels, which round the weights p_j to bf16 (unit
    roundoff u = 2^-8) and use the same rounded weights in P.V and in the
    normaliser: with p~_j = p_j (1 + e_j) and w_j the exact weights,
        y - r = sum_j w_j e_j (v_j - r) / (1 + sum_j w_j e_j),
    bounded by u/(1-u) * A_i with A_i = sum_j w_j |v_ij - r_i| in the worst
    case, and, treating the e_j as independent and zero-mean (the standard
    probabilistic model of rounding errors), by u/(1-u) * 8 sqrt(S2_i),
    S2_i = sum_j w_j^2 (v_ij - r_i)^2, except with probability below 3e-14
    per element (Hoeffding's inequality); delta_i adds the smaller of the two
    to the fp32 term above.
A kernel that lost the lo half of a split, or rounded an operand the design
keeps in fp32, moves some outputs past this bound.
"""
from __future__ import annotations

import os

import numpy as np

TOL_F32 = 1e-4
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 5e-3


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    """Upload a stored tensor: uint16 arrays become bfloat16, others keep dtype."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(a).cuda()


def host(x) -> np.ndarray:
    """Download: bfloat16 tensors come back as uint16 bit patterns."""
    t = torch()
    x = x.detach()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def err_f32(g, r):
    g, r = as_f64(np.asarray(g)), np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    den = np.maximum(np.abs(r), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(g - r) / den)) if r.size else 0.0


def err_bf16(g, r):
    """(max, mean) of |g - r| / RMS of r's output vector (last axis)."""
    g, r = as_f64(np.asarray(g)), np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0, 0.0
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    zero = rms == 0
    d = np.abs(g - r) / np.where(zero, 1.0, rms)
    d = np.where(zero & (g != 0), np.inf, np.where(zero, 0.0, d))
    return float(d.max()), float(d.mean())


def err_bf16_tensor(g, r):
    """(max, mean) of |g - r| / RMS of the whole tensor (reported, not asserted)."""
    g, r = as_f64(np.asarray(g)), np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    d = np.abs(g - r) / (rms if rms > 0 else 1.0)
    return (float(d.max()), float(d.mean())) if r.size else (0.0, 0.0)


def rounding_floor(r):
    """bf16 error of the correctly rounded reference itself, per the bf16 rule."""
    r = np.asarray(r, np.float64)
    rne = (r.astype(np.float32).view(np.uint32).astype(np.uint64))
    rne = ((rne + 0x7FFF + ((rne >> 16) & 1)) >> 16).astype(np.uint16)
    return err_bf16(rne, r)


def assert_f32(g, r, what="", tol=TOL_F32):
    e = err_f32(g, r)
    assert np.isfinite(as_f64(np.asarray(g))).all(), f"{what}: non-finite values"
    assert e <= tol, f"{what}: fp32 max rel error {e:.3e} > {tol:.0e}"
    return e


U_BF16 = 2.0 ** -8  # unit roundoff of bfloat16 (8 significant bits)
# (what, error max, error mean, floor max, floor mean, margin max, margin mean) of every
# bf16 comparison of the session, relative to the RMS of each output vector
BF16_REPORT: list = []


def bf16_floor_elem(r):
    """|RNE_bf16(r_i) - r_i| for each element of a float64 array, exactly: the
    distance from r_i to the nearest bf16 value."""
    a = np.abs(np.asarray(r, np.float64))
    t = (a.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).astype(np.int64)
    best = None
    for d in (-0x10000, 0, 0x10000):
        c = np.clip(t + d, 0, 0x7F7F0000).astype(np.uint32).view(np.float32).astype(np.float64)
        e = np.abs(c - a)
        best = e if best is None else np.minimum(best, e)
    return best


def fp32_delta(r):
    """Pre-rounding error bound of an fp32-faithful kernel: 1e-4 * max(|r_i|, RMS(r_v))."""
    r = np.asarray(r, np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    return TOL_F32 * np.maximum(np.abs(r), rms)


def _p_rounding_term(Q, K, V, npos, scale, R):
    """u/(1-u) * min(A, 8 sqrt(S2)) per element for query rows Q [M, D] over keys K, V
    [n, D] (row i sees keys 0 .. npos[i]-1) with exact outputs R [M, D]."""
    M, D = Q.shape
    n = K.shape[0]
    s = (Q @ K.T) * scale
    s[np.arange(n)[None, :] >= np.asarray(npos)[:, None]] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    out = np.empty((M, D))
    step = 8192  # keys per pass: the temporaries are reused, never reallocated
    dev = np.empty((min(step, n), D))
    tmp = np.empty_like(dev)
    for i in range(M):
        A = np.zeros(D)
        S2 = np.zeros(D)
        w2 = w[i] * w[i]
        for j0 in range(0, n, step):
            j1 = min(n, j0 + step)
            d, t = dev[:j1 - j0], tmp[:j1 - j0]
            np.subtract(V[j0:j1], R[i], out=d)
            A += w[i, j0:j1] @ np.abs(d, out=t)
            S2 += w2[j0:j1] @ np.multiply(d, d, out=t)
        out[i] = U_BF16 / (1 - U_BF16) * np.minimum(A, 8.0 * np.sqrt(S2))
    return out


def attention_delta(q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, scale, want,
                    units=None):
    """Pre-rounding error bound (delta above) of a softmax attention kernel with bf16
    weights, shaped like `want` [N_q][H_q][D]; arguments as for the oracle's
    paged_attention. Rows outside `units` get the fp32 term only."""
    want = np.asarray(want, np.float64)
    delta = fp32_delta(want)
    Nq, Hq, D = want.shape
    H_kv = k_pool.shape[1]
    G = Hq // H_kv
    cu = np.asarray(cu_q_lens, np.int64)
    q64 = as_f64(np.asarray(q))
    if units is None:
        units = [(r, h) for r in range(len(cu) - 1) for h in range(Hq)]
    cache = {}
    for r, h in units:
        ql, c = int(cu[r + 1] - cu[r]), int(context_lens[r])
        if ql == 0 or c == 0:
            continue
        key = (r, h // G)
        if key not in cache:
            nb = (c + 15) // 16
            blocks = np.asarray(block_tables[r][:nb], np.int64)
            cache = {key: (as_f64(k_pool[blocks, h // G]).reshape(nb * 16, D)[:c],
                           as_f64(v_pool[blocks, h // G]).reshape(nb * 16, D)[:c])}
        K, V = cache[key]
        rows = np.arange(int(cu[r]), int(cu[r + 1]))
        npos = c - ql + np.arange(ql) + 1
        delta[rows, h] += _p_rounding_term(q64[rows, h], K, V, npos, scale, want[rows, h])
    return delta


def assert_bf16(g, r, what="", delta=None):
    """The bf16 rule, plus the element-wise bound against the rounding floor:
    |g_i - r_i| <= |RNE(r_i) - r_i| + 2 delta_i (delta: fp32_delta(r) unless given)."""
    g64 = as_f64(np.asarray(g))
    assert np.isfinite(g64).all(), f"{what}: non-finite values"
    r = np.asarray(r, np.float64)
    mx, mean = err_bf16(g, r)
    d = fp32_delta(r) if delta is None else np.broadcast_to(np.asarray(delta, np.float64), r.shape)
    err = np.abs(g64 - r)
    floor = bf16_floor_elem(r)
    slack = 2.0 ** -40 * np.abs(r)
    bad = err > floor + 2.0 * d + slack
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    rel = lambda x: np.where(rms == 0, 0.0, x / np.where(rms == 0, 1.0, rms))
    fmx, fmean = float(rel(floor).max()) if r.size else 0.0, float(rel(floor).mean()) if r.size else 0.0
    mmx, mmean = float(rel(2 * d).max()) if r.size else 0.0, float(rel(2 * d).mean()) if r.size else 0.0
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split("::")[-1].split(" ")[0]
    BF16_REPORT.append((f"{test}: {what}" if test else what, mx, mean, fmx, fmean, mmx, mmean))
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} of {bad.size} outputs beyond rounding floor + 2 delta "
        f"(worst excess {float(rel(err - floor - 2 * d).max()):.3e} of the vector RMS; "
        f"error max {mx:.3e} mean {mean:.3e}, floor max {fmx:.3e} mean {fmean:.3e})")
    assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, (
        f"{what}: bf16 errors max {mx:.3e} (<= {TOL_BF16_MAX}), mean {mean:.3e} (<= {TOL_BF16_MEAN})")
    return mx, mean


def assert_io(g, r, dtype: str, what="", delta=None):
    return assert_f32(g, r, what) if dtype == "f32" else assert_bf16(g, r, what, delta)


def torch_dtype(dtype: str):
    t = torch()
    return t.bfloat16 if dtype == "bf16" else t.float32


def i32(a):
    t = torch()
    return t.as_tensor(np.asarray(a, dtype=np.int32)).cuda()
