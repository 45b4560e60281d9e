"""hyattn_ref -- Python side of the fp64 CPU oracle.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline may import this module. It loads ``libhyattn_ref.so`` (plain C, built
with gcc from ``hyattn_ref.c``) and composes its per-unit routines into the
operations of the hybrid attention step. It never imports the HIP package.

Cited pages: "P2" = "推理框架适配Hybrid Model：KV Cache管理与算子调度实战",
"P1" = "Hybrid Model推理适配：vLLM与SGLang的工程实践指南".

Every function works on host numpy arrays. bf16 tensors are ``uint16`` bit
patterns, fp32 tensors ``float32``; results are float64.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hyattn_ref.c")
_LIB = os.path.join(_HERE, "libhyattn_ref.so")

F32, BF16, F64 = 0, 1, 2
BLOCK = 16

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            L = C.CDLL(_LIB)
            vp, i64, i32p = C.c_void_p, C.c_int64, C.POINTER(C.c_int32)
            dp = C.POINTER(C.c_double)
            for name in ("ref_linear_recurrent", "ref_linear_closed_form"):
                f = getattr(L, name)
                f.argtypes = [C.c_int, C.c_int, C.c_int, vp, vp, vp, i64, i64, dp, dp, i64]
                f.restype = None
            L.ref_linear_chunked.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, vp,
                                             i64, i64, dp, dp, i64]
            L.ref_linear_chunked.restype = None
            for name in ("ref_linear_gated_recurrent", "ref_linear_gated_chunked"):
                f = getattr(L, name)
                head = [C.c_int, C.c_int] if name.endswith("chunked") else [C.c_int]
                f.argtypes = head + [C.c_int, C.c_int, vp, vp, vp, i64, i64, C.c_int, vp, i64,
                                     i64, dp, dp, i64]
                f.restype = None
            L.ref_kv_offset.argtypes = [i32p, C.c_int, C.c_int, C.c_int, C.c_int]
            L.ref_kv_offset.restype = C.c_int64
            L.ref_paged_attention_query.argtypes = [C.c_int, C.c_int, vp, i64, C.c_int, vp, vp,
                                                    C.c_int, C.c_int, i32p, C.c_int, C.c_double,
                                                    dp]
            L.ref_paged_attention_query.restype = C.c_int
            _lib = L
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle input dtype {a.dtype} not supported")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_double))


def n_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _pmap(fn, items, threads=None):
    items = list(items)
    threads = threads or n_threads()
    if threads <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:  # ctypes calls drop the GIL
        return list(ex.map(fn, items))


# ----------------------------------------------------------- linear layers --
def linear_unit(form: str, q, k, v, S, token0: int, T: int, head: int, chunk: int = 0,
                log_gamma=None):
    """Run one (request, head) unit on packed [N_tok][H][D] inputs.

    form: "recurrent" (the token recurrence), "chunked" (P2 §2.4 chunk form with
    chunk size ``chunk``) or "closed" (whole-sequence closed form).
    S: float64 [D][D] prior state, updated in place. Returns out [T][D] f64.
    log_gamma: None (plain layer) or the per-token log forget factors
    [N_tok][H] (float32 or float64) of the gated variant; forms "recurrent"
    and "chunked" only.
    """
    L = lib()
    assert q.dtype == k.dtype == v.dtype and q.shape == k.shape == v.shape
    N, H, D = q.shape
    assert 0 <= token0 and token0 + T <= N and 0 <= head < H
    assert S.dtype == np.float64 and S.shape == (D, D) and S.flags.c_contiguous
    o = np.zeros((max(T, 1), D), dtype=np.float64)
    off, ldx = (token0 * H + head) * D, H * D
    args = (_dt(q), _ptr(q), _ptr(k), _ptr(v), off, ldx, _dptr(S), _dptr(o), D)
    if T > 0 and log_gamma is not None:
        g = np.ascontiguousarray(log_gamma)
        assert g.shape == (N, H) and g.dtype in (np.float32, np.float64)
        gargs = (_dt(q), _ptr(q), _ptr(k), _ptr(v), off, ldx, _dt(g), _ptr(g), token0 * H + head,
                 H, _dptr(S), _dptr(o), D)
        if form == "recurrent":
            L.ref_linear_gated_recurrent(T, D, *gargs)
        elif form == "chunked":
            L.ref_linear_gated_chunked(T, int(chunk), D, *gargs)
        else:
            raise ValueError(form)
    elif T > 0:
        if form == "recurrent":
            L.ref_linear_recurrent(T, D, *args)
        elif form == "chunked":
            L.ref_linear_chunked(T, int(chunk), D, *args)
        elif form == "closed":
            L.ref_linear_closed_form(T, D, *args)
        else:
            raise ValueError(form)
    return o[:T]


def linear_prefill(q, k, v, cu_seqlens, states, chunk: int = 0, form: str = "chunked",
                   units=None, threads=None, log_gamma=None):
    """Prefill of packed requests (P2 §2.1 recurrence, §2.4 chunking).

    states: float64 [n_req][H][D][D], updated in place (the slot's state on
    entry: zero at request start). Returns out float64 [N][H][D] (rows of
    units not listed in ``units`` stay zero). log_gamma [N][H]: the gated
    variant's per-token log forget factors (None: plain layer).
    """
    N, H, D = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n_req = len(cu) - 1
    out = np.zeros((N, H, D), dtype=np.float64)
    if units is None:
        units = [(r, h) for r in range(n_req) for h in range(H)]

    def run(u):
        r, h = u
        S = np.ascontiguousarray(states[r, h])
        t0, T = int(cu[r]), int(cu[r + 1] - cu[r])
        o = linear_unit(form, q, k, v, S, t0, T, h, chunk, log_gamma)
        states[r, h] = S
        out[t0:t0 + T, h] = o

    _pmap(run, units, threads)
    return out


def linear_decode(q, k, v, states, units=None, threads=None, log_gamma=None):
    """One decode step for B requests: per (r, h), S += k (x) v then o = q . S
    (gated variant: S <- exp(g) S + k (x) v with g = log_gamma[r][h]).

    q/k/v: [B][H][D]; states float64 [B][H][D][D] updated in place.
    """
    B, H, D = q.shape
    cu = np.arange(B + 1)
    return linear_prefill(q, k, v, cu, states, form="recurrent", units=units, threads=threads,
                          log_gamma=log_gamma)


# ------------------------------------------------------------- full layers --
def kv_offset(block_table_row, p: int, H_kv: int, g: int, D: int) -> int:
    bt = np.ascontiguousarray(block_table_row, dtype=np.int32)
    return int(lib().ref_kv_offset(bt.ctypes.data_as(C.POINTER(C.c_int32)), int(p), H_kv, g, D))


def append_kv(pool, new, block_tables, context_lens, cu_q_lens):
    """Expected pool after writing new tokens through the block tables.

    pool [n_blocks][H_kv][16][D] (copied), new [N_q][H_kv][D]; the i-th new
    token of request r goes to logical position ctx_r - q_len_r + i.
    """
    out = pool.copy()
    flat = out.reshape(-1)
    n_blocks, H_kv, _, D = pool.shape
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    for r in range(len(cu) - 1):
        ql = int(cu[r + 1] - cu[r])
        for i in range(ql):
            p = int(context_lens[r]) - ql + i
            for g in range(H_kv):
                o = kv_offset(block_tables[r], p, H_kv, g, D)
                flat[o:o + D] = new[cu[r] + i, g]
    return out


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, scale,
                    units=None, threads=None):
    """Softmax attention over paged KV (P2 §2.3), decode or causal prefill.

    q [N_q][H_q][D]; pools [n_blocks][H_kv][16][D]; request r owns query rows
    cu_q_lens[r] .. cu_q_lens[r+1]-1, and its i-th query sits at position
    ctx_r - q_len_r + i, attending to keys 0 .. that position (inclusive).
    ``units``: optional list of (r, h) to compute. Returns float64 [N_q][H_q][D].
    """
    L = lib()
    Nq, Hq, D = q.shape
    n_blocks, H_kv, blk, D2 = k_pool.shape
    assert blk == BLOCK and D2 == D and Hq % H_kv == 0
    group = Hq // H_kv
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    B = len(cu) - 1
    bts = np.ascontiguousarray(block_tables, dtype=np.int32)
    out = np.zeros((Nq, Hq, D), dtype=np.float64)
    if units is None:
        units = [(r, h) for r in range(B) for h in range(Hq)]
    dq, dkv = _dt(q), _dt(k_pool)

    def run(u):
        r, h = u
        ql = int(cu[r + 1] - cu[r])
        btp = bts[r].ctypes.data_as(C.POINTER(C.c_int32))
        buf = np.zeros(D, dtype=np.float64)
        for i in range(ql):
            n_keys = int(context_lens[r]) - ql + i + 1
            row = int(cu[r]) + i
            rc = L.ref_paged_attention_query(D, dq, _ptr(q), (row * Hq + h) * D, dkv,
                                             _ptr(k_pool), _ptr(v_pool), H_kv, h // group,
                                             btp, n_keys, float(scale), _dptr(buf))
            if rc != 0:
                raise ValueError(f"block table of request {r} misses a block")
            out[row, h] = buf

    _pmap(run, units, threads)
    return out


# ------------------------------------------------------- memory estimate --
def memory_estimate(layer_types, H, H_kv, D, context_lens, kv_elem_bytes, state_elem_bytes):
    """Device bytes of the two state kinds (P2 §3.3, P2 §2.1), exact integers.

    Full layers: K and V of every cached token, 2 * L_full * H_kv * D * S *
    elem bytes summed over requests (P2 §3.3's 2 x L x H x D x S x batch x
    dtype with per-request S); the paged pool holds whole 16-token blocks, so
    each S rounds up to a multiple of 16 there (P2 §2.1). Linear layers: one
    H x D x D state per request, L_lin * H * D * D * batch * elem bytes,
    independent of S. layer_types are names or codes as in
    ``parse_layer_types``.
    """
    types = parse_layer_types(layer_types)
    n_full = sum(1 for t in types if t == 1)
    n_lin = sum(1 for t in types if t == 0)
    ctx = [int(c) for c in context_lens]
    if any(c < 0 for c in ctx):
        raise ValueError("negative context length")
    tokens = sum(ctx)
    blocks = sum(-(-c // BLOCK) for c in ctx)
    per_token = 2 * n_full * H_kv * D * kv_elem_bytes
    return {"kv_bytes": per_token * tokens,
            "kv_paged_bytes": per_token * blocks * BLOCK,
            "kv_blocks": blocks,
            "state_bytes": n_lin * H * D * D * len(ctx) * state_elem_bytes,
            "n_full_layers": n_full, "n_linear_layers": n_lin}


# ------------------------------------------------- length-bucketed batches --
def bucket_by_length(lengths, max_padded_tokens, max_requests):
    """Group requests of similar length into batches (P2 §2.4 scheduling).

    Reading of P2 §2.4: a full layer pays for its batch's longest sequence
    (padding), a linear layer does not, so batches are formed from requests of
    similar length. A batch's cost is its request count times its longest
    length; each batch stays within max_padded_tokens of that cost and
    max_requests requests. Requests are taken shortest first (ties by index)
    and a new batch starts when the next request would break a limit.
    Returns a list of batches, each a list of request indices.
    """
    lengths = [int(x) for x in lengths]
    if max_padded_tokens < 1 or max_requests < 1:
        raise ValueError("limits must be >= 1")
    if any(x < 0 or x > max_padded_tokens for x in lengths):
        raise ValueError("a length is negative or exceeds max_padded_tokens")
    ranked = sorted(range(len(lengths)), key=lambda r: (lengths[r], r))
    batches = []
    for r in ranked:
        cur = batches[-1] if batches else None
        if cur is not None and len(cur) + 1 <= max_requests and \
                (len(cur) + 1) * max(lengths[j] for j in cur + [r]) <= max_padded_tokens:
            cur.append(r)
        else:
            batches.append([r])
    return batches


# -------------------------------------------------------- state-pool slots --
class SlotAllocator:
    """Reference simulation of the state-pool slot free list.

    Reading of P2 §1.3/§2.3 (state buffer bound to the request, allocated at
    its start and released at its end): alloc(n) hands out the n lowest free
    ids in ascending order, or nothing at all when fewer than n are free;
    free() returns ids to the pool and rejects ids that are not in use.
    """

    def __init__(self, n_slots: int):
        self.n = n_slots
        self.used = [False] * n_slots

    def alloc(self, n: int):
        free = [i for i in range(self.n) if not self.used[i]]
        if n < 0 or n > len(free):
            return None
        got = free[:n]
        for i in got:
            self.used[i] = True
        return got

    def free(self, ids) -> bool:
        ids = list(ids)
        if len(set(ids)) != len(ids) or any(not (0 <= i < self.n) or not self.used[i] for i in ids):
            return False
        for i in ids:
            self.used[i] = False
        return True

    def in_use(self) -> int:
        return sum(self.used)


# ------------------------------------------------------- the hybrid step --
LAYER_NAMES = {"linear": 0, "linear_attn": 0, "full": 1, "full_attn": 1}


def parse_layer_types(names):
    """Map the config spellings of P2 §2.2 / P1 §3.2 to LINEAR (0) / FULL (1)."""
    out = []
    for i, n in enumerate(names):
        if n not in LAYER_NAMES:
            raise ValueError(f"layer {i}: attention type {n!r} is not supported")
        out.append(LAYER_NAMES[n])
    return out


def hybrid_step(layer_types, layers, batch, linear_states, kv_pools, threads=None,
                units_linear=None, units_full=None):
    """One attention step over all layers of a hybrid model (P2 §2.2, §2.3).

    layer_types: list of 0 (linear) / 1 (full).
    layers[i]: dict with q, k, v (linear: [N][H][D]; full: q [N][Hq][D],
      k, v [N][Hkv][D]); a linear layer may add g, the gated variant's log
      forget factors [N][H].
    batch: dict with prefill_cu (int [n_p+1]), n_decode, block_tables
      ([n_p+n_d][max_blocks]), context_lens ([n_p+n_d]), chunk, scale.
      Token rows: prefill requests first (packed), then one row per decode
      request.
    linear_states: float64 [L_lin][n_p+n_d][H][D][D] -- state of each request
      (prefill requests first), updated in place.
    kv_pools: list over full layers of (k_pool, v_pool), appended in place.
    Returns the list of per-layer outputs (float64).
    """
    cu_p = np.asarray(batch["prefill_cu"], dtype=np.int64)
    n_p = len(cu_p) - 1
    n_d = int(batch["n_decode"])
    Np = int(cu_p[-1])
    cu_all = np.concatenate([cu_p, Np + np.arange(1, n_d + 1)])
    outs = []
    li = fi = 0
    for t, io in zip(layer_types, layers):
        if t == 0:
            st = linear_states[li]
            q, k, v = io["q"], io["k"], io["v"]
            N, H, D = q.shape
            o = np.zeros((N, H, D))
            units_p = None if units_linear is None else [u for u in units_linear if u[0] < n_p]
            g = io.get("g")  # gated variant: log forget factors [N][H]
            o[:Np] = linear_prefill(q[:Np], k[:Np], v[:Np], cu_p, st[:n_p],
                                    chunk=batch["chunk"], form="chunked", units=units_p,
                                    threads=threads,
                                    log_gamma=None if g is None else g[:Np])[:Np]
            units_d = None if units_linear is None else [(r - n_p, h) for r, h in units_linear
                                                         if r >= n_p]
            if n_d:
                o[Np:] = linear_decode(q[Np:], k[Np:], v[Np:], st[n_p:], units=units_d,
                                       threads=threads, log_gamma=None if g is None else g[Np:])
            outs.append(o)
            li += 1
        elif t == 1:
            kp, vp = kv_pools[fi]
            kp[...] = append_kv(kp, io["k"], batch["block_tables"], batch["context_lens"],
                                cu_all)
            vp[...] = append_kv(vp, io["v"], batch["block_tables"], batch["context_lens"],
                                cu_all)
            outs.append(paged_attention(io["q"], kp, vp, batch["block_tables"],
                                        batch["context_lens"], cu_all, batch["scale"],
                                        units=units_full, threads=threads))
            fi += 1
        else:
            raise ValueError(f"unsupported layer type {t}")
    return outs
