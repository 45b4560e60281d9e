"""Thin ctypes binding of libhyattn (the C ABI declared in include/hyattn.h).

Functions carry the C names and argument order. Pointer arguments accept a
torch tensor (its data_ptr() is passed), a plain integer address, or None.
``stream`` defaults to torch's current stream. Every call is argument
marshalling only; all computation happens in the library's HIP kernels. A
non-OK status raises HyattnError with the library's message.

The library must be built (``python -m linear_attention_attn_amd._build`` or
``__graft_entry__.build()``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhyattn.so")

OK, ERR_INVALID_ARG, ERR_OUT_OF_SLOTS, ERR_BAD_SLOT = 0, 1, 2, 3
ERR_UNSUPPORTED_LAYER, ERR_UNSUPPORTED, ERR_HIP = 4, 5, 6
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "OUT_OF_SLOTS", 3: "BAD_SLOT",
                4: "UNSUPPORTED_LAYER", 5: "UNSUPPORTED", 6: "HIP"}
F32, BF16 = 0, 1
LAYER_LINEAR, LAYER_FULL = 0, 1

# Every entry point the header declares (checked by the CPU test suite).
EXPORTS = (
    "hyattn_last_error", "hyattn_abi_version", "hyattn_state_pool_bytes",
    "hyattn_state_pool_create", "hyattn_state_pool_destroy", "hyattn_state_pool_alloc",
    "hyattn_state_pool_zero", "hyattn_state_pool_free", "hyattn_state_pool_in_use",
    "hyattn_state_pool_state_ptr", "hyattn_linear_prefill_chunked", "hyattn_linear_decode",
    "hyattn_paged_append", "hyattn_paged_decode_workspace_bytes", "hyattn_paged_decode",
    "hyattn_paged_prefill", "hyattn_hybrid_workspace_bytes", "hyattn_hybrid_step",
    "hyattn_estimate_memory",
    "hyattn_linear_prefill_chunked_gated", "hyattn_linear_decode_gated",
    "hyattn_bucket_by_length", "hyattn_paged_decode_noalloc",
)


class HyattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hyattn {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class LayerIO(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("o", C.c_void_p),
                ("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("log_gamma", C.c_void_p)]


class Batch(C.Structure):
    _fields_ = [("n_prefill", C.c_int), ("n_decode", C.c_int),
                ("cu_seqlens", C.c_void_p), ("n_prefill_tokens", C.c_int),
                ("max_prefill_len", C.c_int), ("prefill_slots", C.c_void_p),
                ("decode_slots", C.c_void_p), ("block_tables", C.c_void_p),
                ("max_blocks_per_seq", C.c_int), ("context_lens", C.c_void_p),
                ("cu_q_lens", C.c_void_p), ("max_context", C.c_int), ("n_blocks", C.c_int64),
                ("H", C.c_int), ("H_kv", C.c_int), ("D", C.c_int), ("chunk_size", C.c_int),
                ("scale", C.c_float), ("dtype", C.c_int), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t)]


class MemoryEstimate(C.Structure):
    _fields_ = [("kv_bytes", C.c_uint64), ("kv_paged_bytes", C.c_uint64),
                ("kv_blocks", C.c_uint64), ("state_bytes", C.c_uint64),
                ("n_full_layers", C.c_int), ("n_linear_layers", C.c_int)]


_lib = None
ABI_VERSION = 2  # must match hyattn_abi_version() of the loaded library


def lib_path() -> str:
    return LIB_PATH


def load():
    """Load libhyattn.so, building it first only if no built library exists."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import _build
        _build.build()
    L = C.CDLL(LIB_PATH)
    vp, i, i64, sz, f = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_float
    st = C.c_int
    sig = {
        "hyattn_last_error": ([], C.c_char_p),
        "hyattn_abi_version": ([], i),
        "hyattn_state_pool_bytes": ([i, i, i, i], sz),
        "hyattn_state_pool_create": ([vp, sz, i, i, i, i, C.POINTER(vp)], st),
        "hyattn_state_pool_destroy": ([vp], st),
        "hyattn_state_pool_alloc": ([vp, i, vp], st),
        "hyattn_state_pool_zero": ([vp, vp, i, vp], st),
        "hyattn_state_pool_free": ([vp, vp, i], st),
        "hyattn_state_pool_in_use": ([vp], i),
        "hyattn_state_pool_state_ptr": ([vp, i, i], vp),
        "hyattn_linear_prefill_chunked": ([vp, i, vp, vp, vp, vp, vp, vp, i, i, i, vp], st),
        "hyattn_linear_decode": ([vp, i, vp, vp, vp, vp, vp, i, i, vp], st),
        "hyattn_linear_prefill_chunked_gated": ([vp, i, vp, vp, vp, vp, vp, vp, vp, i, i, i, vp],
                                                st),
        "hyattn_linear_decode_gated": ([vp, i, vp, vp, vp, vp, vp, vp, i, i, vp], st),
        "hyattn_paged_append": ([vp, vp, vp, vp, i64, vp, i, vp, vp, i, i, i, i, i, vp], st),
        "hyattn_paged_decode_workspace_bytes": ([i, i, i, i], sz),
        "hyattn_paged_decode": ([vp, vp, vp, vp, i64, vp, i, vp, i, i, i, i, i, f, vp, sz, i,
                                 vp], st),
        "hyattn_paged_prefill": ([vp, vp, vp, vp, i64, vp, i, vp, vp, i, i, i, i, i, f, i, vp],
                                 st),
        "hyattn_paged_decode_noalloc": ([vp, vp, vp, vp, i64, vp, i, vp, i, i, i, i, i, f, i, vp],
                                        st),
        "hyattn_hybrid_workspace_bytes": ([C.POINTER(Batch)], sz),
        "hyattn_hybrid_step": ([vp, i, C.POINTER(LayerIO), C.POINTER(Batch), vp, vp], st),
        "hyattn_estimate_memory": ([vp, i, i, i, i, vp, i, i, i, C.POINTER(MemoryEstimate)], st),
        "hyattn_bucket_by_length": ([vp, i, i64, i, vp, vp, C.POINTER(C.c_int)], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    if L.hyattn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH}: ABI version {L.hyattn_abi_version()}, this binding "
                           f"expects {ABI_VERSION}; rebuild the library")
    _lib = L
    return L


# ------------------------------------------------------------- marshalling --
def ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr() if x.numel() > 0 else None
    if hasattr(x, "ctypes"):  # numpy (host arrays)
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def last_error() -> str:
    return load().hyattn_last_error().decode()


def _check(status: int):
    if status != OK:
        raise HyattnError(status, last_error())


# ------------------------------------------------------------- entry points --
def hyattn_abi_version() -> int:
    return load().hyattn_abi_version()


def hyattn_state_pool_bytes(n_linear_layers, n_slots, H, D) -> int:
    return load().hyattn_state_pool_bytes(n_linear_layers, n_slots, H, D)


def hyattn_state_pool_create(dev_buf, nbytes, n_linear_layers, n_slots, H, D):
    h = C.c_void_p()
    _check(load().hyattn_state_pool_create(ptr(dev_buf), nbytes, n_linear_layers, n_slots, H, D,
                                           C.byref(h)))
    return h.value


def hyattn_state_pool_destroy(pool):
    _check(load().hyattn_state_pool_destroy(pool))


def hyattn_state_pool_alloc(pool, n):
    out = (C.c_int32 * max(n, 1))()
    _check(load().hyattn_state_pool_alloc(pool, n, C.cast(out, C.c_void_p)))
    return [int(out[i]) for i in range(n)]


def hyattn_state_pool_zero(pool, slots_dev, n, stream=None):
    _check(load().hyattn_state_pool_zero(pool, ptr(slots_dev), n, _stream(stream)))


def hyattn_state_pool_free(pool, slots):
    arr = (C.c_int32 * max(len(slots), 1))(*slots)
    _check(load().hyattn_state_pool_free(pool, C.cast(arr, C.c_void_p), len(slots)))


def hyattn_state_pool_in_use(pool) -> int:
    return load().hyattn_state_pool_in_use(pool)


def hyattn_state_pool_state_ptr(pool, linear_layer, slot):
    return load().hyattn_state_pool_state_ptr(pool, linear_layer, slot)


def hyattn_linear_prefill_chunked(pool, linear_layer, q, k, v, o, cu_seqlens, slots, n_req,
                                  chunk_size, dtype, stream=None):
    _check(load().hyattn_linear_prefill_chunked(pool, linear_layer, ptr(q), ptr(k), ptr(v),
                                                ptr(o), ptr(cu_seqlens), ptr(slots), n_req,
                                                chunk_size, dtype, _stream(stream)))


def hyattn_linear_decode(pool, linear_layer, q, k, v, o, slots, B, dtype, stream=None):
    _check(load().hyattn_linear_decode(pool, linear_layer, ptr(q), ptr(k), ptr(v), ptr(o),
                                       ptr(slots), B, dtype, _stream(stream)))


def hyattn_linear_prefill_chunked_gated(pool, linear_layer, q, k, v, log_gamma, o, cu_seqlens,
                                        slots, n_req, chunk_size, dtype, stream=None):
    _check(load().hyattn_linear_prefill_chunked_gated(pool, linear_layer, ptr(q), ptr(k), ptr(v),
                                                      ptr(log_gamma), ptr(o), ptr(cu_seqlens),
                                                      ptr(slots), n_req, chunk_size, dtype,
                                                      _stream(stream)))


def hyattn_linear_decode_gated(pool, linear_layer, q, k, v, log_gamma, o, slots, B, dtype,
                               stream=None):
    _check(load().hyattn_linear_decode_gated(pool, linear_layer, ptr(q), ptr(k), ptr(v),
                                             ptr(log_gamma), ptr(o), ptr(slots), B, dtype,
                                             _stream(stream)))


def hyattn_paged_append(k_new, v_new, k_pool, v_pool, n_blocks, block_tables, max_blocks_per_seq,
                        context_lens, cu_q_lens, B, max_q_len, H_kv, D, dtype, stream=None):
    _check(load().hyattn_paged_append(ptr(k_new), ptr(v_new), ptr(k_pool), ptr(v_pool), n_blocks,
                                      ptr(block_tables), max_blocks_per_seq, ptr(context_lens),
                                      ptr(cu_q_lens), B, max_q_len, H_kv, D, dtype,
                                      _stream(stream)))


def hyattn_paged_decode_workspace_bytes(B, H_q, D, max_context) -> int:
    return load().hyattn_paged_decode_workspace_bytes(B, H_q, D, max_context)


def hyattn_paged_decode(q, o, k_pool, v_pool, n_blocks, block_tables, max_blocks_per_seq,
                        context_lens, max_context, B, H_q, H_kv, D, scale, workspace,
                        workspace_bytes, dtype, stream=None):
    _check(load().hyattn_paged_decode(ptr(q), ptr(o), ptr(k_pool), ptr(v_pool), n_blocks,
                                      ptr(block_tables), max_blocks_per_seq, ptr(context_lens),
                                      max_context, B, H_q, H_kv, D, float(scale), ptr(workspace),
                                      workspace_bytes, dtype, _stream(stream)))


def hyattn_paged_decode_noalloc(q, o, k_pool, v_pool, n_blocks, block_tables, max_blocks_per_seq,
                                context_lens, max_context, B, H_q, H_kv, D, scale, dtype,
                                stream=None):
    _check(load().hyattn_paged_decode_noalloc(ptr(q), ptr(o), ptr(k_pool), ptr(v_pool), n_blocks,
                                              ptr(block_tables), max_blocks_per_seq,
                                              ptr(context_lens), max_context, B, H_q, H_kv, D,
                                              float(scale), dtype, _stream(stream)))


def hyattn_paged_prefill(q, o, k_pool, v_pool, n_blocks, block_tables, max_blocks_per_seq,
                         context_lens, cu_q_lens, max_q_len, B, H_q, H_kv, D, scale, dtype,
                         stream=None):
    _check(load().hyattn_paged_prefill(ptr(q), ptr(o), ptr(k_pool), ptr(v_pool), n_blocks,
                                       ptr(block_tables), max_blocks_per_seq, ptr(context_lens),
                                       ptr(cu_q_lens), max_q_len, B, H_q, H_kv, D, float(scale),
                                       dtype, _stream(stream)))


def make_batch(**kw) -> Batch:
    b = Batch()
    for name, _ in Batch._fields_:
        if name in kw:
            val = kw[name]
            setattr(b, name, ptr(val) if _is_ptr_field(name) else val)
    return b


def _is_ptr_field(name):
    return dict(Batch._fields_)[name] is C.c_void_p


def make_layers(layers) -> "C.Array":
    arr = (LayerIO * max(len(layers), 1))()
    for i, L in enumerate(layers):
        for name, _ in LayerIO._fields_:
            setattr(arr[i], name, ptr(L.get(name)))
    return arr


def hyattn_hybrid_workspace_bytes(batch: Batch) -> int:
    return load().hyattn_hybrid_workspace_bytes(C.byref(batch))


def hyattn_hybrid_step(layer_types, n_layers, layers, batch: Batch, pool, stream=None):
    lt = (C.c_int32 * max(n_layers, 1))(*layer_types)
    arr = layers if isinstance(layers, C.Array) else make_layers(layers)
    _check(load().hyattn_hybrid_step(C.cast(lt, C.c_void_p), n_layers, arr, C.byref(batch), pool,
                                     _stream(stream)))


def hyattn_estimate_memory(layer_types, H, H_kv, D, context_lens, kv_elem_bytes, state_elem_bytes):
    """Host-only memory estimate; returns a dict of the hyattn_memory_estimate fields."""
    import numpy as np
    lt = np.ascontiguousarray(layer_types, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = MemoryEstimate()
    _check(load().hyattn_estimate_memory(ptr(lt) if lt.size else None, int(lt.size), int(H), int(H_kv),
                                         int(D), ptr(cl) if cl.size else None, int(cl.size),
                                         int(kv_elem_bytes), int(state_elem_bytes), C.byref(out)))
    return {name: int(getattr(out, name)) for name, _ in MemoryEstimate._fields_}


def hyattn_bucket_by_length(lengths, max_padded_tokens, max_requests):
    """Host-only length-bucketed batch formation; returns a list of batches,
    each a list of request indices."""
    import numpy as np
    ln = np.ascontiguousarray(lengths, dtype=np.int32)
    order = np.zeros(max(ln.size, 1), np.int32)
    offs = np.zeros(ln.size + 1, np.int32)
    nb = C.c_int(0)
    _check(load().hyattn_bucket_by_length(ptr(ln) if ln.size else None, int(ln.size),
                                          int(max_padded_tokens), int(max_requests), ptr(order),
                                          ptr(offs), C.byref(nb)))
    return [order[offs[b]:offs[b + 1]].tolist() for b in range(nb.value)]
