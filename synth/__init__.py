"""Seeded synthetic inputs for the hybrid full/linear attention step.

This module is shared by the HIP path's tests and bench and by the CPU
oracle's tests. It holds no arithmetic of the method itself: it only draws
random numbers, rounds them to the storage dtype, and lays out block tables,
sequence lengths and slot lists. Every generator takes an explicit seed.

Recipe (stated once, used everywhere):
  * q, k, v ~ N(0, 1) * D**-0.5, drawn in float64, rounded to float32, then
    (for bf16 storage) rounded to bfloat16 with round-to-nearest-even.
  * Prior linear states ~ N(0, 1) * 0.1, float32.
  * Block pools hold 16-token blocks; a request's logical blocks map to
    physical ids through a seeded permutation of the pool, so neighbouring
    logical blocks are scattered.
  * bf16 tensors are carried on the host as ``uint16`` arrays holding the
    raw bit pattern, fp32 as ``float32``.

Large pools (tens to hundreds of GB) are drawn on the device with torch's
seeded generator (``device_normal_bf16``); the oracle side copies back the
sampled parts it needs, so both sides read identical bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16  # tokens per KV block (page 2, section 2.1: fixed 16-token blocks)


# ---------------------------------------------------------------- rounding --
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


def normal(rng: np.random.Generator, shape, scale: float, dtype: str):
    """N(0,1)*scale drawn in float64 -> float32 -> (bf16 bits | float32)."""
    x = (rng.standard_normal(size=shape) * scale).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def small_ints(rng: np.random.Generator, shape, lo: int, hi: int, dtype: str):
    """Integers in [lo, hi], exactly representable in fp32 and bf16."""
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def log_forget(rng: np.random.Generator, shape, p_one: float = 0.05):
    """Per-token log forget factors g = log(gamma) <= 0, float32, shape [N][H].

    Head h draws gamma = 1 - u * 2^-(2 + h % 8) with u ~ U(0, 1), so heads
    range from fast forgetting (gamma in [0.75, 1]) to slow (gamma within
    2^-9 of 1); a fraction p_one of the tokens has gamma = 1 exactly (g = 0).
    """
    N, H = shape
    e = 2.0 + (np.arange(H) % 8)
    gamma = 1.0 - rng.random((N, H)) * np.exp2(-e)[None, :]
    g = np.log(gamma).astype(np.float32)
    g[rng.random((N, H)) < p_one] = 0.0
    return np.minimum(g, 0.0).astype(np.float32)


def to_f32(a: np.ndarray) -> np.ndarray:
    """Widen a stored tensor (uint16 bf16 bits or float32) to float32."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


# ------------------------------------------------------- paged KV layouts --
@dataclass
class PagedLayout:
    """Block tables for B requests over a pool of ``n_blocks`` 16-token blocks.

    ``block_tables[r, j]`` is the physical block holding logical tokens
    16*j .. 16*j+15 of request r; -1 marks unused entries. Physical ids come
    from a seeded permutation, and ``spare`` ids (never referenced) are left
    over for poisoning.
    """
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, max_blocks]
    n_blocks: int
    spare: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]


def paged_layout(rng: np.random.Generator, context_lens, n_spare: int = 0,
                 max_blocks: int | None = None) -> PagedLayout:
    ctx = np.asarray(context_lens, dtype=np.int64)
    need = [(int(c) + BLOCK - 1) // BLOCK for c in ctx]
    total = int(sum(need))
    n_blocks = total + n_spare
    perm = rng.permutation(n_blocks).astype(np.int32)
    mb = max(need) if need else 0
    if max_blocks is not None:
        assert max_blocks >= mb
        mb = max_blocks
    mb = max(mb, 1)
    bt = np.full((len(ctx), mb), -1, dtype=np.int32)
    pos = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[pos:pos + n]
        pos += n
    return PagedLayout(ctx.astype(np.int32), bt, n_blocks, perm[pos:].copy())


def uniform_contexts(rng, B: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def loguniform_contexts(rng, B: int, lo: int, hi: int, force_max: bool = True) -> np.ndarray:
    u = rng.random(B)
    ctx = np.floor(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))).astype(np.int64)
    ctx = np.clip(ctx, lo, hi)
    if force_max and B > 0:
        ctx[int(np.argmax(ctx))] = hi
    return ctx.astype(np.int32)


def cu_lens(lens) -> np.ndarray:
    out = np.zeros(len(lens) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return out


# ------------------------------------------------ device-side generation --
def device_normal_bf16(shape, scale: float, seed: int, device="cuda"):
    """Draw N(0,1)*scale on the device with torch's seeded generator, bf16 (RNE).

    Used for pools far too large to draw on the host. Bits are deterministic
    for a given (seed, shape, device type).
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = x.view(-1)
    step = 1 << 28
    tmp = None
    for s in range(0, flat.numel(), step):
        n = min(step, flat.numel() - s)
        if tmp is None or tmp.numel() < n:
            tmp = torch.empty(n, dtype=torch.float32, device=device)
        t = tmp[:n]
        t.normal_(0.0, 1.0, generator=g)
        t.mul_(scale)
        flat[s:s + n].copy_(t)
    return x


# ------------------------------------------------------ workload recipes --
WORKLOADS = {
    "tiny": dict(seed=0, H=4, D=64, T=256, chunk=64, n_decode=16, dtype="f32",
                 n_blocks=32),
    "linear_decode": dict(seed=1, B=64, H=32, D=128, steps=256, dtype="bf16",
                          state_scale=0.1),
    "linear_prefill": dict(seed=2, B=8, H=32, D=128, T=8192, chunks=(64, 128, 256),
                           dtype="bf16"),
    "paged_decode": dict(seed=3, B=128, Hq=32, Hkv=8, D=128, ctx_lo=512,
                         ctx_hi=32768, dtype="bf16", n_spare=1024),
    "hybrid_step": dict(seed=4, n_layers=32, pattern=("linear", "linear", "linear", "full"),
                        H=32, Hkv=8, D=128, n_prefill=16, prefill_len=4096,
                        n_decode=240, ctx_lo=512, ctx_hi=131072, chunk=128,
                        dtype="bf16"),
}


def device_log_forget(shape, seed: int, device="cuda"):
    """log_forget's distribution drawn on the device (float32 [N][H]): head h
    takes gamma = 1 - u * 2^-(2 + h % 8), u ~ U(0, 1)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    N, H = shape
    u = torch.rand((N, H), generator=g, device=device, dtype=torch.float64)
    e = 2.0 + (torch.arange(H, device=device, dtype=torch.float64) % 8)
    return torch.log1p(-u * torch.exp2(-e)).clamp(max=0.0).to(torch.float32)


def tiny_inputs():
    """The tiny workload's inputs (WORKLOADS["tiny"]): one request of T + n_decode
    tokens, seed 0, fp32. The linear layer and the full layer each get their own q, k,
    v ~ N(0,1) * D^-0.5 of shape [T + n_decode][H][D] (the full layer has H_kv = H).
    The full layer's pool holds n_blocks 16-token blocks, all NaN at first; the
    request's blocks come from a seeded permutation of the pool, so its logical blocks
    are scattered and the blocks it never uses stay NaN."""
    cfg = WORKLOADS["tiny"]
    rng = np.random.default_rng(cfg["seed"])
    H, D, n = cfg["H"], cfg["D"], cfg["T"] + cfg["n_decode"]
    s = D ** -0.5
    lin = {x: normal(rng, (n, H, D), s, cfg["dtype"]) for x in ("q", "k", "v")}
    full = {x: normal(rng, (n, H, D), s, cfg["dtype"]) for x in ("q", "k", "v")}
    n_used = (n + BLOCK - 1) // BLOCK
    lay = paged_layout(rng, [n], n_spare=cfg["n_blocks"] - n_used)
    pool_nan = np.full((lay.n_blocks, H, BLOCK, D), np.nan, np.float32)
    return dict(cfg=cfg, linear=lin, full=full, layout=lay, k_pool=pool_nan,
                v_pool=pool_nan.copy())
