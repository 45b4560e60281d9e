"""Seeded inputs for one hybrid attention step (host arrays, small sizes).

A step serves ``n_prefill`` requests that bring a prompt chunk (rows first,
packed) and ``n_decode`` requests that bring one token each. Linear layers
start prefill requests from a zero state and decode requests from a random
prior state; full layers hold, for every decode request, its earlier
context_len - 1 tokens in the paged pool (prefill requests start empty).
``gated`` adds log forget factors ``g`` [N][H] to every linear layer (the
gated variant). Pure data generation: no arithmetic of the method.
"""
from __future__ import annotations

import numpy as np

from . import cu_lens, log_forget, normal, paged_layout, BF16_NAN

PATTERN = ("linear", "linear", "linear", "full")


def small_case(seed=0, n_layers=4, H=4, Hkv=2, D=128, prefill_lens=(40, 70),
               decode_ctx=(1, 17, 300), chunk=32, dtype="bf16", pattern=PATTERN, n_spare=4,
               gated=False):
    rng = np.random.default_rng(seed)
    types = [pattern[i % len(pattern)] for i in range(n_layers)]
    n_p, n_d = len(prefill_lens), len(decode_ctx)
    cu_p = cu_lens(prefill_lens)
    Np = int(cu_p[-1])
    N = Np + n_d
    ctx = np.array(list(prefill_lens) + list(decode_ctx), np.int32)
    lay = paged_layout(rng, ctx, n_spare=n_spare)
    n_lin = sum(t == "linear" for t in types)
    layers, pools = [], []
    scale_lin = D ** -0.5
    for t in types:
        if t == "linear":
            q, k, v = (normal(rng, (N, H, D), scale_lin, dtype) for _ in range(3))
        else:
            q = normal(rng, (N, H, D), 1.0, dtype)
            k = normal(rng, (N, Hkv, D), 1.0, dtype)
            v = normal(rng, (N, Hkv, D), 1.0, dtype)
            shape = (lay.n_blocks, Hkv, 16, D)
            nan = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
            kp = np.full(shape, nan, np.uint16 if dtype == "bf16" else np.float32)
            vp = kp.copy()
            for r in range(n_p, n_p + n_d):  # earlier tokens of decode requests
                prior = int(ctx[r]) - 1
                for j in range((prior + 15) // 16):
                    b = lay.block_tables[r, j]
                    m = min(16, prior - 16 * j)
                    kp[b, :, :m] = normal(rng, (Hkv, m, D), 1.0, dtype)
                    vp[b, :, :m] = normal(rng, (Hkv, m, D), 1.0, dtype)
            pools.append((kp, vp))
        layers.append(dict(q=q, k=k, v=v))
        if gated and t == "linear":  # the gated variant's log forget factors
            layers[-1]["g"] = log_forget(rng, (N, H))
    states = np.zeros((n_lin, n_p + n_d, H, D, D), np.float32)
    states[:, n_p:] = (rng.standard_normal((n_lin, n_d, H, D, D)) * 0.1).astype(np.float32)
    return dict(types=types, layers=layers, pools=pools, states=states, layout=lay, ctx=ctx,
                prefill_cu=cu_p, n_prefill=n_p, n_decode=n_d, N=N, H=H, Hkv=Hkv, D=D,
                chunk=chunk, scale=D ** -0.5, dtype=dtype,
                cu_q=np.concatenate([cu_p, Np + np.arange(1, n_d + 1)]).astype(np.int32),
                max_prefill_len=max(prefill_lens) if n_p else 0)


def continuation_case(seed=0, n_layers=4, H=4, Hkv=2, D=128, prompts=((40, 17), (70, 32), (129, 64)),
                      decode_prior=(1, 17, 300), decode_tokens=2, chunk=32, dtype="bf16",
                      pattern=PATTERN, n_spare=4, gated=False):
    """Requests whose new tokens are served over several steps.

    ``prompts`` holds (length, first) pairs: a prompt of ``length`` tokens with
    no earlier context, of which the first ``first`` come in one step and the
    rest in the next. ``decode_prior`` holds the cached context of requests
    that then bring ``decode_tokens`` tokens, one per step. Token rows are
    packed request-major (prompts first) with offsets ``cu``; ``prior`` and
    ``new`` give each request's cached and new token counts, ``split`` the
    tokens of each request that belong to the first step. Earlier tokens of
    decode requests sit in the pools, and their linear states are random;
    prompts start from empty pools and zero states. ``gated`` adds log forget
    factors ``g`` [N][H] to every linear layer (the gated variant).
    """
    rng = np.random.default_rng(seed)
    types = [pattern[i % len(pattern)] for i in range(n_layers)]
    prior = np.array([0] * len(prompts) + list(decode_prior), np.int64)
    new = np.array([p[0] for p in prompts] + [decode_tokens] * len(decode_prior), np.int64)
    split = np.array([p[1] for p in prompts] + [1] * len(decode_prior), np.int64)
    assert np.all((split >= 1) & (split < new)), "each request needs tokens in both steps"
    cu = cu_lens(new)
    N = int(cu[-1])
    ctx = (prior + new).astype(np.int32)
    lay = paged_layout(rng, ctx, n_spare=n_spare)
    n_lin = sum(t == "linear" for t in types)
    B = len(new)
    layers, pools = [], []
    for t in types:
        if t == "linear":
            q, k, v = (normal(rng, (N, H, D), D ** -0.5, dtype) for _ in range(3))
        else:
            q = normal(rng, (N, H, D), 1.0, dtype)
            k = normal(rng, (N, Hkv, D), 1.0, dtype)
            v = normal(rng, (N, Hkv, D), 1.0, dtype)
            shape = (lay.n_blocks, Hkv, 16, D)
            nan = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
            kp = np.full(shape, nan, np.uint16 if dtype == "bf16" else np.float32)
            vp = kp.copy()
            for r in range(B):
                for j in range((int(prior[r]) + 15) // 16):
                    b = lay.block_tables[r, j]
                    m = min(16, int(prior[r]) - 16 * j)
                    kp[b, :, :m] = normal(rng, (Hkv, m, D), 1.0, dtype)
                    vp[b, :, :m] = normal(rng, (Hkv, m, D), 1.0, dtype)
            pools.append((kp, vp))
        layers.append(dict(q=q, k=k, v=v))
        if gated and t == "linear":  # the gated variant's log forget factors
            layers[-1]["g"] = log_forget(rng, (N, H))
    states = np.zeros((n_lin, B, H, D, D), np.float32)
    has = prior > 0
    states[:, has] = (rng.standard_normal((n_lin, int(has.sum()), H, D, D)) * 0.1).astype(np.float32)
    return dict(types=types, layers=layers, pools=pools, states=states, layout=lay, ctx=ctx,
                prior=prior, new=new, split=split, cu=cu, n_prompts=len(prompts), N=N, H=H,
                Hkv=Hkv, D=D, chunk=chunk, scale=D ** -0.5, dtype=dtype)
