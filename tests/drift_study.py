"""State-precision drift of the linear layer over long decodes.

Pages: "推理框架适配Hybrid Model：KV Cache管理与算子调度实战" (P2) §2.3 and
§4.1/§4.4 (a state kept at the KV cache's 16-bit precision drifts over long
sequences; fp32 storage with 16-bit compute is the fix) and
"Hybrid Model推理适配：vLLM与SGLang的工程实践指南" (P1) §4.4 (asks for fp16
state storage).

Each arm runs the library's linear decode (hyattn_linear_decode: fp32 state
read, k (x) v added and q . S taken in fp32, state written back) for T
consecutive tokens of B requests x H heads. Arm "fp32" is the library as it
is. Arms "bf16" and "fp16" model a state stored at that precision: after
every decode step the state is rounded to the format and widened back
(round to nearest even), so each step reads a 16-bit-valued state and the
output of the step itself still comes from the fp32 sum, as in an
"fp32 compute, 16-bit storage" kernel. The reference is the oracle's fp64
token recurrence over the same inputs. Inputs are bf16 with the hybrid
workload's scales (q, k, v ~ N(0,1) D^-1/2); the plain layer's state grows
like sqrt(t), the gated layer's (``--gated``) stays bounded.

Test infrastructure: it calls the oracle, so it lives beside the tests.
Run: python tests/drift_study.py [--steps T] [--out FILE] [--gated]
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import ref  # noqa: E402

ARMS = ("fp32", "bf16", "fp16")


def checkpoints(T):
    c, t = [], 16
    while t < T:
        c.append(t)
        t *= 4
    return c + [T]


def run(T=16384, B=2, H=4, D=128, seed=5, gated=False, arms=ARMS, window=16):
    """Returns {arm: [(t, out_max, out_mean, state_max, state_fro), ...]}: errors
    of the outputs of steps t-window .. t-1 (the bf16 rule's max and mean of
    |g - r| / RMS of each output vector) and of the state after step t (max of
    |g - r| / max(|r|, RMS) and the relative Frobenius norm)."""
    import torch
    from linear_attention_attn_amd import hyattn as hy
    from tests import gpu_util as gu
    rng = np.random.default_rng(seed)
    q, k, v = (synth.normal(rng, (T, B, H, D), D ** -0.5, "bf16") for _ in range(3))
    g = synth.log_forget(rng, (T * B, H)).reshape(T, B, H) if gated else None
    cps = checkpoints(T)
    # oracle: per request, the token recurrence in segments between checkpoints
    want_o = np.zeros((T, B, H, D))
    want_S = {t: np.zeros((B, H, D, D)) for t in cps}
    for r in range(B):
        qr, kr, vr = (np.ascontiguousarray(x[:, r]) for x in (q, k, v))
        gr = None if g is None else np.ascontiguousarray(g[:, r])
        for h in range(H):
            S = np.zeros((D, D))
            t0 = 0
            for t in cps:
                want_o[t0:t, r, h] = ref.linear_unit("recurrent", qr, kr, vr, S, t0, t - t0, h,
                                                     log_gamma=gr)
                want_S[t][r, h] = S
                t0 = t
    print(f"[drift] oracle done ({T} steps, {B * H} units)", file=sys.stderr, flush=True)
    dq, dk, dv = gu.dev(q), gu.dev(k), gu.dev(v)
    dg = None if g is None else torch.from_numpy(g).cuda()
    fmt = {"bf16": torch.bfloat16, "fp16": torch.float16}
    results = {}
    for arm in arms:
        nbytes = hy.hyattn_state_pool_bytes(1, B, H, D)
        buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
        pool = hy.hyattn_state_pool_create(buf, nbytes, 1, B, H, D)
        slots = hy.hyattn_state_pool_alloc(pool, B)
        ds = gu.i32(slots)
        hy.hyattn_state_pool_zero(pool, ds, B)
        view = buf.view(B, H, D, D)  # slots 0 .. B-1 of a fresh pool
        out = torch.empty_like(dq)
        rows = []
        for t in range(T):
            if dg is None:
                hy.hyattn_linear_decode(pool, 0, dq[t], dk[t], dv[t], out[t], ds, B, hy.BF16)
            else:
                hy.hyattn_linear_decode_gated(pool, 0, dq[t], dk[t], dv[t], dg[t], out[t], ds, B,
                                              hy.BF16)
            if arm in fmt:  # the state as a 16-bit store would keep it
                view.copy_(view.to(fmt[arm]).to(torch.float32))
            if t + 1 in want_S:
                tt = t + 1
                got_S = gu.host(view)[slots]
                got_o = gu.host(out[tt - window:tt])
                om, oa = gu.err_bf16(got_o, want_o[tt - window:tt])
                ref_S = want_S[tt]
                sm = gu.err_f32(got_S, ref_S)
                sf = float(np.linalg.norm(got_S - ref_S) / max(np.linalg.norm(ref_S), 1e-300))
                rows.append((tt, om, oa, sm, sf))
        hy.hyattn_state_pool_destroy(pool)
        results[arm] = rows
        print(f"[drift] arm {arm} done", file=sys.stderr, flush=True)
    return results


def table(results, gated):
    lines = ["layer: " + ("gated (forget factors as in the gated workload)" if gated else "plain"),
             "",
             "| arm | step t | output max err / RMS | output mean err / RMS | state max rel err | state rel Frobenius err |",
             "|---|---|---|---|---|---|"]
    for arm, rows in results.items():
        for t, om, oa, sm, sf in rows:
            lines.append(f"| {arm} | {t} | {om:.3e} | {oa:.3e} | {sm:.3e} | {sf:.3e} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=16384)
    ap.add_argument("--gated", action="store_true")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    res = run(T=args.steps, gated=args.gated)
    text = table(res, args.gated)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
