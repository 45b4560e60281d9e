"""Benchmark of one hybrid attention step on one MI355X.

Workload (synthetic, seeded): a 32-layer hybrid model, layer types
[linear, linear, linear, full] x 8, H = 32 heads, D = 128, bf16 I/O, fp32
linear states. One step serves 16 requests bringing a 4096-token prompt chunk
(from an empty context; linear chunk size 128) and 240 decode requests whose
contexts are log-uniform in [512, 131072] (the largest forced to 131072),
full layers with 8 KV heads in 16-token blocks. A step = zero the 16 prefill
slots (request start) + hyattn_hybrid_step over all 32 layers. Throughput =
tokens served per second (65 536 prefill + 240 decode tokens per step).

Printed: one JSON line (see the keys below), with
  * the roofline of the dominant kernel (paged decode, HBM-bound; HIP events
    around each of its launches),
  * the step against the sum of its operations' roofline times (step_roofline),
  * the first (cold) step beside the steady state (first_step_ms),
  * each layer operation on a workload of its own (workloads: the 64-request
    linear decode batch cold and back to back, the 8 x 8192-token chunked
    prefill per chunk size with its first call, the B = 128 paged decode, the
    step's 16 x 4096 causal prefill alone; see kernel_workloads()), timed before
    the step's workload is allocated,
  * per-operation times on the step's own data (components_ms_per_call),
  * the fp64 oracle's throughput on a bounded sample of the same workload.

`--kernel-workloads` prints only the per-operation workloads, one JSON line each.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

W = synth.WORKLOADS["hybrid_step"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def rocminfo_gfx950():
    """Compute units and maximum clock of the first gfx950 agent, as rocminfo reports them
    (run as a child process); None where it cannot be read."""
    import subprocess
    try:
        text = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in text.split("Agent ")[1:]:
        fields = {}
        for line in agent.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
        if fields.get("Name", "").startswith("gfx950"):
            def num(key):
                try:
                    return int(fields.get(key, "").split()[0])
                except (ValueError, IndexError):
                    return None
            return {"compute_units": num("Compute Unit"), "max_clock_mhz": num("Max Clock Freq. (MHz)")}
    return None


# ---------------------------------------------------------------- workload --
class Workload:
    """Device-resident inputs of the hybrid step (allocated once)."""

    def __init__(self, scale_ctx: float = 1.0):
        import torch
        from linear_attention_attn_amd import hyattn as hy
        from linear_attention_attn_amd import layer_types
        self.hy = hy
        rng = np.random.default_rng(W["seed"])
        self.H, self.Hkv, self.D = W["H"], W["Hkv"], W["D"]
        H, Hkv, D = self.H, self.Hkv, self.D
        self.types = layer_types.parse([W["pattern"][i % 4] for i in range(W["n_layers"])])
        self.n_lin = sum(t == 0 for t in self.types)
        self.n_full = len(self.types) - self.n_lin
        n_p, n_d, P = W["n_prefill"], W["n_decode"], W["prefill_len"]
        self.n_p, self.n_d = n_p, n_d
        dec_ctx = synth.loguniform_contexts(rng, n_d, W["ctx_lo"], int(W["ctx_hi"] * scale_ctx))
        self.ctx = np.concatenate([np.full(n_p, P, np.int32), dec_ctx]).astype(np.int32)
        lay = synth.paged_layout(rng, self.ctx)
        self.lay = lay
        self.N = n_p * P + n_d
        self.tokens = self.N
        B = n_p + n_d
        dev = "cuda"
        t0 = time.time()
        # state pool [L_lin][B][H][D][D]: decode requests hold a prior state
        nbytes = hy.hyattn_state_pool_bytes(self.n_lin, B, H, D)
        self.state_buf = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        sv = self.state_buf.view(self.n_lin, B, H * D * D)
        g = torch.Generator(device=dev)
        g.manual_seed(W["seed"] * 1000 + 1)
        for l in range(self.n_lin):
            sv[l].normal_(0.0, 0.1, generator=g)
        self.pool = hy.hyattn_state_pool_create(self.state_buf, nbytes, self.n_lin, B, H, D)
        slots = hy.hyattn_state_pool_alloc(self.pool, B)
        self.slots_p = torch.tensor(slots[:n_p], dtype=torch.int32, device=dev)
        self.slots_d = torch.tensor(slots[n_p:], dtype=torch.int32, device=dev)
        # inputs, shared by all layers of one type; outputs one per type
        s = D ** -0.5
        self.lin = dict(q=synth.device_normal_bf16((self.N, H, D), s, W["seed"] * 1000 + 2),
                        k=synth.device_normal_bf16((self.N, H, D), s, W["seed"] * 1000 + 3),
                        v=synth.device_normal_bf16((self.N, H, D), s, W["seed"] * 1000 + 4))
        self.lin["o"] = torch.empty_like(self.lin["q"])
        # log forget factors of the gated linear variant (timed as a component only)
        self.lin_g = synth.device_log_forget((self.N, H), W["seed"] * 1000 + 8)
        self.full = dict(q=synth.device_normal_bf16((self.N, H, D), 1.0, W["seed"] * 1000 + 5),
                         k=synth.device_normal_bf16((self.N, Hkv, D), 1.0, W["seed"] * 1000 + 6),
                         v=synth.device_normal_bf16((self.N, Hkv, D), 1.0, W["seed"] * 1000 + 7))
        self.full["o"] = torch.empty_like(self.full["q"])
        # one K and one V pool per full layer, fully random (prior context of decode requests)
        self.pools = []
        for f in range(self.n_full):
            kp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, W["seed"] * 1000 + 100 + 2 * f)
            vp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, W["seed"] * 1000 + 101 + 2 * f)
            self.pools.append((kp, vp))
        self.bt = torch.as_tensor(lay.block_tables).to(dev)
        self.ctx_d = torch.as_tensor(self.ctx).to(dev)
        cu_p = synth.cu_lens([P] * n_p)
        self.cu_p_host = cu_p
        self.cu_p = torch.as_tensor(cu_p).to(dev)
        self.cu_q = torch.as_tensor(np.concatenate([cu_p, cu_p[-1] + np.arange(1, n_d + 1)])
                                    .astype(np.int32)).to(dev)
        self.max_context = int(self.ctx.max())
        self.ws_bytes = hy.hyattn_paged_decode_workspace_bytes(n_d, H, D, self.max_context)
        self.ws = torch.empty(max(self.ws_bytes, 4) // 4, dtype=torch.float32, device=dev)
        self.layers = []
        fi = 0
        for t in self.types:
            if t == 0:
                self.layers.append(dict(self.lin))
            else:
                kp, vp = self.pools[fi]
                fi += 1
                self.layers.append(dict(self.full, k_pool=kp, v_pool=vp))
        self.layer_arr = hy.make_layers(self.layers)
        self.batch = hy.make_batch(
            n_prefill=n_p, n_decode=n_d, cu_seqlens=self.cu_p, n_prefill_tokens=n_p * P,
            max_prefill_len=P, prefill_slots=self.slots_p, decode_slots=self.slots_d,
            block_tables=self.bt, max_blocks_per_seq=lay.max_blocks, context_lens=self.ctx_d,
            cu_q_lens=self.cu_q, max_context=self.max_context, n_blocks=lay.n_blocks, H=H,
            H_kv=Hkv, D=D, chunk_size=W["chunk"], scale=D ** -0.5, dtype=hy.BF16,
            workspace=self.ws, workspace_bytes=self.ws_bytes)
        torch.cuda.synchronize()
        kv_bytes = 2 * self.n_full * lay.n_blocks * Hkv * 16 * D * 2
        log(f"workload ready in {time.time() - t0:.1f}s: KV {kv_bytes / 1e9:.1f} GB, "
            f"states {nbytes / 1e9:.1f} GB, contexts sum {int(self.ctx.sum())}, "
            f"max {self.max_context}, blocks/layer {lay.n_blocks}")

    def step(self, stream=None):
        hy = self.hy
        hy.hyattn_state_pool_zero(self.pool, self.slots_p, self.n_p, stream)
        hy.hyattn_hybrid_step(self.types, len(self.types), self.layer_arr, self.batch, self.pool,
                              stream)

    # ---- algorithmic work per component (per launch) ----
    def decode_kv_bytes(self):
        c = self.ctx[self.n_p:].astype(np.int64)
        kv = int(c.sum()) * self.Hkv * self.D * 2 * 2           # K and V rows read once
        qo = self.n_d * self.H * self.D * 2 * 2
        return kv + qo

    def linear_decode_bytes(self, gated=False):
        # state read + write, q k v o rows (+ one fp32 gate per request-head)
        return self.n_d * self.H * (2 * self.D * self.D * 4 + 4 * self.D * 2 + (4 if gated else 0))

    def linear_prefill_flops(self, gated=False):
        # the bf16 kernel works in 32-token blocks whatever the chunk size (the sums are the
        # same), so its work per token-head is Q.S (2D^2) + S update (2D^2) + the causal
        # intra-block part 2 (32 + 1) D; the gates' scalings are elementwise and not counted
        C, D, T = 32, self.D, W["prefill_len"]
        per_tok = 4 * D * D + 2 * (C + 1) * D
        return self.n_p * T * self.H * per_tok

    def linear_prefill_bytes(self):
        return self.n_p * W["prefill_len"] * self.H * self.D * 2 * 4 + 2 * self.n_p * self.H * self.D * self.D * 4

    def paged_prefill_flops(self):
        T, D = W["prefill_len"], self.D
        return self.n_p * self.H * 4 * D * (T * (T + 1) // 2)

    def paged_append_bytes(self):
        # each new token's K and V rows read once and written once into the pool
        return self.N * self.Hkv * self.D * 2 * 2 * 2

    def state_zero_bytes(self):
        return self.n_lin * self.n_p * self.H * self.D * self.D * 4

    def component_roofline_ms(self):
        """Each operation of the step at its bound's peak (ms): HBM-bound ones on their
        algorithmic bytes, the causal prefill on its algorithmic flops (MFMA-bound), the
        linear prefill at the larger of its byte and flop times (bytes bind)."""
        hbm = lambda b: b / (HBM_PEAK_GBS * 1e9) * 1e3
        mfma = lambda f: f / (BF16_PEAK_TFLOPS * 1e12) * 1e3
        return {"state_zero": hbm(self.state_zero_bytes()),
                "linear_prefill": max(hbm(self.linear_prefill_bytes()), mfma(self.linear_prefill_flops())),
                "linear_decode": hbm(self.linear_decode_bytes()),
                "paged_append": hbm(self.paged_append_bytes()),
                "paged_prefill": max(mfma(self.paged_prefill_flops()), hbm(self.N * self.H * self.D * 2 * 2)),
                "paged_decode": hbm(self.decode_kv_bytes())}


# ------------------------------------------------------------- components --
def step_component_times(wl, steps=2):
    """Per-call time of each operation inside the step. The step is issued decomposed:
    the same launches as hyattn_hybrid_step, in the same order on the same data, through
    the single-operation entry points, with a HIP event after each call on torch's stream.
    Each interval is one operation with the step's own neighbours before and after it
    (cache contents, clocks); means over its layers and `steps` steps. The sum of the
    intervals is a whole step (reported as step_ms_decomposed)."""
    import torch
    hy = wl.hy
    st = torch.cuda.current_stream()
    n_p, n_d, P = wl.n_p, wl.n_d, W["prefill_len"]
    off = n_p * P
    lin, full = wl.lin, wl.full
    row = lambda t: t[off:]
    marks = []

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        marks.append((name, e))

    wl.step()  # warm
    torch.cuda.synchronize()
    mark("start")
    for _ in range(steps):
        hy.hyattn_state_pool_zero(wl.pool, wl.slots_p, n_p)
        mark("state_zero")
        li = fi = 0
        for t in wl.types:
            if t == 0:
                hy.hyattn_linear_prefill_chunked(wl.pool, li, lin["q"], lin["k"], lin["v"], lin["o"],
                                                 wl.cu_p, wl.slots_p, n_p, W["chunk"], hy.BF16)
                mark("linear_prefill")
                hy.hyattn_linear_decode(wl.pool, li, row(lin["q"]), row(lin["k"]), row(lin["v"]),
                                        row(lin["o"]), wl.slots_d, n_d, hy.BF16)
                mark("linear_decode")
                li += 1
            else:
                kp, vp = wl.pools[fi]
                hy.hyattn_paged_append(full["k"], full["v"], kp, vp, wl.lay.n_blocks, wl.bt,
                                       wl.lay.max_blocks, wl.ctx_d, wl.cu_q, n_p + n_d, P, wl.Hkv,
                                       wl.D, hy.BF16)
                mark("paged_append")
                hy.hyattn_paged_prefill(full["q"], full["o"], kp, vp, wl.lay.n_blocks, wl.bt,
                                        wl.lay.max_blocks, wl.ctx_d, wl.cu_p, P, n_p, wl.H, wl.Hkv,
                                        wl.D, wl.D ** -0.5, hy.BF16)
                mark("paged_prefill")
                hy.hyattn_paged_decode(row(full["q"]), row(full["o"]), kp, vp, wl.lay.n_blocks,
                                       wl.bt[n_p:], wl.lay.max_blocks, wl.ctx_d[n_p:], wl.max_context,
                                       n_d, wl.H, wl.Hkv, wl.D, wl.D ** -0.5, wl.ws, wl.ws_bytes,
                                       hy.BF16)
                mark("paged_decode")
                fi += 1
    torch.cuda.synchronize()
    acc = {}
    for (_, e0), (name, e1) in zip(marks[:-1], marks[1:]):
        acc.setdefault(name, []).append(e0.elapsed_time(e1))
    out = {k: float(np.mean(v)) for k, v in acc.items()}
    out["step_ms_decomposed"] = marks[0][1].elapsed_time(marks[-1][1]) / steps
    return out


def component_times(wl, reps=3, inner=5, names=None):
    """Per-call device time of layer operations on their own, HIP events on torch's stream:
    the median over `reps` event pairs, each around `inner` back-to-back calls of one
    operation on the step's data. Used for the gated variants, which the step does not run;
    the step's own operations are timed in place by step_component_times. `names` selects
    operations (all by default)."""
    import torch
    hy = wl.hy
    st = torch.cuda.current_stream()
    n_p, n_d, P = wl.n_p, wl.n_d, W["prefill_len"]
    off = n_p * P
    lin, full = wl.lin, wl.full
    kp, vp = wl.pools[0]
    row = lambda t: t[off:]
    calls = {
        "state_zero": lambda: hy.hyattn_state_pool_zero(wl.pool, wl.slots_p, n_p),
        "linear_prefill": lambda: hy.hyattn_linear_prefill_chunked(
            wl.pool, 0, lin["q"], lin["k"], lin["v"], lin["o"], wl.cu_p, wl.slots_p, n_p,
            W["chunk"], hy.BF16),
        "linear_decode": lambda: hy.hyattn_linear_decode(
            wl.pool, 0, row(lin["q"]), row(lin["k"]), row(lin["v"]), row(lin["o"]), wl.slots_d,
            n_d, hy.BF16),
        "linear_prefill_gated": lambda: hy.hyattn_linear_prefill_chunked_gated(
            wl.pool, 0, lin["q"], lin["k"], lin["v"], wl.lin_g, lin["o"], wl.cu_p, wl.slots_p,
            n_p, W["chunk"], hy.BF16),
        "linear_decode_gated": lambda: hy.hyattn_linear_decode_gated(
            wl.pool, 0, row(lin["q"]), row(lin["k"]), row(lin["v"]), wl.lin_g[off:], row(lin["o"]),
            wl.slots_d, n_d, hy.BF16),
        "paged_append": lambda: hy.hyattn_paged_append(
            full["k"], full["v"], kp, vp, wl.lay.n_blocks, wl.bt, wl.lay.max_blocks, wl.ctx_d,
            wl.cu_q, n_p + n_d, P, wl.Hkv, wl.D, hy.BF16),
        "paged_prefill": lambda: hy.hyattn_paged_prefill(
            full["q"], full["o"], kp, vp, wl.lay.n_blocks, wl.bt, wl.lay.max_blocks, wl.ctx_d,
            wl.cu_p, P, n_p, wl.H, wl.Hkv, wl.D, wl.D ** -0.5, hy.BF16),
        "paged_decode": lambda: hy.hyattn_paged_decode(
            row(full["q"]), row(full["o"]), kp, vp, wl.lay.n_blocks, wl.bt[n_p:],
            wl.lay.max_blocks, wl.ctx_d[n_p:], wl.max_context, n_d, wl.H, wl.Hkv, wl.D,
            wl.D ** -0.5, wl.ws, wl.ws_bytes, hy.BF16),
    }
    out = {}
    for name, fn in calls.items():
        if names is not None and name not in names:
            continue
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(inner):
                fn()
            e1.record(st)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / inner)
        out[name] = float(np.median(ts))
    return out


PMC_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                           "paged_decode_hbm_traffic.md")
# sources that make up the paged-decode kernel (hashed together, in this order)
DECODE_SOURCES = [os.path.join(os.path.dirname(os.path.abspath(__file__)), "linear_attention_attn_amd",
                               "csrc", f) for f in ("k_paged.hip", "hy_common.hpp", "hy_kernels.hpp")]


def decode_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per paged-decode launch from the committed counter summary.

    The summary holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch of
    k_paged_decode_bf16 on this workload), the factors that map each counter
    onto bytes (from a plain copy of known size) and the SHA-256 of the
    kernel's sources the counters were taken with (k_paged.hip and the two
    headers it includes). Returns None when the file is missing or a source
    has changed since.
    """
    import re
    try:
        text = open(PMC_SUMMARY).read()
        src = decode_source_sha256()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): (\S+)$", text, re.M))
    try:
        if fields["kernel_source_sha256"] != src:
            return None
        kib = (float(fields["fetch_kib_per_dispatch"]) * float(fields["fetch_scale"])
               + float(fields["write_kib_per_dispatch"]) * float(fields["write_scale"]))
    except (KeyError, ValueError):
        return None
    return int(kib * 1024)


def copy_probe(reps=3):
    """A plain 2 GiB device copy (the calibration target of the HBM counters)."""
    import torch
    n = 1 << 29
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                      "reps": reps}), flush=True)


def kernel_workloads(emit=None):
    """Each layer operation on a workload of its own, HIP events on torch's stream:
      * linear decode: B = 64, H = 32, D = 128, 256 steps from prior states ~ N(0, 0.1);
        cold steps (a 1 GiB write between steps, untimed, evicts the 134 MB of state from
        L2 and the MALL) and the mean over 256 back-to-back steps;
      * linear chunked prefill: 8 requests x 8192 tokens from a zeroed state (zeroed
        again before every call, untimed), chunk sizes 64, 128 and 256: the first (cold)
        call, then the median of 10 after 3 warm-ups;
      * paged decode: B = 128, H_q = 32, H_kv = 8, D = 128, contexts uniform in
        [512, 32768], 16-token blocks in a permuted pool with 1024 NaN spare blocks:
        the first call, then the median of 20 after 5 warm-ups;
      * causal prefill: the hybrid step's full-layer prefill (16 requests x 4096 new
        tokens, H_q = 32, H_kv = 8, D = 128) through hyattn_paged_prefill alone: the
        first call, then the median of 10 after 3 warm-ups.
    A GPU-side sleep ahead of each timed call lets the host enqueue the events and the
    launch before the GPU reaches them, so host launch latency is not timed. Returns a
    dict of the four workloads' figures (emit: called with each one as it is done).
    Every device buffer is released before returning."""
    import torch
    from linear_attention_attn_amd import hyattn as hy
    hy.load()
    st = torch.cuda.current_stream()
    dev = "cuda"
    res = {}

    def timed(fn, before=None):
        if before is not None:
            before()
        torch.cuda._sleep(200_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1)

    def done(name, d):
        res[name] = d
        if emit is not None:
            emit(dict({"kernel_workload": name}, **d))

    # ---- linear decode ----
    cfg = synth.WORKLOADS["linear_decode"]
    B, H, D, steps = cfg["B"], cfg["H"], cfg["D"], cfg["steps"]
    nbytes = hy.hyattn_state_pool_bytes(1, B, H, D)
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    pool = hy.hyattn_state_pool_create(buf, nbytes, 1, B, H, D)
    sl = torch.tensor(hy.hyattn_state_pool_alloc(pool, B), dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg["seed"])
    buf.normal_(0.0, cfg["state_scale"], generator=g)
    qkv = synth.device_normal_bf16((steps, 3, B, H, D), D ** -0.5, cfg["seed"] * 1000 + 1)
    out = torch.empty(steps, B, H, D, dtype=torch.bfloat16, device=dev)
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    step_bytes = B * H * (2 * D * D * 4 + 4 * D * 2)
    call = lambda t: hy.hyattn_linear_decode(pool, 0, qkv[t, 0], qkv[t, 1], qkv[t, 2], out[t],
                                             sl, B, hy.BF16)
    first = timed(lambda: call(0), before=lambda: scrub.fill_(-1.0))
    cold = [timed(lambda t=t: call(t), before=lambda t=t: scrub.fill_(float(t)))
            for t in range(steps)]
    torch.cuda._sleep(200_000)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for t in range(steps):
        call(t)
    e1.record(st)
    e1.synchronize()
    warm = e0.elapsed_time(e1) / steps
    tc = float(np.median(cold))
    done("linear_decode", {
        "shape": f"B={B} H={H} D={D} bf16 io, fp32 state", "steps": steps,
        "bytes_per_step": step_bytes, "first_call_ms": round(first, 5),
        "cold_ms_median": round(tc, 5),
        "cold_tokens_per_s": round(B * steps / (sum(cold) * 1e-3), 1),
        "cold_gbs": round(step_bytes / (tc * 1e-3) / 1e9, 1),
        "cold_hbm_frac": round(step_bytes / (tc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "back_to_back_ms": round(warm, 5),
        "back_to_back_gbs": round(step_bytes / (warm * 1e-3) / 1e9, 1),
        "back_to_back_hbm_frac": round(step_bytes / (warm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    hy.hyattn_state_pool_destroy(pool)
    del buf, qkv, out, scrub

    # ---- linear chunked prefill ----
    cfg = synth.WORKLOADS["linear_prefill"]
    B, H, D, T = cfg["B"], cfg["H"], cfg["D"], cfg["T"]
    N = B * T
    q, k, v = (synth.device_normal_bf16((N, H, D), D ** -0.5, cfg["seed"] * 1000 + i)
               for i in range(3))
    o = torch.empty_like(q)
    cu = torch.as_tensor(synth.cu_lens([T] * B)).to(dev)
    nbytes = hy.hyattn_state_pool_bytes(1, B, H, D)
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    pool = hy.hyattn_state_pool_create(buf, nbytes, 1, B, H, D)
    sl = torch.tensor(hy.hyattn_state_pool_alloc(pool, B), dtype=torch.int32, device=dev)
    pf_bytes = N * H * D * 2 * 4 + 2 * B * H * D * D * 4
    zero = lambda: hy.hyattn_state_pool_zero(pool, sl, B)
    calls = {C: (lambda C=C: hy.hyattn_linear_prefill_chunked(pool, 0, q, k, v, o, cu, sl, B, C,
                                                              hy.BF16))
             for C in cfg["chunks"]}
    first = {C: timed(fn, before=zero) for C, fn in calls.items()}
    for _ in range(3):
        for fn in calls.values():
            timed(fn, before=zero)
    # the chunk sizes take turns, so that clock drift over the run favours none of them
    reps = {C: [] for C in calls}
    for _ in range(10):
        for C, fn in calls.items():
            reps[C].append(timed(fn, before=zero))
    per_c = {}
    for C in cfg["chunks"]:
        t = float(np.median(reps[C]))
        # the chunk-size count of the method (Q.S, S update, causal pairs inside each
        # chunk) and the kernel's own count (32-token blocks whatever the chunk size)
        flops_c = N * H * (4 * D * D + 2 * (C + 1) * D)
        flops_k = N * H * (4 * D * D + 2 * 33 * D)
        t_roof = max(pf_bytes / (HBM_PEAK_GBS * 1e9), flops_k / (BF16_PEAK_TFLOPS * 1e12))
        per_c[str(C)] = {
            "first_call_ms": round(first[C], 4), "ms_median": round(t, 4),
            "tokens_per_s": round(N / (t * 1e-3), 1),
            "hbm_frac": round(pf_bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac_chunk_count": round(flops_c / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "attainable_roof_frac": round(t_roof / (t * 1e-3), 4)}
    done("linear_prefill", {"shape": f"{B}x{T} tokens H={H} D={D} bf16 io", "bytes": pf_bytes,
                            "flops_kernel_count": N * H * (4 * D * D + 2 * 33 * D),
                            "chunks": per_c,
                            "note": "the bf16 kernel streams 32-token blocks whatever the chunk "
                                    "size, so the chunk sizes time one kernel (the same output "
                                    "bits); they differ only in the flop count of the chunk form"})
    hy.hyattn_state_pool_destroy(pool)
    del buf, q, k, v, o

    # ---- paged decode ----
    cfg = synth.WORKLOADS["paged_decode"]
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    rng = np.random.default_rng(cfg["seed"])
    ctx = synth.uniform_contexts(rng, B, cfg["ctx_lo"], cfg["ctx_hi"])
    lay = synth.paged_layout(rng, ctx, n_spare=cfg["n_spare"])
    kp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, cfg["seed"] * 1000 + 1)
    vp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, cfg["seed"] * 1000 + 2)
    spare = torch.as_tensor(lay.spare.astype(np.int64)).to(dev)
    kp[spare] = float("nan")
    vp[spare] = float("nan")
    q = synth.device_normal_bf16((B, Hq, D), 1.0, cfg["seed"] * 1000 + 3)
    o = torch.empty_like(q)
    maxc = int(ctx.max())
    wsb = hy.hyattn_paged_decode_workspace_bytes(B, Hq, D, maxc)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    bt = torch.as_tensor(lay.block_tables).to(dev)
    ctx_d = torch.as_tensor(ctx).to(dev)
    call = lambda: hy.hyattn_paged_decode(q, o, kp, vp, lay.n_blocks, bt, lay.max_blocks, ctx_d,
                                          maxc, B, Hq, Hkv, D, D ** -0.5, ws, wsb, hy.BF16)
    first = timed(call)
    for _ in range(5):
        timed(call)
    t = float(np.median([timed(call) for _ in range(20)]))
    kv_bytes = int(ctx.astype(np.int64).sum()) * Hkv * D * 2 * 2
    done("paged_decode", {
        "shape": f"B={B} H_q={Hq} H_kv={Hkv} D={D} bf16 KV, contexts uniform in "
                 f"[{cfg['ctx_lo']}, {cfg['ctx_hi']}]",
        "first_call_ms": round(first, 4), "ms_median": round(t, 4),
        "tokens_per_s": round(B / (t * 1e-3), 1), "kv_bytes": kv_bytes,
        "gbs": round(kv_bytes / (t * 1e-3) / 1e9, 1),
        "hbm_frac": round(kv_bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    del kp, vp, q, o, ws, bt, ctx_d, spare
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ---- causal prefill: the hybrid step's full-layer prefill on its own ----
    P, B = W["prefill_len"], W["n_prefill"]
    Hq, Hkv, D = W["H"], W["Hkv"], W["D"]
    rng = np.random.default_rng(W["seed"] + 100)
    ctx = np.full(B, P, np.int32)
    lay = synth.paged_layout(rng, ctx)
    kp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, W["seed"] * 1000 + 11)
    vp = synth.device_normal_bf16((lay.n_blocks, Hkv, 16, D), 1.0, W["seed"] * 1000 + 12)
    q = synth.device_normal_bf16((B * P, Hq, D), 1.0, W["seed"] * 1000 + 13)
    o = torch.empty_like(q)
    bt = torch.as_tensor(lay.block_tables).to(dev)
    ctx_d = torch.as_tensor(ctx).to(dev)
    cu = torch.as_tensor(synth.cu_lens([P] * B)).to(dev)
    call = lambda: hy.hyattn_paged_prefill(q, o, kp, vp, lay.n_blocks, bt, lay.max_blocks, ctx_d,
                                           cu, P, B, Hq, Hkv, D, D ** -0.5, hy.BF16)
    first = timed(call)
    for _ in range(3):
        timed(call)
    t = float(np.median([timed(call) for _ in range(10)]))
    flops = B * Hq * 4 * D * (P * (P + 1) // 2)
    done("paged_prefill", {
        "shape": f"{B} requests x {P} new tokens (empty context), causal, H_q={Hq} H_kv={Hkv} "
                 f"D={D} bf16, 16-token blocks",
        "first_call_ms": round(first, 4), "ms_median": round(t, 4),
        "tokens_per_s": round(B * P / (t * 1e-3), 1), "flops": flops,
        "tflops": round(flops / (t * 1e-3) / 1e12, 1),
        "mfma_frac": round(flops / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)})
    del kp, vp, q, o, bt, ctx_d, cu
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def dominant_kernel_roofline(wl, steps):
    """Average paged-decode launch time over all full layers of `steps` steps."""
    import torch
    hy = wl.hy
    st = torch.cuda.current_stream()
    n_p, n_d, P = wl.n_p, wl.n_d, W["prefill_len"]
    off = n_p * P
    full = wl.full
    ts = []
    for _ in range(steps):
        for kp, vp in wl.pools:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            hy.hyattn_paged_decode(full["q"][off:], full["o"][off:], kp, vp, wl.lay.n_blocks,
                                   wl.bt[n_p:], wl.lay.max_blocks, wl.ctx_d[n_p:], wl.max_context,
                                   n_d, wl.H, wl.Hkv, wl.D, wl.D ** -0.5, wl.ws, wl.ws_bytes,
                                   hy.BF16)
            e1.record(st)
            ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ts]))
    nbytes = wl.decode_kv_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(kernel="paged_decode (k_decode_plan + k_paged_decode_bf16 + k_paged_merge)",
                bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), traffic=measured_traffic(),
                algorithmic_bytes_per_launch=nbytes, avg_launch_ms=round(ms, 4))


# ------------------------------------------------------------ cpu baseline --
def cpu_baseline(wl):
    """Time the fp64 oracle on a bounded sample of the step; extrapolate to tokens/s.

    Each operation type runs a sample of its independent (request, head) units
    on all host threads at once; its measured rate (work per wall second) is
    applied to the whole step's work of that type.
    """
    import torch
    from oracle import ref
    threads = ref.n_threads()
    rng = np.random.default_rng(123)
    D, H = wl.D, wl.H
    P, C = W["prefill_len"], W["chunk"]
    off = wl.n_p * P

    def host_bf16(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    rates = {}
    # (1) linear chunked prefill: `threads` (request 0, head) units of 4096 tokens
    nu = min(threads, H)
    q, k, v = (host_bf16(wl.lin[n][:P]) for n in ("q", "k", "v"))
    st = np.zeros((1, H, D, D))
    t0 = time.time()
    ref.linear_prefill(q, k, v, [0, P], st, chunk=C, units=[(0, h) for h in range(nu)],
                       threads=threads)
    rates["linear_prefill_units_per_s"] = nu / (time.time() - t0)
    # (2) linear decode: 64 requests x all heads
    nr = 64
    qd, kd, vd = (host_bf16(wl.lin[n][off:off + nr]) for n in ("q", "k", "v"))
    std = rng.standard_normal((nr, H, D, D)) * 0.1
    t0 = time.time()
    ref.linear_decode(qd, kd, vd, std, threads=threads)
    rates["linear_decode_units_per_s"] = nr * H / (time.time() - t0)
    # (3) paged decode: 4 sampled decode requests, all heads, all their keys
    kp, vp = wl.pools[0]
    keys = 0
    t_pd = 0.0
    for r in rng.choice(np.arange(wl.n_p, wl.n_p + wl.n_d), size=4, replace=False):
        n = int(wl.ctx[r]); nb = (n + 15) // 16
        idx = torch.as_tensor(wl.lay.block_tables[r, :nb]).cuda()
        kk, vv = host_bf16(kp[idx]), host_bf16(vp[idx])
        qq = host_bf16(wl.full["q"][off + r - wl.n_p: off + r - wl.n_p + 1])
        t0 = time.time()
        ref.paged_attention(qq, kk, vv, np.arange(nb, dtype=np.int32)[None], [n], [0, 1],
                            D ** -0.5, threads=threads)
        t_pd += time.time() - t0
        keys += n * H
        qq1, kk1, vv1, n1, nb1 = qq, kk, vv, n, nb
    rates["paged_decode_head_keys_per_s"] = keys / t_pd
    # (4) causal prefill: the first 512 queries of request 0, `threads` heads
    nq, nh = 512, min(threads, H)
    idx = torch.as_tensor(wl.lay.block_tables[0, :nq // 16]).cuda()
    kk, vv = host_bf16(kp[idx]), host_bf16(vp[idx])
    qq = host_bf16(wl.full["q"][:nq])
    t0 = time.time()
    ref.paged_attention(qq, kk, vv, np.arange(nq // 16, dtype=np.int32)[None], [nq], [0, nq],
                        D ** -0.5, units=[(0, h) for h in range(nh)], threads=threads)
    rates["paged_prefill_head_pairs_per_s"] = nh * nq * (nq + 1) // 2 / (time.time() - t0)
    # the same four operations on one host thread, on smaller samples
    one = {}
    t0 = time.time()
    ref.linear_prefill(q, k, v, [0, P], np.zeros((1, H, D, D)), chunk=C, units=[(0, 0)], threads=1)
    one["linear_prefill_units_per_s"] = 1 / (time.time() - t0)
    t0 = time.time()
    ref.linear_decode(qd[:8], kd[:8], vd[:8], std[:8].copy(), threads=1)
    one["linear_decode_units_per_s"] = 8 * H / (time.time() - t0)
    t0 = time.time()
    ref.paged_attention(qq1, kk1, vv1, np.arange(nb1, dtype=np.int32)[None], [n1], [0, 1],
                        D ** -0.5, threads=1)
    one["paged_decode_head_keys_per_s"] = n1 * H / (time.time() - t0)
    t0 = time.time()
    ref.paged_attention(qq, kk, vv, np.arange(nq // 16, dtype=np.int32)[None], [nq], [0, nq],
                        D ** -0.5, units=[(0, 0)], threads=1)
    one["paged_prefill_head_pairs_per_s"] = nq * (nq + 1) // 2 / (time.time() - t0)

    # extrapolate one whole step
    dec_keys = int(wl.ctx[wl.n_p:].astype(np.int64).sum())

    def step_seconds(rt):
        return (wl.n_lin * (wl.n_p * H / rt["linear_prefill_units_per_s"]
                            + wl.n_d * H / rt["linear_decode_units_per_s"])
                + wl.n_full * (H * dec_keys / rt["paged_decode_head_keys_per_s"]
                               + wl.n_p * H * (P * (P + 1) // 2) / rt["paged_prefill_head_pairs_per_s"]))
    step_s = step_seconds(rates)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return dict(value=round(wl.tokens / step_s, 3), unit="tokens/s", cores=threads, kind="oracle",
                cpu_model=cpu_model,
                one_thread={"value": round(wl.tokens / step_seconds(one), 4), "unit": "tokens/s",
                            "sample": "1 linear-prefill unit, 8 x 32 linear-decode units, the last "
                                      "sampled paged-decode request, 512-query causal prefill x 1 head",
                            "rates": {k: round(x, 2) for k, x in one.items()}},
                sample=(f"fp64 oracle, {threads} threads, on sampled units of the same step: "
                        f"{nu} linear-prefill (request, head) units of 4096 tokens, {nr * H} "
                        "linear-decode units, 4 paged-decode requests (all heads and keys), "
                        f"512-query causal prefill x {nh} heads; measured rates extrapolated "
                        "to the whole step"),
                extrapolated_step_s=round(step_s, 1),
                rates={k: round(v, 2) for k, v in rates.items()})


# --------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--no-kernel-workloads", action="store_true",
                    help="skip the per-operation workloads (linear decode batch, 8x8192 "
                         "chunked prefill, B=128 paged decode) in the bench line")
    ap.add_argument("--ctx-scale", type=float, default=1.0,
                    help="scale of the longest decode context (1.0 = 131072)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 2 GiB device copy (HBM counter calibration)")
    ap.add_argument("--kernel-workloads", action="store_true",
                    help="only time each layer operation on its own workload (one JSON line each)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the hybrid attention step has no multi-GPU path here", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        copy_probe()
        return
    if args.kernel_workloads:
        kernel_workloads(emit=lambda d: print(json.dumps(d), flush=True))
        return
    from linear_attention_attn_amd import hyattn as hy
    hy.load()
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {props.gcnArchName} CUs={props.multi_processor_count} "
        f"mem={props.total_memory / 2**30:.0f} GiB")
    workloads = None
    if not args.no_kernel_workloads:
        t0 = time.time()
        workloads = kernel_workloads()
        log(f"per-operation workloads took {time.time() - t0:.1f}s")
    wl = Workload(args.ctx_scale)
    st = torch.cuda.current_stream()
    # the first step after the workload is set up, timed on its own (one-time costs
    # such as loading the kernels' code and first-touch of the pools included)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    wl.step()
    e1.record(st)
    e1.synchronize()
    first_ms = e0.elapsed_time(e1)
    log(f"first step {first_ms:.3f} ms")
    for i in range(args.warmup):
        wl.step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    e0.record(st)
    for _ in range(args.steps):
        wl.step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.time() - t0
    ms = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {wall:.2f}s)")
    value = wl.tokens / (ms * 1e-3)
    out = {
        "metric": "hybrid attn tokens/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hybrid 32-layer attention step (24 linear : 8 full), H=32, "
                               "H_kv=8, D=128, 16x4096-token chunked prefill + 240 decode, "
                               "contexts log-uniform to 131072, 16-token KV blocks, fp32 states",
                   "global_batch": wl.n_p + wl.n_d, "tokens_per_step": wl.tokens,
                   "layers": len(wl.types), "chunk": W["chunk"], "seq_len": W["prefill_len"],
                   "max_context": wl.max_context, "parallelism": "none (1 GPU)"},
    }
    out["first_step_ms"] = round(first_ms, 4)
    roof_ms = wl.component_roofline_ms()
    sum_roof = (roof_ms["state_zero"] + wl.n_lin * (roof_ms["linear_prefill"] + roof_ms["linear_decode"])
                + wl.n_full * (roof_ms["paged_append"] + roof_ms["paged_prefill"] + roof_ms["paged_decode"]))
    out["step_roofline"] = {
        "sum_component_roof_ms": round(sum_roof, 4), "frac": round(sum_roof / ms, 4),
        "component_roof_ms": {k: round(v, 5) for k, v in roof_ms.items()},
        "note": "each operation at its bound's peak (HBM 8 TB/s on its algorithmic bytes, or bf16 "
                "MFMA 2.5 PFLOP/s on its algorithmic flops, whichever is longer), summed over the "
                f"step's {wl.n_lin} linear and {wl.n_full} full layers; frac = that sum / ms_per_step"}
    if workloads is not None:
        out["workloads"] = workloads
    roof = dominant_kernel_roofline(wl, max(1, min(args.steps, 3)))
    log(f"dominant kernel: {roof}")
    out["device"] = {"name": props.gcnArchName, "peaks_used": {"hbm_gbs": HBM_PEAK_GBS,
                                                                "bf16_mfma_tflops": BF16_PEAK_TFLOPS},
                     "rocminfo": rocminfo_gfx950()}
    out["roofline"] = {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    out["roofline"]["kernel"] = roof["kernel"]
    out["roofline"]["algorithmic_bytes_per_launch"] = roof["algorithmic_bytes_per_launch"]
    out["roofline"]["avg_launch_ms"] = roof["avg_launch_ms"]
    if not args.no_components:
        comp = step_component_times(wl)
        alone = component_times(wl, names=("linear_prefill_gated", "linear_decode_gated"))
        n_lin, n_full = wl.n_lin, wl.n_full
        lp, ld, pd = comp["linear_prefill"], comp["linear_decode"], comp["paged_decode"]
        out["components_ms_per_call"] = {k: round(v, 4) for k, v in comp.items()}
        out["components_gated_ms_per_call"] = {k: round(v, 4) for k, v in alone.items()}
        out["components"] = {
            "linear_decode_hbm_frac": round(wl.linear_decode_bytes() / (ld * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "paged_decode_hbm_frac": round(wl.decode_kv_bytes() / (pd * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "linear_prefill_mfma_frac": round(wl.linear_prefill_flops() / (lp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "linear_prefill_hbm_frac": round(wl.linear_prefill_bytes() / (lp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "linear_prefill_gated_mfma_frac": round(
                wl.linear_prefill_flops(gated=True) / (alone["linear_prefill_gated"] * 1e-3) / 1e12
                / BF16_PEAK_TFLOPS, 4),
            "linear_decode_gated_hbm_frac": round(
                wl.linear_decode_bytes(gated=True) / (alone["linear_decode_gated"] * 1e-3) / 1e9
                / HBM_PEAK_GBS, 4),
            "paged_prefill_mfma_frac": round(wl.paged_prefill_flops() / (comp["paged_prefill"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "step_ms_from_components": round(comp["state_zero"] + n_lin * (lp + ld) + n_full * (
                comp["paged_append"] + comp["paged_prefill"] + pd), 3),
            "note": "each operation launched alone inside a decomposed step; the step itself runs "
                    "each full layer's decode beside its prefill on a second stream, so "
                    "ms_per_step is below step_ms_from_components",
        }
        roof_ms = out["step_roofline"]["component_roof_ms"]
        out["step_roofline"]["component_frac"] = {
            k: round(roof_ms[k] / comp[k], 4) for k in roof_ms if k in comp}
    if not args.no_cpu_baseline:
        t0 = time.time()
        out["cpu_baseline"] = cpu_baseline(wl)
        log(f"cpu baseline took {time.time() - t0:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
