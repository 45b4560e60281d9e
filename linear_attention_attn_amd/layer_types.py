"""Model-config layer types -> hyattn layer codes.

Configs name the per-layer attention type in a `layer_types` list (page
"推理框架适配Hybrid Model：KV Cache管理与算子调度实战" §2.2 and §4.5 note the
spellings vary). Accepted: "linear"/"linear_attn" -> HYATTN_LAYER_LINEAR (0),
"full"/"full_attn" -> HYATTN_LAYER_FULL (1). Anything else is rejected, as an
unsupported attention type (page "Hybrid Model推理适配：vLLM与SGLang的工程实践指南" §4.3).
"""
from .hyattn import LAYER_FULL, LAYER_LINEAR

SPELLINGS = {"linear": LAYER_LINEAR, "linear_attn": LAYER_LINEAR,
             "full": LAYER_FULL, "full_attn": LAYER_FULL}


def parse(names):
    out = []
    for i, n in enumerate(names):
        code = SPELLINGS.get(n)
        if code is None:
            raise ValueError(f"layer {i}: attention type {n!r} is not supported")
        out.append(code)
    return out
