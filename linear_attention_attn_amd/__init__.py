"""MI355X (gfx950) hybrid full/linear attention step: the hyattn C-ABI library
and its thin Python binding (``linear_attention_attn_amd.hyattn``)."""
from . import hyattn  # noqa: F401
from .hyattn import HyattnError  # noqa: F401
