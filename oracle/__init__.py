"""CPU oracle for the fused RMSNorm + multimodal rotary path.

Test infrastructure only: imported by tests/, by the entry point's smoke check
and by the benchmark's CPU-baseline leg.  The product path never imports it.
"""
from . import positions_oracle  # noqa: F401
from .mrope_oracle import *  # noqa: F401,F403
from .mrope_oracle import (LAYOUT_CHUNKED, LAYOUT_INTERLEAVED, LAYOUT_VISION_2D,  # noqa: F401
                           layout_id)
