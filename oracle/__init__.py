"""CPU oracle of the LatentMoE layer forward. Test infrastructure only: it may be
imported by the tests, the smoke check and the benchmark's CPU-baseline leg, and
by nothing on the library path."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
from .mxfp8 import (MX_BLOCK, dequantize_mxfp8, e4m3_decode, e4m3_encode,  # noqa: F401
                    quantize_mxfp8)
from .block import RMS_EPS, bias_update, block_forward, f64_to_bf16_bits, rmsnorm  # noqa: F401
from .mxfp4 import dequantize_mxfp4, e2m1_decode, e2m1_encode, quantize_mxfp4  # noqa: F401
