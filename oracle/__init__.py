"""CPU oracle of the W4A16 routed-expert MoE layer -- test infrastructure only.

Only the tests, the package smoke check and the bench's CPU-baseline leg may
import this package. It shares no code with the GPU library and never imports
it.
"""
from .oracle import (  # noqa: F401
    align,
    build,
    dense_moe,
    dequant_int4,
    forward,
    int4_code_c,
    pack_int4,
    route,
    silu_c,
    unpack_int4,
)
