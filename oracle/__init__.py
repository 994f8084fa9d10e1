"""CPU oracle for the W4A16 group-32 path: test infrastructure only.

Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The library under
``int4_w4a16_group_g32_amd`` never imports, links or calls it, and this package
shares no code with it: no kernels, helpers, tables or constants.
"""
from .w4a16 import (  # noqa: F401
    GROUP,
    quantize_w4a16,
    pack_nibbles,
    unpack,
    dequant32,
    dequant64,
    gemm64,
    gemm_abs64,
    silu64,
    swiglu_mlp64,
    route,
    moe_topk,
    moe64,
    moe_shared64,
    rel_frobenius,
)
