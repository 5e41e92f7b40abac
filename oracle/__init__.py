"""CPU oracle for the one-GPU share of an expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``combine_router_softmax_amd``) never imports, calls or links it, and this
package imports nothing from the product path: the two share no code apart from
the seeded input generators in ``synth``.

It is plain, slow and written for reading: NumPy in float64 for floating point,
Python loops where a loop states the definition most directly, and library
primitives (a stable sort, a matmul) only as whole steps.

Every function is pinned by ``tests/test_oracle_*.py`` to facts that do not come
from the oracle itself (brute force, closed forms, library routines, invariants
the pages state, hand-worked fixtures under ``tests/golden/``). Parity pins by
function are listed in each docstring; none of them is "parity unpinned".
"""
from .e4m3 import decode_e4m3fn, e4m3fn_table, dequant_blockwise  # noqa: F401
from .moe_oracle import (  # noqa: F401
    COMPACT,
    PADDED,
    STATUS_OVERFLOW,
    route_topk,
    dispatch_layout,
    dispatch,
    silu,
    swiglu_ffn,
    group_rows,
    grouped_ffn,
    combine,
    moe_layer,
    worst_case_rows,
)
from .w8a8 import (  # noqa: F401
    encode_e4m3fn_rne,
    quantize_1x128,
    dequant_1x128,
    gemm_w8a8,
    w8a8_ffn,
    w8a8_ffn_q,
    moe_layer_w8a8,
)
