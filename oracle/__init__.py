"""CPU oracle for the W4A16 group-quantized GEMM (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and this
package imports nothing from the product.
"""

from .w4a16_ref import (  # noqa: F401
    GROUP,
    ABS_TOL,
    REL_TOL,
    check_k,
    quantize,
    pack,
    unpack,
    dequantize,
    gemm,
    abs_gemm,
    gemm_entries,
    bound,
    compare,
    compare_to,
    compare_entries,
    pack_split,
    silu,
    check_routing,
    grouped_gemm,
    compare_grouped,
    swiglu,
    swiglu_bound,
    compare_swiglu,
    unpack_split,
    pack_grouped,
    unpack_grouped,
    TILE_ROWS,
    STEP_GROUPS,
    SLAB,
    STAGE_GROUPS,
)
