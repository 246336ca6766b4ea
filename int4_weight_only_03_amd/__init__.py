"""MI355X (gfx950) W4A16 group-quantized GEMM: C-ABI library and its Python binding."""

from .binding import (  # noqa: F401
    GROUP,
    W4A16_PATH_AUTO,
    W4A16_PATH_GEMV,
    W4A16_PATH_TILE,
    W4A16_PATH_SPLIT,
    W4A16Error,
    load,
    w4a16_abi_version,
    w4a16_gemm,
    w4a16_gemm_grouped,
    w4a16_grouped_kernel,
    w4a16_gemm_path,
    w4a16_gemm_split,
    w4a16_gemm_swiglu,
    w4a16_gemm_split_packed,
    w4a16_load_quantized,
    w4a16_save_quantized,
    w4a16_split_pack,
    w4a16_split_pack_bytes,
    w4a16_split_workspace_bytes,
    w4a16_quantize,
    w4a16_select_path,
    w4a16_status_str,
)
from .bundle import WeightBundle  # noqa: F401,E402
