"""MI355X (gfx950) mixture-of-experts layer with groupwise-affine 4-bit experts.

The compute path is libmoeq4.so (hand-written HIP kernels behind a C ABI,
declared in include/moeq4.h); this package holds its ctypes binding (same
names as the C entry points), device-memory plumbing and the seeded synthetic
workloads.  Build the library with ``python -m bit_grouped_expert_amd.build``.
"""
from ._lib import (ENGINES, MoEError, layer_opts, lib, moe_chunked_workspace_bytes,  # noqa: F401
                   moe_combine, moe_grouped_gemm_q4, moe_grouped_gemm_q4_ex,
                   moe_grouped_gemm_q4_workspace_bytes, moe_layer_forward,
                   moe_layer_forward_chunked, moe_layer_forward_ex, moe_permute, moe_route,
                   moe_route_ex, moe_workspace_bytes, moe_workspace_layout, q4, q4_ffn, shape,
                   status_string)
