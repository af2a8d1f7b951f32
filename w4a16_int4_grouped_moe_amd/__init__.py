"""MI355X (gfx950) W4A16 INT4 grouped MoE layer.

A thin binding over the C ABI declared in include/moe_w4a16.h: argument
marshalling only, every step of the layer runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.

    out = forward(x, topk_ids, topk_weights, packed_w13, scales_w13,
                  packed_w2, scales_w2, shared_w=None, out=None, expert_base=0)
    ids, weights = route(scores, top_k)              # router step
    out, ids, weights = forward_scores(x, scores, top_k, packed_w13, ...)
    pk = prepack(packed_w13, scales_w13, packed_w2, scales_w2)   # once
    out = forward_prepacked(x, topk_ids, topk_weights, pk, shared_w=None)
"""
from ._binding import (  # noqa: F401
    MOE_ERR_ALIGNMENT,
    MOE_ERR_HIP,
    MOE_ERR_NULL,
    MOE_ERR_SHAPE,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_OK,
    LIB_PATH,
    MoeError,
    Prepacked,
    Problem,
    align,
    align_capacity,
    align_scratch_size,
    forward,
    forward_block_m,
    forward_split_max_pairs,
    forward_noalloc,
    forward_prepacked,
    forward_scores,
    library,
    noalloc_workspace_limit,
    prepack,
    prepack_size,
    problem,
    route,
    status_string,
    workspace_size,
)
