"""ctypes binding of libmoe_w4a16.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_w4a16.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGNMENT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_UNSUPPORTED = -5
MOE_ERR_HIP = -6
MOE_MAX_EXPERTS = 512
MOE_MAX_SCORED = 1024

GROUP = 32


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("expert_base", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def library():
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m w4a16_int4_grouped_moe_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PP = ctypes.POINTER(Problem)
        lib.moe_w4a16_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
        lib.moe_w4a16_forward_block_m.argtypes = [PP, ctypes.POINTER(ctypes.c_int32)]
        lib.moe_w4a16_forward_split_max_pairs.argtypes = [PP, ctypes.POINTER(ctypes.c_int32)]
        lib.moe_w4a16_align_capacity.argtypes = [PP, ctypes.c_int32,
                                                 ctypes.POINTER(ctypes.c_int64),
                                                 ctypes.POINTER(ctypes.c_int64)]
        lib.moe_w4a16_align.argtypes = [P, PP, ctypes.c_int32, P, ctypes.c_int64, P,
                                        ctypes.c_int64, P, P, ctypes.c_size_t, P]
        lib.moe_w4a16_align_scratch_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
        lib.moe_w4a16_forward.argtypes = [P] * 9 + [PP, P, ctypes.c_size_t, P]
        lib.moe_w4a16_forward_timed.argtypes = [P] * 9 + [PP, P, ctypes.c_size_t, P, P]
        lib.moe_w4a16_route.argtypes = [P, ctypes.c_int32, PP, P, P, P]
        lib.moe_w4a16_forward_scores.argtypes = ([P, P, ctypes.c_int32] + [P] * 8 +
                                                 [PP, P, ctypes.c_size_t, P])
        lib.moe_w4a16_prepack_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
        lib.moe_w4a16_prepack.argtypes = [P] * 4 + [PP, P, ctypes.c_size_t, P]
        lib.moe_w4a16_forward_prepacked.argtypes = ([P] * 3 + [P, ctypes.c_size_t, P, P] +
                                                    [PP, P, ctypes.c_size_t, P])
        lib.moe_w4a16_forward_prepacked_timed.argtypes = (
            [P] * 3 + [P, ctypes.c_size_t, P, P] + [PP, P, ctypes.c_size_t, P, P])
        lib.moe_w4a16_forward_noalloc.argtypes = [P] * 9 + [PP, P]
        lib.moe_w4a16_noalloc_workspace_limit.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
        lib.moe_w4a16_status_string.argtypes = [ctypes.c_int]
        lib.moe_w4a16_status_string.restype = ctypes.c_char_p
        for f in ("workspace_size", "forward_block_m", "align_capacity", "align",
                  "align_scratch_size", "forward", "forward_timed", "route",
                  "forward_scores", "prepack_size", "prepack", "forward_prepacked",
                  "forward_prepacked_timed", "forward_noalloc", "noalloc_workspace_limit"):
            getattr(lib, "moe_w4a16_" + f).restype = ctypes.c_int
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().moe_w4a16_status_string(status).decode()


def _check(status: int):
    if status != MOE_OK:
        msg = status_string(status)
        if status == MOE_ERR_HIP:
            raise MoeError(status, msg)
        raise ValueError(f"{msg} (status {status})")


def problem(num_tokens: int, hidden: int, inter: int, num_experts: int, top_k: int,
            expert_base: int = 0, group_size: int = GROUP) -> Problem:
    return Problem(num_tokens, hidden, inter, num_experts, expert_base, top_k, group_size)


def workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(library().moe_w4a16_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def forward_block_m(p: Problem) -> int:
    v = ctypes.c_int32(0)
    _check(library().moe_w4a16_forward_block_m(ctypes.byref(p), ctypes.byref(v)))
    return v.value


def forward_split_max_pairs(p: Problem) -> int:
    """Experts with at most this many pairs take 4-row buckets beside the
    96-row ones in this call (0: no split)."""
    v = ctypes.c_int32(0)
    _check(library().moe_w4a16_forward_split_max_pairs(ctypes.byref(p), ctypes.byref(v)))
    return v.value


def align_capacity(p: Problem, block_m: int):
    s, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(library().moe_w4a16_align_capacity(ctypes.byref(p), block_m, ctypes.byref(s),
                                              ctypes.byref(b)))
    return s.value, b.value


def _torch():
    import torch

    return torch


def _stream_handle(device) -> Optional[int]:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, ndim, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _layer(x, k, packed_w13, scales_w13, packed_w2, scales_w2, shared_w, out, expert_base,
           workspace):
    """Checks the layer's tensors; returns (problem, out, workspace)."""
    torch = _torch()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    _need(x, "x", torch.bfloat16, 2, dev)
    T, H = x.shape
    _need(packed_w13, "packed_w13", torch.int32, 3, dev)
    E, I2, _ = packed_w13.shape
    I = I2 // 2
    _need(scales_w13, "scales_w13", torch.bfloat16, 3, dev)
    _need(packed_w2, "packed_w2", torch.int32, 3, dev)
    _need(scales_w2, "scales_w2", torch.bfloat16, 3, dev)
    shapes = {
        "packed_w13": (tuple(packed_w13.shape), (E, 2 * I, H // 8)),
        "scales_w13": (tuple(scales_w13.shape), (E, 2 * I, H // GROUP)),
        "packed_w2": (tuple(packed_w2.shape), (E, H, I // 8)),
        "scales_w2": (tuple(scales_w2.shape), (E, H, I // GROUP)),
    }
    for name, (got, want) in shapes.items():
        if got != want:
            raise ValueError(f"{name} has shape {got}, expected {want}")
    if shared_w is not None:
        _need(shared_w, "shared_w", torch.bfloat16, 1, dev)
        if shared_w.numel() != 3 * I * H:
            raise ValueError(f"shared_w must hold {3 * I * H} values")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 2, dev)
        if tuple(out.shape) != (T, H):
            raise ValueError("out must be [T, H]")
    p = problem(T, H, I, E, k, expert_base)
    need = workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    return p, out, workspace


def _routing(topk_ids, topk_weights, T, k, dev):
    torch = _torch()
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, 2, dev)
    _need(topk_weights, "topk_weights", torch.float32, 2, dev)
    for name, t in (("topk_ids", topk_ids), ("topk_weights", topk_weights)):
        if tuple(t.shape) != (T, k):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(T, k)}")
    return topk_ids, topk_weights


def forward(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
            shared_w=None, out=None, expert_base: int = 0, workspace=None,
            stage_events=None):
    """The W4A16 MoE layer (see include/moe_w4a16.h for the definition).

    x bf16 [T, H]; topk_ids int32 [T, k]; topk_weights fp32 [T, k];
    packed_w13 int32 [E, 2I, H/8]; scales_w13 bf16 [E, 2I, H/32];
    packed_w2 int32 [E, H, I/8]; scales_w2 bf16 [E, H, I/32];
    shared_w bf16 [2I*H + H*I] or None. Returns out bf16 [T, H].
    stage_events: optional sequence of 7 raw hipEvent_t handles (int or None)
    recorded between the stages (see moe_w4a16_forward_timed).
    """
    torch = _torch()
    _need(topk_ids, "topk_ids", torch.int32, 2, x.device)
    k = topk_ids.shape[1]
    p, out, workspace = _layer(x, k, packed_w13, scales_w13, packed_w2, scales_w2, shared_w,
                               out, expert_base, workspace)
    _routing(topk_ids, topk_weights, x.shape[0], k, x.device)
    args = (x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(), packed_w13.data_ptr(),
            scales_w13.data_ptr(), packed_w2.data_ptr(), scales_w2.data_ptr(),
            None if shared_w is None else shared_w.data_ptr(), out.data_ptr(), ctypes.byref(p),
            workspace.data_ptr(), workspace.numel(), _stream_handle(x.device))
    if stage_events is None:
        st = library().moe_w4a16_forward(*args)
    else:
        if len(stage_events) != 7:
            raise ValueError("stage_events needs 7 entries")
        ev = (ctypes.c_void_p * 7)(*[e or None for e in stage_events])
        st = library().moe_w4a16_forward_timed(*args, ev)
    _check(st)
    return out


def noalloc_workspace_limit() -> int:
    """Bytes of the device array that forward_noalloc uses as its workspace."""
    n = ctypes.c_size_t(0)
    _check(library().moe_w4a16_noalloc_workspace_limit(ctypes.byref(n)))
    return n.value


def forward_noalloc(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
                    shared_w=None, out=None, expert_base: int = 0):
    """forward with the library's own device array as the workspace
    (moe_w4a16_forward_noalloc): nothing is allocated by the library; `out`
    should be given by callers that cannot allocate. Calls that overlap on one
    GPU race."""
    torch = _torch()
    _need(topk_ids, "topk_ids", torch.int32, 2, x.device)
    k = topk_ids.shape[1]
    # an empty placeholder: the workspace argument is not used
    p, out, _ = _layer(x, k, packed_w13, scales_w13, packed_w2, scales_w2, shared_w, out,
                       expert_base, torch.empty(0, dtype=torch.uint8, device=x.device))
    _routing(topk_ids, topk_weights, x.shape[0], k, x.device)
    st = library().moe_w4a16_forward_noalloc(
        x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(), packed_w13.data_ptr(),
        scales_w13.data_ptr(), packed_w2.data_ptr(), scales_w2.data_ptr(),
        None if shared_w is None else shared_w.data_ptr(), out.data_ptr(), ctypes.byref(p),
        _stream_handle(x.device))
    _check(st)
    return out


class Prepacked:
    """Expert weights in the library's prepacked form (moe_w4a16_prepack):
    a uint8 device buffer and the widths it was written for."""

    def __init__(self, buffer, hidden: int, inter: int, num_experts: int):
        self.buffer = buffer
        self.hidden = hidden
        self.inter = inter
        self.num_experts = num_experts


def prepack_size(hidden: int, inter: int, num_experts: int) -> int:
    """Bytes of the prepacked form of num_experts experts (host only)."""
    n = ctypes.c_size_t()
    _check(library().moe_w4a16_prepack_size(
        ctypes.byref(problem(0, hidden, inter, num_experts, 1)), ctypes.byref(n)))
    return n.value


def prepack(packed_w13, scales_w13, packed_w2, scales_w2, out=None) -> Prepacked:
    """One-time repack of the four weight tensors (layouts as for forward)
    into the prepacked form that forward_prepacked reads; out: an optional
    uint8 device buffer of at least prepack_size bytes."""
    torch = _torch()
    dev = packed_w13.device
    if dev.type != "cuda":
        raise ValueError("the weights must be GPU tensors")
    _need(packed_w13, "packed_w13", torch.int32, 3, dev)
    E, I2, H8 = packed_w13.shape
    H, I = 8 * H8, I2 // 2
    for name, t, dtype, shape in (("scales_w13", scales_w13, torch.bfloat16, (E, 2 * I, H // GROUP)),
                                  ("packed_w2", packed_w2, torch.int32, (E, H, I // 8)),
                                  ("scales_w2", scales_w2, torch.bfloat16, (E, H, I // GROUP))):
        _need(t, name, dtype, 3, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    need = prepack_size(H, I, E)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=dev)
    else:
        _need(out, "out", torch.uint8, 1, dev)
    p = problem(0, H, I, E, 1)
    _check(library().moe_w4a16_prepack(
        packed_w13.data_ptr(), scales_w13.data_ptr(), packed_w2.data_ptr(),
        scales_w2.data_ptr(), ctypes.byref(p), out.data_ptr(), out.numel(),
        _stream_handle(dev)))
    return Prepacked(out, H, I, E)


def forward_prepacked(x, topk_ids, topk_weights, prepacked: Prepacked, shared_w=None, out=None,
                      expert_base: int = 0, workspace=None, stage_events=None):
    """forward with the expert weights in prepacked form (see prepack); the
    same results, bit for bit."""
    torch = _torch()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(topk_ids, "topk_ids", torch.int32, 2, dev)
    T, H = x.shape
    k = topk_ids.shape[1]
    if H != prepacked.hidden:
        raise ValueError(f"x has width {H}, the prepacked weights {prepacked.hidden}")
    I, E = prepacked.inter, prepacked.num_experts
    _need(prepacked.buffer, "prepacked.buffer", torch.uint8, 1, dev)
    if shared_w is not None:
        _need(shared_w, "shared_w", torch.bfloat16, 1, dev)
        if shared_w.numel() != 3 * I * H:
            raise ValueError(f"shared_w must hold {3 * I * H} values")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 2, dev)
        if tuple(out.shape) != (T, H):
            raise ValueError("out must be [T, H]")
    _routing(topk_ids, topk_weights, T, k, dev)
    p = problem(T, H, I, E, k, expert_base)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(p), 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    args = (x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(),
            prepacked.buffer.data_ptr(), prepacked.buffer.numel(),
            None if shared_w is None else shared_w.data_ptr(), out.data_ptr(), ctypes.byref(p),
            workspace.data_ptr(), workspace.numel(), _stream_handle(dev))
    if stage_events is None:
        st = library().moe_w4a16_forward_prepacked(*args)
    else:
        if len(stage_events) != 7:
            raise ValueError("stage_events needs 7 entries")
        ev = (ctypes.c_void_p * 7)(*[e or None for e in stage_events])
        st = library().moe_w4a16_forward_prepacked_timed(*args, ev)
    _check(st)
    return out


def route(scores, top_k: int, num_experts: Optional[int] = None, expert_base: int = 0,
          topk_ids=None, topk_weights=None):
    """The router step (see moe_w4a16_route): scores fp32 [T, S] -> (topk_ids
    int32 [T, top_k], topk_weights fp32 [T, top_k]). num_experts / expert_base
    describe the local experts of the layer that follows (default: the first
    min(S, MOE_MAX_EXPERTS))."""
    torch = _torch()
    dev = scores.device
    _need(scores, "scores", torch.float32, 2, dev)
    T, S = scores.shape
    topk_ids, topk_weights = _routing(topk_ids, topk_weights, T, top_k, dev)
    if num_experts is None:
        num_experts = min(S, MOE_MAX_EXPERTS)
    p = problem(T, 128, 128, num_experts, top_k, expert_base)
    _check(library().moe_w4a16_route(scores.data_ptr(), S, ctypes.byref(p), topk_ids.data_ptr(),
                                     topk_weights.data_ptr(), _stream_handle(dev)))
    return topk_ids, topk_weights


def forward_scores(x, scores, top_k: int, packed_w13, scales_w13, packed_w2, scales_w2,
                   shared_w=None, out=None, expert_base: int = 0, workspace=None,
                   topk_ids=None, topk_weights=None):
    """The router step followed by the layer (moe_w4a16_forward_scores).
    Returns (out, topk_ids, topk_weights)."""
    torch = _torch()
    _need(scores, "scores", torch.float32, 2, x.device)
    T, S = scores.shape
    if T != x.shape[0]:
        raise ValueError("scores and x must have the same number of tokens")
    p, out, workspace = _layer(x, top_k, packed_w13, scales_w13, packed_w2, scales_w2,
                               shared_w, out, expert_base, workspace)
    topk_ids, topk_weights = _routing(topk_ids, topk_weights, T, top_k, x.device)
    st = library().moe_w4a16_forward_scores(
        x.data_ptr(), scores.data_ptr(), S, packed_w13.data_ptr(), scales_w13.data_ptr(),
        packed_w2.data_ptr(), scales_w2.data_ptr(),
        None if shared_w is None else shared_w.data_ptr(), out.data_ptr(),
        topk_ids.data_ptr(), topk_weights.data_ptr(), ctypes.byref(p), workspace.data_ptr(),
        workspace.numel(), _stream_handle(x.device))
    _check(st)
    return out, topk_ids, topk_weights


def align_scratch_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(library().moe_w4a16_align_scratch_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def align(topk_ids, num_experts: int, block_m: int, expert_base: int = 0,
          many_groups: bool = False):
    """Token/expert bucketing: returns (sorted_ids, block_expert, n_padded)
    int32 device tensors sized to the capacities; only the first n_padded
    sorted_ids and n_padded/block_m block_expert entries are meaningful.
    many_groups: use the many-work-group form (with its scratch)."""
    torch = _torch()
    dev = topk_ids.device
    _need(topk_ids, "topk_ids", torch.int32, 2, dev)
    T, k = topk_ids.shape
    p = problem(T, 128, 128, num_experts, k, expert_base)
    cap_s, cap_b = align_capacity(p, block_m)
    sorted_ids = torch.empty(max(cap_s, 4), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(cap_b, 4), dtype=torch.int32, device=dev)
    n_padded = torch.empty(4, dtype=torch.int32, device=dev)
    scratch, nbytes = None, 0
    if many_groups:
        nbytes = align_scratch_size(p)
        scratch = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    st = library().moe_w4a16_align(
        topk_ids.data_ptr(), ctypes.byref(p), block_m, sorted_ids.data_ptr(), cap_s,
        block_expert.data_ptr(), cap_b, n_padded.data_ptr(),
        None if scratch is None else scratch.data_ptr(), nbytes, _stream_handle(dev))
    _check(st)
    return sorted_ids, block_expert, n_padded[:1]
