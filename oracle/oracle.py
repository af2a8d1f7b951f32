"""CPU oracle of the W4A16 routed-expert MoE layer -- test infrastructure only.

Only the tests, the package smoke check and the bench's CPU-baseline leg may
use this module. It shares no code with the GPU library and never imports it.

Contents
  forward      fp64 layer output, C implementation (moe_oracle.c), threaded
               over tokens; optional token subset.
  dense_moe    the same layer written a second, independent way in numpy
               (dense [T, E] routing matrix, every expert run on every token),
               for tiny shapes only; used to cross-check `forward`.
  unpack_int4 / pack_int4 / dequant_int4
               the int4 storage format in numpy.
  align        the token/expert bucketing: a stable sort of the valid
               (token, slot) pairs by local expert, each bucket padded to a
               multiple of block_m with the sentinel T*k.
  route        the router step in front of the layer: top-k experts per
               token from fp32 scores, weights = softmax over the selected.

Readings of the pages (Kimi-K2.6 catalog entry: QUANT paragraph -- INT4,
compressed-tensors pack-quantized, group 32, symmetric; PARAMS paragraph --
int4 values in int32 containers): element c of a row sits in word c//8 at bits
4*(c%8)..4*(c%8)+3 (low nibble first), the stored field u encodes q = u - 8,
and the bf16 scale of group c//32 multiplies q. Gate rows [0, I) come before up
rows [I, 2I); the activation is SwiGLU silu(gate)*up; routing weights apply as
given; ids outside [base, base + E) (including -1) contribute nothing.

The pages print no layer output, so parity against the pages' numbers is
unpinned; the tests pin this module to closed forms, library routines,
brute force and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
GROUP = 32

_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into oracle/libmoe_oracle.so."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_forward.argtypes = [P] * 9 + [I64] * 6 + [P, I64, I64]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_int4_code.argtypes = [P, I64]
        lib.oracle_int4_code.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
            shared_w=None, expert_base: int = 0, rows=None, threads: Optional[int] = None):
    """fp64 reference output [len(rows) or T, H] (C implementation)."""
    lib = _load()
    x = _c(x, np.uint16)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    pw13 = _c(packed_w13, np.int32)
    s13 = _c(scales_w13, np.uint16)
    pw2 = _c(packed_w2, np.int32)
    s2 = _c(scales_w2, np.uint16)
    sh = _c(shared_w, np.uint16)
    T, H = x.shape
    E, I2, _ = pw13.shape
    I = I2 // 2
    k = ids.shape[1]
    assert ids.shape == (T, k) and wts.shape == (T, k)
    assert pw13.shape == (E, 2 * I, H // 8) and s13.shape == (E, 2 * I, H // GROUP)
    assert pw2.shape == (E, H, I // 8) and s2.shape == (E, H, I // GROUP)
    if sh is not None:
        assert sh.size == 2 * I * H + H * I
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = T if r is None else r.size
    out = np.zeros((n, H), np.float64)
    rc = lib.oracle_forward(_ptr(x), _ptr(ids), _ptr(wts), _ptr(pw13), _ptr(s13), _ptr(pw2),
                            _ptr(s2), _ptr(sh), _ptr(out), T, H, I, E, expert_base, k,
                            _ptr(r), n, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments")
    return out


def silu_c(z: float) -> float:
    return _load().oracle_silu(float(z))


def int4_code_c(words: np.ndarray, c: int) -> int:
    w = np.ascontiguousarray(words, dtype=np.int32)
    return _load().oracle_int4_code(_ptr(w), int(c))


# ----------------------------------------------------------------------------
# numpy side
# ----------------------------------------------------------------------------
def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """int32 [..., C/8] -> signed codes int8 [..., C] (low nibble first,
    excess-8)."""
    u = np.ascontiguousarray(packed).view(np.uint32)
    fields = (u[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    q = fields.astype(np.int16) - 8
    return q.reshape(*packed.shape[:-1], packed.shape[-1] * 8).astype(np.int8)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """signed codes in [-8, 7], [..., C] -> int32 [..., C/8]."""
    q = np.asarray(q)
    assert q.shape[-1] % 8 == 0
    assert q.min() >= -8 and q.max() <= 7
    u = (q.astype(np.int64) + 8).astype(np.uint32)
    u = u.reshape(*q.shape[:-1], q.shape[-1] // 8, 8)
    word = np.zeros(u.shape[:-1], np.uint32)
    for i in range(8):
        word |= u[..., i] << np.uint32(4 * i)
    return word.view(np.int32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_int4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[..., n, c] = q[..., n, c] * s[..., n, c // 32] in fp64."""
    q = unpack_int4(packed).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales), GROUP, axis=-1)
    return q * s


def _swiglu_mlp(X, W13, W2, I):
    A = X @ W13.T
    g, u = A[:, :I], A[:, I:]
    return ((g / (1.0 + np.exp(-g))) * u) @ W2.T


def dense_moe(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
              shared_w=None, expert_base: int = 0) -> np.ndarray:
    """The layer as a dense mixture: R[t, e] = sum of the weights of the slots of
    token t that select local expert e; out = S(X) + sum_e R[:, e] * F_e(X).
    Every expert runs on every token (tiny shapes only)."""
    X = bf16_to_f64(x)
    T, H = X.shape
    E, I2, _ = packed_w13.shape
    I = I2 // 2
    ids = np.asarray(topk_ids, np.int64)
    wts = np.asarray(topk_weights, np.float64)
    R = np.zeros((T, E))
    local = (ids >= expert_base) & (ids < expert_base + E)
    tt, jj = np.nonzero(local)
    np.add.at(R, (tt, ids[tt, jj] - expert_base), wts[tt, jj])
    out = np.zeros((T, H))
    if shared_w is not None:
        sw = bf16_to_f64(shared_w)
        out += _swiglu_mlp(X, sw[: 2 * I * H].reshape(2 * I, H), sw[2 * I * H:].reshape(H, I), I)
    for e in range(E):
        if not R[:, e].any():
            continue
        W13 = dequant_int4(packed_w13[e], scales_w13[e])
        W2 = dequant_int4(packed_w2[e], scales_w2[e])
        out += R[:, e:e + 1] * _swiglu_mlp(X, W13, W2, I)
    return out


def align(topk_ids, num_experts: int, expert_base: int, block_m: int):
    """Bucket the (token, slot) pairs by local expert.

    A pair p = t*k + j is valid when expert_base <= id < expert_base + E; its
    local expert is id - expert_base. Bucket e holds the valid pairs of expert
    e in ascending p, padded with the sentinel T*k up to a multiple of block_m
    (an expert without pairs gets an empty bucket). Buckets follow each other
    in expert order.

    Returns (sorted_ids int32 [n_padded], block_expert int32 [n_padded/block_m],
    n_padded).
    """
    ids = np.asarray(topk_ids, np.int64).ravel()
    P = ids.size
    valid = (ids >= expert_base) & (ids < expert_base + num_experts)
    p_valid = np.nonzero(valid)[0]
    e_valid = ids[p_valid] - expert_base
    order = np.argsort(e_valid, kind="stable")
    p_sorted, e_sorted = p_valid[order], e_valid[order]
    cnt = np.bincount(e_valid, minlength=num_experts)
    pad = -(-cnt // block_m) * block_m
    off = np.concatenate([[0], np.cumsum(pad)[:-1]])
    n_padded = int(pad.sum())
    sorted_ids = np.full(n_padded, P, np.int32)
    first = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    rank = np.arange(p_sorted.size) - first[e_sorted]
    sorted_ids[off[e_sorted] + rank] = p_sorted
    block_expert = np.repeat(np.arange(num_experts, dtype=np.int32), pad // block_m)
    return sorted_ids, block_expert, n_padded


def route(scores, top_k: int):
    """The router step that produces the layer's routing inputs.

    The lmdeploy pull request (Runtime Validation) lists MoE routing among the
    validated paths without giving a formula; the plainest rule, the one the
    synthetic inputs follow, is taken: for each token the top_k experts with
    the largest scores, in descending score order, equal scores in ascending
    expert id (-0.0 equals +0.0); weights = softmax over the selected scores,
    which is the softmax over all experts renormalised over the selected ones.
    Selection compares the fp32 scores as given; the weights are computed in
    fp64. Scores must not be NaN.

    Returns (ids int32 [T, top_k], weights float64 [T, top_k]).
    """
    s = np.asarray(scores, np.float32).astype(np.float64)
    T, E = s.shape
    assert 1 <= top_k <= E
    ids = np.argsort(-s, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])  # the first selected score is the largest
    return ids, z / z.sum(axis=1, keepdims=True)
