"""Seeded synthetic inputs for the W4A16 routed-expert MoE layer.

This module is shared by the tests, the bench and the oracle checks. It only
draws random numbers and lays them out in the storage formats of the layer; it
holds none of the layer's arithmetic (no unpacking, dequantisation, GEMM,
activation or combine).

Formats (all row-major, little-endian):
  x            bf16 bit patterns, uint16 [T, H]
  topk_ids     int32 [T, k]
  topk_weights float32 [T, k]
  packed_w13   int32 [E, 2I, H/8]   eight 4-bit codes per word
  scales_w13   bf16 bits, uint16 [E, 2I, H/32]
  packed_w2    int32 [E, H, I/8]
  scales_w2    bf16 bits, uint16 [E, H, I/32]
  shared_w     bf16 bits, uint16 [2I*H + H*I]  (gate/up [2I, H], then down [H, I])

Every expert has its own random stream, keyed by (seed, tag, expert), so any
subset of a weight bank can be regenerated without drawing the rest.

Distributions (Kimi-K2.6 catalog entry, MoE/QUANT paragraphs, give the
geometry and the int4 group-32 symmetric format; the value distributions are
this project's synthetic recipe):
  * packed words: uniform random 32-bit words, i.e. every 4-bit code uniform
    in [0, 15];
  * scales: bf16 of U(0.005, 0.02);
  * x: bf16 of N(0, 1);
  * routing: k distinct experts per token (uniform, or Zipf-skewed via
    Gumbel-top-k), weights = softmax over the k selected N(0, 1) logits;
  * shared expert: bf16 of q*s with q uniform in [-8, 7] and s ~ U(0.005, 0.02)
    per (row, group of 32 inputs).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

GROUP = 32

TAG_W13 = 13
TAG_W2 = 2
TAG_SHARED = 7
TAG_X = 11
TAG_ROUTE = 17
TAG_ZIPF_PERM = 19
TAG_SCORES = 23

SCALE_LO = 0.005
SCALE_HI = 0.02


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns
    the 16-bit patterns. Finite inputs only."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    hidden: int
    inter: int
    n_experts: int   # experts in the bank (global id space)
    top_k: int
    shared: bool

    @property
    def words_w13(self) -> int:
        return self.hidden // 8

    @property
    def words_w2(self) -> int:
        return self.inter // 8


# Kimi-K2.6 text config: hidden 7168, 384 routed experts, 8 per token,
# one shared expert, moe_intermediate_size 2048 (catalog entry, GEOMETRY / MoE).
KIMI = Geometry(hidden=7168, inter=2048, n_experts=384, top_k=8, shared=True)
TINY = Geometry(hidden=256, inter=128, n_experts=8, top_k=2, shared=False)
# one GPU's share of the same layer split 8 ways by tensor parallelism: every
# expert (and the shared expert) keeps all 7168 inputs and outputs but only
# 2048 / 8 = 256 intermediate columns (8 whole scale groups)
TP8_SHARE = Geometry(hidden=7168, inter=256, n_experts=384, top_k=8, shared=True)


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------
def _uniform_f32(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return rng.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)


def _scales(rng: np.random.Generator, rows: int, groups: int) -> np.ndarray:
    return f32_to_bf16_bits(_uniform_f32(rng, (rows, groups), SCALE_LO, SCALE_HI))


def _random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform random 32-bit words (two per 64-bit output of the generator)."""
    n = int(np.prod(shape))
    raw = rng.bit_generator.random_raw((n + 1) // 2)
    return raw.view("<i4")[:n].reshape(shape)


def expert_weights(seed: int, e: int, hidden: int, inter: int):
    """One routed expert: (packed_w13 [2I, H/8], scales_w13 [2I, H/32],
    packed_w2 [H, I/8], scales_w2 [H, I/32])."""
    r13 = _rng(seed, TAG_W13, e)
    pw13 = _random_words(r13, (2 * inter, hidden // 8))
    s13 = _scales(r13, 2 * inter, hidden // GROUP)
    r2 = _rng(seed, TAG_W2, e)
    pw2 = _random_words(r2, (hidden, inter // 8))
    s2 = _scales(r2, hidden, inter // GROUP)
    return pw13, s13, pw2, s2


@dataclass
class Bank:
    packed_w13: np.ndarray
    scales_w13: np.ndarray
    packed_w2: np.ndarray
    scales_w2: np.ndarray

    @property
    def n_experts(self) -> int:
        return self.packed_w13.shape[0]


def weight_bank(seed: int, hidden: int, inter: int, experts: Sequence[int]) -> Bank:
    """Stack the given experts (in the given order) into [E, ...] arrays."""
    E = len(experts)
    pw13 = np.empty((E, 2 * inter, hidden // 8), np.int32)
    s13 = np.empty((E, 2 * inter, hidden // GROUP), np.uint16)
    pw2 = np.empty((E, hidden, inter // 8), np.int32)
    s2 = np.empty((E, hidden, inter // GROUP), np.uint16)
    for i, e in enumerate(experts):
        a, b, c, d = expert_weights(seed, e, hidden, inter)
        pw13[i], s13[i], pw2[i], s2[i] = a, b, c, d
    return Bank(pw13, s13, pw2, s2)


def shared_weights(seed: int, hidden: int, inter: int) -> np.ndarray:
    """bf16 shared expert, flat: gate/up [2I, H] followed by down [H, I]."""
    r = _rng(seed, TAG_SHARED)

    def mat(rows: int, cols: int) -> np.ndarray:
        q = (_random_words(r, (rows * cols + 3) // 4).view(np.uint8)[:rows * cols] & 15).astype(np.float32) - 8.0
        s = _uniform_f32(r, (rows, cols // GROUP), SCALE_LO, SCALE_HI)
        w = q.reshape(rows, cols // GROUP, GROUP) * s[:, :, None]
        return f32_to_bf16_bits(w.reshape(rows, cols))

    return np.concatenate([mat(2 * inter, hidden).ravel(), mat(hidden, inter).ravel()])


# --------------------------------------------------------------------------
# activations and routing
# --------------------------------------------------------------------------
def activations(seed: int, T: int, hidden: int) -> np.ndarray:
    r = _rng(seed, TAG_X)
    return f32_to_bf16_bits(r.standard_normal(size=(T, hidden), dtype=np.float32))


def _softmax_weights(r: np.random.Generator, T: int, k: int) -> np.ndarray:
    logits = r.standard_normal(size=(T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def routing_uniform(seed: int, T: int, n_experts: int, k: int):
    """k distinct experts per token, uniform: the first k of a random
    permutation of the experts."""
    r = _rng(seed, TAG_ROUTE)
    keys = r.random(size=(T, n_experts))
    ids = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    return np.ascontiguousarray(ids), _softmax_weights(r, T, k)


def routing_zipf(seed: int, T: int, n_experts: int, k: int, s: float = 1.2):
    """k distinct experts per token drawn without replacement from a Zipf(s)
    law over ranks 1..n (Gumbel-top-k on log p); ranks map to expert ids via
    a seeded permutation."""
    r = _rng(seed, TAG_ROUTE)
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    logp = -s * np.log(ranks)
    logp -= np.log(np.exp(logp).sum())
    g = r.gumbel(size=(T, n_experts))
    top = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :k]
    perm = _rng(seed, TAG_ZIPF_PERM).permutation(n_experts)
    ids = perm[top].astype(np.int32)
    return np.ascontiguousarray(ids), _softmax_weights(r, T, k)


def router_scores(seed: int, T: int, n_experts: int) -> np.ndarray:
    """fp32 router scores [T, n_experts], N(0, 1): the input of the router step."""
    return _rng(seed, TAG_SCORES).standard_normal(size=(T, n_experts), dtype=np.float32)


# --------------------------------------------------------------------------
# tensor-parallel shards (slicing only)
# --------------------------------------------------------------------------
def tp_shard(bank: Bank, shared_w: Optional[np.ndarray], hidden: int, inter: int,
             rank: int, n: int):
    """Rank `rank` of an n-way split of the intermediate dimension: gate rows
    and up rows [rank*I/n, (rank+1)*I/n) of W13 (with their scales), the same
    input columns of W2 (packed words and scale groups), and the same cut of
    the shared expert. I/n must be a whole number of scale groups."""
    Is = inter // n
    assert Is * n == inter and Is % GROUP == 0
    lo, hi = rank * Is, (rank + 1) * Is
    rows = np.r_[lo:hi, inter + lo:inter + hi]
    b = Bank(np.ascontiguousarray(bank.packed_w13[:, rows]),
             np.ascontiguousarray(bank.scales_w13[:, rows]),
             np.ascontiguousarray(bank.packed_w2[:, :, lo // 8:hi // 8]),
             np.ascontiguousarray(bank.scales_w2[:, :, lo // GROUP:hi // GROUP]))
    sh = None
    if shared_w is not None:
        gu = shared_w[:2 * inter * hidden].reshape(2 * inter, hidden)
        dn = shared_w[2 * inter * hidden:].reshape(hidden, inter)
        sh = np.concatenate([gu[rows].ravel(), dn[:, lo:hi].ravel()])
    return b, sh


# --------------------------------------------------------------------------
# crafted bit patterns for invariant tests (no arithmetic of the layer)
# --------------------------------------------------------------------------
def const_code_word(code: int) -> np.int32:
    """A 32-bit word whose eight 4-bit fields all hold `code` (0..15)."""
    assert 0 <= code < 16
    return np.array([code * 0x11111111], dtype=np.uint32).view(np.int32)[0]


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    geo: Geometry
    T: int
    n_local: int          # experts present in the packed tensors
    expert_base: int      # global id of local expert 0
    routing: str          # "uniform" | "zipf"
    seed_bank: int = 1
    seed_x: int = 100
    seed_route: int = 200

    def bank_experts(self) -> list:
        return list(range(self.expert_base, self.expert_base + self.n_local))


def workload(name: str, T: Optional[int] = None) -> Workload:
    """Named synthetic workloads.

    tiny     hidden 256, inter 128, 8 experts, top-2, 16 tokens, no shared expert
    decode   Kimi-K2.6 shape (7168 / 2048, 384 experts, top-8, bf16 shared
             expert), T in {1, 8, 32, 64}, uniform distinct routing
    prefill  same layer, 4096 tokens, uniform routing
    skew     same layer, 512 tokens, Zipf(1.2) routing
    ep       48 local experts (global ids 0..47) of the same bank, 2048 tokens
             routed uniformly over all 384; only local pairs are computed
    tp8_decode   one GPU's share of the layer under 8-way tensor parallelism
             (moe_intermediate 256 per expert and for the shared expert),
             T in {1, 8, 32, 64}; an independent bank (seed 2) with the same
             value distributions, routing identical to `decode`
    tp8_prefill  the same share at 4096 tokens, routing identical to `prefill`
    """
    if name == "tiny":
        return Workload("tiny", TINY, T or 16, 8, 0, "uniform", seed_bank=5)
    if name == "decode":
        return Workload("decode", KIMI, T or 64, 384, 0, "uniform")
    if name == "prefill":
        return Workload("prefill", KIMI, T or 4096, 384, 0, "uniform")
    if name == "skew":
        return Workload("skew", KIMI, T or 512, 384, 0, "zipf")
    if name == "ep":
        return Workload("ep", KIMI, T or 2048, 48, 0, "uniform")
    if name == "tp8_decode":
        return Workload("tp8_decode", TP8_SHARE, T or 64, 384, 0, "uniform", seed_bank=2)
    if name == "tp8_prefill":
        return Workload("tp8_prefill", TP8_SHARE, T or 4096, 384, 0, "uniform", seed_bank=2)
    raise ValueError(f"unknown workload {name!r}")


def make_routing(w: Workload):
    g = w.geo
    if w.routing == "uniform":
        return routing_uniform(w.seed_route + w.T, w.T, g.n_experts, g.top_k)
    return routing_zipf(w.seed_route + w.T, w.T, g.n_experts, g.top_k)


def make_inputs(w: Workload, bank: Optional[Bank] = None):
    """Everything the layer needs for workload `w` (host arrays)."""
    g = w.geo
    if bank is None:
        bank = weight_bank(w.seed_bank, g.hidden, g.inter, w.bank_experts())
    x = activations(w.seed_x + w.T, w.T, g.hidden)
    ids, wts = make_routing(w)
    shared = shared_weights(w.seed_bank, g.hidden, g.inter) if g.shared else None
    return dict(x=x, topk_ids=ids, topk_weights=wts, bank=bank, shared_w=shared,
                expert_base=w.expert_base)


# --------------------------------------------------------------------------
# host <-> device (uint16 arrays are bf16 bit patterns)
# --------------------------------------------------------------------------
def to_device(a: np.ndarray, device):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch

    b = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f32(b).astype(np.float64)


def device_bank(seed: int, hidden: int, inter: int, experts: Sequence[int], device) -> dict:
    """The bank of `experts` generated expert by expert straight into device
    tensors (no host copy of the whole bank)."""
    import torch

    E = len(experts)
    pw13 = torch.empty((E, 2 * inter, hidden // 8), dtype=torch.int32, device=device)
    s13 = torch.empty((E, 2 * inter, hidden // GROUP), dtype=torch.bfloat16, device=device)
    pw2 = torch.empty((E, hidden, inter // 8), dtype=torch.int32, device=device)
    s2 = torch.empty((E, hidden, inter // GROUP), dtype=torch.bfloat16, device=device)
    for i, e in enumerate(experts):
        a, b, c, d = expert_weights(seed, e, hidden, inter)
        pw13[i].copy_(to_device(a, device))
        s13[i].copy_(to_device(b, device))
        pw2[i].copy_(to_device(c, device))
        s2[i].copy_(to_device(d, device))
    return dict(packed_w13=pw13, scales_w13=s13, packed_w2=pw2, scales_w2=s2)


def compact_routing(topk_ids: np.ndarray, rows, expert_base: int, n_local: int):
    """For the tokens `rows`: the sorted global ids of the local experts they
    use, and their ids renumbered into that list (non-local ids -> -1)."""
    ids = np.asarray(topk_ids)[np.asarray(rows)]
    local = (ids >= expert_base) & (ids < expert_base + n_local)
    used = np.unique(ids[local])
    remap = np.full(ids.shape, -1, np.int32)
    remap[local] = np.searchsorted(used, ids[local]).astype(np.int32)
    return [int(u) for u in used], remap
