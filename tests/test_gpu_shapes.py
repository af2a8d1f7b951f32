"""Layer parity over a spread of shapes that reach every kernel path and its
edges: K not a multiple of the small-batch iteration (partial last
iteration), down widths that take the narrow-K kernel (I = 128, 384), the
streamed down kernel with several slice groups per work-group, the
largest top-k (16) and expert count (512), expert bases with non-local ids,
the decode launches that bucket the pairs themselves (at most 64 pairs and 8
tokens) with their down-and-combine kernel's partial column slices,
ragged token counts, both block sizes (4 and 96), and on the 96-row path
widths that are not whole tiles (hidden % 512, inter % 256: masked column
tiles) with an odd number of 128-input chunks.

Every routed product on the 96-row path uses the exact dequantised weights
(fp16), as the small-batch path does; the cases without a shared expert and
with hundreds of thousands to over a million outputs are the ones whose
largest elementwise error is most exposed (heavy-tailed outputs, no shared
term), so each reports max_small_err_over_rms and must stay below 0.015."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.helpers import check, run_layer

pytestmark = pytest.mark.gpu

CASES = [
    # T, H, I, E, k, base, shared, expected block_m
    (3, 640, 384, 8, 2, 0, True, 4),       # K = 640: one full and one partial iteration
    (5, 1152, 640, 6, 3, 1, False, 4),     # K = 1152 and a down K of 640 (partial iterations)
    (1, 384, 128, 16, 16, 0, True, 4),     # top-16, narrow down (I = 128)
    (8, 256, 128, 512, 8, 0, True, 4),     # 512 local experts
    (120, 2048, 640, 128, 4, 0, True, 4),  # streamed down: 3 slice groups per work-group, last run of 2
    # at most 64 pairs and 8 tokens: the launches bucket the pairs themselves
    # and the down launch also combines
    (4, 2176, 256, 8, 4, 0, True, 4),      # 3 row-sets per work-group, a partial last one
    (8, 512, 256, 4, 2, 0, True, 4),       # four local experts of six
    (4, 384, 128, 64, 16, 0, False, 4),    # 64 pairs on up to 64 experts, non-local ids
    (6, 640, 1152, 12, 4, 3, True, 4),     # expert base, down K = 1152 (partial iteration)
    (33, 640, 384, 8, 4, 0, True, 96),     # 96-row blocks: masked tiles both phases, 5 / 3 chunks
    (97, 384, 640, 6, 2, 2, True, 96),     # masked tiles, 3 / 5 chunks, expert base
    (150, 1024, 512, 8, 2, 1, True, 96),   # whole tiles, expert base
    (700, 1536, 512, 10, 2, 0, True, 96),  # whole tiles, shared expert in 8 token blocks
    (301, 1024, 768, 4, 3, 0, False, 96),  # no shared expert, 308k outputs
    (1100, 1024, 768, 4, 3, 0, False, 96), # no shared expert, 1.13M outputs
    (260, 896, 1152, 5, 2, 0, False, 96),  # no shared expert, masked tiles, 7 / 9 chunks
    (200, 512, 128, 4, 2, 0, True, 96),    # down K = 128: a single chunk; gate_up tile half masked
    (2, 14336, 256, 8, 4, 0, True, 96),    # two tokens on 96-row blocks: the 4-row kernel's staged
                                           # scales for K = 14336 exceed its LDS; one-row blocks
]



@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    return torch.device("cuda:0")


@pytest.mark.parametrize("T,H,I,E,k,base,shared,bm", CASES)
def test_shape(dev, T, H, I, E, k, base, shared, bm):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    got_bm = moe.forward_block_m(moe.problem(T, H, I, E, k, base))
    assert got_bm == bm, got_bm
    seed = 1000 + T + H + I
    n_global = base + E + 2
    bank = mi.weight_bank(seed, H, I, list(range(base, base + E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    x = mi.activations(seed + 1, T, H)
    ids, w = mi.routing_uniform(seed + 2, T, n_global, min(k, n_global))
    if base:
        ids[::5, 0] = -1
    sw = mi.shared_weights(seed + 3, H, I) if shared else None
    print(f"[case] T={T} H={H} I={I} E={E} k={k} base={base} shared={shared} bm={bm}",
          flush=True)
    out = run_layer(dev, x, ids, w, bank_dev, sw, expert_base=base)
    torch.cuda.synchronize()
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw, base)
    res = check(mi.bf16_tensor_to_f64(out), ref, f"T={T} H={H} I={I} E={E} k={k} bm={bm}")
    assert res["max_small_err_over_rms"] <= 0.015, res


def test_local_buckets_spanning_blocks(dev):
    """The launches that bucket the pairs themselves (at most 64 pairs and 8
    tokens), with buckets longer than one 4-row block: experts 0 and 1 take
    six and eight pairs (two blocks each), an invalid id and a non-local one
    drop their pairs."""
    import torch

    T, H, I, E, k = 8, 640, 384, 8, 2
    ids = np.zeros((T, k), np.int32)
    ids[:, 0] = 1
    ids[:6, 1] = 0
    ids[6, 1] = 5
    ids[7, 1] = -1
    ids[5, 0] = 9  # not a local expert
    w = np.random.default_rng(7).uniform(0.1, 1.0, (T, k)).astype(np.float32)
    bank = mi.weight_bank(71, H, I, list(range(E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    x = mi.activations(72, T, H)
    sw = mi.shared_weights(73, H, I)
    out = run_layer(dev, x, ids, w, bank_dev, sw)
    torch.cuda.synchronize()
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw, 0)
    check(mi.bf16_tensor_to_f64(out), ref, "local buckets spanning blocks")


@pytest.mark.parametrize("shared", [True, False])
def test_split_buckets(dev, shared):
    """A call with 96-row buckets and fewer than 8192 pairs: experts with at
    most 4 pairs (here 1, 3 and exactly 4) are bucketed in 4 rows and take the
    decode-sized kernels, the others (5 pairs, just over, and 40 and more)
    keep 96-row buckets; an expert without pairs, a non-local id and an
    invalid id drop out. Both sets in one call, against the oracle, and the
    prepacked form equal to it bit for bit."""
    import torch

    import w4a16_int4_grouped_moe_amd as moe

    H, I, E, k, base = 1024, 512, 10, 2, 3  # widths the prepacked layout serves
    want = [40, 1, 3, 4, 5, 0, 57, 4, 1, 3]  # pairs per local expert
    valid = np.repeat(np.arange(E, dtype=np.int32), want) + base  # sorted by expert
    T = (len(valid) + 2) // k
    s = np.concatenate([valid, np.array([1, -7], np.int32)])  # non-local, invalid
    # token t takes positions t and t + T of the sorted list: distinct experts,
    # as no expert holds T or more pairs
    assert max(want) < T and len(s) == T * k
    ids = np.stack([s[:T], s[T:]], axis=1)
    ids = ids[np.random.default_rng(11).permutation(T)]
    assert moe.forward_block_m(moe.problem(T, H, I, E, k, base)) == 96
    loc = ids[(ids >= base) & (ids < base + E)] - base
    assert np.bincount(loc, minlength=E).tolist() == want
    assert all(ids[t, 0] != ids[t, 1] for t in range(T))
    w = np.random.default_rng(12).uniform(0.1, 1.0, (T, k)).astype(np.float32)
    bank = mi.weight_bank(81, H, I, list(range(base, base + E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    x = mi.activations(82, T, H)
    sw = mi.shared_weights(83, H, I) if shared else None
    print(f"[case] split buckets T={T} shared={shared}", flush=True)
    out = run_layer(dev, x, ids, w, bank_dev, sw, base)
    d = lambda a: mi.to_device(a, dev)
    pk = moe.prepack(bank_dev["packed_w13"], bank_dev["scales_w13"], bank_dev["packed_w2"],
                     bank_dev["scales_w2"])
    out_pk = moe.forward_prepacked(d(x), d(ids), d(w), pk, None if sw is None else d(sw),
                                   expert_base=base)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_pk.view(torch.int16))
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw, base)
    check(mi.bf16_tensor_to_f64(out), ref, f"split buckets shared={shared}")


def _random_cases(seed, n):
    """Seeded random shapes of the 96-row path: widths any multiple of 128 up
    to 3968 (an odd or even number of 128-input chunks, masked column
    tiles), 1-16 local experts with an expert base, top-1..8, with and
    without a shared expert, enough pairs per expert for 96-row buckets (and
    the split bucketing wherever an expert has at most 4 pairs)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = 128 * int(rng.integers(1, 32))
        I = 128 * int(rng.integers(1, 17))
        E = int(rng.integers(1, 17))
        k = int(rng.integers(1, min(E, 8) + 1))
        base = int(rng.integers(0, 3))
        T = int(rng.integers(4 * E // k + 8, 4 * E // k + 1200))
        out.append((T, H, I, E, k, base, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("T,H,I,E,k,base,shared", _random_cases(2026, 12))
def test_random_shapes_96(dev, T, H, I, E, k, base, shared):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    assert moe.forward_block_m(moe.problem(T, H, I, E, k, base)) == 96
    seed = 7000 + T + H + I
    bank = mi.weight_bank(seed, H, I, list(range(base, base + E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    x = mi.activations(seed + 1, T, H)
    n_global = base + E + 2
    ids, w = mi.routing_uniform(seed + 2, T, n_global, min(k, n_global))
    if base:
        ids[::7, 0] = -1
    sw = mi.shared_weights(seed + 3, H, I) if shared else None
    print(f"[case] random T={T} H={H} I={I} E={E} k={k} base={base} shared={shared}", flush=True)
    out = run_layer(dev, x, ids, w, bank_dev, sw, expert_base=base)
    torch.cuda.synchronize()
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw, base)
    res = check(mi.bf16_tensor_to_f64(out), ref, f"random T={T} H={H} I={I} E={E} k={k}")
    assert res["max_small_err_over_rms"] <= 0.015, res
