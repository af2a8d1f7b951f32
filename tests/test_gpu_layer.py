"""Layer parity: the HIP path against the fp64 oracle, elementwise, on the
seeded synthetic workloads (full rows where the oracle is quick, sampled
tokens at full size -- tokens are independent, so a sampled row is checked
exactly as in a full run)."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.helpers import block_edge_tokens, check, oracle_rows, run_layer, sample_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    return torch.device("cuda:0")


# ---------------------------------------------------------------- tiny shapes
@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("T", [1, 5, 16, 100])
def test_tiny(dev, shared, T):
    import torch

    g = mi.TINY
    bank = mi.weight_bank(5, g.hidden, g.inter, list(range(g.n_experts)))
    bank_dev = {k: mi.to_device(v, dev) for k, v in bank.__dict__.items()}
    x = mi.activations(6 + T, T, g.hidden)
    ids, w = mi.routing_uniform(7 + T, T, g.n_experts, g.top_k)
    sw = mi.shared_weights(5, g.hidden, g.inter) if shared else None
    print(f"[case] tiny T={T} shared={shared}", flush=True)
    out = run_layer(dev, x, ids, w, bank_dev, sw)
    torch.cuda.synchronize()
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw)
    check(mi.bf16_tensor_to_f64(out), ref, f"tiny T={T} shared={shared}")


@pytest.mark.parametrize("T,E,k,base,bm_rows", [
    (300, 12, 4, 0, "many rows per expert"),
    (40, 20, 6, 5, "expert base with invalid ids"),
])
def test_mid_shapes(dev, T, E, k, base, bm_rows):
    import torch

    H, I = 512, 384
    n_global = base + E + 4
    bank = mi.weight_bank(9, H, I, list(range(base, base + E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    x = mi.activations(10, T, H)
    ids, w = mi.routing_uniform(11, T, n_global, k)
    ids[::7, 0] = -1
    sw = mi.shared_weights(9, H, I)
    print(f"[case] mid T={T} E={E} k={k} base={base}", flush=True)
    out = run_layer(dev, x, ids, w, bank_dev, sw, expert_base=base)
    torch.cuda.synchronize()
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw, base)
    check(mi.bf16_tensor_to_f64(out), ref, f"mid T={T} ({bm_rows})")


@pytest.mark.parametrize("T,H,I,E,k,base,shared", [
    (500, 1024, 512, 6, 2, 0, True),     # two column tiles per phase, 2-3 blocks per expert
    (400, 512, 256, 5, 4, 3, True),      # expert base, non-local and invalid ids
    (130, 2048, 256, 2, 2, 0, True),     # several scale buffers per block (K = 2048)
])
def test_prefill_shapes(dev, T, H, I, E, k, base, shared):
    """Shapes that take the prefill kernel (many rows per expert, widths that
    fit its tiles): block row counts from a few rows to full blocks."""
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    n_global = base + E + 3
    bm = moe.forward_block_m(moe.problem(T, H, I, E, k, base))
    assert bm > 64, bm
    bank = mi.weight_bank(40 + H, H, I, list(range(base, base + E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    x = mi.activations(41, T, H)
    ids, w = mi.routing_uniform(42, T, n_global, k)
    ids[::11, -1] = -1
    sw = mi.shared_weights(43, H, I) if shared else None
    print(f"[case] prefill T={T} H={H} I={I} E={E} k={k} base={base} bm={bm}", flush=True)
    out = run_layer(dev, x, ids, w, bank_dev, sw, expert_base=base)
    torch.cuda.synchronize()
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw, base)
    check(mi.bf16_tensor_to_f64(out), ref, f"prefill T={T} H={H} I={I}")


# ------------------------------------------------------- Kimi-K2.6 layer shape
@pytest.fixture(scope="module")
def kimi(dev):
    g = mi.KIMI
    print("[fixture] generating the 384-expert Kimi-shape bank on the device", flush=True)
    bank = mi.device_bank(1, g.hidden, g.inter, list(range(g.n_experts)), dev)
    shared = mi.shared_weights(1, g.hidden, g.inter)
    return bank, shared


def _kimi_case(dev, kimi, name, T, rows=None, n_sample=None):
    import torch

    bank, shared = kimi
    w = mi.workload(name, T)
    g = w.geo
    x = mi.activations(w.seed_x + w.T, w.T, g.hidden)
    ids, wts = mi.make_routing(w)
    if rows is None:
        rows = np.arange(T) if n_sample is None else np.sort(
            np.random.default_rng(T).choice(T, n_sample, replace=False))
    print(f"[case] {name} T={T} rows={len(rows)}", flush=True)
    sub = {k: v[w.expert_base:w.expert_base + w.n_local] for k, v in bank.items()}
    out = run_layer(dev, x, ids, wts, sub, shared, expert_base=w.expert_base)
    torch.cuda.synchronize()
    got = mi.bf16_tensor_to_f64(out)
    assert np.isfinite(got).all()
    ref = oracle_rows(w.seed_bank, g, x, ids, wts, shared, w.expert_base, w.n_local, rows)
    return check(got[rows], ref, f"{name} T={T}")


@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_kimi_decode(dev, kimi, T):
    _kimi_case(dev, kimi, "decode", T)


def _edge_sample(name, T, n_min=256):
    """At least n_min tokens of the workload, among them the first and last
    rows of every local expert's last 96-row block."""
    import w4a16_int4_grouped_moe_amd as moe

    w = mi.workload(name, T)
    ids, _ = mi.make_routing(w)
    bm = moe.forward_block_m(moe.problem(T, w.geo.hidden, w.geo.inter, w.n_local, w.geo.top_k,
                                         w.expert_base))
    must = block_edge_tokens(ids, w.expert_base, w.n_local, bm)
    return sample_tokens(T, must, n_min, seed=T)


def test_kimi_prefill_sampled(dev, kimi):
    # 4096 tokens: every expert's last block (about one in nine experts
    # overflows its first 96-row block), ~400 tokens checked
    _kimi_case(dev, kimi, "prefill", 4096, rows=_edge_sample("prefill", 4096))


def test_kimi_skew_full(dev, kimi):
    # all 512 tokens of the Zipf batch (hot experts span several blocks)
    _kimi_case(dev, kimi, "skew", 512)


def test_kimi_expert_parallel_share_sampled(dev, kimi):
    _kimi_case(dev, kimi, "ep", 2048, rows=_edge_sample("ep", 2048))


# ------------------------------------- 8-way tensor-parallel share (I = 256)
@pytest.fixture(scope="module")
def tp8(dev):
    w = mi.workload("tp8_decode")
    g = w.geo
    print("[fixture] generating the 384-expert I=256 bank on the device", flush=True)
    bank = mi.device_bank(w.seed_bank, g.hidden, g.inter, list(range(g.n_experts)), dev)
    shared = mi.shared_weights(w.seed_bank, g.hidden, g.inter)
    return bank, shared


@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_tp8_share_decode(dev, tp8, T):
    _kimi_case(dev, tp8, "tp8_decode", T)


def test_tp8_share_prefill_sampled(dev, tp8):
    import w4a16_int4_grouped_moe_amd as moe

    g = mi.TP8_SHARE
    print(f"[case] tp8_prefill block_m "
          f"{moe.forward_block_m(moe.problem(4096, g.hidden, g.inter, 384, 8, 0))}", flush=True)
    _kimi_case(dev, tp8, "tp8_prefill", 4096, rows=_edge_sample("tp8_prefill", 4096))


def test_tp8_share_prefill_prepacked_bit_exact(dev, tp8):
    """One GPU's share (intermediate 256) at 4096 tokens. Its down projection
    is two 128-input chunks per column tile, so each work-group of the down
    launch takes several consecutive tiles (four here: ~420 real blocks of 14
    tiles) with one copy stream across them. The layer on prepacked weights
    takes the same path and must equal the checkpoint-layout layer bit for
    bit (the sampled rows above are checked against the oracle)."""
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    bank, shared = tp8
    w = mi.workload("tp8_prefill", 4096)
    x = mi.activations(w.seed_x + w.T, w.T, w.geo.hidden)
    ids, wts = mi.make_routing(w)
    print("[case] tp8_prefill T=4096 prepacked vs checkpoint layout", flush=True)
    ref = run_layer(dev, x, ids, wts, bank, shared)
    pk = moe.prepack(bank["packed_w13"], bank["scales_w13"], bank["packed_w2"], bank["scales_w2"])
    d = lambda a: mi.to_device(a, dev)
    got = moe.forward_prepacked(d(x), d(ids), d(wts), pk, d(shared))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
