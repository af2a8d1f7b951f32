"""Router step (top-k + softmax over the selected) on the GPU against the
oracle: expert ids bit-exact, weights within a few fp32 rounding steps; and
the combined router + layer entry point against the two separate calls."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.helpers import check

pytestmark = pytest.mark.gpu

# fp32 softmax (expf, one IEEE division) against the fp64 oracle
WEIGHT_RTOL = 2e-6


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _route(dev, scores, k, **kw):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    ids, w = moe.route(torch.from_numpy(scores).to(dev), k, **kw)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _compare(dev, scores, k, label):
    print(f"[case] route {label} T={scores.shape[0]} S={scores.shape[1]} k={k}", flush=True)
    ids, w = _route(dev, scores, k)
    rid, rw = oracle.route(scores, k)
    assert np.array_equal(ids, rid), label
    np.testing.assert_allclose(w, rw, rtol=WEIGHT_RTOL, atol=1e-30, err_msg=label)


@pytest.mark.parametrize("T", [1, 5, 64, 4096])
def test_route_random_scores(dev, T):
    _compare(dev, mi.router_scores(300 + T, T, 384), 8, "N(0,1)")


@pytest.mark.parametrize("S,k", [(7, 1), (7, 7), (100, 6), (64, 16), (1000, 16), (1024, 8),
                                 (384, 1)])
def test_route_widths(dev, S, k):
    _compare(dev, mi.router_scores(400 + S + k, 37, S), k, "widths")


def test_route_ties_signed_zeros_and_infinities(dev):
    rng = np.random.default_rng(5)
    s = rng.integers(-3, 4, size=(50, 384)).astype(np.float32)  # many equal scores
    s[rng.random(s.shape) < 0.2] = np.float32(-0.0)
    s[rng.random(s.shape) < 0.2] = np.float32(0.0)
    s[rng.random(s.shape) < 0.05] = -np.inf
    s[3] = 0.0
    s[4] = -np.inf
    s[4, 17] = 1.0
    _compare(dev, s, 8, "ties")


def test_route_is_deterministic(dev):
    s = mi.router_scores(9, 512, 384)
    a = _route(dev, s, 8)
    b = _route(dev, s, 8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name,T", [("decode", 8), ("decode", 64), ("ep", 2048)])
def test_forward_scores_matches_route_then_forward(dev, name, T):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    w = mi.workload(name, T)
    g = w.geo
    E = w.n_local
    experts = list(range(w.expert_base, w.expert_base + E))
    # a small bank slice keeps the test quick; the router scores all 384 experts
    bank = mi.device_bank(w.seed_bank, 512, 256, experts, dev)
    shared = mi.to_device(mi.shared_weights(w.seed_bank, 512, 256), dev)
    x = mi.to_device(mi.activations(w.seed_x + T, T, 512), dev)
    scores = mi.router_scores(500 + T, T, g.n_experts)
    sc = torch.from_numpy(scores).to(dev)
    print(f"[case] forward_scores {name} T={T}", flush=True)
    out, ids, wts = moe.forward_scores(x, sc, g.top_k, bank["packed_w13"], bank["scales_w13"],
                                       bank["packed_w2"], bank["scales_w2"], shared,
                                       expert_base=w.expert_base)
    ids2, wts2 = moe.route(sc, g.top_k, num_experts=E, expert_base=w.expert_base)
    out2 = moe.forward(x, ids2, wts2, bank["packed_w13"], bank["scales_w13"],
                       bank["packed_w2"], bank["scales_w2"], shared, expert_base=w.expert_base)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(wts, wts2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    rid, rw = oracle.route(scores, g.top_k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    # the layer on the oracle's routing (fp32 weights, as the layer receives them)
    hb = mi.weight_bank(w.seed_bank, 512, 256, experts)
    ref = oracle.forward(mi.activations(w.seed_x + T, T, 512), rid, rw.astype(np.float32),
                         hb.packed_w13, hb.scales_w13, hb.packed_w2, hb.scales_w2,
                         mi.shared_weights(w.seed_bank, 512, 256), w.expert_base)
    check(mi.bf16_tensor_to_f64(out), ref, f"forward_scores {name} T={T}")
