"""Properties of the HIP path that hold at any size: determinism, zero and
invalid routing, exact power-of-two scaling, token permutation, empty input,
and replay of a captured HIP graph."""
import numpy as np
import pytest

import moe_inputs as mi
from tests.helpers import run_layer

pytestmark = pytest.mark.gpu

E, K = 16, 4
# (tokens, hidden, inter): 96-row blocks on widths that are not whole tiles
# (masked), 4-row blocks (32 pairs: bucketed inside the GEMM launches, down
# and combine in one; 16 tokens: the bucketing kernel and the combine kernel),
# and 96-row blocks on whole tiles
SHAPES = {"masked": (96, 640, 384), "small-batch": (8, 512, 256),
          "small-batch-bucketed": (16, 512, 256), "prefill": (300, 512, 256)}


@pytest.fixture(scope="module", params=sorted(SHAPES))
def setup(request):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    T, H, I = SHAPES[request.param]
    want = {"masked": 96, "small-batch": 4, "small-batch-bucketed": 4,
            "prefill": 96}[request.param]
    assert moe.forward_block_m(moe.problem(T, H, I, E, K)) == want
    dev = torch.device("cuda:0")
    bank = mi.weight_bank(3, H, I, list(range(E)))
    bank_dev = {k: mi.to_device(v, dev) for k, v in bank.__dict__.items()}
    x = mi.activations(4, T, H)
    ids, w = mi.routing_uniform(5, T, E, K)
    sw = mi.shared_weights(3, H, I)
    return dev, bank, bank_dev, x, ids, w, sw, H, I


def bits(t):
    import torch

    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().copy()


def test_deterministic(setup):
    dev, bank, bank_dev, x, ids, w, sw, H, I = setup
    a = bits(run_layer(dev, x, ids, w, bank_dev, sw))
    for _ in range(10):
        assert np.array_equal(bits(run_layer(dev, x, ids, w, bank_dev, sw)), a)


def test_zero_weights_and_invalid_ids_give_shared_only(setup):
    dev, bank, bank_dev, x, ids, w, sw, H, I = setup
    a = bits(run_layer(dev, x, ids, np.zeros_like(w), bank_dev, sw))
    b = bits(run_layer(dev, x, np.full_like(ids, -1), w, bank_dev, sw))
    c = bits(run_layer(dev, x, ids + E, w, bank_dev, sw))  # all ids beyond the local range
    assert np.array_equal(a, b) and np.array_equal(a, c)
    # and without a shared expert the output is exactly zero
    z = bits(run_layer(dev, x, np.full_like(ids, -1), w, bank_dev, None))
    assert not z.any()


def test_doubling_down_scales_doubles_output_exactly(setup):
    import torch

    dev, bank, bank_dev, x, ids, w, sw, H, I = setup
    base = run_layer(dev, x, ids, w, bank_dev, None)
    doubled_dev = dict(bank_dev)
    doubled_dev["scales_w2"] = bank_dev["scales_w2"] * 2
    dbl = run_layer(dev, x, ids, w, doubled_dev, None)
    torch.cuda.synchronize()
    assert torch.equal(dbl.float(), 2 * base.float())


def test_token_permutation(setup):
    import torch

    dev, bank, bank_dev, x, ids, w, sw, H, I = setup
    perm = np.random.default_rng(1).permutation(x.shape[0])
    a = run_layer(dev, x, ids, w, bank_dev, sw).float()
    b = run_layer(dev, x[perm], ids[perm], w[perm], bank_dev, sw).float()
    torch.cuda.synchronize()
    assert torch.equal(a[torch.from_numpy(perm).to(dev)], b)


def test_empty_batch(setup):
    import torch

    import w4a16_int4_grouped_moe_amd as moe

    dev, bank, bank_dev, x, ids, w, sw, H, I = setup
    out = run_layer(dev, x[:0], ids[:0], w[:0], bank_dev, sw)
    assert out.shape == (0, H)
    p = moe.problem(0, H, I, E, K)
    assert moe.workspace_size(p) == 0


def test_graph_capture_replay(setup):
    import torch

    import w4a16_int4_grouped_moe_amd as moe

    dev, bank, bank_dev, x, ids, w, sw, H, I = setup
    d = lambda a: mi.to_device(a, dev)
    xs, ids_d, w_d, sw_d = d(x), d(ids), d(w), d(sw)
    T = x.shape[0]
    p = moe.problem(T, H, I, E, K)
    ws = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    args = (xs, ids_d, w_d, bank_dev["packed_w13"], bank_dev["scales_w13"],
            bank_dev["packed_w2"], bank_dev["scales_w2"], sw_d)
    # captured before any call of this shape: the library keeps no state and
    # allocates nothing, so no warm-up call is needed
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(*args, out=out, workspace=ws)
    eager = moe.forward(*args).clone()
    for i in range(4):
        out.zero_()
        ws.fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        # unrelated eager work between replays
        moe.forward(xs[:7], ids_d[:7], w_d[:7], *args[3:])
        torch.cuda.synchronize()


def test_timed_entry_point(setup):
    """moe_w4a16_forward_timed: the same output as the plain call, and its seven
    events recorded in stream order."""
    import ctypes
    import torch

    dev, bank, bank_dev, x, ids, w, sw, H, I = setup
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    ev = []
    for _ in range(7):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        ev.append(e.value)
    import w4a16_int4_grouped_moe_amd as moe

    d = lambda a: mi.to_device(a, dev)
    plain = bits(run_layer(dev, x, ids, w, bank_dev, sw))
    out = moe.forward(d(x), d(ids), d(w), bank_dev["packed_w13"], bank_dev["scales_w13"],
                      bank_dev["packed_w2"], bank_dev["scales_w2"], d(sw), stage_events=ev)
    assert np.array_equal(bits(out), plain)
    ms = ctypes.c_float()
    for a, b in [(0, 1), (1, 5), (5, 2), (2, 6), (6, 3), (3, 4)]:
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[a], ev[b]) == 0
        assert ms.value >= 0.0
