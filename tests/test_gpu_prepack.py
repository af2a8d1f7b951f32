"""The prepacked-weight variant (moe_w4a16_prepack, moe_w4a16_forward_prepacked).

The repack is a pure reordering, checked byte for byte against a host re-layout
written here from the layout's definition (per expert and matrix, tiles of 512
weight rows; W13 rows in the order gate 0-15, gate 16-31, up 0-15, up 16-31 of
each 64-row slice; codes [chunk of 128 inputs][row][4 groups x 16 B], scales
[period of 16 groups][row][16 x 2 B], zero-padded). The layer on prepacked
weights does the same arithmetic on the same values as the layer on the
original weights, so the two outputs must be equal bit for bit; that is
checked on every kernel path the prepacked form reaches: the small-batch
kernels (the narrow down kernel for inter <= 512, streamed down up to 2048, the
general down kernel beyond), and prefill blocks with 2, 4 and 6 active
sub-tiles; one case is also compared with the oracle directly."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.helpers import check

pytestmark = pytest.mark.gpu

ROWS, CHUNK = 512, 128


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def tile_order(Nw, I, w13):
    """Destination slot (tile * 512 + row in tile) of each weight row n."""
    dest = np.empty(Nw, np.int64)
    for t in range(Nw // ROWS):
        for R in range(ROWS):
            if w13:
                w, s, r = R // 64, (R % 64) // 16, R % 16
                c = t * (ROWS // 2) + w * 32 + 16 * (s % 2) + r
                n = c if s < 2 else I + c
            else:
                n = t * ROWS + R
            dest[n] = t * ROWS + R
    assert np.array_equal(np.sort(dest), np.arange(Nw))
    return dest


def host_prepack(packed, scales, I, w13):
    E, Nw, K8 = packed.shape
    K = 8 * K8
    nch, ng = K // CHUNK, K // 32
    nper = (ng + 15) // 16
    dest = tile_order(Nw, I, w13)
    codes = np.empty((E, Nw, nch, 4, 4), np.int32)
    codes[:, dest] = packed.reshape(E, Nw, nch, 4, 4)
    codes = codes.reshape(E, Nw // ROWS, ROWS, nch, 4, 4).transpose(0, 1, 3, 2, 4, 5)
    sc = np.zeros((E, Nw, nper * 16), np.uint16)
    sc[:, :, :ng] = scales
    s2 = np.empty((E, Nw, nper, 16), np.uint16)
    s2[:, dest] = sc.reshape(E, Nw, nper, 16)
    s2 = s2.reshape(E, Nw // ROWS, ROWS, nper, 16).transpose(0, 1, 3, 2, 4)
    return (np.ascontiguousarray(codes).view(np.uint8).ravel(),
            np.ascontiguousarray(s2).view(np.uint8).ravel())


def device_bank(bank, dev):
    return {k: mi.to_device(v, dev) for k, v in bank.__dict__.items()}


def test_prepack_bytes_match_the_layout(dev):
    import w4a16_int4_grouped_moe_amd as moe

    H, I, E = 512, 768, 3  # W2 rows: 24 scale groups, the second period padded
    bank = mi.weight_bank(71, H, I, list(range(E)))
    pk = moe.prepack(*[device_bank(bank, dev)[k] for k in
                       ("packed_w13", "scales_w13", "packed_w2", "scales_w2")])
    got = pk.buffer.cpu().numpy()
    rnd = lambda v: (v + 255) // 256 * 256
    c13, s13 = host_prepack(bank.packed_w13, bank.scales_w13, I, True)
    c2, s2 = host_prepack(bank.packed_w2, bank.scales_w2, I, False)
    o = 0
    for name, want in (("w13 codes", c13), ("w13 scales", s13), ("w2 codes", c2),
                       ("w2 scales", s2)):
        assert np.array_equal(got[o:o + want.size], want), name
        o = rnd(o + want.size)
    assert o == got.size == moe.prepack_size(H, I, E)


CASES = [
    # T, H, I, E, k, base, shared, expected block_m, path
    (3, 512, 768, 8, 2, 0, True, 4),       # small-batch; streamed down, K tail, padded scales
    (5, 1024, 2304, 6, 2, 1, False, 4),    # small-batch; general down kernel (K > 2048)
    (40, 512, 768, 16, 2, 0, True, 96),    # prefill blocks, ~5 rows per expert (2 sub-tiles)
    (120, 512, 1024, 8, 4, 0, True, 96),   # ~50 rows per expert (4 sub-tiles)
    (300, 1024, 1024, 4, 2, 2, False, 96),  # ~100 rows per expert (6 + 2 sub-tiles), base
    (6, 1024, 256, 8, 4, 0, True, 4),      # narrow down kernel, K = 256 (two tiles of rows)
    (9, 512, 512, 8, 3, 1, False, 4),      # narrow down kernel, K = 512, expert base
    (200, 1024, 256, 8, 4, 0, True, 96),   # prefill blocks with K = 256 for down
]


def _compare(dev, T, H, I, E, k, base, shared, bm, seed, with_oracle=False):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    assert moe.forward_block_m(moe.problem(T, H, I, E, k, base)) == bm
    bank = mi.weight_bank(seed, H, I, list(range(base, base + E)))
    bd = device_bank(bank, dev)
    x = mi.activations(seed + 1, T, H)
    ids, w = mi.routing_uniform(seed + 2, T, base + E + 2, min(k, base + E + 2))
    sw = mi.shared_weights(seed + 3, H, I) if shared else None
    d = lambda a: None if a is None else mi.to_device(a, dev)
    print(f"[prepack] T={T} H={H} I={I} E={E} k={k} base={base} shared={shared} bm={bm}",
          flush=True)
    ref = moe.forward(d(x), d(ids), d(w), bd["packed_w13"], bd["scales_w13"], bd["packed_w2"],
                      bd["scales_w2"], d(sw), expert_base=base)
    pk = moe.prepack(bd["packed_w13"], bd["scales_w13"], bd["packed_w2"], bd["scales_w2"])
    got = moe.forward_prepacked(d(x), d(ids), d(w), pk, d(sw), expert_base=base)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    if with_oracle:
        want = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                              bank.scales_w2, sw, base)
        check(mi.bf16_tensor_to_f64(got), want, f"prepacked T={T} H={H} I={I}")


@pytest.mark.parametrize("T,H,I,E,k,base,shared,bm", CASES)
def test_prepacked_equals_forward(dev, T, H, I, E, k, base, shared, bm):
    _compare(dev, T, H, I, E, k, base, shared, bm, seed=500 + T + H + I, with_oracle=(T == 3))


@pytest.mark.parametrize("T", [1, 8, 64])
def test_prepacked_equals_forward_layer_widths(dev, T):
    """The full layer's widths (7168 / 2048, shared expert) with 24 local
    experts: T = 1 and 8 in the small-batch kernels (T = 8: several slice
    groups per streamed down work-group), T = 64 in prefill blocks."""
    bm = 4 if T * 8 <= 4 * 24 else 96
    _compare(dev, T, 7168, 2048, 24, 8, 0, True, bm, seed=900)


def test_prepacked_zero_tokens(dev):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    bank = mi.weight_bank(3, 512, 768, [0, 1])
    bd = device_bank(bank, dev)
    pk = moe.prepack(bd["packed_w13"], bd["scales_w13"], bd["packed_w2"], bd["scales_w2"])
    x = torch.empty((0, 512), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((0, 2), dtype=torch.int32, device=dev)
    w = torch.empty((0, 2), dtype=torch.float32, device=dev)
    out = moe.forward_prepacked(x, ids, w, pk)
    assert out.shape == (0, 512)


@pytest.mark.parametrize("T,H,I,E,k", [(6, 1024, 768, 8, 2), (150, 1024, 768, 8, 4)])
def test_prepacked_graph_capture_replay(dev, T, H, I, E, k):
    """A captured prepacked forward (small-batch kernels; prefill blocks with
    the shared expert in the library GEMM, whose handle the eager call creates
    first) replays to the eager result, with eager work between replays."""
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    bank = mi.weight_bank(31 + T, H, I, list(range(E)))
    bd = device_bank(bank, dev)
    pk = moe.prepack(bd["packed_w13"], bd["scales_w13"], bd["packed_w2"], bd["scales_w2"])
    d = lambda a: mi.to_device(a, dev)
    ids, w = mi.routing_uniform(32 + T, T, E, k)
    xs, ids_d, w_d = d(mi.activations(33 + T, T, H)), d(ids), d(w)
    sw = d(mi.shared_weights(34 + T, H, I))
    p = moe.problem(T, H, I, E, k)
    ws = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    eager = moe.forward_prepacked(xs, ids_d, w_d, pk, sw, workspace=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward_prepacked(xs, ids_d, w_d, pk, sw, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward_prepacked(xs, ids_d, w_d, pk, sw, out=out, workspace=ws)
    for i in range(4):
        out.zero_()
        ws.fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        moe.forward_prepacked(xs[:5], ids_d[:5], w_d[:5], pk, sw)
        torch.cuda.synchronize()
