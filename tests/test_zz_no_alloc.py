"""moe_w4a16_forward_noalloc (the entry point for callers that cannot
allocate): through the C ABI it gives the same output, bit for bit, as
moe_w4a16_forward with a caller workspace, on two calls in a row (the second
smaller, on the other kernel path, so the device array keeps the first call's
contents), and matches the fp64 oracle."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.helpers import check

pytestmark = pytest.mark.gpu

H, I, E, K = 1024, 512, 8, 2


@pytest.fixture(scope="module")
def setup():
    import torch

    dev = torch.device("cuda:0")
    bank = mi.weight_bank(77, H, I, list(range(E)))
    bank_dev = {k: mi.to_device(v, dev) for k, v in bank.__dict__.items()}
    sw = mi.shared_weights(77, H, I)
    return dev, bank, bank_dev, sw


@pytest.mark.parametrize("shared", [True, False])
def test_noalloc_equals_forward(setup, shared):
    import torch

    import w4a16_int4_grouped_moe_amd as moe

    dev, bank, bank_dev, sw = setup
    d = lambda a: mi.to_device(a, dev)
    wts = (bank_dev["packed_w13"], bank_dev["scales_w13"], bank_dev["packed_w2"],
           bank_dev["scales_w2"])
    swd = d(sw) if shared else None
    # 40 tokens (96-row blocks), then 6 tokens (4-row buckets)
    for T, bm in [(40, 96), (6, 4)]:
        assert moe.forward_block_m(moe.problem(T, H, I, E, K)) == bm
        x = mi.activations(78 + T, T, H)
        ids, w = mi.routing_uniform(79 + T, T, E, K)
        print(f"[case] noalloc T={T} bm={bm} shared={shared}", flush=True)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
        got = moe.forward_noalloc(d(x), d(ids), d(w), *wts, swd, out=out)
        ref_gpu = moe.forward(d(x), d(ids), d(w), *wts, swd)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), ref_gpu.view(torch.int16)), T
        ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                             bank.scales_w2, sw if shared else None)
        check(mi.bf16_tensor_to_f64(got), ref, f"noalloc T={T} shared={shared}")


def test_noalloc_limit(setup):
    import w4a16_int4_grouped_moe_amd as moe

    assert moe.noalloc_workspace_limit() == 64 << 20
    # the Kimi-K2.6 decode batches fit; 193 tokens (96-row blocks) do not
    for T, fits in [(1, True), (64, True), (192, True), (193, False)]:
        p = moe.problem(T, 7168, 2048, 384, 8)
        assert (moe.workspace_size(p) <= moe.noalloc_workspace_limit()) is fits, T
