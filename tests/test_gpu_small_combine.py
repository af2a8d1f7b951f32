"""The small-batch path (4-row buckets) on routing edge cases, against the
fp64 oracle: k = 1 and k = 16 slots, duplicated expert ids in a token, tokens
with no local slot (zero rows, or the shared expert alone), and a workspace
left by a larger call. The output buffer starts as NaN so that every element
must be written."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.helpers import check, run_layer

pytestmark = pytest.mark.gpu

H, I = 512, 384


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _routing(seed, T, E, k, base, dup, orphans):
    ids, w = mi.routing_uniform(seed, T, base + E + 3, k)
    if dup and k > 1:
        ids[1::3, 1] = ids[1::3, 0]          # one expert twice in a token
    if orphans:
        ids[0, :] = -1                        # no slot at all
        ids[2, :] = base + E + 1              # only non-local experts
        if base > 0:
            ids[4 % T, :] = base - 1
    return ids, w


@pytest.mark.parametrize("T,E,k,base,shared,dup,orphans", [
    (6, 64, 16, 0, True, False, False),
    (5, 40, 1, 0, False, False, False),
    (7, 40, 1, 0, True, False, True),
    (9, 24, 6, 8, False, True, True),
    (9, 24, 6, 8, True, True, True),
    (3, 300, 8, 0, True, True, False),
])
def test_small_path_combine(dev, T, E, k, base, shared, dup, orphans):
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    assert moe.forward_block_m(moe.problem(T, H, I, E, k, base)) == 4
    bank = mi.weight_bank(21, H, I, list(range(base, base + E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    x = mi.activations(22 + T, T, H)
    ids, w = _routing(23 + T, T, E, k, base, dup, orphans)
    sw = mi.shared_weights(21, H, I) if shared else None
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
    print(f"[case] small combine T={T} E={E} k={k} base={base} shared={shared}", flush=True)
    run_layer(dev, x, ids, w, bank_dev, sw, expert_base=base, out=out)
    torch.cuda.synchronize()
    ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                         bank.scales_w2, sw, base)
    got = mi.bf16_tensor_to_f64(out)
    assert np.isfinite(got).all()
    if orphans and not shared:
        assert (got[0] == 0).all() and (got[2] == 0).all()
    check(got, ref, f"small combine T={T} k={k}")


def test_small_path_reused_workspace(dev):
    """A call after a larger one on the same workspace: the buckets and partial
    results left behind must not leak into the next result."""
    import torch
    import w4a16_int4_grouped_moe_amd as moe

    E, k = 32, 4
    bank = mi.weight_bank(31, H, I, list(range(E)))
    bank_dev = {kk: mi.to_device(v, dev) for kk, v in bank.__dict__.items()}
    sw = mi.shared_weights(31, H, I)
    ws_bytes = moe.workspace_size(moe.problem(24, H, I, E, k, 0))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    d = lambda a: mi.to_device(a, dev)
    for T in (24, 5, 24, 1):
        x = mi.activations(32 + T, T, H)
        ids, w = mi.routing_uniform(33 + T, T, E, k)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
        print(f"[case] reused workspace T={T}", flush=True)
        moe.forward(d(x), d(ids), d(w), bank_dev["packed_w13"], bank_dev["scales_w13"],
                    bank_dev["packed_w2"], bank_dev["scales_w2"], d(sw), out=out,
                    workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.forward(x, ids, w, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                             bank.scales_w2, sw)
        check(mi.bf16_tensor_to_f64(out), ref, f"reused workspace T={T}")
