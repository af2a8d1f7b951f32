"""Bucketing on the GPU equals the oracle's stable sort, bit for bit, in both
forms: one work-group, and many work-groups with per-chunk counts."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def gpu_align(dev, ids, E, base, bm, many_groups=False):
    import torch

    import w4a16_int4_grouped_moe_amd as moe

    s, b, n = moe.align(mi.to_device(ids, dev), E, bm, expert_base=base,
                        many_groups=many_groups)
    torch.cuda.synchronize()
    n = int(n.cpu()[0])
    return s.cpu().numpy()[:n], b.cpu().numpy()[:n // bm], n


def compare(dev, ids, E, base, bm, label):
    print(f"[align] {label} T={ids.shape[0]} k={ids.shape[1]} E={E} base={base} bm={bm}",
          flush=True)
    rs, rb, rn = oracle.align(ids, E, base, bm)
    for many in (False, True):
        s, b, n = gpu_align(dev, ids, E, base, bm, many)
        assert n == rn, (label, many, n, rn)
        assert np.array_equal(s, rs), (label, many)
        assert np.array_equal(b, rb), (label, many)


WORKLOADS = [("tiny", None), ("decode", 1), ("decode", 8), ("decode", 32), ("decode", 64),
             ("prefill", 4096), ("skew", 512), ("ep", 2048)]


@pytest.mark.parametrize("name,T", WORKLOADS)
@pytest.mark.parametrize("bm", [1, 4, 16, 64, 96, 128])
def test_align_workloads(dev, name, T, bm):
    w = mi.workload(name, T)
    ids, _ = mi.make_routing(w)
    compare(dev, ids, w.n_local, w.expert_base, bm, f"{name}")


def test_align_edge_cases(dev):
    rng = np.random.default_rng(5)
    # invalid, duplicate and out-of-range ids
    ids = np.array([[2, 0], [0, 1], [2, -1], [5, 2]], np.int32)
    compare(dev, ids, 3, 0, 2, "hand")
    compare(dev, ids, 3, 1, 2, "hand-base")
    ids = rng.integers(-3, 12, size=(777, 6)).astype(np.int32)
    for bm in (1, 3, 16, 64):
        compare(dev, ids, 9, 2, bm, "random-with-invalid")
    # all pairs to one expert; a single token; no valid pair at all
    compare(dev, np.zeros((1000, 8), np.int32), 4, 0, 16, "one-expert")
    compare(dev, np.array([[7, 3, 1, 0, 2, 5, 6, 4]], np.int32), 384, 0, 16, "T=1")
    compare(dev, np.full((33, 2), -1, np.int32), 5, 0, 16, "none-valid")
    # largest expert count and a long pair list
    ids = rng.integers(0, 512, size=(8192, 8)).astype(np.int32)
    compare(dev, ids, 512, 0, 64, "E=512,P=65536")
    ids = rng.integers(0, 2, size=(3000, 16)).astype(np.int32)
    compare(dev, ids, 1, 1, 16, "E=1")


def test_align_deterministic(dev):
    w = mi.workload("skew", 512)
    ids, _ = mi.make_routing(w)
    for many in (False, True):
        first = gpu_align(dev, ids, 384, 0, 16, many)
        for _ in range(10):
            again = gpu_align(dev, ids, 384, 0, 16, many)
            assert again[2] == first[2]
            assert np.array_equal(again[0], first[0]) and np.array_equal(again[1], first[1])
