"""Shared helpers of the GPU tests: run the library and the oracle on the same
seeded inputs."""
import numpy as np

import moe_inputs as mi
import oracle
from oracle import tolerance


def run_layer(dev, x, ids, w, bank_dev, shared=None, expert_base=0, out=None):
    import w4a16_int4_grouped_moe_amd as moe

    d = lambda a: mi.to_device(a, dev)
    return moe.forward(d(x), d(ids), d(w), bank_dev["packed_w13"], bank_dev["scales_w13"],
                       bank_dev["packed_w2"], bank_dev["scales_w2"],
                       None if shared is None else d(shared), out=out,
                       expert_base=expert_base)


def oracle_rows(seed, geo, x, ids, w, shared, expert_base, n_local, rows):
    """fp64 reference for tokens `rows`, using a bank of only the experts those
    tokens reach (same values: each expert has its own random stream)."""
    rows = np.asarray(rows, np.int64)
    used, remap = mi.compact_routing(ids, rows, expert_base, n_local)
    if used:
        bank = mi.weight_bank(seed, geo.hidden, geo.inter, used)
    else:
        bank = mi.weight_bank(seed, geo.hidden, geo.inter, [0])
    return oracle.forward(x[rows], remap, w[rows], bank.packed_w13, bank.scales_w13,
                          bank.packed_w2, bank.scales_w2, shared, 0)


def check(got_f64, ref, label=""):
    res = tolerance.check(got_f64, ref)
    print(f"[parity] {label} {res}", flush=True)
    assert res["ok"], f"{label}: {res}"
    return res
