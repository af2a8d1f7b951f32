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


def block_edge_tokens(ids, expert_base, n_local, block_m):
    """Tokens holding the first and the last row of every local expert's last
    bucket block (rows of an expert are its valid pairs p = t*k + j in
    ascending p, in blocks of block_m): together they reach every expert's
    last block, including every overflow block past a full one."""
    flat = np.asarray(ids).ravel()
    k = np.asarray(ids).shape[1]
    toks = set()
    for e in range(n_local):
        ps = np.nonzero(flat == expert_base + e)[0]
        if ps.size == 0:
            continue
        toks.add(int(ps[-1] // k))
        toks.add(int(ps[(ps.size - 1) // block_m * block_m] // k))
    return sorted(toks)


def sample_tokens(T, must, n_min, seed):
    """`must` plus seeded random tokens up to n_min (sorted, distinct)."""
    rest = np.setdiff1d(np.arange(T), np.asarray(must, np.int64))
    extra = max(0, n_min - len(must))
    pick = np.random.default_rng(seed).choice(rest, min(extra, rest.size), replace=False)
    return np.sort(np.concatenate([np.asarray(must, np.int64), pick]))
