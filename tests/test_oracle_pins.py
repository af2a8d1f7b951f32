"""Pins of the CPU oracle to things other than itself.

Each test compares the oracle with a value printed on the pages, a closed form,
a library routine (torch fp64 SwiGLU MLP), an independent dense formulation or
an invariant of the layer -- chosen so that a dropped term, a wrong sign, a
wrong index or a transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _tiny_inputs(seed=0, T=6, H=64, I=32, E=4, k=2, shared=True, base=0, n_global=None):
    n_global = n_global or E
    bank = mi.weight_bank(seed, H, I, list(range(base, base + E)))
    x = mi.activations(seed, T, H)
    ids, w = mi.routing_uniform(seed, T, n_global, k)
    sw = mi.shared_weights(seed, H, I) if shared else None
    return dict(x=x, topk_ids=ids, topk_weights=w, packed_w13=bank.packed_w13,
                scales_w13=bank.scales_w13, packed_w2=bank.packed_w2,
                scales_w2=bank.scales_w2, shared_w=sw, expert_base=base)


def _bf16_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# int4 storage format
# --------------------------------------------------------------------------
def test_unpack_hand_examples(oracle_lib):
    g = _load("unpack_examples.json")
    for ex in g["examples"]:
        word = np.array([int(ex["word_hex"], 16)], np.uint32).view(np.int32)
        assert oracle.unpack_int4(word).tolist() == ex["codes"], ex
        assert [oracle.int4_code_c(word, c) for c in range(8)] == ex["codes"], ex
        assert oracle.pack_int4(np.array(ex["codes"])).view(np.uint32)[0] == int(ex["word_hex"], 16)


def test_unpack_exhaustive_fields():
    # every value in every field position, others held at code 0 (field 8)
    for pos in range(8):
        for q in range(-8, 8):
            codes = np.zeros(8, np.int64)
            codes[pos] = q
            w = oracle.pack_int4(codes)
            expect = 0x88888888 & ~(0xF << (4 * pos)) | ((q + 8) << (4 * pos))
            assert int(w.view(np.uint32)[0]) == expect
            assert oracle.unpack_int4(w).tolist() == codes.tolist()
            assert oracle.int4_code_c(w, pos) == q


def test_pack_unpack_roundtrip_random_words():
    rng = np.random.default_rng(3)
    words = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint32).view(np.int32)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(words)), words)
    # C and numpy unpackers agree on a random row
    row = words[:64]
    q = oracle.unpack_int4(row)
    assert [oracle.int4_code_c(row, c) for c in range(512)] == q.tolist()


def test_random_words_give_uniform_codes():
    # uniform random words -> each code in [-8, 7] equally likely
    rng = np.random.default_rng(4)
    words = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint32).view(np.int32)
    counts = np.bincount(oracle.unpack_int4(words).astype(np.int64).ravel() + 8, minlength=16)
    assert counts.size == 16
    exp = counts.sum() / 16
    assert np.all(np.abs(counts - exp) < 6 * math.sqrt(exp))


# --------------------------------------------------------------------------
# geometry printed on the pages
# --------------------------------------------------------------------------
def test_geometry_matches_int32_count():
    g = _load("geometry.json")
    moe_layers = g["layers"] - g["first_k_dense_replace"]
    # three matrices per expert (gate, up, down) of hidden x intermediate
    int4_weights = moe_layers * g["routed_experts"] * 3 * g["hidden"] * g["moe_intermediate_size"]
    assert int4_weights == g["params_i32"] == 1_014_686_023_680
    assert (mi.KIMI.hidden, mi.KIMI.inter, mi.KIMI.n_experts, mi.KIMI.top_k) == (
        g["hidden"], g["moe_intermediate_size"], g["routed_experts"], g["experts_per_token"])
    assert g["hidden"] % g["group_size"] == 0 and g["moe_intermediate_size"] % g["group_size"] == 0


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def _silu(z):
    return z / (1.0 + math.exp(-z))


def test_silu_identity():
    for z in [-30.0, -3.5, -1.0, -1e-3, 0.0, 0.25, 2.0, 17.0]:
        assert abs((oracle.silu_c(z) - oracle.silu_c(-z)) - z) <= 1e-15 * max(1.0, abs(z))
        assert abs(oracle.silu_c(z) - _silu(z)) <= 1e-15 * max(1.0, abs(z))


def test_constant_weights_closed_form(oracle_lib):
    # all gate/up codes c1 with scale s1, all down codes c2 with scale s2:
    # g = u = c1*s1*sum(x) =: A,  h = silu(A)*A,  y_n = c2*s2*I*h,  out = w*y
    H, I, E, T = 64, 32, 3, 5
    c1, c2 = 3, -5
    s1_bits = mi.f32_to_bf16_bits(np.array([0.0078125], np.float32))[0]  # exact 2^-7
    s2_bits = mi.f32_to_bf16_bits(np.array([0.01171875], np.float32))[0]  # 3 * 2^-8
    pw13 = np.full((E, 2 * I, H // 8), mi.const_code_word(c1 + 8), np.int32)
    pw2 = np.full((E, H, I // 8), mi.const_code_word(c2 + 8), np.int32)
    s13 = np.full((E, 2 * I, H // 32), s1_bits, np.uint16)
    s2 = np.full((E, H, I // 32), s2_bits, np.uint16)
    x = mi.activations(9, T, H)
    ids = np.array([[1], [0], [2], [1], [-1]], np.int32)
    w = np.array([[0.75], [1.0], [-0.5], [2.0], [1.0]], np.float32)
    out = oracle.forward(x, ids, w, pw13, s13, pw2, s2)
    X = _bf16_f64(x)
    for t in range(T):
        if ids[t, 0] < 0:
            assert np.all(out[t] == 0.0)
            continue
        A = c1 * 0.0078125 * math.fsum(X[t])
        y = c2 * 0.01171875 * I * _silu(A) * A
        np.testing.assert_allclose(out[t], float(w[t, 0]) * y, rtol=1e-12, atol=1e-12)


def test_per_group_scales_closed_form(oracle_lib):
    # all codes +1, scales s13[n][g] distinct per (row, group):
    # a_n = sum_g s13[n][g] * sum_{c in group g} x_c ; gate row n, up row I+n
    H, I, E, T = 96, 64, 1, 3
    rng = np.random.default_rng(11)
    pw13 = np.full((E, 2 * I, H // 8), mi.const_code_word(9), np.int32)
    pw2 = np.full((E, H, I // 8), mi.const_code_word(9), np.int32)
    s13 = mi.f32_to_bf16_bits(rng.uniform(0.01, 0.05, (E, 2 * I, H // 32)).astype(np.float32))
    s2 = mi.f32_to_bf16_bits(rng.uniform(0.01, 0.05, (E, H, I // 32)).astype(np.float32))
    x = mi.activations(12, T, H)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out = oracle.forward(x, ids, w, pw13, s13, pw2, s2)
    X = _bf16_f64(x)
    S13 = _bf16_f64(s13[0])
    S2 = _bf16_f64(s2[0])
    for t in range(T):
        gs = [math.fsum(X[t, 32 * g:32 * g + 32]) for g in range(H // 32)]
        a = [math.fsum(S13[n, g] * gs[g] for g in range(H // 32)) for n in range(2 * I)]
        h = [_silu(a[i]) * a[I + i] for i in range(I)]
        hg = [math.fsum(h[32 * g:32 * g + 32]) for g in range(I // 32)]
        y = [math.fsum(S2[n, g] * hg[g] for g in range(I // 32)) for n in range(H)]
        np.testing.assert_allclose(out[t], y, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# library routine: one-hot routing == textbook SwiGLU MLP (torch, fp64)
# --------------------------------------------------------------------------
def _torch_mlp(X, W13, W2, I):
    A = torch.from_numpy(X) @ torch.from_numpy(W13).T
    h = torch.nn.functional.silu(A[:, :I]) * A[:, I:]
    return (h @ torch.from_numpy(W2).T).numpy()


def test_one_hot_routing_is_textbook_swiglu(oracle_lib):
    d = _tiny_inputs(seed=21, T=5, H=128, I=64, E=3, k=1, shared=False)
    for e in range(3):
        ids = np.full((5, 1), e, np.int32)
        w = np.ones((5, 1), np.float32)
        out = oracle.forward(d["x"], ids, w, d["packed_w13"], d["scales_w13"],
                             d["packed_w2"], d["scales_w2"])
        W13 = oracle.dequant_int4(d["packed_w13"][e], d["scales_w13"][e])
        W2 = oracle.dequant_int4(d["packed_w2"][e], d["scales_w2"][e])
        ref = _torch_mlp(_bf16_f64(d["x"]), W13, W2, 64)
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_zero_routing_weights_give_shared_expert_only(oracle_lib):
    d = _tiny_inputs(seed=22, T=4, H=128, I=64, E=3, k=2, shared=True)
    w0 = np.zeros_like(d["topk_weights"])
    out = oracle.forward(d["x"], d["topk_ids"], w0, d["packed_w13"], d["scales_w13"],
                         d["packed_w2"], d["scales_w2"], d["shared_w"])
    sw = _bf16_f64(d["shared_w"])
    H, I = 128, 64
    ref = _torch_mlp(_bf16_f64(d["x"]), sw[:2 * I * H].reshape(2 * I, H),
                     sw[2 * I * H:].reshape(H, I), I)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


# --------------------------------------------------------------------------
# brute force: independent dense formulation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", [
    dict(seed=31, T=7, H=64, I=32, E=4, k=2, shared=True),
    dict(seed=32, T=5, H=96, I=64, E=5, k=3, shared=False),
    dict(seed=33, T=6, H=64, I=32, E=3, k=4, shared=True, base=2, n_global=8),
])
def test_dense_formulation_agrees(oracle_lib, case):
    d = _tiny_inputs(**case)
    args = (d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"], d["scales_w13"],
            d["packed_w2"], d["scales_w2"], d["shared_w"], d["expert_base"])
    out = oracle.forward(*args)
    ref = oracle.dense_moe(*args)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_dense_formulation_duplicates_and_invalid_ids(oracle_lib):
    d = _tiny_inputs(seed=34, T=4, H=64, I=32, E=3, k=3, shared=True)
    ids = np.array([[0, 0, 2], [-1, 5, 1], [2, 2, 2], [3, -7, 0]], np.int32)
    args = (d["x"], ids, d["topk_weights"], d["packed_w13"], d["scales_w13"],
            d["packed_w2"], d["scales_w2"], d["shared_w"], 0)
    np.testing.assert_allclose(oracle.forward(*args), oracle.dense_moe(*args), rtol=1e-12,
                               atol=1e-9)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_sum_of_single_slot_runs(oracle_lib):
    d = _tiny_inputs(seed=41, T=5, H=64, I=32, E=4, k=3, shared=True)
    full = oracle.forward(d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"],
                          d["scales_w13"], d["packed_w2"], d["scales_w2"], d["shared_w"])
    shared_only = oracle.forward(d["x"], d["topk_ids"], np.zeros_like(d["topk_weights"]),
                                 d["packed_w13"], d["scales_w13"], d["packed_w2"],
                                 d["scales_w2"], d["shared_w"])
    acc = shared_only.copy()
    for j in range(3):
        w = np.zeros_like(d["topk_weights"])
        w[:, j] = d["topk_weights"][:, j]
        acc += oracle.forward(d["x"], d["topk_ids"], w, d["packed_w13"], d["scales_w13"],
                              d["packed_w2"], d["scales_w2"], None)
    np.testing.assert_allclose(full, acc, rtol=1e-12, atol=1e-12 * np.abs(full).max())


def test_token_permutation(oracle_lib):
    d = _tiny_inputs(seed=42, T=6, H=64, I=32, E=4, k=2, shared=True)
    perm = np.random.default_rng(0).permutation(6)
    a = oracle.forward(d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"],
                       d["scales_w13"], d["packed_w2"], d["scales_w2"], d["shared_w"])
    b = oracle.forward(d["x"][perm], d["topk_ids"][perm], d["topk_weights"][perm],
                       d["packed_w13"], d["scales_w13"], d["packed_w2"], d["scales_w2"],
                       d["shared_w"])
    np.testing.assert_array_equal(a[perm], b)


def test_slot_permutation_and_expert_relabelling(oracle_lib):
    d = _tiny_inputs(seed=43, T=5, H=64, I=32, E=4, k=3, shared=False)
    a = oracle.forward(d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"],
                       d["scales_w13"], d["packed_w2"], d["scales_w2"])
    sp = [2, 0, 1]
    b = oracle.forward(d["x"], d["topk_ids"][:, sp], d["topk_weights"][:, sp],
                       d["packed_w13"], d["scales_w13"], d["packed_w2"], d["scales_w2"])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13 * np.abs(a).max())
    # relabel experts: new expert pi[e] holds old expert e
    pi = np.array([3, 1, 0, 2])
    inv = np.argsort(pi)
    c = oracle.forward(d["x"], pi[d["topk_ids"]].astype(np.int32), d["topk_weights"],
                       d["packed_w13"][inv], d["scales_w13"][inv], d["packed_w2"][inv],
                       d["scales_w2"][inv])
    np.testing.assert_array_equal(a, c)


def test_doubling_down_scales_doubles_routed_part(oracle_lib):
    d = _tiny_inputs(seed=44, T=4, H=64, I=32, E=3, k=2, shared=True)
    base = oracle.forward(d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"],
                          d["scales_w13"], d["packed_w2"], d["scales_w2"], d["shared_w"])
    shared_only = oracle.forward(d["x"], d["topk_ids"], np.zeros_like(d["topk_weights"]),
                                 d["packed_w13"], d["scales_w13"], d["packed_w2"],
                                 d["scales_w2"], d["shared_w"])
    s2x = (d["scales_w2"].astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1
    assert np.array_equal(_bf16_f64(s2x), 2 * _bf16_f64(d["scales_w2"]))
    doubled = oracle.forward(d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"],
                             d["scales_w13"], d["packed_w2"], s2x, d["shared_w"])
    np.testing.assert_allclose(doubled - shared_only, 2 * (base - shared_only), rtol=1e-12,
                               atol=1e-12 * np.abs(base).max())


@pytest.mark.parametrize("n", [2, 4])
def test_tensor_parallel_shards_sum_to_full(oracle_lib, n):
    """SwiGLU acts column by column on the intermediate dimension and the
    down projection is linear in it, so splitting the intermediate columns of
    every expert and of the shared expert n ways (gate and up rows, W2 input
    columns and their scale groups) and adding the n partial layers gives the
    whole layer: the one-GPU share of a tensor-parallel deployment."""
    H, I = 64, 128
    d = _tiny_inputs(seed=46, T=5, H=H, I=I, E=4, k=3, shared=True)
    bank = mi.Bank(d["packed_w13"], d["scales_w13"], d["packed_w2"], d["scales_w2"])
    full = oracle.forward(d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"],
                          d["scales_w13"], d["packed_w2"], d["scales_w2"], d["shared_w"])
    acc = np.zeros_like(full)
    for r in range(n):
        b, sh = mi.tp_shard(bank, d["shared_w"], H, I, r, n)
        assert b.packed_w13.shape == (4, 2 * I // n, H // 8)
        assert b.scales_w2.shape == (4, H, I // n // 32)
        part = oracle.forward(d["x"], d["topk_ids"], d["topk_weights"], b.packed_w13,
                              b.scales_w13, b.packed_w2, b.scales_w2, sh)
        assert np.abs(part).max() > 0
        acc += part
    np.testing.assert_allclose(acc, full, rtol=1e-11, atol=1e-12 * np.abs(full).max())


def test_token_subset_matches_full(oracle_lib):
    d = _tiny_inputs(seed=45, T=9, H=64, I=32, E=4, k=2, shared=True)
    args = (d["x"], d["topk_ids"], d["topk_weights"], d["packed_w13"], d["scales_w13"],
            d["packed_w2"], d["scales_w2"], d["shared_w"])
    full = oracle.forward(*args, threads=3)
    rows = np.array([8, 0, 4, 4])
    np.testing.assert_array_equal(oracle.forward(*args, rows=rows, threads=2), full[rows])


# --------------------------------------------------------------------------
# align (bucketing)
# --------------------------------------------------------------------------
def test_align_hand_examples():
    for ex in _load("align_examples.json")["examples"]:
        s, b, n = oracle.align(np.array(ex["topk_ids"], np.int32).reshape(len(ex["topk_ids"]), -1),
                               ex["num_experts"], ex["expert_base"], ex["block_m"])
        assert s.tolist() == ex["sorted_ids"], ex
        assert b.tolist() == ex["block_expert"], ex
        assert n == ex["n_padded"]


def _align_brute(ids, E, base, bm):
    # pure-Python definition: walk the experts in order, then the pairs in order
    flat = [int(v) for v in np.asarray(ids).ravel()]
    P = len(flat)
    out, blocks = [], []
    for e in range(E):
        members = [p for p in range(P) if flat[p] - base == e and base <= flat[p] < base + E]
        padded = members + [P] * ((-len(members)) % bm)
        out += padded
        blocks += [e] * (len(padded) // bm)
    return out, blocks


@pytest.mark.parametrize("seed", range(6))
def test_align_brute_force_and_invariants(seed):
    rng = np.random.default_rng(seed)
    T, k = int(rng.integers(0, 40)), int(rng.integers(1, 9))
    E, base, bm = int(rng.integers(1, 20)), int(rng.integers(0, 4)), int(rng.choice([1, 2, 4, 16]))
    ids = rng.integers(-2, base + E + 3, size=(T, k)).astype(np.int32)
    s, b, n = oracle.align(ids, E, base, bm)
    bs, bb = _align_brute(ids, E, base, bm)
    assert s.tolist() == bs and b.tolist() == bb and n == len(bs)
    P = T * k
    flat = ids.ravel()
    valid = (flat >= base) & (flat < base + E)
    real = s[s < P]
    assert sorted(real.tolist()) == np.nonzero(valid)[0].tolist()  # each valid pair once
    assert n % bm == 0 and b.size == n // bm
    for blk in range(b.size):
        rows = s[blk * bm:(blk + 1) * bm]
        assert all(flat[p] - base == b[blk] for p in rows if p < P)
        assert np.all(np.diff(rows[rows < P]) > 0)  # ascending within a block
    assert (s == P).sum() == n - valid.sum()


def test_workload_routing_shapes():
    ids, w = mi.routing_uniform(1, 64, 384, 8)
    assert ids.shape == (64, 8) and w.shape == (64, 8)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
    zi, zw = mi.routing_zipf(1, 512, 384, 8)
    assert all(len(set(r)) == 8 for r in zi.tolist())
    counts = np.bincount(zi.ravel(), minlength=384)
    assert counts.max() > 300 and (counts == 0).sum() > 10  # heavy skew, idle experts


# --------------------------------------------------------------------------
# router step (top-k + softmax over the selected)
# --------------------------------------------------------------------------
def _route_case(scores, k):
    return oracle.route(np.array([scores], np.float32), k)


def test_route_hand_examples():
    e = math.e
    ids, w = _route_case([1.0, 3.0, 2.0, 0.5], 2)  # top two: 3 and 2, one apart
    assert ids.tolist() == [[1, 2]]
    np.testing.assert_allclose(w[0], [e / (e + 1), 1 / (e + 1)], rtol=1e-15)
    # ties go to the lower expert id, and the selection keeps descending order
    ids, w = _route_case([2.0, 5.0, 2.0, 5.0, 2.0], 3)
    assert ids.tolist() == [[1, 3, 0]]
    d = 2 + math.exp(-3)
    np.testing.assert_allclose(w[0], [1 / d, 1 / d, math.exp(-3) / d], rtol=1e-15)
    # -0.0 and +0.0 are equal scores
    ids, w = _route_case([-0.0, 0.0, -1.0], 2)
    assert ids.tolist() == [[0, 1]] and w.tolist() == [[0.5, 0.5]]
    ids, w = _route_case([-0.0, -1.0, 0.0], 2)
    assert ids.tolist() == [[0, 2]]
    # equal scores: the first k experts, equal weights
    ids, w = _route_case([0.25] * 6, 4)
    assert ids.tolist() == [[0, 1, 2, 3]] and w.tolist() == [[0.25] * 4]
    # large magnitudes: only differences matter
    ids, w = _route_case([-100.0, -101.0, -99.0], 2)
    assert ids.tolist() == [[2, 0]]
    np.testing.assert_allclose(w[0], [e / (e + 1), 1 / (e + 1)], rtol=1e-13)
    # k = E: every expert, sorted
    ids, w = _route_case([0.0, 2.0, 1.0], 3)
    assert ids.tolist() == [[1, 2, 0]]
    np.testing.assert_allclose(w[0], np.array([e * e, e, 1.0]) / (e * e + e + 1), rtol=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_route_brute_force(seed):
    """Against an exhaustive search: the selected set is the k-subset with the
    largest score sum, the lexicographically smallest id tuple among equal
    sums, listed by descending score then id."""
    import itertools

    rng = np.random.default_rng(seed)
    E, k, T = int(rng.integers(1, 8)), 0, 5
    k = int(rng.integers(1, E + 1))
    scores = rng.integers(-2, 3, size=(T, E)).astype(np.float32)  # many ties
    scores[:, :: 3] *= np.float32(0.5)
    ids, w = oracle.route(scores, k)
    for t in range(T):
        s = scores[t].astype(np.float64)
        best = max(itertools.combinations(range(E), k),
                   key=lambda c: (sum(s[list(c)]), tuple(-i for i in c)))
        want = sorted(best, key=lambda e: (-s[e], e))
        assert ids[t].tolist() == want, (t, scores[t], ids[t], want)
        z = np.exp(s[want] - s[want].max())
        np.testing.assert_allclose(w[t], z / z.sum(), rtol=1e-14)


def test_route_equals_renormalised_full_softmax():
    from scipy.special import softmax

    rng = np.random.default_rng(3)
    scores = rng.standard_normal((7, 384)).astype(np.float32)
    ids, w = oracle.route(scores, 8)
    p = softmax(scores.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12)
    # every unselected score is at most the smallest selected one
    for t in range(7):
        rest = np.setdiff1d(np.arange(384), ids[t])
        assert scores[t, rest].max() <= scores[t, ids[t]].min()
        assert np.all(np.diff(scores[t, ids[t]]) <= 0)


def test_route_shift_and_permutation():
    rng = np.random.default_rng(4)
    scores = rng.integers(-50, 50, size=(6, 40)).astype(np.float32)  # exact under shifts
    ids, w = oracle.route(scores, 6)
    ids2, w2 = oracle.route(scores + np.float32(1000), 6)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-14)
    d = rng.permutation(40 * 6).reshape(6, 40).astype(np.float32)  # distinct scores
    perm = rng.permutation(40)  # new column perm[e] holds old expert e
    moved = np.empty_like(d)
    moved[:, perm] = d
    a, wa = oracle.route(d, 5)
    b, wb = oracle.route(moved, 5)
    assert np.array_equal(perm[a], b) and np.array_equal(wa, wb)
