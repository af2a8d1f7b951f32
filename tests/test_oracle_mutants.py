"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/moe_oracle.c (on the CPU),
builds it, points the oracle module at the copy and runs the pin tests: at
least one of them must fail.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import oracle.oracle as oo
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "moe_oracle.c")

MUTANTS = {
    "gate_up_swapped": ("h[i] = silu(a[i]) * a[I + i];", "h[i] = silu(a[I + i]) * a[i];", 2),
    "gate_up_interleaved": ("h[i] = silu(a[i]) * a[I + i];",
                            "h[i] = silu(a[2 * i]) * a[2 * i + 1];", 2),
    "twos_complement_codes": ("return field - 8;", "return (field ^ 8) - 8;", 1),
    "high_nibble_first": ("(word >> (4 * (c % 8)))", "(word >> (4 * (7 - c % 8)))", 1),
    "scale_group_reversed": ("scales[n * (C / GROUP) + c / GROUP]",
                             "scales[n * (C / GROUP) + (C / GROUP - 1 - c / GROUP)]", 1),
    "shared_dropped": ("for (int64_t n = 0; n < H; ++n) o[n] += y[n];", "", 1),
    "routing_weight_ignored": ("o[n] += w * y[n];", "o[n] += y[n];", 1),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));", 1),
    "expert_base_ignored": ("int64_t e = id - jb->base;", "int64_t e = id;", 1),
    "down_uses_gate_scales": ("jb->s2 + e * H * (I / GROUP)", "jb->s13 + e * H * (I / GROUP)", 1),
    "bf16_truncated_to_8_bits": ("uint32_t u = (uint32_t)bits << 16;",
                                 "uint32_t u = ((uint32_t)bits & 0xFF00u) << 16;", 1),
}

PIN_TESTS = [
    lambda: pins.test_unpack_hand_examples(None),
    pins.test_unpack_exhaustive_fields,
    pins.test_pack_unpack_roundtrip_random_words,
    pins.test_silu_identity,
    lambda: pins.test_constant_weights_closed_form(None),
    lambda: pins.test_per_group_scales_closed_form(None),
    lambda: pins.test_one_hot_routing_is_textbook_swiglu(None),
    lambda: pins.test_zero_routing_weights_give_shared_expert_only(None),
    lambda: pins.test_dense_formulation_agrees(
        None, dict(seed=31, T=7, H=64, I=32, E=4, k=2, shared=True)),
    lambda: pins.test_dense_formulation_agrees(
        None, dict(seed=33, T=6, H=64, I=32, E=3, k=4, shared=True, base=2, n_global=8)),
    lambda: pins.test_doubling_down_scales_doubles_routed_part(None),
    lambda: pins.test_tensor_parallel_shards_sum_to_full(None, 2),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new, count = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == count, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", "-o",
                           str(so), str(mutated), "-lm"])
    lib = ctypes.CDLL(str(so))
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_forward.argtypes = [P] * 9 + [I64] * 6 + [P, I64, I64]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_int4_code.argtypes = [P, I64]
    lib.oracle_int4_code.restype = ctypes.c_int
    monkeypatch.setattr(oo, "_lib", lib)
    failed = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught the planted mistake {name}"
    assert oracle.forward is oo.forward
