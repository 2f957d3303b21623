"""Plant plausible mistakes in a copy of the oracle (CPU only) and check the pins catch each.

Every mutation below is a one-token slip of the kind a hand-written oracle
could contain; each must make at least one pin in test_oracle_pins fail.
"""
import os

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pkv_oracle.c")

MUTATIONS = [
    ("scale dropped", "z[j] = scale * dot;", "z[j] = dot;", ["test_weights_are_softmax_and_sum_to_one"]),
    ("causal range off by one", "j <= p; ++j", "j < p; ++j", ["test_prefill_causal_range_is_exact"]),
    ("GQA head mapping", "hq / G,", "hq % Hkv,", ["test_constant_values_and_gqa_head_mapping"]),
    ("block-table index", "bt_row[j / B]", "bt_row[j % B]", ["test_scatter_then_gather_round_trip"]),
    ("slot offset", "int off = (int)(s % B);", "int off = (int)((s + 1) % B);",
     ["test_scatter_then_gather_round_trip"]),
    ("K piece order", "* B + off) * X + e % X", "* B + off) * X + (e + 1) % X", ["test_slot_worked_example"]),
    ("V layout transposed", "* d + e) * B + off", "* B + off) * d + e", ["test_slot_worked_example"]),
    ("normaliser sign", "Z += z[j];", "Z -= z[j];", ["test_weights_are_softmax_and_sum_to_one"]),
    ("normalisation dropped", "double w = z[j] / Z;", "double w = z[j];",
     ["test_zero_query_gives_mean_of_values"]),
    ("decode position", "rp[s] = context_lens[s] - 1;", "rp[s] = context_lens[s] - 2;",
     ["test_decode_matches_brute_force_on_unpaged_kv"]),
    ("prefill position", "rp[query_start_loc[s] + i] = hist + i;",
     "rp[query_start_loc[s] + i] = hist + i / 2;", ["test_prefill_causal_range_is_exact"]),
    ("f16 exponent bias", "expo - 25", "expo - 24", ["test_f16_decoder_known_encodings"]),
    ("fp8 exponent bias", "expo - 10", "expo - 9", ["test_fp8_decoder_known_encodings"]),
    ("fp8 ties away from zero", "(int)rint(ldexp(a, 3 - E))", "(int)floor(ldexp(a, 3 - E) + 0.5)",
     ["test_fp8_encoder_is_nearest_even_by_brute_force"]),
    ("fp8 scale not applied on write", "fp8_from_float(x / scale)", "fp8_from_float(x)",
     ["test_fp8_scatter_stores_codes_of_fp32_quotients"]),
    ("fp8 key scale not applied on read", "Kc[dst] = ks *", "Kc[dst] =",
     ["test_fp8_decode_matches_brute_force_on_dequantised_kv"]),
    ("query dot uses wrong operand", "dot += q[e] * k[e];", "dot += q[e] * q[e];",
     ["test_weights_are_softmax_and_sum_to_one"]),
    ("window start off by one", "p - window + 1 > 0 ? p - window + 1 : 0",
     "p - window > 0 ? p - window : 0", ["test_sliding_window_range_is_exact"]),
    ("window ignored", "int lo = window > 0 &&", "int lo = 0 &&",
     ["test_sliding_window_range_is_exact"]),
]


def _run(name, golden_dir):
    fn = getattr(pins, name)
    import inspect
    params = inspect.signature(fn).parameters
    if "dtype" in params:      # parametrised pins: try every case, any failure counts
        cases = {"test_scatter_then_gather_round_trip": [dict(dtype=d) for d in (0, 1, 2)],
                 "test_decode_matches_brute_force_on_unpaged_kv": [dict(dtype=0, G=1), dict(dtype=2, G=4)]}[name]
        for kw in cases:
            fn(**kw)
    elif "golden_dir" in params:
        fn(golden_dir)
    else:
        fn()


@pytest.mark.parametrize("label,old,new,tests", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, golden_dir, label, old, new, tests):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(out_path=str(tmp_path / "libmutant.so"), src=str(mutated))
    oracle.use_library(lib)
    try:
        caught = False
        for t in tests:
            try:
                _run(t, golden_dir)
            except (AssertionError, oracle.OracleError):
                caught = True
        assert caught, f"no pin caught mutation '{label}'"
    finally:
        oracle.use_library(None)
