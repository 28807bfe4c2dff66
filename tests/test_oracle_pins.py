"""The oracle against its pins, and the pins against planted mistakes.

Every mutant below is a plausible slip in the oracle (wrong zero point, nibble
order, group index, dropped scale, swapped gate/up, eps placement, ...). It is
planted in a copy of the oracle source on the CPU, compiled with gcc, and must
fail at least one pin.
"""
import os

import pytest

import oracle
import oracle_pins as P

SRC = open(oracle.SRC).read()


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


# (name, text in q4_oracle.c, replacement)
MUTANTS = [
    ("zero_point_8", "(double)(q - 7) * s", "(double)(q - 8) * s"),
    ("nibble_order_reversed", "(w >> (4 * (k % 8)))", "(w >> (4 * (7 - k % 8)))"),
    ("pack_order_reversed", "<< (4 * i)", "<< (4 * (7 - i))"),
    ("group_index_off_by_one", "S[r * (k_total / 32) + k / 32]",
     "S[r * (k_total / 32) + (k / 32 + 1) % (k_total / 32)]"),
    ("group_of_16", "S[r * (k_total / 32) + k / 32]", "S[r * (k_total / 32) + (k / 16) % (k_total / 32)]"),
    ("scale_dropped", "return (double)(q - 7) * s;", "return (double)(q - 7);"),
    ("h2d_subnormal_scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("d2h_truncates", "double m = rint(ldexp(a, 10 - E));", "double m = floor(ldexp(a, 10 - E));"),
    ("gate_up_swapped", "double g = q4o_h2d(gu[b * 2 * f + i]);", "double g = q4o_h2d(gu[b * 2 * f + f + i]);"),
    ("silu_sign", "exp(-z)", "exp(z)"),
    ("eps_outside_sqrt", "sqrt(ss / (double)d + eps)", "(sqrt(ss / (double)d) + eps)"),
    ("mean_over_d_minus_1", "ss / (double)d + eps", "ss / (double)(d - 1) + eps"),
    ("residual_add_dropped", "q4o_h2d(a[b * d + i]) + q4o_h2d(rr[i])", "q4o_h2d(rr[i])"),
    ("gamma_dropped", "* inv * q4o_h2d(gamma[i])", "* inv"),
    ("moe_weight_ignored", "y[i * n + r] += w * v[r];", "y[i * n + r] += v[r];"),
    ("moe_slot_activation_ignored", "x + i * ldx + s * x_slot_stride", "x + i * ldx"),
    ("moe_gu_not_rounded", "vh[r] = q4o_d2h(v[r]);", "vh[r] = q4o_d2h(v[r] * 1.0009765625);"),
    ("stack_wrong_v_slice", "qkv + v_off, d, dv", "qkv, d, dv"),
    ("stack_gamma_next_is_current", "gamma_in + (L + 1) * d", "gamma_in + L * d"),
    ("layer_second_norm_uses_first_residual", "q4o_add_rmsnorm(dn, r1, gamma_next", "q4o_add_rmsnorm(dn, r_in, gamma_next"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_some_pin(name, old, new):
    assert SRC.count(old) == 1, "mutation anchor must match exactly once: %r" % old
    bad = oracle.load_variant(SRC.replace(old, new), name)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(bad)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
