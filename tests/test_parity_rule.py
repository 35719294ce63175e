"""CPU: the comparison rules the GPU parity tests enforce (tests/parity.py), checked on outputs
built here, so that a rule that is too loose or too strict shows without a GPU.

bf16 rule: |g - o| <= 2 ulp_bf16(max(|o|, 2^-14 S)), o the fp32 oracle rounded to bf16, S the
sum of absolute terms; copies are compared bit for bit.
"""
import numpy as np
import pytest

import oracle
from parity import compare_head, ulp_bf16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16_bits(x) -> np.ndarray:
    return oracle.to_bf16(np.asarray(x, np.float64))


def bits_to_f64(b) -> np.ndarray:
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def check(z, S, g_values, m=16):
    exp = {"copy": False, "z": np.asarray(z, np.float64), "S": np.asarray(S, np.float64)}
    return compare_head(exp, bf16_bits(g_values), "bf16", m, "rule test")


def test_two_ulps_pass_three_fail():
    z = np.array([1.0, -3.0, 1e-3, 123.0])
    S = np.abs(z)
    u = ulp_bf16(z)
    assert check(z, S, z).float_fail == 0
    assert check(z, S, z + 2 * u).float_fail == 0
    assert check(z, S, z - 2 * u).float_fail == 0
    r = check(z, S, z + 3 * u)
    assert r.float_fail == 4 and r.unfloored_fail == 4 and r.floor_active == 0
    assert r.max_ulp == pytest.approx(3.0)


def test_wrong_sign_and_dropped_term_fail():
    z = np.array([0.75, -2.5])
    S = np.array([1.5, 4.0])
    assert check(z, S, -z).float_fail == 2
    # a dropped patch term of size 0.25 S
    assert check(z, S, z - 0.25 * S).float_fail == 2


def test_floor_acts_only_where_terms_cancel():
    # |o| = 2^-20 while S = 4: the floor 2^-14 S = 2^-12 sets the tolerance 2 ulp(2^-12) = 2^-18
    z = np.array([2.0 ** -20])
    S = np.array([4.0])
    r = check(z, S, z + 2.0 ** -19)
    assert r.float_fail == 0 and r.floor_active == 1 and r.unfloored_fail == 1
    assert check(z, S, z + 2.0 ** -17).float_fail == 1
    # without cancellation the floor is inactive: |o| = 1 >> 2^-14 S
    r = check(np.array([1.0]), np.array([1.5]), np.array([1.0]))
    assert r.floor_active == 0


def test_zero_result_with_zero_terms_must_be_zero():
    r = check(np.zeros(3), np.zeros(3), np.zeros(3))
    assert r.float_fail == 0
    assert check(np.zeros(1), np.zeros(1), np.array([2.0 ** -100])).float_fail == 1


def test_copy_rule_is_bitwise():
    src = np.array([0x8000, 0x0000, 0x7FC1, 0xFF81, 0x0001], np.uint16)   # -0, +0, NaNs, subnormal
    exp = {"copy": True, "bits": src}
    assert compare_head(exp, src.copy(), "bf16", 0, "copy").copy_mismatches == 0
    flipped = src.copy()
    flipped[0] = 0x0000                     # -0.0 -> +0.0, as a float add of zero would do
    assert compare_head(exp, flipped, "bf16", 0, "copy").copy_mismatches == 1


def _round_f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("m", [16, 32, 64])
def test_fp32_chain_of_the_kernel_meets_the_rule(m):
    """A model of the GPU's arithmetic (fp32 cos/sin, the rotation as one product and one
    fused multiply-add, then m exact bf16 products summed in fp32 in order) passes the bf16
    rule on rotated, patched elements: the rule is achievable by fp32 arithmetic."""
    rng = np.random.Generator(np.random.PCG64(m))
    n, width = 512, 128
    x = bf16_bits(rng.standard_normal((n, width)))
    U = bf16_bits(0.05 * rng.standard_normal((n, m)))
    V = bf16_bits(0.05 * rng.standard_normal((width, m)))
    delta, theta = 12345, 1e4
    z, S = oracle.segment(x, rotate=True, delta=delta, theta=theta, U=U, V=V)
    c, s = oracle.phase(delta, theta, width)
    c32, s32 = _round_f32(c), _round_f32(s)
    xv, Uv, Vv = bits_to_f64(x), bits_to_f64(U), bits_to_f64(V)
    half = width // 2
    a, b = xv[:, :half], xv[:, half:]
    ra = _round_f32(a * c32 - _round_f32(b * s32))     # fma(x, c, -(y s)): one rounding
    rb = _round_f32(b * c32 + _round_f32(a * s32))
    acc = np.concatenate([ra, rb], axis=1)
    for r in range(m):                                  # exact products, fp32 sums
        acc = _round_f32(acc + np.outer(Uv[:, r], Vv[:, r]))
    g = bf16_bits(acc)
    exp = {"copy": False, "z": z, "S": S}
    rep = compare_head(exp, g, "bf16", m, f"fp32 chain model m={m}")
    assert rep.float_fail == 0, rep.details
    assert rep.chain_fail == 0
