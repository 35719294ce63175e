"""The patch-compile checker (tests/compile_cases.py) on the CPU: the oracle's own factors,
rounded to the element type, pass it; factors with a planted mistake do not."""
import numpy as np
import pytest

import oracle
import compile_cases as cc


def _factors(case, e):
    U, V = e["U"], e["V"]
    m = case.chunks[0].m
    if U.shape[1] < m:          # rank below m: complete V with orthonormal directions
        W = V.shape[0]
        extra = np.random.default_rng(0).standard_normal((W, m - V.shape[1]))
        V, _ = np.linalg.qr(np.concatenate([V, extra], axis=1))
        U = e["delta"] @ V
    if case.dtype == "bf16":
        U = cc.decode(oracle.to_bf16(U), "bf16")
        V = cc.decode(oracle.to_bf16(V), "bf16")
    return U, V


@pytest.mark.parametrize("case", cc.small_cases() + cc.degenerate_cases()[1:],
                         ids=lambda c: c.name)
def test_oracle_factors_pass_and_planted_mistakes_fail(case):
    inputs = cc.build(case)
    rng = np.random.default_rng(1)
    for ch in range(2):
        H, W, _ = case.geometry(ch)
        e = cc.expected(case, inputs, 0, ch, 0, H - 1)
        U, V = _factors(case, e)
        assert cc.check_head(U, V, e, case.dtype).ok
        if not e["full_rank"]:
            continue
        # a dropped direction
        assert not cc.check_head(U[:, :-1], V[:, :-1], e, case.dtype).ok
        # a sign flip of one basis vector with U left alone
        V2 = V.copy()
        V2[:, 0] *= -1
        assert not cc.check_head(U, V2, e, case.dtype).ok
        # a basis rotated slightly out of the subspace (there is no outside when m == width)
        if V.shape[1] < W:
            Q, _ = np.linalg.qr(V + 0.02 * rng.standard_normal(V.shape))
            assert not cc.check_head(e["delta"] @ Q, Q, e, case.dtype).ok
        # an unrotated deficit (the relocation left out of Delta)
        if ch == 0 and case.chunks[0].delta != 0:
            canon = inputs[0]["canonical"][ch][0, :, (H - 1) * W:H * W]
            cond = inputs[0]["conditioned"][ch][0, :, (H - 1) * W:H * W]
            wrong = oracle.values(cond) - oracle.values(canon)
            u, s, vt = np.linalg.svd(wrong, full_matrices=False)
            m = case.chunks[0].m
            assert not cc.check_head(u[:, :m] * s[:m], vt[:m].T, e, case.dtype).ok


def test_rotation_invariance_of_the_check():
    """Any orthonormal basis of the same subspace passes (U V^T and V V^T are basis-free)."""
    case = cc.small_cases()[1]
    inputs = cc.build(case)
    e = cc.expected(case, inputs, 0, 0, 0, 0)
    m = case.chunks[0].m
    R, _ = np.linalg.qr(np.random.default_rng(3).standard_normal((m, m)))
    assert cc.check_head(e["U"] @ R, e["V"] @ R, e, case.dtype).ok


def test_orbit_checker_accepts_the_oracle_and_rejects_one_ordering():
    """The orbit tolerance passes the oracle's own orbit factors (rounded to bf16) and fails
    the plain compile of a single ordering (which is not the orbit patch)."""
    case = cc.Case("orbit_check", "gqa", "bf16", 1, 1, 64, 64, oracle.HALF_SPLIT, 1e4,
                   [cc.ChunkSpec(120, 8, 0)], seed=5)
    inp = cc.build_orbit(case, [0, 700, 1400, -300], own_level=0.3)
    e = cc.expected_orbit(case, inp, 0, 0, 0)
    U = cc.decode(oracle.to_bf16(e["U"]), "bf16")
    V = cc.decode(oracle.to_bf16(e["V"]), "bf16")
    assert cc.check_head(U, V, e, "bf16").ok
    one = oracle.compile_patch(inp["conditioned"][1][0][0], inp["canonical"][0][0], m=8,
                               rotate=True, delta=700, theta=1e4)
    assert not cc.check_head(one["U"], one["V"], e, "bf16").ok
