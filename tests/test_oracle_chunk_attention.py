"""Pins of the relocation-free chunk attention oracle (oracle/attention.py chunk_attention).

The oracle builds each chunk's keys and values with the reuse operator's own definition
(oracle.segment) and attends over them. These tests recompute the same attention in the
form a relocation-free reader uses, written out independently with explicit 2x2 rotations:
    <q, R(delta) k + Uk Vk^T row> = <R(-delta) q, k> + Uk row . (Vk^T q)
    sum_t p_t (v_t + Uv row Vv^T)  = sum_t p_t v_t + (sum_t p_t Uv row) Vv^T
(R orthogonal per pair, R(delta)^T = R(-delta)), and check the state-merge identity across
chunks, the rank-0 / shift-0 reduction to plain attention, and that a query turned the wrong
way fails."""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as att


def _bf16(x):
    return oracle.to_bf16(np.asarray(x, np.float64))


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _chunk(rng, T, D, m_k, m_v, delta):
    c = {"K": _bf16(rng.standard_normal((T, D))), "V": _bf16(rng.standard_normal((T, D))),
         "delta": delta}
    if m_k:
        c["Uk"] = _bf16(0.1 * rng.standard_normal((T, m_k)))
        c["Vk"] = _bf16(0.1 * rng.standard_normal((D, m_k)))
    if m_v:
        c["Uv"] = _bf16(0.1 * rng.standard_normal((T, m_v)))
        c["Vv"] = _bf16(0.1 * rng.standard_normal((D, m_v)))
    return c


def _pairs(D, R, layout):
    if layout == oracle.HALF_SPLIT:
        return [(i, i + R // 2) for i in range(R // 2)]
    return [(2 * i, 2 * i + 1) for i in range(R // 2)]


def _turn(q, angle_of_pair, pairs):
    """Each pair (a, b) of every row turned by its angle: (x c - y s, y c + x s)."""
    out = q.copy()
    for i, (a, b) in enumerate(pairs):
        ang = angle_of_pair[i]
        rot = np.array([[math.cos(ang), -math.sin(ang)], [math.sin(ang), math.cos(ang)]])
        xy = q[:, [a, b]] @ rot.T
        out[:, a], out[:, b] = xy[:, 0], xy[:, 1]
    return out


def _counter_rotated(q, chunks, scale, layout, theta, R=None):
    D = q.shape[1]
    R = D if R is None else R
    pairs = _pairs(D, R, layout)
    freq = np.array([theta ** (-2.0 * i / R) for i in range(R // 2)])
    s_all, v_all = [], []
    for c in chunks:
        K, V = _f64(c["K"]), _f64(c["V"])
        qr = _turn(q, -c["delta"] * freq, pairs)            # R(-delta) q
        s = qr @ K.T
        if "Uk" in c:
            s = s + (q @ _f64(c["Vk"])) @ _f64(c["Uk"]).T   # Uk row . (Vk^T q)
        s_all.append(scale * s)
        v_all.append((V, c))
    s = np.concatenate(s_all, axis=1)
    mx = s.max(axis=1, keepdims=True)
    w = np.exp(s - mx)
    z = w.sum(axis=1, keepdims=True)
    p = w / z
    o = np.zeros_like(q)
    t0 = 0
    for V, c in v_all:
        pc = p[:, t0:t0 + V.shape[0]]
        o += pc @ V
        if "Uv" in c:
            o += (pc @ _f64(c["Uv"])) @ _f64(c["Vv"]).T     # (sum_t p_t Uv row) Vv^T
        t0 += V.shape[0]
    return o, (mx + np.log(z))[:, 0]


@pytest.mark.parametrize("layout", [oracle.HALF_SPLIT, oracle.INTERLEAVED])
@pytest.mark.parametrize("ranks", [(0, 0), (8, 4), (16, 16)])
def test_matches_the_counter_rotated_form(layout, ranks):
    rng = np.random.default_rng(3 + ranks[0] + layout)
    D, theta = 32, 1e4
    chunks = [_chunk(rng, 9, D, *ranks, 1000), _chunk(rng, 5, D, *ranks, -37),
              _chunk(rng, 12, D, *ranks, 65536)]
    q = rng.standard_normal((3, D))
    o, lse = att.chunk_attention(q, chunks, 0.2, layout=layout, theta=theta)
    o2, lse2 = _counter_rotated(q, chunks, 0.2, layout, theta)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_partial_rotary_turns_only_the_first_pairs():
    rng = np.random.default_rng(11)
    D, R = 32, 16
    chunks = [_chunk(rng, 7, D, 4, 4, 321), _chunk(rng, 6, D, 4, 4, -5)]
    q = rng.standard_normal((2, D))
    o, lse = att.chunk_attention(q, chunks, 0.3, layout=oracle.HALF_SPLIT, theta=1e4, rot_dim=R)
    o2, lse2 = _counter_rotated(q, chunks, 0.3, oracle.HALF_SPLIT, 1e4, R=R)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_rank_zero_at_shift_zero_is_plain_attention():
    rng = np.random.default_rng(5)
    chunks = [_chunk(rng, 10, 16, 0, 0, 0), _chunk(rng, 4, 16, 0, 0, 0)]
    q = rng.standard_normal((2, 16))
    o, lse = att.chunk_attention(q, chunks, 0.5, layout=oracle.HALF_SPLIT, theta=1e4)
    K = np.concatenate([_f64(c["K"]) for c in chunks])
    V = np.concatenate([_f64(c["V"]) for c in chunks])
    o2, lse2 = att.decode_attention(q, K, V, 0.5)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


def test_chunks_merge_by_the_state_merge():
    rng = np.random.default_rng(9)
    chunks = [_chunk(rng, 8, 32, 8, 8, 17), _chunk(rng, 11, 32, 8, 8, -900)]
    q = rng.standard_normal((4, 32))
    kw = dict(layout=oracle.HALF_SPLIT, theta=1e6)
    whole = att.chunk_attention(q, chunks, 0.1, **kw)
    parts = [att.chunk_attention(q, [c], 0.1, **kw) for c in chunks]
    o, lse = att.state_merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, whole[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, whole[1], rtol=0, atol=1e-12)


def test_a_query_turned_the_wrong_way_fails():
    """Planted mistake: turning q by +delta (instead of -delta) is not the same attention."""
    rng = np.random.default_rng(13)
    chunks = [_chunk(rng, 10, 32, 0, 0, 50)]
    q = rng.standard_normal((2, 32))
    o, _ = att.chunk_attention(q, chunks, 0.5, layout=oracle.HALF_SPLIT, theta=1e4)
    flipped = [dict(chunks[0], delta=-50)]
    o_wrong, _ = _counter_rotated(q, flipped, 0.5, oracle.HALF_SPLIT, 1e4)
    assert np.max(np.abs(o - o_wrong)) > 1e-3
