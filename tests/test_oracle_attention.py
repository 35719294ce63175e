"""Pins of the attention / state-merge oracle (oracle/attention.py) against a library routine
and closed forms: torch's scaled_dot_product_attention in fp64; one key returns its value;
equal scores average the values; the merge of a split equals attention over the whole
(the state-merge identity the Kamera abstract relies on); empty parts drop out."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as att


def _rand(rng, h, t, d):
    return rng.standard_normal((h, d)), rng.standard_normal((t, d)), rng.standard_normal((t, d))


@pytest.mark.parametrize("t", [1, 7, 300])
def test_matches_torch_sdpa_fp64(t):
    rng = np.random.default_rng(t)
    q, K, V = _rand(rng, 7, t, 128)
    scale = 1 / math.sqrt(128)
    o, lse = att.decode_attention(q, K, V, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None], torch.from_numpy(K)[None, None].expand(1, 7, t, 128),
        torch.from_numpy(V)[None, None].expand(1, 7, t, 128), scale=scale)[0, :, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = scale * q @ K.T
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=1e-13, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(1)
    q, K, V = _rand(rng, 3, 1, 16)
    o, lse = att.decode_attention(q, K, V, 0.5)
    np.testing.assert_array_equal(o, np.repeat(V, 3, axis=0))           # one key: its value
    np.testing.assert_allclose(lse, 0.5 * (q @ K.T)[:, 0], rtol=0, atol=1e-15)
    K = np.zeros((5, 16))
    V = rng.standard_normal((5, 16))
    o, lse = att.decode_attention(q, K, V, 1.0)                          # equal scores
    np.testing.assert_allclose(o, np.repeat(V.mean(axis=0, keepdims=True), 3, axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, np.log(5.0), rtol=1e-15)


@pytest.mark.parametrize("cuts", [(100,), (1, 50, 299), (0, 150)])
def test_merge_of_a_split_is_the_whole(cuts):
    rng = np.random.default_rng(7)
    q, K, V = _rand(rng, 4, 300, 64)
    scale = 0.125
    whole = att.decode_attention(q, K, V, scale)
    edges = [0, *cuts, 300]
    parts = [att.decode_attention(q, K[a:b], V[a:b], scale) for a, b in zip(edges, edges[1:])]
    o, lse = att.state_merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, whole[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, whole[1], rtol=0, atol=1e-12)


def test_empty_parts_drop_out_and_all_empty_is_empty():
    rng = np.random.default_rng(9)
    q, K, V = _rand(rng, 2, 10, 8)
    full = att.decode_attention(q, K, V, 1.0)
    empty = att.decode_attention(q, K[:0], V[:0], 1.0)
    assert np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)
    o, lse = att.state_merge([empty[0], full[0], empty[0]], [empty[1], full[1], empty[1]])
    np.testing.assert_allclose(o, full[0], atol=1e-15)
    np.testing.assert_allclose(lse, full[1], atol=1e-15)
    o, lse = att.state_merge([empty[0]], [empty[1]])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_a_wrong_merge_weight_fails_the_identity():
    """A merge that forgets the lse weights (plain average) is not attention over the whole."""
    rng = np.random.default_rng(11)
    q, K, V = _rand(rng, 3, 40, 16)
    a = att.decode_attention(q, K[:10], V[:10], 1.0)
    b = att.decode_attention(q, K[10:], V[10:], 1.0)
    whole = att.decode_attention(q, K, V, 1.0)
    assert np.max(np.abs((a[0] + b[0]) / 2 - whole[0])) > 1e-3
