"""Plain fp64 oracle of the consumer side: decode attention over a (paged) KV cache and the
standard state merge.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): the tests, the smoke check and the
benchmark's CPU-baseline leg are the only callers.

The Kamera abstract (the authors' publication page and the summary page) states that the
direct readout of a cached chunk is recovered exactly by the standard state merge: attention
of a query over a concatenation of chunks equals the log-sum-exp weighted combination of its
attention over each chunk. Definitions (one query head, scores s_t = scale * <q, k_t>):
    lse = log sum_t exp(s_t),   o = sum_t exp(s_t - lse) v_t
    merge of parts (o_i, lse_i):  L = log sum_i exp(lse_i),  o = sum_i exp(lse_i - L) o_i
An empty part has lse = -inf and o = 0 and drops out of a merge.

chunk_attention: decode attention over cached chunks that are read where they are stored,
never relocated. Each chunk contributes the keys and values the reuse operator defines for it
(relocation by its shift plus its rank-m patch, the technical summary's reuse equation), kept
exact in fp64; the result is attention over all chunks' tokens together.
"""
from __future__ import annotations

import numpy as np

import oracle as _core


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """q (heads x D), K and V (tokens x D), all fp64 -> (o (heads x D), lse (heads,))."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    heads, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((heads, D)), np.full(heads, -np.inf)
    s = scale * (q @ K.T)                       # heads x tokens
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    z = w.sum(axis=1, keepdims=True)
    return (w @ V) / z, (m + np.log(z))[:, 0]


def state_merge(outs: list, lses: list):
    """Merge attention states (o_i (rows x D), lse_i (rows,)) of disjoint key sets."""
    lse = np.stack([np.asarray(x, np.float64) for x in lses])        # parts x rows
    o = np.stack([np.asarray(x, np.float64) for x in outs])          # parts x rows x D
    M = lse.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lse), np.exp(lse - Ms), 0.0)            # parts x rows
    Z = w.sum(axis=0)
    out = np.where(finite[:, None], (w[:, :, None] * o).sum(axis=0) / np.where(Z > 0, Z, 1.0)[:, None], 0.0)
    return out, np.where(finite, Ms + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)


def score_bounds(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """sum_d |q_d k_td| * scale per head and token: the scale of each score's terms."""
    return abs(scale) * (np.abs(np.asarray(q, np.float64)) @ np.abs(np.asarray(K, np.float64)).T)


def chunk_keys_values(chunk: dict, *, layout: int, theta: float, rot_dim: int | None = None,
                      inv_freq=None, pair_section=None):
    """(K', V') of one chunk and one KV head in fp64: K' = R(delta) K + Uk Vk^T and
    V' = V + Uv Vv^T (the reuse operator's rows, unrounded). chunk: 'K', 'V' (tokens x D, in
    the model's element type), 'delta' (and 'section_delta' when pair_section is given),
    optional 'Uk', 'Vk', 'Uv', 'Vv'."""
    pd = None
    if pair_section is not None:
        pd = _core.pair_deltas(pair_section, chunk["section_delta"])
    k, _ = _core.segment(chunk["K"], rotate=True, layout=layout, delta=int(chunk["delta"]),
                         theta=theta, U=chunk.get("Uk"), V=chunk.get("Vk"), rot_dim=rot_dim,
                         inv_freq=inv_freq, pair_delta=pd)
    v, _ = _core.segment(chunk["V"], rotate=False, U=chunk.get("Uv"), V=chunk.get("Vv"))
    return k, v


def chunk_attention(q: np.ndarray, chunks: list, scale: float, *, layout: int, theta: float,
                    rot_dim: int | None = None, inv_freq=None, pair_section=None):
    """q (heads x D, fp64) over the tokens of every chunk (see chunk_keys_values) ->
    (o (heads x D), lse (heads,))."""
    D = np.asarray(q).shape[1]
    Ks, Vs = [np.zeros((0, D))], [np.zeros((0, D))]
    for c in chunks:
        k, v = chunk_keys_values(c, layout=layout, theta=theta, rot_dim=rot_dim,
                                 inv_freq=inv_freq, pair_section=pair_section)
        Ks.append(k)
        Vs.append(v)
    return decode_attention(q, np.concatenate(Ks), np.concatenate(Vs), scale)
