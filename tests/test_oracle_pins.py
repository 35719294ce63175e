"""Pins of the CPU oracle to facts other than itself (no GPU).

The pages print no worked example, so the oracle is pinned by:
  * library RoPE routines (Hugging Face transformers: Llama's half-split rotate_half form,
    GPT-J's interleaved rotate_every_two form, Llama's default inverse-frequency ladder);
  * high-precision trigonometry (mpmath at 50 digits);
  * the Eckart-Young theorem through numpy's SVD (a rank-m deficit is recovered exactly by
    its top-m factors, technical summary §2: the patch is the top-m SVD factors of the
    deficit Delta = KV(B|A) - KV(B|empty) of §1);
  * torch's fp32 -> bf16 rounding and numpy's fp64 -> fp32 rounding;
  * group properties of the rotation and brute force over tiny inputs.
Each test names the mistake it would catch.
"""
import math

import mpmath
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle

mpmath.mp.dps = 50


# ----------------------------------------------------------------------------------------
# independent references
# ----------------------------------------------------------------------------------------

def mp_cos_sin(positions, theta, d):
    """cos/sin of pos * theta^(-2i/d) for every position and pair, at 50 digits."""
    positions = list(positions)
    c = np.empty((len(positions), d // 2))
    s = np.empty((len(positions), d // 2))
    th = mpmath.mpf(theta)
    for a, pos in enumerate(positions):
        for i in range(d // 2):
            ang = mpmath.mpf(int(pos)) * mpmath.power(th, mpmath.mpf(-2 * i) / d)
            c[a, i] = float(mpmath.cos(ang))
            s[a, i] = float(mpmath.sin(ang))
    return c, s


def lib_rope_half(x, positions, theta):
    """RoPE at absolute positions via transformers' Llama apply_rotary_pos_emb (fp64).
    x: [T, H, D] -> [T, H, D]."""
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    T, H, D = x.shape
    c, s = mp_cos_sin(positions, theta, D)
    cos = torch.from_numpy(np.concatenate([c, c], axis=1))[None]        # [1, T, D]
    sin = torch.from_numpy(np.concatenate([s, s], axis=1))[None]
    q = torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]   # [1, H, T, D]
    _, k = apply_rotary_pos_emb(q, q, cos, sin, unsqueeze_dim=1)
    return k[0].numpy().transpose(1, 0, 2)


def lib_rope_interleaved(x, positions, theta):
    """RoPE at absolute positions via transformers' GPT-J apply_rotary_pos_emb (fp64).
    x: [T, H, D] -> [T, H, D]."""
    from transformers.models.gptj.modeling_gptj import apply_rotary_pos_emb
    T, H, D = x.shape
    c, s = mp_cos_sin(positions, theta, D)
    t = torch.from_numpy(np.ascontiguousarray(x))[None]                     # [1, T, H, D]
    out = apply_rotary_pos_emb(t, torch.from_numpy(s)[None], torch.from_numpy(c)[None])
    return out[0].numpy()


LIB = {oracle.HALF_SPLIT: lib_rope_half, oracle.INTERLEAVED: lib_rope_interleaved}


def relocate_heads(x, layout, delta, theta, U=None, V=None):
    """Apply the oracle head by head to a [T, H, D] array."""
    out = np.empty(x.shape, np.float64)
    for h in range(x.shape[1]):
        uu = None if U is None else U[h]
        vv = None if V is None else V[h]
        out[:, h, :], _ = oracle.segment(np.ascontiguousarray(x[:, h, :]), rotate=True,
                                         layout=layout, delta=delta, theta=theta, U=uu, V=vv)
    return out


# ----------------------------------------------------------------------------------------
# frequencies and phases
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("theta,d", [(1e4, 128), (1e6, 128), (1e4, 64), (5e5, 256)])
def test_inv_freq_matches_transformers_llama_ladder(theta, d):
    """Catches a wrong exponent (i/d instead of 2i/d, a missing minus) or a wrong base."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
    cfg = LlamaConfig(hidden_size=4 * d, num_attention_heads=4, head_dim=d, rope_theta=theta)
    lib, _ = LlamaRotaryEmbedding.compute_default_rope_parameters(cfg)
    ours = oracle.inv_freq(theta, d)
    np.testing.assert_allclose(ours, lib.double().numpy(), rtol=1e-6, atol=0)


@pytest.mark.parametrize("theta,d", [(1e4, 128), (1e6, 64)])
def test_inv_freq_endpoints_closed_form(theta, d):
    """Pair 0 turns at frequency 1, the last pair at theta^(-(d-2)/d) (the slowest)."""
    inv = oracle.inv_freq(theta, d)
    assert inv[0] == 1.0
    last = float(mpmath.power(mpmath.mpf(theta), mpmath.mpf(-(d - 2)) / d))
    assert abs(inv[-1] - last) <= 4e-16 * last
    assert np.all(np.diff(inv) < 0)


@pytest.mark.parametrize("delta", [0, 1, -1, 1000, -32768, 65536, 2**31 - 1])
def test_phase_pair0_is_delta_radians(delta):
    """Pair 0 rotates by exactly delta radians: cos/sin(delta) at 50 digits."""
    c, s = oracle.phase(delta, 1e4, 128)
    assert abs(c[0] - float(mpmath.cos(delta))) <= 2e-16
    assert abs(s[0] - float(mpmath.sin(delta))) <= 2e-16


@pytest.mark.parametrize("delta", [1000, -32768, 65536])
def test_phase_is_fp64_accurate_at_large_shift(delta):
    """The angle is formed in fp64: an fp32 angle would be off by ~1e-3 rad at these shifts."""
    c, s = oracle.phase(delta, 1e6, 128)
    mc, ms = mp_cos_sin([delta], 1e6, 128)
    assert np.max(np.abs(c - mc[0])) < 1e-10
    assert np.max(np.abs(s - ms[0])) < 1e-10


# ----------------------------------------------------------------------------------------
# P1: relocating a canonical key equals RoPE applied at the target position (library form)
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", [oracle.HALF_SPLIT, oracle.INTERLEAVED])
@pytest.mark.parametrize("delta", [1, 37, 1000, -500, 65536])
@pytest.mark.parametrize("theta,d", [(1e4, 128), (1e6, 128), (1e4, 64)])
def test_relocation_equals_library_rope_at_target(layout, delta, theta, d):
    """R(delta) RoPE(k, j) == RoPE(k, j + delta); at j = 0 RoPE is the identity.
    Catches a wrong sign, a wrong pairing (half-split vs interleaved) or a wrong frequency."""
    rng = np.random.default_rng(1)
    T, H = 6, 2
    raw = rng.standard_normal((T, H, d))
    j = np.arange(T)
    canonical = LIB[layout](raw, j, theta)
    if layout == oracle.HALF_SPLIT:
        np.testing.assert_allclose(canonical[0], raw[0], rtol=0, atol=1e-15)  # RoPE(k, 0) = k
    target = LIB[layout](raw, j + delta, theta)
    got = relocate_heads(canonical, layout, delta, theta)
    tol = 4e-16 * (abs(delta) + 16) * np.max(np.abs(raw))
    assert np.max(np.abs(got - target)) <= tol


def test_relocation_matches_transformers_fp32_pipeline():
    """End to end against the library's own fp32 cos/sin pipeline (frequencies + angles +
    apply), at shifts where fp32 angles are still accurate to ~1e-4."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import (LlamaRotaryEmbedding,
                                                          apply_rotary_pos_emb)
    d, theta = 128, 1e4
    cfg = LlamaConfig(hidden_size=4 * d, num_attention_heads=4, head_dim=d, rope_theta=theta,
                      max_position_embeddings=4096)
    emb = LlamaRotaryEmbedding(cfg)
    rng = np.random.default_rng(2)
    raw = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    for delta in (1, 5, 100, 1000):
        cos, sin = emb(torch.zeros(1, 1, d), torch.tensor([[delta]]))
        _, lib = apply_rotary_pos_emb(torch.from_numpy(raw), torch.from_numpy(raw), cos, sin)
        got, _ = oracle.segment(raw[0, 0].astype(np.float32), rotate=True, delta=delta,
                                theta=theta)
        assert np.max(np.abs(got[0] - lib[0, 0, 0].double().numpy())) < 2e-4 * max(1, delta / 100)


def test_mla_k_rope_relocation_64_dims():
    """MLA moves only the 64-dim k_rope: a 64-wide head, same rule (Irminsul's delta-rotation
    rule for k_r is the same case)."""
    rng = np.random.default_rng(3)
    raw = rng.standard_normal((5, 1, 64))
    for layout in (oracle.HALF_SPLIT, oracle.INTERLEAVED):
        canonical = LIB[layout](raw, np.arange(5), 1e4)
        got = relocate_heads(canonical, layout, 40000, 1e4)
        target = LIB[layout](raw, np.arange(5) + 40000, 1e4)
        assert np.max(np.abs(got - target)) < 1e-10


# ----------------------------------------------------------------------------------------
# P2, P6, P7: group properties of the rotation
# ----------------------------------------------------------------------------------------

@settings(max_examples=60, deadline=None)
@given(a=st.integers(-2**20, 2**20), b=st.integers(-2**20, 2**20),
       theta=st.sampled_from([1e4, 5e5, 1e6]), layout=st.sampled_from([0, 1]),
       d=st.sampled_from([2, 8, 64, 128]))
def test_composition_and_inverse(a, b, theta, layout, d):
    """R(a)R(b) = R(a+b) and R(-a)R(a) = I."""
    rng = np.random.default_rng(abs(a) + 7 * abs(b))
    x = rng.standard_normal((3, d))
    ra, _ = oracle.segment(x, rotate=True, layout=layout, delta=a, theta=theta)
    rab, _ = oracle.segment(ra, rotate=True, layout=layout, delta=b, theta=theta)
    direct, _ = oracle.segment(x, rotate=True, layout=layout, delta=a + b, theta=theta)
    tol = 1e-15 * (abs(a) + abs(b) + 16) * 8
    assert np.max(np.abs(rab - direct)) <= tol
    back, _ = oracle.segment(ra, rotate=True, layout=layout, delta=-a, theta=theta)
    assert np.max(np.abs(back - x)) <= tol


@pytest.mark.parametrize("layout", [0, 1])
def test_pair_norms_and_scores_preserved(layout):
    """Each pair keeps its norm and <R q, R k> = <q, k>: attention scores are unchanged by a
    common shift (the relative-position property that makes relocation exact)."""
    rng = np.random.default_rng(4)
    d = 128
    q = rng.standard_normal((4, d))
    k = rng.standard_normal((4, d))
    rq, _ = oracle.segment(q, rotate=True, layout=layout, delta=12345, theta=1e6)
    rk, _ = oracle.segment(k, rotate=True, layout=layout, delta=12345, theta=1e6)
    np.testing.assert_allclose(np.sum(rq * rk, axis=1), np.sum(q * k, axis=1), rtol=1e-12)
    if layout == 0:
        pn = lambda v: v[:, : d // 2] ** 2 + v[:, d // 2:] ** 2
    else:
        pn = lambda v: v[:, 0::2] ** 2 + v[:, 1::2] ** 2
    np.testing.assert_allclose(pn(rq), pn(q), rtol=1e-12)


def test_zero_shift_no_patch_is_identity():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 128))
    for layout in (0, 1):
        z, S = oracle.segment(x, rotate=True, layout=layout, delta=0, theta=1e4)
        assert np.array_equal(z, x)
        assert np.array_equal(S, np.abs(x))


# ----------------------------------------------------------------------------------------
# P3, P4, P9: the patch
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("m", [1, 8, 32])
def test_svd_of_rank_m_deficit_restores_conditioned_kv(layout, m):
    """KV(B|A) := RoPE(k, j + delta) + Delta with Delta of rank m. The top-m SVD factors of
    KV(B|A) - R(delta) KV(B|empty), added by the oracle, give back KV(B|A); m - 1 factors do
    not. Tokens (L = 48) != features (D = 128), so a transposed U/V fails."""
    rng = np.random.default_rng(10 + m)
    L, D, theta, delta = 48, 128, 1e6, 777
    raw = rng.standard_normal((L, 1, D))
    j = np.arange(L)
    canonical = LIB[layout](raw, j, theta)[:, 0]
    deficit = rng.standard_normal((L, m)) @ rng.standard_normal((m, D)) * 0.05
    conditioned = LIB[layout](raw, j + delta, theta)[:, 0] + deficit
    reloc, _ = oracle.segment(canonical, rotate=True, layout=layout, delta=delta, theta=theta)
    u, s, vt = np.linalg.svd(conditioned - reloc)
    assert s[m:].max(initial=0.0) < 1e-10 * s[0]
    U = np.ascontiguousarray(u[:, :m] * s[:m])
    V = np.ascontiguousarray(vt[:m].T)
    patched, _ = oracle.segment(canonical, rotate=True, layout=layout, delta=delta,
                                theta=theta, U=U, V=V)
    assert np.max(np.abs(patched - conditioned)) < 1e-10
    if m > 1:
        short, _ = oracle.segment(canonical, rotate=True, layout=layout, delta=delta,
                                  theta=theta, U=U[:, : m - 1].copy(), V=V[:, : m - 1].copy())
        assert np.max(np.abs(short - conditioned)) > 1e-3


def test_plain_channel_patch_is_u_vt():
    """Unrotated channel (values, c_KV): out = x + U V^T, compared with numpy's matmul."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((40, 512))
    U = rng.standard_normal((40, 32)) * 0.05
    V = rng.standard_normal((512, 32)) * 0.05
    z, S = oracle.segment(x, rotate=False, U=U, V=V)
    np.testing.assert_allclose(z, x + U @ V.T, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, np.abs(x) + np.abs(U) @ np.abs(V).T, rtol=1e-13)


@pytest.mark.parametrize("layout", [0, 1])
def test_linearity_reuse_minus_relocate_is_patch(layout):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((33, 128))
    U = rng.standard_normal((33, 16))
    V = rng.standard_normal((128, 16))
    reuse, _ = oracle.segment(x, rotate=True, layout=layout, delta=-4242, theta=1e4, U=U, V=V)
    reloc, _ = oracle.segment(x, rotate=True, layout=layout, delta=-4242, theta=1e4)
    np.testing.assert_allclose(reuse - reloc, U @ V.T, rtol=0, atol=1e-12)


def test_rank_zero_is_pure_relocation_and_plain_copy():
    """m = 0 reduces to relocation; an unrotated, unpatched channel is a bit copy."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((9, 128)).astype(np.float32)
    a, _ = oracle.segment(x, rotate=True, delta=99, theta=1e4)
    b, _ = oracle.segment(x, rotate=True, delta=99, theta=1e4,
                          U=np.zeros((9, 0), np.float32), V=np.zeros((128, 0), np.float32))
    assert np.array_equal(a, b)
    bits = (rng.integers(0, 2**16, size=(9, 512))).astype(np.uint16)
    e = oracle.expected_head(bits, rotate=False, layout=0, delta=5, theta=1e4, U=None, V=None)
    assert e["copy"] and e["bits"] is bits


# ----------------------------------------------------------------------------------------
# P10: brute force on tiny inputs (explicit 2x2 matrices, Python loops, 50-digit trig)
# ----------------------------------------------------------------------------------------

def brute_force(x, layout, delta, theta, U, V):
    T, D = len(x), len(x[0])
    out = [[0.0] * D for _ in range(T)]
    pairs = ([(i, i + D // 2) for i in range(D // 2)] if layout == 0
             else [(2 * i, 2 * i + 1) for i in range(D // 2)])
    for t in range(T):
        for i, (a, b) in enumerate(pairs):
            ang = mpmath.mpf(delta) * mpmath.power(mpmath.mpf(theta), mpmath.mpf(-2 * i) / D)
            rot = [[mpmath.cos(ang), -mpmath.sin(ang)], [mpmath.sin(ang), mpmath.cos(ang)]]
            va, vb = mpmath.mpf(float(x[t][a])), mpmath.mpf(float(x[t][b]))
            out[t][a] = rot[0][0] * va + rot[0][1] * vb
            out[t][b] = rot[1][0] * va + rot[1][1] * vb
        for f in range(D):
            acc = mpmath.mpf(0)
            for r in range(len(U[0]) if U is not None else 0):
                acc += mpmath.mpf(float(U[t][r])) * mpmath.mpf(float(V[f][r]))
            out[t][f] = float(out[t][f] + acc)
    return np.array(out, dtype=np.float64)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("D", [2, 4, 8])
@pytest.mark.parametrize("m", [0, 1, 3])
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_brute_force_tiny(layout, D, m, dtype):
    rng = np.random.default_rng(100 * D + 10 * m + layout)
    T = 5
    x = rng.standard_normal((T, D)).astype(dtype)
    U = rng.standard_normal((T, m)).astype(dtype) if m else None
    V = rng.standard_normal((D, m)).astype(dtype) if m else None
    delta = int(rng.integers(-70000, 70000))
    z, S = oracle.segment(x, rotate=True, layout=layout, delta=delta, theta=1e4, U=U, V=V)
    ref = brute_force(x.tolist(), layout, delta, 1e4, None if U is None else U.tolist(),
                      None if V is None else V.tolist())
    assert np.max(np.abs(z - ref)) < 1e-10
    assert np.all(S >= np.abs(z) - 1e-12)


def test_bf16_inputs_decode_exactly():
    """bf16 bit patterns decode to the same values torch gives them."""
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 2**16, size=(4, 64)).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80          # drop inf/nan patterns
    z, _ = oracle.segment(bits, rotate=False, U=np.zeros((4, 1), np.uint16),
                          V=np.zeros((64, 1), np.uint16))
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(z, ref)


# ----------------------------------------------------------------------------------------
# rounding of the oracle's output
# ----------------------------------------------------------------------------------------

def _bf16_probe_values():
    rng = np.random.default_rng(11)
    base = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    crafted = ((rng.integers(0, 2**16, size=(400, 1)).astype(np.uint32) << 16) | lows).ravel()
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x7F7F8000,
                        0x00000001, 0x00008000, 0x00018000, 0x807F8000, 0x3F808000, 0x3F818000],
                       np.uint32)
    u = np.concatenate([base, crafted, special])
    f = u.view(np.float32)
    return f[~np.isnan(f)]


def test_to_bf16_matches_torch_rounding():
    """Round to nearest even, ties, overflow to inf, subnormals and signed zero."""
    f = _bf16_probe_values()
    ours = oracle.to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = oracle.to_bf16(np.array([np.nan]))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


def test_to_f32_matches_numpy_rounding():
    rng = np.random.default_rng(12)
    z = rng.standard_normal(10000) * np.exp(rng.uniform(-30, 30, 10000))
    assert np.array_equal(oracle.to_f32(z).view(np.uint32), z.astype(np.float32).view(np.uint32))


# ----------------------------------------------------------------------------------------
# P11: page-table placement
# ----------------------------------------------------------------------------------------

def test_slots_brute_force_and_bijection():
    rng = np.random.default_rng(13)
    ps, n_logical, n_pages = 16, 40, 50
    table = rng.permutation(n_pages)[:n_logical].astype(np.int32)
    chunks = [(0, 100), (100, 37), (137, 1), (138, 502)]       # (offset, tokens), ragged
    seen = set()
    for off, n in chunks:
        got = oracle.slots(table, ps, off, n)
        for t in range(n):
            p = off + t
            assert got[t] == int(table[p // ps]) * ps + (p % ps)
            seen.add(int(got[t]))
    assert len(seen) == sum(n for _, n in chunks)
    assert max(seen) < n_pages * ps
    ident = oracle.slots(None, ps, 77, 10)
    assert np.array_equal(ident, np.arange(77, 87))
    with pytest.raises(ValueError):
        oracle.slots(table, ps, n_logical * ps - 3, 4)


# ----------------------------------------------------------------------------------------
# patch compile: deficit and top-m factors
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", [0, 1])
def test_deficit_is_conditioned_minus_relocated_canonical(layout):
    """Delta of KV(B|A) = RoPE(k, j + delta) + E against KV(B|empty) = RoPE(k, j) is E
    (RoPE from the transformers routines, E arbitrary)."""
    rng = np.random.default_rng(20)
    L, D, theta, delta = 24, 64, 1e4, 3000
    raw = rng.standard_normal((L, 1, D))
    j = np.arange(L)
    E = rng.standard_normal((L, D)) * 0.1
    canonical = LIB[layout](raw, j, theta)[:, 0]
    conditioned = LIB[layout](raw, j + delta, theta)[:, 0] + E
    d = oracle.deficit(conditioned, canonical, rotate=True, layout=layout, delta=delta, theta=theta)
    np.testing.assert_allclose(d, E, rtol=0, atol=1e-11)
    # unrotated channel: a plain difference
    d2 = oracle.deficit(conditioned, canonical, rotate=False)
    np.testing.assert_allclose(d2, conditioned - canonical, rtol=0, atol=0)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_compile_recovers_exact_rank_m_deficit(m):
    rng = np.random.default_rng(21 + m)
    L, D = 40, 128
    canonical = rng.standard_normal((L, D))
    E = rng.standard_normal((L, m)) @ rng.standard_normal((m, D))
    reloc, _ = oracle.segment(canonical, rotate=True, delta=-777, theta=1e6)
    r = oracle.compile_patch(reloc + E, canonical, m=m, rotate=True, delta=-777, theta=1e6)
    np.testing.assert_allclose(r["UV"], E, rtol=0, atol=1e-10)
    np.testing.assert_allclose(r["V"].T @ r["V"], np.eye(m), atol=1e-12)     # orthonormal V
    np.testing.assert_allclose(r["U"], r["delta"] @ r["V"], atol=1e-10)       # U = Delta V


def test_compile_is_the_best_rank_m_approximation():
    """Eckart-Young: the residual's squared Frobenius norm is the sum of the discarded
    squared singular values, and a random rank-m projection does worse."""
    rng = np.random.default_rng(30)
    L, D, m = 60, 64, 8
    canonical = rng.standard_normal((L, D))
    conditioned = rng.standard_normal((L, D))
    r = oracle.compile_patch(conditioned, canonical, m=m, rotate=False)
    resid = np.sum((r["delta"] - r["UV"]) ** 2)
    assert abs(resid - np.sum(r["s"][m:] ** 2)) < 1e-9 * resid
    q, _ = np.linalg.qr(rng.standard_normal((D, m)))
    other = r["delta"] @ q @ q.T
    assert np.sum((r["delta"] - other) ** 2) > resid


# ----------------------------------------------------------------------------------------
# orbit patch: the mean deficit over orderings, then its top-m factors
# ----------------------------------------------------------------------------------------

def _orbit_set(rng, T=40, D=64, K=4, m=6, theta=1e4, layout=oracle.HALF_SPLIT):
    """K orderings of a chunk: shifts d_k, conditioned = R(d_k) canonical + shared low-rank
    deficit + an ordering-specific deficit (all fp64)."""
    canonical = rng.standard_normal((T, D))
    shared = rng.standard_normal((T, m)) @ rng.standard_normal((m, D)) * 0.1
    members = []
    for k in range(K):
        d = int(rng.integers(-5000, 5000))
        own = rng.standard_normal((T, 2)) @ rng.standard_normal((2, D)) * 0.02
        reloc, _ = oracle.segment(canonical, rotate=True, layout=layout, delta=d, theta=theta)
        members.append((reloc + shared + own, d, own))
    return canonical, shared, members


def test_orbit_patch_of_one_ordering_is_the_compile():
    rng = np.random.default_rng(31)
    canonical, _, members = _orbit_set(rng, K=1)
    a = oracle.orbit_patch([members[0][:2]], canonical, m=6, rotate=True)
    b = oracle.compile_patch(members[0][0], canonical, m=6, rotate=True, delta=members[0][1])
    np.testing.assert_allclose(a["UV"], b["UV"], rtol=0, atol=1e-12)


def test_orbit_deficit_is_the_mean_of_the_orderings_deficits():
    """Closed form: each member contributes shared + own; the mean is shared + mean(own)."""
    rng = np.random.default_rng(32)
    canonical, shared, members = _orbit_set(rng, K=5)
    r = oracle.orbit_patch([mm[:2] for mm in members], canonical, m=6, rotate=True)
    expect = shared + sum(mm[2] for mm in members) / len(members)
    np.testing.assert_allclose(r["delta"], expect, rtol=0, atol=1e-11)


def test_orbit_patch_serves_every_ordering_better_than_no_patch():
    """With a shared rank-m deficit and small ordering-specific parts, the one orbit patch
    leaves each ordering with only (roughly) its own part."""
    rng = np.random.default_rng(33)
    canonical, shared, members = _orbit_set(rng, K=6)
    r = oracle.orbit_patch([mm[:2] for mm in members], canonical, m=6, rotate=True)
    for cond, d, own in members:
        dk = oracle.deficit(cond, canonical, rotate=True, delta=d)
        left = np.linalg.norm(dk - r["UV"])
        assert left < 0.5 * np.linalg.norm(dk)
        assert left < 3.0 * np.linalg.norm(own) + 1e-9


def test_orbit_patch_members_in_the_same_frame_average_conditioned_kv():
    """All orderings at one shift: the mean deficit is the deficit of the mean conditioned KV."""
    rng = np.random.default_rng(34)
    canonical = rng.standard_normal((30, 32))
    conds = [rng.standard_normal((30, 32)) for _ in range(3)]
    r = oracle.orbit_patch([(c, 123) for c in conds], canonical, m=4, rotate=True)
    d = oracle.deficit(sum(conds) / 3, canonical, rotate=True, delta=123)
    np.testing.assert_allclose(r["delta"], d, rtol=0, atol=1e-12)
