"""Patch compile on the GPU (kamera_patch_compile through the C ABI) against the oracle.

The oracle is the exact fp64 deficit of the same stored inputs and its LAPACK SVD
(oracle.compile_patch). What is unique is compared: the rank-m truncation U V^T and the
projector V V^T; the GPU basis itself must be orthonormal. Tolerances are derived in
tests/compile_cases.py.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from position_invariant_kv_kamera_amd import binding as kb
import compile_cases as cc

pytestmark = pytest.mark.gpu

SENT_BF16 = 0x7FC1
SENT_F32 = 0x7FC00001


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _torch_dtype(case):
    return torch.bfloat16 if case.dtype == "bf16" else torch.float32


def _to_device(bits: np.ndarray, case) -> torch.Tensor:
    if case.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda()


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _sentinel(shape, case) -> torch.Tensor:
    t = torch.empty(shape, dtype=_torch_dtype(case), device="cuda")
    if case.dtype == "bf16":
        t.view(torch.int16).fill_(SENT_BF16)
    else:
        t.view(torch.int32).fill_(SENT_F32)
    return t


def model_of(case) -> kb.KameraModel:
    return kb.make_model(case.family, case.dtype, case.n_layers, case.n_kv_heads,
                         case.head_dim, case.rope_dim, case.layout, case.theta)


def device_items(case, inputs):
    """CompileItems (device tensors) for every chunk of the case; keeps the tensors alive."""
    items, keep = [], []
    for c, spec in enumerate(case.chunks):
        canon, cond = [], []
        if case.family == "mla" and case.mla_shared_rows:
            # one [c_KV | k_rope] row per token, channels as views into it
            for key, dst in (("canonical", canon), ("conditioned", cond)):
                rows = np.concatenate([inputs[c][key][1], inputs[c][key][0]], axis=-1)
                t = _to_device(rows, case)
                keep.append(t)
                dst.extend([t[..., case.head_dim:], t[..., :case.head_dim]])
        else:
            for ch in range(2):
                canon.append(_to_device(inputs[c]["canonical"][ch], case))
                cond.append(_to_device(inputs[c]["conditioned"][ch], case))
        U, V = [], []
        for ch in range(2):
            H, W, _ = case.geometry(ch)
            U.append(_sentinel((case.n_layers, H, spec.n_tokens, spec.m), case))
            V.append(_sentinel((case.n_layers, H, W, spec.m), case))
        keep += canon + cond
        items.append(kb.CompileItem(spec.n_tokens, spec.m, spec.delta, canon, cond, U, V))
    return items, keep


def run(case, inputs=None, n_iter=None):
    inputs = inputs if inputs is not None else cc.build(case)
    items, keep = device_items(case, inputs)
    _log(f"[compile] case={case.name} dtype={case.dtype} chunks={len(items)}")
    kb.run_compile(model_of(case), items, n_iter=n_iter or case.n_iter)
    torch.cuda.synchronize()
    return inputs, items


def outputs(case, items, c, ch):
    U = cc.decode(_bits(items[c].U[ch]), case.dtype)
    V = cc.decode(_bits(items[c].V[ch]), case.dtype)
    return U, V


def check_case(case, inputs, items, heads=None):
    worst = []
    for c, spec in enumerate(case.chunks):
        for ch in range(2):
            H, W, _ = case.geometry(ch)
            U, V = outputs(case, items, c, ch)
            assert np.all(np.isfinite(U)) and np.all(np.isfinite(V)), \
                f"{case.name}: unwritten or non-finite factors (chunk {c} channel {ch})"
            units = heads if heads is not None else [(l, h) for l in range(case.n_layers)
                                                     for h in range(H)]
            for (l, h) in units:
                if h >= H:
                    continue
                e = cc.expected(case, inputs, c, ch, l, h)
                r = cc.check_head(U[l, h], V[l, h], e, case.dtype)
                worst.append((r.patch_excess, r.proj_excess, r.orth_err / r.orth_tol,
                              (c, ch, l, h)))
                assert r.ok, (f"{case.name} chunk {c} channel {ch} layer {l} head {h}: "
                              f"patch {r.patch_excess:.3g} proj {r.proj_excess:.3g} "
                              f"orth {r.orth_err:.3g}/{r.orth_tol:.3g}")
    w = max(worst)
    _log(f"[compile] {case.name}: worst patch/tol {w[0]:.3g} proj/tol "
         f"{max(x[1] for x in worst):.3g} orth/tol {max(x[2] for x in worst):.3g}")


@pytest.mark.parametrize("case", cc.small_cases(), ids=lambda c: c.name)
def test_compile_matches_oracle_svd(case):
    inputs, items = run(case)
    check_case(case, inputs, items)


def test_zero_deficit_gives_a_zero_patch():
    case = cc.degenerate_cases()[0]
    inputs, items = run(case)
    for ch in range(2):
        U, V = outputs(case, items, 0, ch)
        assert np.all(U == 0.0), "Delta == 0 must give U == 0 exactly"
        for l in range(case.n_layers):
            for h in range(case.geometry(ch)[0]):
                g = V[l, h].T @ V[l, h]
                assert np.all(np.isfinite(g))
                assert np.max(np.abs(g - np.eye(g.shape[0]))) <= 2 * 2.0 ** -8 * 1.02 + 2.0 ** -20


@pytest.mark.parametrize("idx", [1, 2, 3], ids=["rank16", "rank64", "mla_rank32"])
def test_fewer_tokens_than_rank_reconstructs_delta(idx):
    case = cc.degenerate_cases()[idx]
    inputs, items = run(case)
    check_case(case, inputs, items)


def test_deterministic_and_independent_of_the_batch():
    """The same chunk compiles to the same bits twice, and alone or beside other chunks."""
    base = cc.small_cases()[0]
    inputs, items = run(base)
    _, again = run(base, inputs)
    both = cc.Case(**{**base.__dict__, "name": "pair", "chunks": base.chunks + [
        cc.ChunkSpec(700, 32, -5000)]})
    extra = cc.build(cc.Case(**{**both.__dict__, "chunks": both.chunks, "seed": 99}))
    _, pair = run(both, [inputs[0], extra[1]])
    for ch in range(2):
        for a in (again, pair):
            assert np.array_equal(_bits(items[0].U[ch]), _bits(a[0].U[ch]))
            assert np.array_equal(_bits(items[0].V[ch]), _bits(a[0].V[ch]))


def test_wide_heads_independent_of_the_launch_rank_class():
    """A rank-12 MLA chunk compiles to the same bits alone (rank-16 class) and beside a rank-32
    chunk (its latent heads then run in the rank-32 class)."""
    base = cc.Case("mla_alone", "mla", "bf16", 1, 1, 512, 64, oracle.HALF_SPLIT, 1e4,
                   [cc.ChunkSpec(260, 12, 555)], seed=17)
    inputs, items = run(base)
    both = cc.Case(**{**base.__dict__, "name": "mla_pair",
                      "chunks": base.chunks + [cc.ChunkSpec(180, 32, -90)]})
    extra = cc.build(cc.Case(**{**both.__dict__, "seed": 98}))
    _, pair = run(both, [inputs[0], extra[1]])
    for ch in range(2):
        assert np.array_equal(_bits(items[0].U[ch]), _bits(pair[0].U[ch]))
        assert np.array_equal(_bits(items[0].V[ch]), _bits(pair[0].V[ch]))


def test_projection_block_length_leaves_the_bits_unchanged(monkeypatch):
    """U rows are formed token by token, so the streamed projection's tokens per block (512 by
    default at this size; 2048, cut into equal 16-token multiples, when the block-count floor is
    lowered) change no bit; 3000 tokens split into two blocks of 1504 there."""
    case = cc.Case("proj_blocks", "gqa", "bf16", 1, 2, 128, 128, oracle.HALF_SPLIT, 1e6,
                   [cc.ChunkSpec(3000, 16, 321), cc.ChunkSpec(4096, 32, -77)], seed=19)
    inputs, items = run(case)
    check_case(case, inputs, items)
    monkeypatch.setenv("KAMERA_PROJ_MIN_BLOCKS", "1")
    _, long_blocks = run(case, inputs)
    for i in range(2):
        for ch in range(2):
            assert np.array_equal(_bits(items[i].U[ch]), _bits(long_blocks[i].U[ch]))
            assert np.array_equal(_bits(items[i].V[ch]), _bits(long_blocks[i].V[ch]))


def test_compiled_patch_restores_the_conditioned_kv():
    """Relocate + compiled patch (kamera_reuse_batch) reproduces KV(B|A): within the rank-m
    residual of the deficit, the patch tolerance and one rounding of the output."""
    for case in (cc.small_cases()[0], cc.small_cases()[1]):
        inputs, items = run(case)
        spec = case.chunks[0]
        T = spec.n_tokens
        ps = 16
        n_pages = -(-T // ps)
        pools = []
        cache = kb.KameraCache()
        row = case.n_kv_heads * case.head_dim
        for ch in range(2):
            pools.append(_sentinel((case.n_layers, n_pages * ps, row), case))
            cache.pool[ch] = pools[ch].data_ptr()
        cache.layer_stride = pools[0].stride(0)
        cache.token_stride = pools[0].stride(1)
        cache.page_table = None
        cache.n_logical_pages = n_pages
        cache.page_size = ps
        cache.n_pages = n_pages
        chunks = (kb.KameraChunk * 1)()
        k = chunks[0]
        k.n_tokens, k.dst_token_offset, k.delta = T, 0, spec.delta
        it = items[0]
        for ch in range(2):
            s = it.canonical[ch]
            k.src[ch] = kb.KameraSrc(s.data_ptr(), s.stride(0), s.stride(1))
            U, V = it.U[ch], it.V[ch]
            k.patch[ch] = kb.KameraPatchRef(spec.m, 0, U.data_ptr(), U.stride(0), U.stride(1),
                                            V.data_ptr(), V.stride(0), V.stride(1))
        ws = kb.Workspace(1)
        kb.check(kb.kamera_reuse_batch(model_of(case), cache, chunks, 1, ws.ptr, ws.nbytes,
                                       kb.current_stream_ptr()))
        torch.cuda.synchronize()
        u = 2.0 ** -8 if case.dtype == "bf16" else 2.0 ** -24
        for ch in range(2):
            H, W, _ = case.geometry(ch)
            got = cc.decode(_bits(pools[ch][:, :T]), case.dtype)
            for l in range(case.n_layers):
                for h in range(H):
                    e = cc.expected(case, inputs, 0, ch, l, h)
                    cond = oracle.values(inputs[0]["conditioned"][ch][l, :, h * W:(h + 1) * W])
                    Vo = e["V"]
                    pf = np.sqrt(np.diag(Vo @ Vo.T))
                    dm = np.linalg.norm(e["UV"], axis=1)
                    dn = np.linalg.norm(e["delta"], axis=1)
                    r = 2 * u * (1 + 2.0 ** -6)
                    patch_tol = r * np.outer(dm, pf) + (2 * e["eps_sub"] + 1e-6) * dn[:, None]
                    resid = np.abs(e["delta"] - e["UV"])
                    g = got[l, :, h * W:(h + 1) * W]
                    # one rounding of the output, plus the fp32 chain of the reuse kernel
                    out_round = (u * np.abs(cond) * 1.02
                                 + 2 * (spec.m + 4) * 2.0 ** -24 * (np.abs(cond) + 1))
                    tol = resid + patch_tol + out_round
                    bad = np.abs(g - cond) > tol
                    assert not bad.any(), (f"{case.name} ch {ch} l {l} h {h}: "
                                           f"{int(bad.sum())} elements off")


def test_full_size_chunk_sampled_heads():
    """A full 28-layer, 4-head, 1296-token chunk (split Gram, assembled G); every head's
    factors are finite and orthonormal, 12 sampled heads are checked against the oracle."""
    case = cc.full_case()
    inputs, items = run(case)
    rng = np.random.default_rng(5)
    heads = [(0, 0), (27, 3)] + [(int(rng.integers(28)), int(rng.integers(4)))
                                 for _ in range(10)]
    check_case(case, inputs, items, heads=heads)
    for ch in range(2):
        _, V = outputs(case, items, 0, ch)
        g = np.einsum("lhfr,lhfs->lhrs", V, V)
        assert np.max(np.abs(g - np.eye(16))) <= 2 * 2.0 ** -8 * 1.02 + 2.0 ** -20


def test_full_size_mla_chunk_sampled_heads():
    """A full 27-layer, 2048-token MLA chunk (the latent's Gram over 64 token steps without
    splits, its block-per-head subspace); every head's factors are orthonormal, six sampled
    layers of both channels are checked against the oracle."""
    case = cc.full_mla_case()
    inputs, items = run(case)
    rng = np.random.default_rng(6)
    heads = [(0, 0), (26, 0)] + [(int(rng.integers(27)), 0) for _ in range(4)]
    check_case(case, inputs, items, heads=heads)
    for ch in range(2):
        _, V = outputs(case, items, 0, ch)
        g = np.einsum("lhfr,lhfs->lhrs", V, V)
        assert np.max(np.abs(g - np.eye(32))) <= 2 * 2.0 ** -8 * 1.02 + 2.0 ** -20


def test_rank64_chunk_sampled_heads():
    """Rank 64 at the MHA reorder workload's per-head geometry (4096 tokens, 32 heads, the
    blocked factorisation of rank 64): every head orthonormal, eight sampled heads checked
    against the oracle."""
    case = cc.full_rank64_case()
    inputs, items = run(case)
    rng = np.random.default_rng(7)
    heads = [(0, 0), (3, 31)] + [(int(rng.integers(4)), int(rng.integers(32))) for _ in range(6)]
    check_case(case, inputs, items, heads=heads)
    for ch in range(2):
        _, V = outputs(case, items, 0, ch)
        g = np.einsum("lhfr,lhfs->lhrs", V, V)
        assert np.max(np.abs(g - np.eye(64))) <= 2 * 2.0 ** -8 * 1.02 + 2.0 ** -20
