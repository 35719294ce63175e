"""The orbit patch on the GPU (kamera_patch_compile_orbit through the C ABI) against the
oracle's mean-deficit SVD (oracle.orbit_patch): unique quantities U V^T and V V^T under the
tolerance of tests/compile_cases.py (with the orbit's extra formation term), one ordering
bit-identical to the plain compile, and multimodal sections per ordering."""
import numpy as np
import pytest
import torch

import oracle
import compile_cases as cc
from position_invariant_kv_kamera_amd import binding as kb
from test_gpu_compile import _bits, _sentinel, _to_device, model_of, outputs

pytestmark = pytest.mark.gpu


def _orbit_items(case, inp, sections=None):
    spec = case.chunks[0]
    canon = [_to_device(inp["canonical"][ch], case) for ch in range(2)]
    members = []
    for k, d in enumerate(inp["deltas"]):
        cond = [_to_device(inp["conditioned"][k][ch], case) for ch in range(2)]
        members.append((d, cond) if sections is None else (d, cond, sections[k]))
    U, V = [], []
    for ch in range(2):
        H, W, _ = case.geometry(ch)
        U.append(_sentinel((case.n_layers, H, spec.n_tokens, spec.m), case))
        V.append(_sentinel((case.n_layers, H, W, spec.m), case))
    return [kb.OrbitItem(spec.n_tokens, spec.m, canon, members, U, V)]


def _check(case, inp, items, rope=None):
    worst = 0.0
    for ch in range(2):
        H, W, _ = case.geometry(ch)
        U, V = outputs(case, items, 0, ch)
        assert np.all(np.isfinite(U)) and np.all(np.isfinite(V))
        for l in range(case.n_layers):
            for h in range(H):
                e = cc.expected_orbit(case, inp, ch, l, h, rope=rope)
                r = cc.check_head(U[l, h], V[l, h], e, case.dtype)
                worst = max(worst, r.patch_excess, r.proj_excess)
                assert r.ok, (case.name, ch, l, h, r)
    print(f"[orbit] {case.name}: worst excess {worst:.3g}", flush=True)


ORBITS = [
    (cc.Case("orbit_bf16_k6", "gqa", "bf16", 2, 2, 128, 128, oracle.HALF_SPLIT, 1e6,
             [cc.ChunkSpec(300, 16, 0)], seed=41), [0, 1296, 2592, -1296, 5000, 77]),
    (cc.Case("orbit_f32_k3", "gqa", "f32", 1, 2, 64, 64, oracle.INTERLEAVED, 1e4,
             [cc.ChunkSpec(200, 8, 0)], seed=42), [0, 4096, 8192]),
    (cc.Case("orbit_mla_bf16_k4", "mla", "bf16", 1, 1, 512, 64, oracle.HALF_SPLIT, 1e4,
             [cc.ChunkSpec(260, 32, 0)], seed=43), [0, 2048, 4096, 6144]),
]


@pytest.mark.parametrize("case,deltas", ORBITS, ids=[c.name for c, _ in ORBITS])
def test_orbit_matches_oracle(case, deltas):
    inp = cc.build_orbit(case, deltas)
    items = _orbit_items(case, inp)
    print(f"[orbit] case={case.name} members={len(deltas)}", flush=True)
    kb.run_orbit_compile(model_of(case), items, n_iter=case.n_iter)
    torch.cuda.synchronize()
    _check(case, inp, items)


def test_orbit_of_one_ordering_is_the_compile_bit_for_bit():
    from test_gpu_compile import device_items
    case = cc.small_cases()[0]
    inputs = cc.build(case)
    items, keep = device_items(case, inputs)
    kb.run_compile(model_of(case), items, n_iter=case.n_iter)
    orbit = [kb.OrbitItem(it.n_tokens, it.m, it.canonical, [(it.delta, it.conditioned)],
                          [torch.empty_like(u) for u in it.U], [torch.empty_like(v) for v in it.V])
             for it in items]
    print("[orbit] one ordering vs compile", flush=True)
    kb.run_orbit_compile(model_of(case), orbit, n_iter=case.n_iter)
    torch.cuda.synchronize()
    for ch in range(2):
        assert np.array_equal(_bits(items[0].U[ch]), _bits(orbit[0].U[ch]))
        assert np.array_equal(_bits(items[0].V[ch]), _bits(orbit[0].V[ch]))


def test_orbit_with_sections_per_ordering():
    sec = np.repeat(np.array([0, 1, 2], np.uint8), [16, 24, 24])
    rope = {"pair_section": sec}
    case = cc.Case("orbit_sections", "gqa", "f32", 1, 2, 128, 128, oracle.HALF_SPLIT, 1e6,
                   [cc.ChunkSpec(160, 16, 0)], seed=44)
    deltas = [0, 900, 1800]
    shifts = [(0, 0), (12, -30), (40, 7)]
    # the conditioned KV of ordering k moves section s by shifts[k][s-1] (sections 1, 2)
    orig = cc.oracle_rope

    def rope_k(case_, spec_, ch_, rope_):
        kw = orig(case_, spec_, ch_, rope_)
        if "pair_delta" in kw:
            k = deltas.index(spec_.delta)
            kw["pair_delta"] = oracle.pair_deltas(sec, (spec_.delta, *shifts[k]))
        return kw

    cc.oracle_rope = rope_k
    try:
        inp = cc.build_orbit(case, deltas, rope=rope)
        items = _orbit_items(case, inp, sections=shifts)
        model = kb.make_model(case.family, case.dtype, case.n_layers, case.n_kv_heads,
                              case.head_dim, case.rope_dim, case.layout, case.theta,
                              pair_section=sec)
        print("[orbit] sections", flush=True)
        kb.run_orbit_compile(model, items, n_iter=case.n_iter)
        torch.cuda.synchronize()
        _check(case, inp, items, rope=rope)
    finally:
        cc.oracle_rope = orig


def test_orbit_rank64_at_the_full_head_geometry_sampled_heads():
    """The orbit at the MHA reorder workload's per-head geometry and rank (4096 tokens, 32
    heads x 128, interleaved RoPE, rank 64, three orderings, as the benchmark's orbit leg), on
    one layer: every head's V orthonormal, sampled heads of both channels against the oracle."""
    case = cc.Case("orbit_rank64_full_heads", "gqa", "bf16", 1, 32, 128, 128, oracle.INTERLEAVED,
                   1e4, [cc.ChunkSpec(4096, 64, 0)], seed=44)
    deltas = [0, 4096, 8192]
    inp = cc.build_orbit(case, deltas)
    items = _orbit_items(case, inp)
    print(f"[orbit] case={case.name} members={len(deltas)}", flush=True)
    kb.run_orbit_compile(model_of(case), items, n_iter=case.n_iter)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    worst = 0.0
    for ch in range(2):
        U, V = outputs(case, items, 0, ch)
        assert np.all(np.isfinite(U)) and np.all(np.isfinite(V))
        g = np.einsum("lhfr,lhfs->lhrs", V, V)
        assert np.max(np.abs(g - np.eye(64))) <= 2 * 2.0 ** -8 * 1.02 + 2.0 ** -20
        for h in [0, 31] + [int(x) for x in rng.integers(32, size=2)]:
            e = cc.expected_orbit(case, inp, ch, 0, h)
            r = cc.check_head(U[0, h], V[0, h], e, case.dtype)
            worst = max(worst, r.patch_excess, r.proj_excess)
            assert r.ok, (case.name, ch, h, r)
    print(f"[orbit] {case.name}: worst excess {worst:.3g}", flush=True)
