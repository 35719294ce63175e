"""GPU parity for the RoPE variants of real backbones, through the C ABI, against the oracle
(whose variant arithmetic is pinned to library RoPE in tests/test_oracle_rope_variants.py):
multimodal sections with a different shift per position component (contiguous and
interleaved section maps), partial rotary (MFMA and VALU sub-heads, both pair layouts), an
explicit frequency table (bf16 and fp32), and the patch compile with these variants.
"""
import numpy as np
import pytest
import torch

import oracle
import compile_cases as cc
from position_invariant_kv_kamera_amd import binding as kb
from position_invariant_kv_kamera_amd import workloads as wl

from parity import compare_batch, rope_kwargs, to_numpy_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def run(op, batch):
    print(f"[kamera] {op} {batch.plan.name} chunks={batch.plan.n_chunks} "
          f"layers={batch.plan.n_layers} rope_dim={batch.plan.rope_dim} "
          f"sections={batch.plan.n_sections} table={batch.plan.inv_freq is not None}", flush=True)
    kb.run_batch(op, batch)
    torch.cuda.synchronize()


def assert_report(rep, label):
    print(f"[kamera] {label}: {rep.line()}", flush=True)
    assert rep.ok, rep.details


CASES = {
    "mrope_sections": lambda: wl.plan("qwen25vl_mrope_bf16", n_layers=2,
                                      chunk_tokens=(1296, 200, 37, 1)),
    "mrope_interleaved_map": lambda: wl.plan("qwen25vl_mrope_bf16", n_layers=2,
                                             chunk_tokens=(700, 45), interleaved_map=True),
    "partial_64_of_128": lambda: wl.plan("neox_partial_bf16", n_layers=2,
                                         chunk_tokens=(512, 100, 3)),
    "partial_64_interleaved": lambda: wl.plan("neox_partial_bf16", n_layers=2,
                                              chunk_tokens=(300, 17),
                                              rope_layout=wl.INTERLEAVED),
    "partial_32_of_128_valu": lambda: wl.plan("neox_partial_bf16", n_layers=2,
                                              chunk_tokens=(256, 9), rope_dim=32),
    "scaled_table_bf16": lambda: wl.plan("scaled_table_bf16", n_layers=2,
                                         chunk_tokens=(1024, 77)),
    "scaled_table_f32": lambda: wl.plan("scaled_table_bf16", n_layers=2, chunk_tokens=(256, 33),
                                        dtype="f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_variant_reuse_matches_oracle(name):
    batch = wl.materialize(CASES[name](), DEV)
    run("reuse", batch)
    assert_report(compare_batch(batch, "reuse"), name)


@pytest.mark.parametrize("name", ["partial_64_of_128", "partial_32_of_128_valu"])
def test_partial_rotary_passes_features_through_bit_for_bit(name):
    """Relocation only: the features past rope_dim of every key head keep their bits."""
    batch = wl.materialize(CASES[name](), DEV)
    run("relocate", batch)
    p = batch.plan
    assert_report(compare_batch(batch, "relocate"), name + " relocate")
    R, W = p.rope_dim, p.head_dim
    for c in range(p.n_chunks):
        L = p.chunk_tokens[c]
        slots = torch.from_numpy(oracle.slots(None, p.page_size, p.dst_offsets[c], L)).to(DEV)
        for l in range(p.n_layers):
            got = to_numpy_bits(batch.pools[0][l].reshape(-1, p.n_kv_heads * W).index_select(0, slots))
            src = to_numpy_bits(batch.chunks[c].src[0][l])
            for h in range(p.n_kv_heads):
                assert np.array_equal(got[:, h * W + R:(h + 1) * W], src[:, h * W + R:(h + 1) * W])


def test_sections_with_equal_shifts_equal_plain_relocation():
    """All three components moved alike = plain RoPE relocation, bit for bit."""
    a = wl.plan("qwen25vl_mrope_bf16", n_layers=1, chunk_tokens=(300, 64))
    a.delta_sections = [(d, d) for d in a.deltas]
    b = wl.plan("qwen25vl_gqa_bf16", n_layers=1, chunk_tokens=(300, 64))
    ba, bb = wl.materialize(a, DEV), wl.materialize(b, DEV)
    run("reuse", ba)
    run("reuse", bb)
    for ch in range(2):
        assert torch.equal(ba.pools[ch].view(torch.int16), bb.pools[ch].view(torch.int16))


# ---- patch compile with the variants ----------------------------------------------------

def _compile_variant(case, rope):
    """Build compile inputs whose conditioned KV is relocated with the variant (oracle), run
    kamera_patch_compile with the same variant, and check every head."""
    from test_gpu_compile import device_items, outputs
    inputs = cc.build(case, rope=rope)
    items, keep = device_items(case, inputs)
    for it, spec in zip(items, case.chunks):
        it.delta_sections = spec.delta_sections or (spec.delta, spec.delta)
    model = kb.make_model(case.family, case.dtype, case.n_layers, case.n_kv_heads,
                          case.head_dim, case.rope_dim, case.layout, case.theta,
                          inv_freq=rope.get("inv_freq"),
                          pair_section=rope.get("pair_section"))
    print(f"[compile] variant case={case.name} rope={sorted(rope)}", flush=True)
    kb.run_compile(model, items, n_iter=case.n_iter)
    torch.cuda.synchronize()
    for ch in range(2):
        H, W, _ = case.geometry(ch)
        U, V = outputs(case, items, 0, ch)
        for l in range(case.n_layers):
            for h in range(H):
                e = cc.expected(case, inputs, 0, ch, l, h, rope=rope)
                r = cc.check_head(U[l, h], V[l, h], e, case.dtype)
                assert r.ok, (case.name, ch, l, h, r)


def test_compile_with_partial_rotary():
    case = cc.Case("partial_compile", "gqa", "bf16", 2, 2, 128, 64, oracle.HALF_SPLIT, 1e4,
                   [cc.ChunkSpec(300, 16, 999)], seed=21)
    _compile_variant(case, {})


@pytest.mark.parametrize("head_dim,rope_dim,layout", [
    (128, 96, oracle.HALF_SPLIT),     # pairs (i, i + 48): pieces paired across lane groups
    (128, 32, oracle.HALF_SPLIT),
    (64, 32, oracle.HALF_SPLIT),
    (128, 32, oracle.INTERLEAVED),
    (128, 48, oracle.INTERLEAVED),    # three whole 16-feature groups turn, five pass through
])
def test_compile_with_partial_rotary_other_widths(head_dim, rope_dim, layout):
    case = cc.Case(f"partial_{rope_dim}_of_{head_dim}_{layout}", "gqa", "bf16", 2, 2, head_dim,
                   rope_dim, layout, 1e4,
                   [cc.ChunkSpec(333, 16, -4321), cc.ChunkSpec(40, 32, 77)], seed=23)
    _compile_variant(case, {})


def test_compile_with_sections_and_table():
    sec = np.repeat(np.array([0, 1, 2], np.uint8), [16, 24, 24])
    table = np.sort(10.0 ** np.random.default_rng(3).uniform(-6, 0, 64))[::-1].copy()
    case = cc.Case("sections_table_compile", "gqa", "f32", 1, 2, 128, 128, oracle.HALF_SPLIT,
                   1e6, [cc.ChunkSpec(260, 16, 1500, delta_sections=(-20, 333))], seed=22)
    _compile_variant(case, {"pair_section": sec, "inv_freq": table})
