"""GPU parity: the HIP operator (through the C ABI) against the CPU oracle, every element.

Sizes are cut down in layers and chunks so that the oracle finishes in seconds, while each
case still spans many 16-token tiles, several blocks, ragged tails and page boundaries.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from position_invariant_kv_kamera_amd import binding as kb
from position_invariant_kv_kamera_amd import workloads as wl

from parity import compare_batch, count_sentinel_damage, to_numpy_bits, ulp_bf16, bf16_bits_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def run(op, batch, **kw):
    print(f"[kamera] {op} {batch.plan.name} chunks={batch.plan.n_chunks} "
          f"layers={batch.plan.n_layers}", flush=True)
    ws = kb.run_batch(op, batch, **kw)
    torch.cuda.synchronize()
    return ws


def assert_report(rep, label):
    print(f"[kamera] {label}: {rep.line()}", flush=True)
    assert rep.ok, rep.details


SMALL = {
    "tiny_gqa_f32": lambda: wl.plan("tiny_gqa_f32"),
    "tiny_gqa_f32_ragged": lambda: wl.plan("tiny_gqa_f32", n_layers=2, chunk_tokens=(256, 37, 1)),
    "qwen25vl_gqa_bf16": lambda: wl.plan("qwen25vl_gqa_bf16", n_layers=2,
                                         chunk_tokens=(1296, 1296, 37, 1, 200)),
    "dsv2lite_mla_bf16": lambda: wl.plan("dsv2lite_mla_bf16", n_layers=2,
                                         chunk_tokens=(2048, 300, 17)),
    "dsv2lite_mla_bf16_interleaved": lambda: wl.plan("dsv2lite_mla_bf16", n_layers=2,
                                                     chunk_tokens=(512, 45),
                                                     rope_layout=wl.INTERLEAVED),
    "mha7b_reorder_bf16": lambda: wl.plan("mha7b_reorder_bf16", n_layers=2, n_chunks=3,
                                          chunk_len=512),
    "qwen3vl_window_bf16": lambda: wl.plan("qwen3vl_window_bf16", n_layers=2, n_slots=16,
                                           n_recall=4, max_slide=4),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_reuse_batch_matches_oracle(name):
    batch = wl.materialize(SMALL[name](), DEV)
    run("reuse", batch)
    assert_report(compare_batch(batch, "reuse"), name)


@pytest.mark.parametrize("name", ["qwen25vl_gqa_bf16", "dsv2lite_mla_bf16", "mha7b_reorder_bf16",
                                  "tiny_gqa_f32"])
def test_relocate_matches_oracle_and_copies_bits(name):
    """R(delta) only: keys rotate, values / c_KV come out bit for bit (copy path)."""
    batch = wl.materialize(SMALL[name](), DEV)
    run("relocate", batch)
    rep = compare_batch(batch, "relocate")
    assert_report(rep, name + " relocate")
    assert rep.copies > 0


@pytest.mark.parametrize("name", ["qwen25vl_gqa_bf16", "dsv2lite_mla_bf16", "qwen3vl_window_bf16",
                                  "tiny_gqa_f32"])
def test_relocate_is_reuse_with_rank_zero_bitwise(name):
    a = wl.materialize(SMALL[name](), DEV)
    run("relocate", a)
    b = wl.materialize(SMALL[name](), DEV)
    run("reuse", b, m_override=0)
    for pa, pb in zip(a.pool_storage, b.pool_storage):
        assert torch.equal(pa.view(torch.int16) if pa.dtype == torch.bfloat16 else pa.view(torch.int32),
                           pb.view(torch.int16) if pb.dtype == torch.bfloat16 else pb.view(torch.int32))


@pytest.mark.parametrize("name", ["qwen25vl_gqa_bf16", "mha7b_reorder_bf16", "qwen3vl_window_bf16"])
def test_two_runs_are_bitwise_identical(name):
    a = wl.materialize(SMALL[name](), DEV)
    b = wl.materialize(SMALL[name](), DEV)
    run("reuse", a)
    run("reuse", b)
    for pa, pb in zip(a.pool_storage, b.pool_storage):
        assert torch.equal(pa.view(torch.int16), pb.view(torch.int16))


def _seed_pool_slots(batch, seed=5):
    """Write seeded values into every slot the chunks address; return them per chunk and
    channel as host arrays [layers, L, row]."""
    p = batch.plan
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    inputs = []
    for c in range(p.n_chunks):
        L = p.chunk_tokens[c]
        slots = torch.from_numpy(oracle.slots(p.page_table, p.page_size, p.dst_offsets[c], L)).to(DEV)
        per_ch = []
        for ch in range(2):
            row = p.heads(ch) * p.width(ch)
            vals = torch.randn((p.n_layers, L, row), generator=g, device=DEV).to(batch.pools[ch].dtype)
            for l in range(p.n_layers):
                pool_rows = batch.pools[ch][l].view(-1, batch.pools[ch].shape[-1])
                pool_rows[slots] = vals[l]
            per_ch.append(to_numpy_bits(vals))
        inputs.append(per_ch)
    torch.cuda.synchronize()
    return inputs


@pytest.mark.parametrize("name", ["qwen25vl_gqa_bf16", "dsv2lite_mla_bf16", "tiny_gqa_f32",
                                  "qwen3vl_window_bf16"])
def test_patch_in_place_matches_oracle(name):
    """kamera_patch: dst = round(dst + U V^T), no rotation, on seeded cache contents."""
    batch = wl.materialize(SMALL[name](), DEV)
    inputs = _seed_pool_slots(batch)
    run("patch", batch)
    assert_report(compare_batch(batch, "patch", patch_inputs=inputs), name + " patch")


@pytest.mark.parametrize("name", ["qwen25vl_gqa_bf16", "dsv2lite_mla_bf16"])
def test_relocate_then_patch_within_one_rounding_of_fused(name):
    fused = wl.materialize(SMALL[name](), DEV)
    run("reuse", fused)
    split = wl.materialize(SMALL[name](), DEV)
    run("relocate", split)
    reloc = [t.clone() for t in split.pool_storage]
    run("patch", split)
    for pf, ps, pr in zip(fused.pool_storage, split.pool_storage, reloc):
        a = bf16_bits_to_f64(to_numpy_bits(pf).ravel())
        b = bf16_bits_to_f64(to_numpy_bits(ps).ravel())
        r = bf16_bits_to_f64(to_numpy_bits(pr).ravel())
        live = ~np.isnan(a)
        assert np.array_equal(live, ~np.isnan(b))
        a, b, r = a[live], b[live], r[live]
        # one extra rounding of the relocated value: at most one ulp of the larger operand
        tol = ulp_bf16(np.maximum(np.maximum(np.abs(a), np.abs(b)), np.abs(r)))
        assert np.all(np.abs(a - b) <= tol)


# ----------------------------------------------------------------------------------------
# edge cases and the less common kernel paths
# ----------------------------------------------------------------------------------------

def _variant(base, **kw):
    p = SMALL[base]()
    n = p.n_chunks
    if "m" in kw:
        m = kw.pop("m")
        kw["m_rot"] = [m] * n
        kw["m_plain"] = [m] * n
    return dataclasses.replace(p, **kw)


def _paged(base, page_size, slack=1.25, seed=11, **kw):
    """The base plan written through a shuffled table of pages of `page_size` tokens (sizes
    that are not powers of two take the kernel's division path), 25 % spare pages."""
    p = _variant(base, **kw)
    total = max(o + L for o, L in zip(p.dst_offsets, p.chunk_tokens))
    n_logical = -(-total // page_size)
    n_pages = int(n_logical * slack) + 1
    rng = np.random.Generator(np.random.PCG64(seed))
    table = rng.permutation(n_pages)[:n_logical].astype(np.int32)
    return dataclasses.replace(p, page_size=page_size, n_pages=n_pages, page_table=table,
                               n_logical_pages=n_logical)


EDGE = {
    "rank5_scalar_uv_loads": lambda: _variant("qwen25vl_gqa_bf16", m=5),
    "rank8_partial_kstep": lambda: _variant("qwen25vl_gqa_bf16", m=8),
    "rank64_two_ksteps": lambda: _variant("qwen25vl_gqa_bf16", m=64),
    "rank96_streamed_v": lambda: _variant("qwen25vl_gqa_bf16", m=96),
    "rank256_max": lambda: _variant("qwen25vl_gqa_bf16", m=256, chunk_tokens=[300, 17]),
    "head64_halfsplit": lambda: _variant("qwen25vl_gqa_bf16", head_dim=64, rope_dim=64),
    "head64_interleaved": lambda: _variant("qwen25vl_gqa_bf16", head_dim=64, rope_dim=64,
                                           rope_layout=wl.INTERLEAVED),
    "head96_valu_fallback": lambda: _variant("qwen25vl_gqa_bf16", head_dim=96, rope_dim=96,
                                             chunk_tokens=[300, 17]),
    "mla_fp32_valu": lambda: _variant("dsv2lite_mla_bf16", dtype="f32", chunk_tokens=[100, 33]),
    "one_head_gqa": lambda: _variant("qwen25vl_gqa_bf16", n_kv_heads=1),
    "three_heads": lambda: _variant("qwen25vl_gqa_bf16", n_kv_heads=3),
    "max_abs_delta": lambda: _variant("qwen25vl_gqa_bf16", deltas=[2**31 - 1, -(2**31 - 1), 0, 1, -1]),
    "empty_chunk_in_batch": lambda: _variant("qwen25vl_gqa_bf16", chunk_tokens=[1296, 0, 37, 1, 200]),
    "page12_shuffled": lambda: _paged("qwen25vl_gqa_bf16", 12),
    "page24_reorder_rank64": lambda: _paged("mha7b_reorder_bf16", 24),
    "page1_window": lambda: _paged("qwen3vl_window_bf16", 1),
    "page7_mla": lambda: _paged("dsv2lite_mla_bf16", 7),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases_match_oracle(name):
    p = EDGE[name]()
    if name == "empty_chunk_in_batch":   # keep the destinations disjoint and in range
        p = dataclasses.replace(p, dst_offsets=[0, 1296, 1296, 1333, 1334])
    batch = wl.materialize(p, DEV)
    run("reuse", batch)
    assert_report(compare_batch(batch, "reuse"), name)


def test_zero_chunks_is_a_no_op():
    batch = wl.materialize(SMALL["qwen25vl_gqa_bf16"](), DEV)
    model, cache = kb.model_of(batch.plan), kb.cache_of(batch)
    ws = kb.Workspace(1)
    chunks = (kb.KameraChunk * 1)()
    kb.check(kb.kamera_reuse_batch(model, cache, chunks, 0, ws.ptr, ws.nbytes,
                                   kb.current_stream_ptr()))
    torch.cuda.synchronize()
    assert count_sentinel_damage(batch) == 0
    for pool in batch.pool_storage:
        assert bool((pool.view(torch.int16) == wl.SENTINEL_BF16).all())


def test_out_of_range_page_entries_are_skipped_and_counted():
    """Rows whose table entry points outside the pool are not written, counted instead; all
    other rows are still correct."""
    p = SMALL["mha7b_reorder_bf16"]()
    table = p.page_table.copy()
    n_bad_pages = 2
    bad_logical = [3, 40]                     # logical pages 3 and 40 (chunk placement varies)
    table[bad_logical[0]] = p.n_pages + 5
    table[bad_logical[1]] = -1
    p = dataclasses.replace(p, page_table=table)
    batch = wl.materialize(p, DEV)
    ws = run("reuse", batch)
    st, count = kb.kamera_read_fault_count(ws.ptr, kb.current_stream_ptr())
    assert st == 0
    # each skipped token row is counted once per layer and 128-feature window of each channel
    windows = 2 * p.n_kv_heads * p.head_dim // 128
    assert count == n_bad_pages * p.page_size * windows * p.n_layers
    # chunks that do not touch the bad pages are exact
    clean = [c for c in range(p.n_chunks)
             if not any(p.dst_offsets[c] // 16 <= b < (p.dst_offsets[c] + p.chunk_tokens[c]) // 16
                        for b in bad_logical)]
    assert clean
    rep = compare_batch(batch, "reuse", chunks=clean, check_sentinel=False)
    assert_report(rep, "clean chunks with a damaged table")
    # physical pages that no valid entry points to were never written
    live = {int(table[i]) for i in range(len(table)) if i not in bad_logical}
    dead = torch.tensor([q for q in range(p.n_pages) if q not in live], device=DEV)
    for pool in batch.pool_storage:
        rows = pool.index_select(1, dead)
        assert bool((rows.view(torch.int16) == wl.SENTINEL_BF16).all())


def _first_full_page(p, c):
    """A logical page that chunk c writes from its first slot to its last."""
    lp = -(-p.dst_offsets[c] // p.page_size)
    assert (lp + 1) * p.page_size <= p.dst_offsets[c] + p.chunk_tokens[c]
    return lp


@pytest.mark.parametrize("op", ["reuse", "relocate", "patch"])
@pytest.mark.parametrize("damage", ["out_of_range", "negative", "aliased"])
def test_validate_mode_rejects_a_bad_table_before_enqueueing(monkeypatch, op, damage):
    """KAMERA_VALIDATE=1: a table entry outside the pool, or two written logical pages mapped
    to one physical page, is refused on the host with INVALID_ARGUMENT, and nothing reaches
    the cache."""
    monkeypatch.setenv("KAMERA_VALIDATE", "1")
    p = SMALL["mha7b_reorder_bf16"]()
    table = p.page_table.copy()
    a, b = _first_full_page(p, 0), _first_full_page(p, 1)
    table[b] = {"out_of_range": p.n_pages + 5, "negative": -1, "aliased": table[a]}[damage]
    batch = wl.materialize(dataclasses.replace(p, page_table=table), DEV)
    print(f"[kamera] validate {op} {damage}", flush=True)
    with pytest.raises(kb.KameraError) as err:
        kb.run_batch(op, batch)
    torch.cuda.synchronize()
    assert err.value.status == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert ("outside" if damage != "aliased" else "both write") in str(err.value)
    for pool in batch.pool_storage:
        assert bool((pool.view(torch.int16) == wl.SENTINEL_BF16).all())


def test_validate_mode_passes_a_good_table(monkeypatch):
    """KAMERA_VALIDATE=1 on a valid shuffled table (page size 7, 25 % spare pages): the call
    goes through and matches the oracle, as without the check."""
    monkeypatch.setenv("KAMERA_VALIDATE", "1")
    p = _paged("dsv2lite_mla_bf16", 7)
    batch = wl.materialize(p, DEV)
    run("reuse", batch)
    assert_report(compare_batch(batch, "reuse"), "validated paged MLA")


def test_workspace_reused_across_calls_of_different_sizes():
    big = wl.materialize(SMALL["qwen25vl_gqa_bf16"](), DEV)
    ws = kb.Workspace(big.plan.n_chunks)
    kb.run_batch("reuse", big, workspace=ws)
    small = wl.materialize(wl.plan("qwen25vl_gqa_bf16", n_layers=2, chunk_tokens=(64,)), DEV)
    kb.run_batch("reuse", small, workspace=ws)
    torch.cuda.synchronize()
    assert_report(compare_batch(big, "reuse"), "first call")
    assert_report(compare_batch(small, "reuse"), "second, smaller call")
