"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The oracle computes sampled rows one by one; properties that hold at any size are checked on
every element: copies are bit-exact, untouched pool slots keep the sentinel, and every chunk
token lands at its page-table slot.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from position_invariant_kv_kamera_amd import binding as kb
from position_invariant_kv_kamera_amd import workloads as wl

from parity import count_sentinel_damage, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def copies_exact(batch, op) -> tuple[int, int]:
    """Every element of every unpatched plain channel (values / c_KV) equals its input bits.
    Returns (rows checked, rows that differ)."""
    p = batch.plan
    checked = bad = 0
    for c in range(p.n_chunks):
        if op == "reuse" and p.m_plain[c] > 0:
            continue
        L = p.chunk_tokens[c]
        slots = torch.from_numpy(oracle.slots(p.page_table, p.page_size, p.dst_offsets[c], L)).to(DEV)
        for l in range(p.n_layers):
            pool = batch.pools[1][l]
            got = pool.view(-1, pool.shape[-1]).index_select(0, slots)
            src = batch.chunks[c].src[1][l]
            same = (got.view(torch.int16) == src.view(torch.int16)).all(dim=1)
            checked += L
            bad += int((~same).sum().item())
    return checked, bad


@pytest.mark.parametrize("name", ["tiny_gqa_f32", "qwen25vl_gqa_bf16", "dsv2lite_mla_bf16",
                                  "qwen3vl_window_bf16", "mha7b_reorder_bf16"])
def test_full_size_sampled_rows_and_properties(name):
    p = wl.plan(name)
    print(f"[kamera] full-size {name}: {p.n_chunks} chunks x {p.chunk_tokens[0]} tokens, "
          f"{p.n_layers} layers", flush=True)
    batch = wl.materialize(p, DEV)
    kb.run_batch("reuse", batch)
    torch.cuda.synchronize()
    rep = sample_rows(batch, 1500, seed=11)
    print(f"[kamera] sampled: {rep.line()}", flush=True)
    assert rep.ok, rep.details
    assert count_sentinel_damage(batch) == 0
    if p.dtype == "bf16":
        checked, bad = copies_exact(batch, "reuse")
        print(f"[kamera] bit-exact copies: {checked} rows checked, {bad} differ", flush=True)
        assert bad == 0
        if name == "qwen3vl_window_bf16":
            assert checked == 192 * 256 * p.n_layers          # every survivor's values


@pytest.mark.parametrize("name", ["dsv2lite_mla_bf16", "qwen25vl_gqa_bf16"])
def test_full_size_relocate_copies_plain_channel_bits(name):
    """MLA c_KV (and GQA values) are reused byte for byte by R(delta), at full size."""
    p = wl.plan(name)
    batch = wl.materialize(p, DEV)
    kb.run_batch("relocate", batch)
    torch.cuda.synchronize()
    checked, bad = copies_exact(batch, "relocate")
    print(f"[kamera] {name} relocate: {checked} rows checked, {bad} differ", flush=True)
    assert checked == p.total_tokens * p.n_layers and bad == 0
    rep = sample_rows(batch, 500, seed=12, op="relocate")
    assert rep.ok, rep.details
