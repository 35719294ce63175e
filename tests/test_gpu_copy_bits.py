"""GPU: channels that are neither rotated nor patched move bit for bit, on the bit patterns that
tell a copy from a float round trip.

The technical summary (§2, "Unified Architecture Support") reuses MLA's c_KV byte for byte;
sliding-window survivors (§3) keep their values as they are. A float load, add and store
would turn -0.0 + 0.0 into +0.0, quiet signalling NaNs, drop NaN payloads or flush
subnormals; Gaussian test data cannot show any of that. Here the sources of the copied
channels hold every one of the 65,536 bf16 bit patterns (-0.0, subnormals, +-inf, quiet and
signalling NaNs with payloads), or, for fp32, the IEEE special values and random bit patterns,
and the output bits must equal the input bits. The other channel of the same call still
matches the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from position_invariant_kv_kamera_amd import binding as kb
from position_invariant_kv_kamera_amd import workloads as wl

from parity import compare_batch, count_sentinel_damage, record, Report

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def all_bf16_patterns(n: int, seed: int) -> np.ndarray:
    """n bf16 bit patterns (int16 view): every one of the 65,536 patterns, in a seeded order,
    repeated to length n (n >= 65,536 so each appears at least once)."""
    assert n >= 1 << 16
    rng = np.random.Generator(np.random.PCG64(seed))
    reps = -(-n // (1 << 16))
    pats = np.concatenate([rng.permutation(1 << 16) for _ in range(reps)])[:n]
    return pats.astype(np.uint16).view(np.int16)


def fp32_specials(n: int, seed: int) -> np.ndarray:
    """n fp32 bit patterns (int32 view): the IEEE special values (+-0, +-inf, quiet and
    signalling NaNs with payloads, subnormals, extreme normals) interleaved with random bit
    patterns."""
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000,
                        0x7FC00001, 0x7FFFFFFF, 0xFFFFFFFF, 0x7F800001, 0xFF800001, 0x7FA5A5A5,
                        0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00400000, 0x00800000,
                        0x80800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x3F800000, 0xBF800000, 0x7FC1 << 16],
                       dtype=np.uint32)
    rng = np.random.Generator(np.random.PCG64(seed))
    out = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    pos = rng.permutation(n)[: min(n, 64 * special.size)]
    out[pos] = np.resize(special, pos.size)
    return out.view(np.int32)


def fill_bits(t: torch.Tensor, bits: np.ndarray) -> None:
    """Overwrite the elements of t (a contiguous bf16 or fp32 view) with the given bit patterns."""
    iv = t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
    iv.copy_(torch.from_numpy(np.ascontiguousarray(bits[: iv.numel()])).view(iv.shape).to(t.device))


def fill_channel(batch: wl.Batch, ch: int, kind: str, seed: int, chunks=None) -> int:
    """Give channel ch of the chosen chunks adversarial source bits; returns elements filled."""
    filled = 0
    for c in (range(batch.plan.n_chunks) if chunks is None else chunks):
        src = batch.chunks[c].src[ch]
        if src.numel() == 0:
            continue
        n = max(src.numel(), 1 << 16)
        bits = all_bf16_patterns(n, seed + c) if kind == "bf16" else fp32_specials(n, seed + c)
        if src.is_contiguous():
            fill_bits(src, bits)
        else:   # MLA: c_KV is a strided view into the shared rows
            tmp = torch.empty(src.shape, dtype=src.dtype, device=src.device)
            fill_bits(tmp, bits)
            src.copy_(tmp)   # same dtype: a bit copy
        filled += src.numel()
    torch.cuda.synchronize()
    return filled


def patterns_seen(batch: wl.Batch, ch: int, chunks) -> int:
    """Distinct bf16 patterns among the chosen chunks' channel ch sources."""
    seen = set()
    for c in chunks:
        seen.update(np.unique(batch.chunks[c].src[ch].contiguous().view(torch.int16)
                              .cpu().numpy()).tolist())
    return len(seen)


def copy_report(batch: wl.Batch, ch: int, chunks, feats=None) -> Report:
    """Bitwise check of channel ch (features `feats` of every head, default all) of the chosen
    chunks, read back through the page table."""
    p = batch.plan
    rep = Report()
    for c in chunks:
        L = p.chunk_tokens[c]
        if L == 0:
            continue
        slots = torch.from_numpy(oracle.slots(p.page_table, p.page_size, p.dst_offsets[c], L)).to(DEV)
        for l in range(p.n_layers):
            pool = batch.pools[ch][l]
            got = pool.reshape(-1, pool.shape[-1]).index_select(0, slots)
            src = batch.chunks[c].src[ch][l]
            if feats is not None:
                W = p.width(ch)
                idx = torch.tensor([h * W + f for h in range(p.heads(ch)) for f in feats], device=DEV)
                got, src = got.index_select(1, idx), src.index_select(1, idx)
            iv = torch.int16 if got.dtype == torch.bfloat16 else torch.int32
            diff = int((got.contiguous().view(iv) != src.contiguous().view(iv)).sum().item())
            rep.elements += got.numel()
            rep.copies += got.numel()
            rep.copy_mismatches += diff
            if diff:
                rep.details.append(f"chunk {c} layer {l}: {diff} copied elements differ")
    return record(rep, f"{p.name} channel {ch} bit copy")


def run(op, batch, **kw):
    print(f"[kamera] {op} {batch.plan.name} chunks={batch.plan.n_chunks} layers={batch.plan.n_layers}",
          flush=True)
    kb.run_batch(op, batch, **kw)
    torch.cuda.synchronize()


def check(rep: Report, label: str):
    print(f"[kamera] {label}: {rep.line()}", flush=True)
    assert rep.ok, rep.details


@pytest.mark.parametrize("op", ["relocate", "reuse_rot_patch_only"])
def test_mla_c_kv_moves_every_bf16_pattern_bit_for_bit(op):
    """MLA at the DeepSeek-V2-Lite-like geometry (2 layers, ragged chunks): c_KV holds all
    65,536 bf16 patterns; with no c_KV patch (relocation, or a reuse that patches only k_rope)
    it comes out bit for bit, and k_rope matches the oracle."""
    p = wl.plan("dsv2lite_mla_bf16", n_layers=2, chunk_tokens=(2048, 300, 17))
    if op != "relocate":
        p = dataclasses.replace(p, m_plain=[0] * p.n_chunks)
    batch = wl.materialize(p, DEV)
    n = fill_channel(batch, 1, "bf16", seed=101)
    assert patterns_seen(batch, 1, range(p.n_chunks)) == 1 << 16
    run("relocate" if op == "relocate" else "reuse", batch)
    check(copy_report(batch, 1, range(p.n_chunks)), f"c_KV {op}: {n} patterned elements")
    rot = compare_batch(batch, "relocate" if op == "relocate" else "reuse", check_sentinel=True)
    check(rot, f"k_rope {op} (c_KV copies included)")


def test_window_survivor_values_move_every_bf16_pattern_bit_for_bit():
    """The sliding-window batch (Qwen3-VL-like heads, paged, shuffled): every survivor's V holds
    all 65,536 bf16 patterns and is moved bit for bit in the same launch that rotates the
    survivors' keys and patches the recalled chunks."""
    p = wl.plan("qwen3vl_window_bf16", n_layers=2, n_slots=16, n_recall=4, max_slide=4)
    batch = wl.materialize(p, DEV)
    survivors = [c for c in range(p.n_chunks) if p.m_plain[c] == 0]
    assert survivors and len(survivors) < p.n_chunks
    fill_channel(batch, 1, "bf16", seed=202, chunks=survivors)
    assert patterns_seen(batch, 1, survivors) == 1 << 16
    run("reuse", batch)
    check(copy_report(batch, 1, survivors), "survivor V copies")
    check(compare_batch(batch, "reuse"), "whole window batch (survivor V as copies)")


def test_gqa_relocate_values_move_every_bf16_pattern_bit_for_bit():
    """Relocation of the Qwen2.5-VL-like heads: V (all 65,536 patterns) comes out bit for bit."""
    p = wl.plan("qwen25vl_gqa_bf16", n_layers=2, chunk_tokens=(1296, 37, 1, 200))
    batch = wl.materialize(p, DEV)
    fill_channel(batch, 1, "bf16", seed=303)
    run("relocate", batch)
    check(compare_batch(batch, "relocate"), "relocate, patterned V")


def test_valu_path_bf16_copy_every_pattern():
    """A head width the MFMA path does not take (96): the VALU kernel's copy of V."""
    p = wl.plan("qwen25vl_gqa_bf16", n_layers=2, chunk_tokens=(300, 17), head_dim=96, rope_dim=96)
    batch = wl.materialize(p, DEV)
    fill_channel(batch, 1, "bf16", seed=404)
    assert patterns_seen(batch, 1, range(p.n_chunks)) == 1 << 16
    run("relocate", batch)
    check(compare_batch(batch, "relocate"), "VALU bf16 relocate, patterned V")


@pytest.mark.parametrize("op", ["relocate", "reuse_m0"])
def test_valu_path_fp32_copy_special_values(op):
    """fp32 (the tiny GQA shape, 2 layers, ragged chunks): V holds the IEEE special values and
    random bit patterns; relocation and a rank-0 reuse move them bit for bit."""
    p = wl.plan("tiny_gqa_f32", n_layers=2, chunk_tokens=(256, 37, 1))
    batch = wl.materialize(p, DEV)
    fill_channel(batch, 1, "f32", seed=505)
    if op == "relocate":
        run("relocate", batch)
    else:
        run("reuse", batch, m_override=0)
    check(compare_batch(batch, "relocate"), f"fp32 {op}, special V values")


def test_partial_rotary_pass_through_features_every_bf16_pattern():
    """GPT-NeoX-style partial rotary (rope_dim 64 of 128): the key features past rope_dim pass
    through R(delta) unchanged; under relocation they are a bit copy of every bf16 pattern,
    while the rotated features match the oracle."""
    p = wl.plan("neox_partial_bf16", n_layers=2, chunk_tokens=(512, 45))
    batch = wl.materialize(p, DEV)
    W, R = p.head_dim, p.rope_dim
    # patterns in the pass-through features of every key head; the rotated part stays Gaussian
    for c in range(p.n_chunks):
        k = batch.chunks[c].src[0].view(p.n_layers, -1, p.n_kv_heads, W)
        n = k[..., R:].numel()
        tmp = torch.empty(k[..., R:].shape, dtype=k.dtype, device=DEV)
        fill_bits(tmp, all_bf16_patterns(max(n, 1 << 16), 606 + c))
        k[..., R:].copy_(tmp)
    torch.cuda.synchronize()
    run("relocate", batch)
    check(copy_report(batch, 0, range(p.n_chunks), feats=range(R, W)), "pass-through features")
    # rotated features: the oracle, over the first rope_dim features of every head
    ref = wl.materialize(p, DEV)          # same seed: the same Gaussian rotated features
    run("relocate", ref)
    for l in range(p.n_layers):
        a = batch.pools[0][l].reshape(-1, p.n_kv_heads, W)[..., :R]
        b = ref.pools[0][l].reshape(-1, p.n_kv_heads, W)[..., :R]
        assert torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
    check(compare_batch(ref, "relocate"), "partial rotary relocate (Gaussian reference)")
    assert count_sentinel_damage(batch) == 0
