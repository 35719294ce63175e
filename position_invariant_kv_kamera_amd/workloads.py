"""Seeded synthetic workloads for the Kamera reuse operator.

This module only draws inputs: canonical KV, patch factors, shifts, destinations and page
tables. It holds none of the operator's arithmetic, imports nothing from the GPU binding or
the oracle, and is the one piece of code both sides share.

The five workloads follow the backbone shapes the Kamera pages name (GQA Qwen-VL family,
MLA DeepSeek-VL/V2 family, MHA) and the three window operations of the technical summary
§3 (reorder, sliding-window survival, recall). The pages use video frames, screenshots and
benchmark suites (MM-NIAH, MileBench, two-page doc-QA); none of those are used: seeded
Gaussian KV of the same shapes stands in for them.

Value recipe (sigma is a standard deviation):
  * canonical K/V (c_KV, k_rope): N(0, 1); the Qwen2.5-VL-like workload multiplies every
    feature by a scale s ~ U[0.5, 2] drawn once per (layer, channel, head, feature);
  * patch factors U, V: N(0, sigma_patch) (0.1 for the tiny fp32 case, 0.05 otherwise);
  * shifts, destinations and page tables: see each plan builder.

Device tensors are drawn with torch's seeded generator on the target device; plan metadata
(shifts, permutations, tables) with numpy's PCG64. Same seed + same device => same bytes.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

GQA, MLA = "gqa", "mla"
HALF_SPLIT, INTERLEAVED = "half_split", "interleaved"
SENTINEL_BF16 = 0x7FC1          # a quiet-NaN bit pattern never produced by the operator
SENTINEL_F32 = 0x7FC00001


@dataclass
class Plan:
    """Everything that defines one batch, except the random tensor contents."""
    name: str
    family: str
    dtype: str                  # "f32" | "bf16"
    n_layers: int
    n_kv_heads: int
    head_dim: int               # GQA: per-head dim; MLA: c_KV width (kv_lora_rank)
    rope_dim: int               # GQA: == head_dim; MLA: k_rope width
    rope_layout: str
    theta: float
    chunk_tokens: list[int]
    deltas: list[int]
    dst_offsets: list[int]      # logical cache token of each chunk's token 0
    m_rot: list[int]            # patch rank on channel 0 (K / k_rope)
    m_plain: list[int]          # patch rank on channel 1 (V / c_KV)
    page_size: int
    n_pages: int                # physical pages per layer in the pool
    page_table: np.ndarray | None   # int32 logical -> physical, None = identity (dense)
    n_logical_pages: int
    seed: int = 0
    kv_channel_scale: bool = False
    patch_sigma: float = 0.05
    notes: dict = field(default_factory=dict)
    # RoPE variants: an explicit frequency table (rope_dim/2 entries), multimodal sections
    # (section index per pair) with per-chunk shifts of sections 1 and 2
    inv_freq: np.ndarray | None = None
    pair_section: np.ndarray | None = None
    n_sections: int = 0
    delta_sections: list | None = None    # per chunk (shift of section 1, of section 2)

    @property
    def n_chunks(self) -> int:
        return len(self.chunk_tokens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.chunk_tokens))

    def width(self, channel: int) -> int:
        """Features per head of channel 0 (rotated) or 1 (plain)."""
        if self.family == MLA:
            return self.rope_dim if channel == 0 else self.head_dim
        return self.head_dim

    def heads(self, channel: int) -> int:
        return 1 if self.family == MLA else self.n_kv_heads

    def row_elems(self) -> int:
        """Elements of one cache row (one token, one layer) per pool."""
        if self.family == MLA:
            return self.head_dim + self.rope_dim
        return self.n_kv_heads * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# ----------------------------------------------------------------------------------------
# plan builders, one per workload
# ----------------------------------------------------------------------------------------

def _dense_layout(chunk_tokens, page_size):
    offs = np.concatenate([[0], np.cumsum(chunk_tokens)[:-1]]).astype(np.int64)
    total = int(np.sum(chunk_tokens))
    n_logical = max(1, -(-total // page_size))
    return [int(o) for o in offs], n_logical


def _shuffled_table(rng, n_logical, n_pages):
    """Distinct physical pages for every logical page, in random order."""
    return rng.permutation(n_pages)[:n_logical].astype(np.int32)


def tiny_gqa_f32(seed=0, n_layers=1, chunk_tokens=(256,), **kw) -> Plan:
    """Tiny GQA, fp32: 1 layer, one 256-token chunk, 2 KV heads x 128, half-split RoPE,
    theta 1e4, delta +1000, rank-8 patch on K and V with U, V ~ N(0, 0.1), dense output."""
    chunk_tokens = list(chunk_tokens)
    offs, n_logical = _dense_layout(chunk_tokens, 16)
    n = len(chunk_tokens)
    p = Plan("tiny_gqa_f32", GQA, "f32", n_layers, 2, 128, 128, HALF_SPLIT, 1e4, chunk_tokens,
             [1000] * n, offs, [8] * n, [8] * n, 16, n_logical, None, n_logical, seed,
             patch_sigma=0.1)
    return dataclasses.replace(p, **kw)


def qwen25vl_gqa_bf16(seed=0, n_layers=28, chunk_tokens=(1296,) * 32, **kw) -> Plan:
    """GQA, Qwen2.5-VL-7B-like, bf16: 28 layers, 4 KV heads x 128, theta 1e6, half-split;
    32 video-frame chunks of 1296 tokens, each delta ~ U{-32768..32768}; rank-16 patches on K
    and V, U, V ~ N(0, 0.05); K, V ~ N(0,1) times a per-feature scale U[0.5, 2]; dense cache,
    chunk c written after chunk c-1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    chunk_tokens = list(chunk_tokens)
    n = len(chunk_tokens)
    deltas = [int(d) for d in rng.integers(-32768, 32768, size=n, endpoint=True)]
    offs, n_logical = _dense_layout(chunk_tokens, 16)
    p = Plan("qwen25vl_gqa_bf16", GQA, "bf16", n_layers, 4, 128, 128, HALF_SPLIT, 1e6,
             chunk_tokens, deltas, offs, [16] * n, [16] * n, 16, n_logical, None, n_logical,
             seed, kv_channel_scale=True)
    return dataclasses.replace(p, **kw)


def dsv2lite_mla_bf16(seed=0, n_layers=27, chunk_tokens=(2048,) * 64, rope_layout=HALF_SPLIT,
                      m=32, **kw) -> Plan:
    """MLA, DeepSeek-V2-Lite-like, bf16: 27 layers, rows of c_KV (512) + k_rope (64), theta
    1e4; 64 chunks of 2048 tokens, delta ~ U{0..65536}; rank-32 patches on both channels,
    U, V ~ N(0, 0.05); dense cache."""
    rng = np.random.Generator(np.random.PCG64(seed))
    chunk_tokens = list(chunk_tokens)
    n = len(chunk_tokens)
    deltas = [int(d) for d in rng.integers(0, 65536, size=n, endpoint=True)]
    offs, n_logical = _dense_layout(chunk_tokens, 16)
    p = Plan("dsv2lite_mla_bf16", MLA, "bf16", n_layers, 1, 512, 64, rope_layout, 1e4,
             chunk_tokens, deltas, offs, [m] * n, [m] * n, 16, n_logical, None, n_logical,
             seed)
    return dataclasses.replace(p, **kw)


def mha7b_reorder_bf16(seed=0, n_layers=32, n_chunks=16, chunk_len=4096, slack=1.25,
                       **kw) -> Plan:
    """MHA, 7B-like, bf16: 32 layers, 32 heads x 128, interleaved RoPE, theta 1e4; 16 chunks of
    4096 tokens with rank-64 patches on K and V. Reorder: chunk c is placed at slot pi(c) of a
    random permutation pi, so it lands at logical token pi(c)*4096 and shifts by the same
    amount from its canonical position 0. Paged cache, page size 16, a shuffled page table
    over a pool with 25 % spare pages that must stay untouched."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pi = rng.permutation(n_chunks)
    offs = [int(pi[c]) * chunk_len for c in range(n_chunks)]
    n_logical = n_chunks * chunk_len // 16
    n_pages = int(n_logical * slack)
    table = _shuffled_table(rng, n_logical, n_pages)
    p = Plan("mha7b_reorder_bf16", GQA, "bf16", n_layers, 32, 128, 128, INTERLEAVED, 1e4,
             [chunk_len] * n_chunks, list(offs), offs, [64] * n_chunks, [64] * n_chunks, 16,
             n_pages, table, n_logical, seed, notes={"permutation": pi.tolist()})
    return dataclasses.replace(p, **kw)


def qwen3vl_window_bf16(seed=0, n_layers=36, n_slots=256, chunk_len=256, n_recall=64,
                        max_slide=64, recall_m=32, slack=1.25, **kw) -> Plan:
    """GQA long-video sliding window, Qwen3-VL-8B-like, bf16: 36 layers, 8 KV heads x 128,
    theta 1e6, half-split. A window of 256 frame-chunks x 256 tokens slides by k ~ U{1..64}
    chunks. A seeded permutation assigns 192 survivors and 64 recalls to the 256 slots.
    Survivor in slot s: its KV sits at old start (s+k)*256 and moves by delta = -k*256, rotation
    only (m = 0). Recall in slot s: canonical chunk at 0, delta = s*256, rank-32 patch on K and
    V. One mixed batch into a paged cache (page size 16, shuffled table, 25 % spare pages)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = int(rng.integers(1, max_slide, endpoint=True))
    slot_of = rng.permutation(n_slots)
    recalled = np.zeros(n_slots, bool)
    recalled[rng.permutation(n_slots)[:n_recall]] = True   # by chunk index
    deltas, offs, m = [], [], []
    for c in range(n_slots):
        s = int(slot_of[c])
        offs.append(s * chunk_len)
        if recalled[c]:
            deltas.append(s * chunk_len)
            m.append(recall_m)
        else:
            deltas.append(-k * chunk_len)
            m.append(0)
    n_logical = n_slots * chunk_len // 16
    n_pages = int(n_logical * slack)
    table = _shuffled_table(rng, n_logical, n_pages)
    p = Plan("qwen3vl_window_bf16", GQA, "bf16", n_layers, 8, 128, 128, HALF_SPLIT, 1e6,
             [chunk_len] * n_slots, deltas, offs, list(m), list(m), 16, n_pages, table,
             n_logical, seed, notes={"slide_k": k, "recalled": recalled.tolist()})
    return dataclasses.replace(p, **kw)


def qwen25vl_mrope_bf16(seed=0, n_layers=28, chunk_tokens=(1296,) * 32, interleaved_map=False,
                        **kw) -> Plan:
    """The Qwen2.5-VL-like batch with multimodal 3-D positions: pairs 0-15 encode time, 16-39
    height, 40-63 width (contiguous sections; or every third pair per component with
    interleaved_map, the map Qwen3-VL uses), and each chunk moves its three components by
    different seeded amounts."""
    p = qwen25vl_gqa_bf16(seed=seed, n_layers=n_layers, chunk_tokens=chunk_tokens)
    rng = np.random.Generator(np.random.PCG64(seed + 101))
    n = len(p.chunk_tokens)
    if interleaved_map:
        sec = np.array([i % 3 for i in range(64)], np.uint8)
    else:
        sec = np.repeat(np.array([0, 1, 2], np.uint8), [16, 24, 24])
    ds = [(int(a), int(b)) for a, b in rng.integers(-4096, 4096, size=(n, 2), endpoint=True)]
    name = "qwen3vl_mrope_bf16" if interleaved_map else "qwen25vl_mrope_bf16"
    return dataclasses.replace(p, name=name, pair_section=sec, n_sections=3, delta_sections=ds,
                               **kw)


def neox_partial_bf16(seed=0, n_layers=4, chunk_tokens=(512,) * 8, rope_dim=64,
                      rope_layout=HALF_SPLIT, **kw) -> Plan:
    """Partial rotary: 8 KV heads x 128 of which the first rope_dim features carry RoPE
    (GPT-NeoX style), theta 1e4, rank-16 patches, dense cache."""
    rng = np.random.Generator(np.random.PCG64(seed))
    chunk_tokens = list(chunk_tokens)
    n = len(chunk_tokens)
    deltas = [int(d) for d in rng.integers(0, 65536, size=n)]
    offs, n_logical = _dense_layout(chunk_tokens, 16)
    p = Plan("neox_partial_bf16", GQA, "bf16", n_layers, 8, 128, rope_dim, rope_layout, 1e4,
             chunk_tokens, deltas, offs, [16] * n, [16] * n, 16, n_logical, None, n_logical, seed)
    return dataclasses.replace(p, **kw)


def scaled_table_bf16(seed=0, n_layers=4, chunk_tokens=(1024,) * 8, dtype="bf16", **kw) -> Plan:
    """An explicit per-pair frequency table (a seeded, decreasing table spanning [1e-6, 1],
    standing in for a model's scaled frequencies), 4 KV heads x 128, rank-16 patches,
    shifts up to 2^20."""
    rng = np.random.Generator(np.random.PCG64(seed))
    chunk_tokens = list(chunk_tokens)
    n = len(chunk_tokens)
    deltas = [int(d) for d in rng.integers(-(1 << 20), 1 << 20, size=n)]
    offs, n_logical = _dense_layout(chunk_tokens, 16)
    table = np.sort(10.0 ** rng.uniform(-6.0, 0.0, size=64))[::-1].copy()
    p = Plan("scaled_table_" + dtype, GQA, dtype, n_layers, 4, 128, 128, HALF_SPLIT, 5e5,
             chunk_tokens, deltas, offs, [16] * n, [16] * n, 16, n_logical, None, n_logical, seed,
             inv_freq=table)
    return dataclasses.replace(p, **kw)


PLANS = {
    "tiny_gqa_f32": tiny_gqa_f32,
    "qwen25vl_gqa_bf16": qwen25vl_gqa_bf16,
    "dsv2lite_mla_bf16": dsv2lite_mla_bf16,
    "mha7b_reorder_bf16": mha7b_reorder_bf16,
    "qwen3vl_window_bf16": qwen3vl_window_bf16,
    "qwen25vl_mrope_bf16": qwen25vl_mrope_bf16,
    "neox_partial_bf16": neox_partial_bf16,
    "scaled_table_bf16": scaled_table_bf16,
}


def plan(name: str, **kw) -> Plan:
    return PLANS[name](**kw)


# ----------------------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------------------

@dataclass
class ChunkTensors:
    src: list            # per channel: tensor [n_layers, L, row_elems_of_that_source] view
    U: list              # per channel: [n_layers, heads, L, m] or None
    V: list              # per channel: [n_layers, heads, width, m] or None


@dataclass
class Batch:
    plan: Plan
    chunks: list         # ChunkTensors per chunk
    pools: list          # per channel: cache pool view [n_layers, n_pages, page_size, row]
    pool_storage: list   # underlying tensors (1 for MLA, 2 for GQA)
    page_table: object   # device int32 tensor or None
    src_storage: list = field(default_factory=list)


def _torch():
    import torch
    return torch


def torch_dtype(plan: Plan):
    torch = _torch()
    return torch.float32 if plan.dtype == "f32" else torch.bfloat16


def sentinel_fill(t):
    """Fill a cache pool with the sentinel NaN bit pattern."""
    torch = _torch()
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(SENTINEL_BF16)
    else:
        t.view(torch.int32).fill_(SENTINEL_F32)
    return t


def materialize(p: Plan, device="cpu") -> Batch:
    """Draw every tensor of the plan on `device` (seeded), and allocate sentinel-filled pools."""
    torch = _torch()
    dt = torch_dtype(p)
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(p.seed * 1000003 + 17)
    L_tot = p.total_tokens

    def randn(shape, sigma=1.0):
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        return x.to(dt)

    chunks = []
    src_storage = []
    if p.family == GQA:
        H, D = p.n_kv_heads, p.head_dim
        scale = None
        if p.kv_channel_scale:
            scale = (torch.rand((2, p.n_layers, 1, H, D), generator=g, device=dev) * 1.5 + 0.5)
        for c, L in enumerate(p.chunk_tokens):
            srcs = []
            for ch in range(2):
                x = torch.randn((p.n_layers, L, H, D), generator=g, device=dev,
                                dtype=torch.float32)
                if scale is not None:
                    x.mul_(scale[ch])
                srcs.append(x.to(dt).view(p.n_layers, L, H * D))
            chunks.append(ChunkTensors(srcs, [None, None], [None, None]))
    else:
        W = p.head_dim + p.rope_dim
        for c, L in enumerate(p.chunk_tokens):
            rows = randn((p.n_layers, L, W))
            # channel 0 (k_rope) starts at element head_dim of each row; channel 1 at 0
            chunks.append(ChunkTensors([rows[:, :, p.head_dim:], rows[:, :, :p.head_dim]],
                                       [None, None], [None, None]))
    for c, L in enumerate(p.chunk_tokens):
        for ch, m in ((0, p.m_rot[c]), (1, p.m_plain[c])):
            if m > 0:
                chunks[c].U[ch] = randn((p.n_layers, p.heads(ch), L, m), p.patch_sigma)
                chunks[c].V[ch] = randn((p.n_layers, p.heads(ch), p.width(ch), m), p.patch_sigma)

    row = p.row_elems()
    shape = (p.n_layers, p.n_pages, p.page_size, row)
    if p.family == GQA:
        storage = [sentinel_fill(torch.empty(shape, dtype=dt, device=dev)) for _ in range(2)]
        pools = storage
    else:
        storage = [sentinel_fill(torch.empty(shape, dtype=dt, device=dev))]
        pools = [storage[0][..., p.head_dim:], storage[0][..., :p.head_dim]]
    table = None
    if p.page_table is not None:
        table = torch.from_numpy(p.page_table.astype(np.int32)).to(dev)
    del L_tot
    return Batch(p, chunks, pools, storage, table, src_storage)
