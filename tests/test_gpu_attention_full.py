"""Decode attention and attention over chunks read in place at the benchmark's full size, in
the launch configuration bench.py times, checked on sampled queries against the fp64 oracle
(oracle/attention.py).

GQA: 64 sequences x 16384 tokens, 4 KV heads x 128, 28 query heads, paged 16 over a shuffled
table (2048-token segments on 512 whole-row blocks). MLA: 64 sequences x 16384 tokens, rows
[c_KV 512 | k_rope 64], 16 query heads, paged 16 shuffled (512-token segments). Inputs follow
the benchmark's seeded recipe. Every query of the call is computed on the GPU; three of them
(first, middle, last) are compared head by head with the oracle under the derived tolerance of
test_gpu_attention.py, their rows gathered from the device pools through the page table.
Chunks: 64 sequences x 16 chunks x 1024 tokens with rank-16 patches, checked the same way
under test_gpu_chunk_attention.py's tolerance.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from position_invariant_kv_kamera_amd import binding as kb
from test_gpu_attention import _bits_to_f64, _expect, check_mla_query

pytestmark = pytest.mark.gpu

N_SEQ, CTX, PS = 64, 16384, 16
SAMPLES = (0, 29, 63)


class PagedRows:
    """The rows of a one-layer paged pool, fetched from the device on demand (fp64 on the
    host), in the interface _expect uses (D, n_kv, rows)."""

    def __init__(self, pools, table, n_kv, D):
        self.pools, self.table = pools, table
        self.n_kv, self.D = n_kv, D

    def rows(self, layer, ch, start, n):
        p = np.arange(start, start + n)
        phys = torch.from_numpy(self.table[p // PS].astype(np.int64)).cuda()
        slot = torch.from_numpy(p % PS).cuda()
        return _bits_to_f64(self.pools[ch][layer][phys, slot])


def test_full_size_decode_attention_sampled_queries():
    n_kv, D, n_q = 4, 128, 28
    n_pages = N_SEQ * CTX // PS
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    row = n_kv * D
    pools = [torch.randn((1, n_pages, PS, row), generator=g, device="cuda").to(torch.bfloat16)
             for _ in range(2)]
    table = np.random.default_rng(77).permutation(n_pages).astype(np.int32)
    table_dev = torch.from_numpy(table).cuda()
    model = kb.make_model("gqa", "bf16", 1, n_kv, D, D, "half_split", 1e6)
    cache = kb.KameraCache()
    cache.pool[0], cache.pool[1] = pools[0].data_ptr(), pools[1].data_ptr()
    cache.layer_stride = pools[0].stride(0)
    cache.token_stride = row
    cache.page_table = table_dev.data_ptr()
    cache.n_logical_pages = n_pages
    cache.page_size = PS
    cache.n_pages = n_pages
    q = torch.randn((N_SEQ, n_q, D), generator=g, device="cuda").to(torch.bfloat16)
    ranges = [(i * CTX, CTX) for i in range(N_SEQ)]
    scale = 1.0 / math.sqrt(D)
    print(f"[attn-full] gqa {N_SEQ} x {CTX} tokens, {n_kv} KV heads, {n_q} query heads", flush=True)
    out, lse = kb.run_decode_attention(model, cache, 0, q, ranges, scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    q64 = _bits_to_f64(q)
    src = PagedRows(pools, table, n_kv, D)
    worst = 0.0
    for j in SAMPLES:
        a, n = ranges[j]
        o, l, otol, ltol = _expect(src, 0, q64[j], a, n, n_q, scale)
        err = np.abs(out[j] - o)
        assert np.all(err <= otol + 1e-30), (j, float((err / (otol + 1e-30)).max()))
        lerr = np.abs(lse[j] - l)
        assert np.all(lerr <= ltol), (j, float((lerr / ltol).max()))
        worst = max(worst, float((err / (otol + 1e-30)).max()), float((lerr / ltol).max()))
    print(f"[attn-full] gqa worst error / tolerance {worst:.3g}", flush=True)


def test_full_size_mla_decode_attention_sampled_queries():
    n_q = 16
    n_pages = N_SEQ * CTX // PS
    g = torch.Generator(device="cuda")
    g.manual_seed(79)
    rows = torch.randn((1, n_pages, PS, 576), generator=g, device="cuda").to(torch.bfloat16)
    table = np.random.default_rng(79).permutation(n_pages).astype(np.int32)
    table_dev = torch.from_numpy(table).cuda()
    model = kb.make_model("mla", "bf16", 1, 1, 512, 64, "half_split", 1e4)
    cache = kb.KameraCache()
    cache.pool[1], cache.pool[0] = rows.data_ptr(), rows.data_ptr() + 512 * 2
    cache.layer_stride = rows.stride(0)
    cache.token_stride = 576
    cache.page_table = table_dev.data_ptr()
    cache.n_logical_pages = n_pages
    cache.page_size = PS
    cache.n_pages = n_pages
    q = torch.randn((N_SEQ, n_q, 576), generator=g, device="cuda").to(torch.bfloat16)
    ranges = [(i * CTX, CTX) for i in range(N_SEQ)]
    scale = 1.0 / math.sqrt(576)
    print(f"[attn-full] mla {N_SEQ} x {CTX} tokens, {n_q} query heads", flush=True)
    out, lse = kb.run_decode_attention(model, cache, 0, q, ranges, scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    q64 = _bits_to_f64(q)
    worst = 0.0
    for j in SAMPLES:
        a, n = ranges[j]
        p = np.arange(a, a + n)
        phys = torch.from_numpy(table[p // PS].astype(np.int64)).cuda()
        slot = torch.from_numpy(p % PS).cuda()
        K = _bits_to_f64(rows[0][phys, slot])
        worst = max(worst, check_mla_query(q64[j], K, K[:, :512], n, scale, out[j], lse[j], j))
    print(f"[attn-full] mla worst error / tolerance {worst:.3g}", flush=True)


class _SampledChunks:
    """The case interface test_gpu_chunk_attention._check reads, over the chunks of the sampled
    queries only (spans renumbered into that list)."""

    def __init__(self, K, V, UK, VK, UV, VV, deltas, samples, n_ck, n_kv, D, G):
        self.D, self.G, self.n_kv, self.R = D, G, n_kv, D
        self.layout, self.theta = oracle.HALF_SPLIT, 1e6   # as the model below
        self.inv_freq = self.pair_section = None
        self.spans = [(k * n_ck, n_ck) for k in range(len(samples))]
        self.ids = [j * n_ck + c for j in samples for c in range(n_ck)]
        self.t = dict(K=K, V=V, UK=UK, VK=VK, UV=UV, VV=VV)
        self.deltas = deltas

    def oracle_chunks(self, layer, h):
        from test_gpu_chunk_attention import _bits
        D, t = self.D, self.t
        res = []
        for c in self.ids:
            res.append({"K": _bits(t["K"][c, layer, :, h * D:(h + 1) * D]),
                        "V": _bits(t["V"][c, layer, :, h * D:(h + 1) * D]),
                        "delta": int(self.deltas[c]),
                        "section_delta": np.array([int(self.deltas[c])] * 3, np.int64),
                        "Uk": _bits(t["UK"][c, layer, h]), "Vk": _bits(t["VK"][c, layer, h]),
                        "Uv": _bits(t["UV"][c, layer, h]), "Vv": _bits(t["VV"][c, layer, h])})
        return res


def test_full_size_chunk_attention_sampled_queries():
    """Attention over chunks read in place at the benchmark's size (64 sequences x 16 chunks
    x 1024 tokens, 4 KV heads x 128, 28 query heads, rank-16 patches; whole-row blocks over
    whole chunks), the benchmark's seeded recipe, three queries checked head by head."""
    from test_gpu_chunk_attention import _check
    n_seq, n_ck, T, n_kv, D, n_q, m = N_SEQ, 16, 1024, 4, 128, 28, 16
    n_chunks = n_seq * n_ck
    row = n_kv * D
    g = torch.Generator(device="cuda")
    g.manual_seed(78)
    K = torch.randn((n_chunks, T, row), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((n_chunks, T, row), generator=g, device="cuda").to(torch.bfloat16)
    UK, UV = [(0.05 * torch.randn((n_chunks, n_kv, T, m), generator=g, device="cuda"))
              .to(torch.bfloat16) for _ in range(2)]
    VK, VV = [(0.05 * torch.randn((n_chunks, n_kv, D, m), generator=g, device="cuda"))
              .to(torch.bfloat16) for _ in range(2)]
    deltas = np.random.default_rng(78).integers(0, 65536, n_chunks)
    es = 2
    items = []
    for c in range(n_chunks):
        items.append({"n_tokens": T, "delta": int(deltas[c]),
                      "src": [(K.data_ptr() + c * K.stride(0) * es, K.stride(0), row),
                              (V.data_ptr() + c * V.stride(0) * es, V.stride(0), row)],
                      "patch": [(m, UK.data_ptr() + c * UK.stride(0) * es, UK.stride(0),
                                 UK.stride(1), VK.data_ptr() + c * VK.stride(0) * es,
                                 VK.stride(0), VK.stride(1)),
                                (m, UV.data_ptr() + c * UV.stride(0) * es, UV.stride(0),
                                 UV.stride(1), VV.data_ptr() + c * VV.stride(0) * es,
                                 VV.stride(0), VV.stride(1))]})
    model = kb.make_model("gqa", "bf16", 1, n_kv, D, D, "half_split", 1e6)
    q = torch.randn((n_seq, n_q, D), generator=g, device="cuda").to(torch.bfloat16)
    spans = [(s * n_ck, n_ck) for s in range(n_seq)]
    scale = 1.0 / math.sqrt(D)
    print(f"[attn-full] chunks {n_seq} x {n_ck} x {T} tokens, rank {m}", flush=True)
    out, lse = kb.run_chunk_attention(model, 0, items, spans, q, scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    sel = list(SAMPLES)
    case = _SampledChunks(K[:, None], V[:, None], UK[:, None], VK[:, None], UV[:, None],
                          VV[:, None], deltas, sel, n_ck, n_kv, D, n_q // n_kv)
    _check(case, 0, q[sel], scale, out[sel], lse[sel])
