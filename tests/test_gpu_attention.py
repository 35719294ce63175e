"""Decode attention over the paged cache and the state merge on the GPU (through the C ABI)
against the fp64 oracle (oracle/attention.py).

The cache is filled directly with seeded bf16 values (the attention reads whatever the
relocation wrote; its own inputs do not come from the HIP path here).

Tolerance (derived): the scores' products are exact (bf16 x bf16) and summed in fp32 over D
terms, then scaled by fl(scale log2 e) (the kernels work in base 2: two roundings), so
|ds_t| <= eps_s = 2 D 2^-24 max_t(scale sum_d |q_d k_td|) + 2 2^-24 max|s|; the
softmax weights then carry a relative error <= 2 eps_s + c u (u = 2^-24, c = 64 + number of
16-token tiles for the fp32 exp, running sums and the merges), so
    |o_g - o|_f <= (2 eps_s + c u) sum_t w_t |v_tf|,   |lse_g - lse| <= eps_s + c u (1 + |lse|).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from position_invariant_kv_kamera_amd import binding as kb

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _bits_to_f64(t):
    b = t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Setup:
    def __init__(self, n_layers=2, n_kv=4, D=128, page_size=16, n_pages=320, n_logical=300,
                 shuffled=True, bad_pages=(), seed=0):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        self.D, self.n_kv, self.ps = D, n_kv, page_size
        row = n_kv * D
        self.pools = [torch.randn((n_layers, n_pages, page_size, row), generator=g,
                                  device="cuda").to(torch.bfloat16) for _ in range(2)]
        rng = np.random.default_rng(seed)
        self.table = None
        if shuffled:
            t = rng.permutation(n_pages)[:n_logical].astype(np.int32)
            for b in bad_pages:
                t[b] = n_pages + 3                      # outside the pool: masked
            self.table = t
            self.table_dev = torch.from_numpy(t).cuda()
        self.model = kb.make_model("gqa", "bf16", n_layers, n_kv, D, D, "half_split", 1e6)
        c = kb.KameraCache()
        c.pool[0] = self.pools[0].data_ptr()
        c.pool[1] = self.pools[1].data_ptr()
        c.layer_stride = self.pools[0].stride(0)
        c.token_stride = row
        c.page_table = None if self.table is None else self.table_dev.data_ptr()
        c.n_logical_pages = n_logical
        c.page_size = page_size
        c.n_pages = n_pages
        self.cache = c
        self.host = [_bits_to_f64(p) for p in self.pools]      # [L, pages, ps, row]
        self.n_pages = n_pages

    def rows(self, layer, ch, start, n):
        """Rows of logical tokens [start, start + n) whose page is inside the pool."""
        p = np.arange(start, start + n)
        page, slot = p // self.ps, p % self.ps
        phys = page if self.table is None else self.table[page].astype(np.int64)
        ok = (phys >= 0) & (phys < self.n_pages)
        return self.host[ch][layer][phys[ok], slot[ok]]


def _expect(setup, layer, q64, start, n, n_q, scale):
    """Oracle (o, lse, o_tol, lse_tol) for one query: q64 [n_q, D]."""
    D, G = setup.D, n_q // setup.n_kv
    K, V = setup.rows(layer, 0, start, n), setup.rows(layer, 1, start, n)
    o = np.zeros((n_q, D))
    lse = np.full(n_q, -np.inf)
    otol = np.zeros((n_q, D))
    ltol = np.zeros(n_q)
    tiles = -(-max(n, 1) // 16)
    c = 64 + tiles
    for h in range(setup.n_kv):
        qh = q64[h * G:(h + 1) * G]
        Kh, Vh = K[:, h * D:(h + 1) * D], V[:, h * D:(h + 1) * D]
        oh, lh = att.decode_attention(qh, Kh, Vh, scale)
        o[h * G:(h + 1) * G], lse[h * G:(h + 1) * G] = oh, lh
        if Kh.shape[0]:
            s = scale * qh @ Kh.T
            eps = (2 * D * U * att.score_bounds(qh, Kh, scale).max(axis=1)
                   + 2 * U * np.abs(s).max(axis=1))
            w = np.exp(s - s.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            otol[h * G:(h + 1) * G] = (2 * eps + c * U)[:, None] * (w @ np.abs(Vh))
            ltol[h * G:(h + 1) * G] = eps + c * U * (1 + np.abs(lh))
    return o, lse, otol, ltol


def _run_and_check(setup, layer, ranges, n_q, scale, seed=1):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((len(ranges), n_q, setup.D), generator=g, device="cuda").to(torch.bfloat16)
    print(f"[attn] D={setup.D} n_q={n_q} ranges={list(ranges)[:6]}... layer={layer}", flush=True)
    out, lse = kb.run_decode_attention(setup.model, setup.cache, layer, q, ranges, scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    q64 = _bits_to_f64(q)
    worst = 0.0
    for j, (a, n) in enumerate(ranges):
        o, l, otol, ltol = _expect(setup, layer, q64[j], a, n, n_q, scale)
        if np.all(np.isneginf(l)):
            assert np.all(out[j] == 0) and np.all(np.isneginf(lse[j])), f"query {j}: empty range"
            continue
        err = np.abs(out[j] - o)
        assert np.all(err <= otol + 1e-30), (j, float((err / (otol + 1e-30)).max()))
        lerr = np.abs(lse[j] - l)
        assert np.all(lerr <= ltol), (j, float((lerr / ltol).max()))
        worst = max(worst, float((err / (otol + 1e-30)).max()), float((lerr / ltol).max()))
    print(f"[attn] worst error / tolerance {worst:.3g}", flush=True)
    return out, lse


RANGES = [(0, 1), (0, 17), (5, 511), (0, 512), (3, 513), (100, 2000), (0, 4096), (7, 0),
          (4000, 800)]


def test_decode_attention_paged_shuffled_gqa7():
    s = Setup()
    _run_and_check(s, 1, RANGES, 28, 1 / math.sqrt(128))


def test_decode_attention_head64_group8_dense_odd_pages():
    s = Setup(D=64, n_kv=2, page_size=12, n_pages=400, n_logical=400, shuffled=False, seed=3)
    _run_and_check(s, 0, [(0, 4800), (11, 13), (1000, 1025)], 16, 0.125, seed=4)


def test_decode_attention_head64_four_kv_heads():
    """Whole-row blocks (a quad of KV heads per block) at head_dim 64, page size 8."""
    s = Setup(D=64, n_kv=4, page_size=8, n_pages=700, n_logical=600, seed=17)
    _run_and_check(s, 1, RANGES, 12, 0.125)


def test_decode_attention_twelve_kv_heads_full_groups():
    """Three quads of KV heads per segment, 16 query heads per KV head (the largest group)."""
    s = Setup(D=64, n_kv=12, page_size=16, n_pages=320, n_logical=300, seed=21)
    _run_and_check(s, 0, RANGES, 192, 0.125, seed=22)


def test_decode_attention_one_kv_head_sixteen_query_heads():
    """One KV head (a block per head) with the largest query group."""
    s = Setup(n_kv=1, seed=19)
    _run_and_check(s, 0, RANGES, 16, 1 / math.sqrt(128))


def test_decode_attention_mha_one_head_per_kv():
    s = Setup(n_kv=8, n_pages=64, n_logical=64, seed=5)
    _run_and_check(s, 0, [(0, 1024), (16, 300)], 8, 1 / math.sqrt(128), seed=6)


def test_pages_outside_the_pool_are_masked():
    s = Setup(bad_pages=(2, 3, 40), seed=7)
    _run_and_check(s, 0, [(0, 100), (20, 700), (32, 16)], 28, 0.09, seed=8)


def test_state_merge_of_segments_equals_attention_over_the_whole():
    """The state-merge identity on the device: attention over [0, 1500) equals the merge of
    the attention over [0, 700) and [700, 1500) (both checked against the oracle)."""
    s = Setup(seed=9)
    n_q, scale = 28, 1 / math.sqrt(128)
    whole_o, whole_l = _run_and_check(s, 0, [(0, 1500)], n_q, scale, seed=10)
    a_o, a_l = _run_and_check(s, 0, [(0, 700)], n_q, scale, seed=10)
    b_o, b_l = _run_and_check(s, 0, [(700, 800)], n_q, scale, seed=10)
    part_o = torch.from_numpy(np.stack([a_o, b_o]).astype(np.float32)).cuda()   # [2, 1, n_q, D]
    part_l = torch.from_numpy(np.stack([a_l, b_l]).astype(np.float32)).cuda()
    out = torch.empty((n_q, s.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_q,), dtype=torch.float32, device="cuda")
    kb.check(kb.kamera_state_merge(2, n_q, s.D, part_o.data_ptr(), part_l.data_ptr(),
                                   out.data_ptr(), lse.data_ptr(), kb.current_stream_ptr()))
    torch.cuda.synchronize()
    ref_o, ref_l = att.state_merge([a_o[0], b_o[0]], [a_l[0], b_l[0]])
    np.testing.assert_allclose(out.cpu().numpy(), ref_o, rtol=0, atol=1e-5)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_l, rtol=0, atol=1e-5)
    np.testing.assert_allclose(out.cpu().numpy(), whole_o[0], rtol=0, atol=2e-5)
    np.testing.assert_allclose(lse.cpu().numpy(), whole_l[0], rtol=0, atol=2e-5)


def test_state_merge_with_empty_parts():
    rows, D = 5, 64
    rng = np.random.default_rng(12)
    po = rng.standard_normal((3, rows, D)).astype(np.float32)
    pl = rng.standard_normal((3, rows)).astype(np.float32)
    pl[1, :] = -np.inf                      # part 1 empty everywhere
    pl[:, 4] = -np.inf                      # row 4 empty in every part
    po[1, :] = 0
    po[:, 4] = 0
    dpo, dpl = torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda()
    out = torch.empty((rows, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    kb.check(kb.kamera_state_merge(3, rows, D, dpo.data_ptr(), dpl.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), kb.current_stream_ptr()))
    torch.cuda.synchronize()
    ref_o, ref_l = att.state_merge(list(po.astype(np.float64)), list(pl.astype(np.float64)))
    np.testing.assert_allclose(out.cpu().numpy(), ref_o, rtol=0, atol=1e-5)
    got_l = lse.cpu().numpy()
    assert np.isneginf(got_l[4]) and np.all(out.cpu().numpy()[4] == 0)
    np.testing.assert_allclose(got_l[:4], ref_l[:4], rtol=0, atol=1e-5)


@pytest.mark.parametrize("n_parts,rows,D,offset", [
    (5, 3, 37, 0),       # odd width: one float per column, 6 groups of threads over the parts
    (7, 4, 128, 1),      # part_out 4 bytes past 16-byte alignment: one float per column
    (9, 2, 300, 0),      # 75 columns of 4: 3 groups, the block's last 31 threads idle
    (600, 2, 1024, 0),   # 256 columns of 4, parts in 3 chunks of weights
    (40, 3, 999, 0),     # 999 columns of 1: four columns per thread
])
def test_state_merge_widths_alignments_and_many_parts(n_parts, rows, D, offset):
    """Every merge layout against the fp64 state merge. Empty parts (lse = -inf) hold NaN on
    the device: their outputs must not be read. Bound (derived): each feature is a sum of at
    most n_parts + 8 fp32 terms e_i o_i / Z, so |out - ref| <= (n_parts + 8) u sum_i w_i |o_i|
    + 2 u |ref|, and |lse - ref| <= (n_parts + 8) u + u |ref|."""
    rng = np.random.default_rng(1000 + D)
    po = rng.standard_normal((n_parts, rows, D)).astype(np.float32)
    pl = (3.0 * rng.standard_normal((n_parts, rows))).astype(np.float32)
    empty = rng.random((n_parts, rows)) < 0.2
    empty[:, -1] = True                                  # the last row has no parts at all
    pl[empty] = -np.inf
    dev_po = po.copy()
    dev_po[empty] = np.nan
    po[empty] = 0.0
    flat = torch.zeros(offset + dev_po.size, dtype=torch.float32)
    flat[offset:] = torch.from_numpy(dev_po.reshape(-1))
    dflat, dpl = flat.cuda(), torch.from_numpy(pl).cuda()
    out = torch.empty((rows, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    args = (n_parts, rows, D, dflat.data_ptr() + 4 * offset, dpl.data_ptr(), out.data_ptr(),
            lse.data_ptr(), kb.current_stream_ptr())
    kb.check(kb.kamera_state_merge(*args))
    torch.cuda.synchronize()
    got_o, got_l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = att.state_merge(list(po.astype(np.float64)), list(pl.astype(np.float64)))
    assert np.isneginf(got_l[-1]) and np.all(got_o[-1] == 0)
    live = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(got_l), live)
    M = np.where(live, ref_l, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl.astype(np.float64) - M), 0.0)   # parts x rows
    bound = (n_parts + 8) * U * np.einsum("pr,prd->rd", w, np.abs(po.astype(np.float64)))
    bound += 2 * U * np.abs(ref_o)
    assert np.all(np.abs(got_o - ref_o) <= bound + 1e-30)
    assert np.all(np.abs(got_l[live] - ref_l[live]) <= (n_parts + 8) * U + U * np.abs(ref_l[live]))
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    kb.check(kb.kamera_state_merge(*args[:5], out2.data_ptr(), lse2.data_ptr(), args[7]))
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


def _segment_tokens(ranges, n_kv):
    """The segment length the library picks: the longest of 2048, 1024, 512 that still gives
    the call 2048 blocks (segments x blocks per segment: one per quad of KV heads when
    n_kv is a multiple of 4, else one per KV head)."""
    per_segment = n_kv // 4 if n_kv % 4 == 0 else n_kv
    for seg in (2048, 1024, 512):
        if sum(-(-n // seg) for _, n in ranges) * per_segment >= 2048:
            return seg
    return 512


def test_many_queries_take_2048_token_segments():
    s = Setup(n_kv=8, n_pages=400, n_logical=350, seed=13)
    ranges = [((17 * i) % 5000, 1 + (i % 37)) for i in range(1010)]
    ranges += [(0, 5000), (1, 4999), (100, 4097), (2047, 2049), (0, 2048), (600, 4000),
               (3, 5597), (0, 5600), (2048, 2048), (4000, 1)]
    assert _segment_tokens(ranges, 8) == 2048
    _run_and_check(s, 0, ranges, 16, 1 / math.sqrt(128), seed=14)


def test_mid_size_calls_take_1024_token_segments():
    s = Setup(n_kv=8, n_pages=400, n_logical=350, seed=15)
    ranges = [(i % 300, 1 + (i % 5)) for i in range(960)]
    ranges += [(i * 37, 4096) for i in range(20)]
    ranges += [(1023, 1025), (5000, 600)]
    assert _segment_tokens(ranges, 8) == 1024
    _run_and_check(s, 1, ranges, 8, 0.1, seed=16)


# ---- MLA cache (absorbed form) -------------------------------------------------------------

class MlaSetup:
    """Pools of one layer-pair MLA cache: rows [c_KV (512) | k_rope (64)] shared (pool[1] is
    the row start, pool[0] 512 elements in) or two separate pools."""

    def __init__(self, n_layers=2, page_size=16, n_pages=300, n_logical=280, shared=True,
                 bad_pages=(), seed=0):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        rng = np.random.default_rng(seed)
        self.ps, self.n_pages = page_size, n_pages
        t = rng.permutation(n_pages)[:n_logical].astype(np.int32)
        for b in bad_pages:
            t[b] = -1                                  # outside the pool: masked
        self.table = t
        self.table_dev = torch.from_numpy(t).cuda()
        self.model = kb.make_model("mla", "bf16", n_layers, 1, 512, 64, "half_split", 1e4)
        c = kb.KameraCache()
        if shared:
            self.rows = torch.randn((n_layers, n_pages, page_size, 576), generator=g,
                                    device="cuda").to(torch.bfloat16)
            c.pool[1] = self.rows.data_ptr()
            c.pool[0] = self.rows.data_ptr() + 512 * 2
            c.layer_stride = self.rows.stride(0)
            c.token_stride = 576
            host = _bits_to_f64(self.rows)
            self.lat, self.rope = host[..., :512], host[..., 512:]
        else:
            self.lat_t = torch.randn((n_layers, n_pages, page_size, 512), generator=g,
                                     device="cuda").to(torch.bfloat16)
            self.rope_t = torch.randn((n_layers, n_pages, page_size, 512), generator=g,
                                      device="cuda").to(torch.bfloat16)   # rows of 512, 64 used
            c.pool[1] = self.lat_t.data_ptr()
            c.pool[0] = self.rope_t.data_ptr()
            c.layer_stride = self.lat_t.stride(0)
            c.token_stride = 512
            self.lat = _bits_to_f64(self.lat_t)
            self.rope = _bits_to_f64(self.rope_t)[..., :64]
        c.page_table = self.table_dev.data_ptr()
        c.n_logical_pages = n_logical
        c.page_size = page_size
        c.n_pages = n_pages
        self.cache = c

    def kv(self, layer, start, n):
        p = np.arange(start, start + n)
        phys = self.table[p // self.ps].astype(np.int64)
        ok = (phys >= 0) & (phys < self.n_pages)
        lat = self.lat[layer][phys[ok], (p % self.ps)[ok]]
        rope = self.rope[layer][phys[ok], (p % self.ps)[ok]]
        return np.concatenate([lat, rope], axis=1), lat


def check_mla_query(q64, K, V, n, scale, out, lse, j):
    """One MLA query (q64 [n_q, 576], rows K [n, 576] and V [n, 512] in fp64) against the
    oracle under the derived tolerance; returns the worst error / tolerance."""
    o, l = att.decode_attention(q64, K, V, scale)
    if K.shape[0] == 0:
        assert np.all(out == 0) and np.all(np.isneginf(lse)), f"query {j}: empty"
        return 0.0
    sc = scale * q64 @ K.T
    eps = (2 * (576 + 4) * U * att.score_bounds(q64, K, scale).max(axis=1)
           + 2 * U * np.abs(sc).max(axis=1))
    w = np.exp(sc - sc.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    c = 64 + -(-max(n, 1) // 16)
    otol = (2 * eps + c * U)[:, None] * (w @ np.abs(V))
    ltol = eps + c * U * (1 + np.abs(l))
    err = np.abs(out - o)
    assert np.all(err <= otol + 1e-30), (j, float((err / (otol + 1e-30)).max()))
    lerr = np.abs(lse - l)
    assert np.all(lerr <= ltol), (j, float((lerr / ltol).max()))
    return max(float((err / (otol + 1e-30)).max()), float((lerr / ltol).max()))


def _run_mla(s, layer, ranges, n_q, scale, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((len(ranges), n_q, 576), generator=g, device="cuda").to(torch.bfloat16)
    print(f"[attn-mla] n_q={n_q} ranges={list(ranges)[:6]} layer={layer}", flush=True)
    out, lse = kb.run_decode_attention(s.model, s.cache, layer, q, ranges, scale)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (len(ranges), n_q, 512)
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    q64 = _bits_to_f64(q)
    worst = 0.0
    for j, (a, n) in enumerate(ranges):
        K, V = s.kv(layer, a, n)
        worst = max(worst, check_mla_query(q64[j], K, V, n, scale, out[j], lse[j], j))
    print(f"[attn-mla] worst error / tolerance {worst:.3g}", flush=True)


def test_mla_decode_shared_rows_16_heads_masked_pages():
    s = MlaSetup(bad_pages=(3, 50), seed=21)
    _run_mla(s, 1, [(0, 1), (0, 17), (5, 511), (100, 2000), (0, 4480), (7, 0)], 16,
             1 / math.sqrt(192), seed=22)


def test_mla_decode_separate_pools_fewer_heads():
    s = MlaSetup(shared=False, n_pages=200, n_logical=200, page_size=12, seed=23)
    _run_mla(s, 0, [(0, 2400), (11, 13), (1000, 1025)], 5, 0.07, seed=24)
