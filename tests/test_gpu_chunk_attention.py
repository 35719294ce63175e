"""Attention over chunks read in place (kamera_chunk_attention) on the GPU, through the C ABI,
against the fp64 oracle (oracle/attention.py chunk_attention: each chunk's keys and values as
the reuse operator defines them, attended exactly).

Tolerance (derived): the query turned by -delta and w = V_K^T q are fp32 (rotation: two
products and a sum; w: D products summed) and each is split into two bf16 terms, so every
score term carries a relative error below 2^-15 + (D + m + 2) 2^-24 < 2^-13 (the last two
roundings: the scale, times log2 e, for the kernel's base-2 scores) of its magnitude
bound B_t = scale (sum_d |q~_d||k_td| + sum_r W~_r |U_K,tr|), with q~_d = |q_a| + |q_b| on a
rotated pair and W~_r = sum_d |q_d||V_K,dr|. With eps = 2^-13 max_t B_t, the softmax weights
carry a relative error below 2 eps + c u (u = 2^-24, c = 64 + tiles + m_V for the exp, running
sums, merges and the value patch sum), so
    |o_g - o|_f <= (2 eps + c u) sum_t w_t (|v_tf| + sum_r |U_V,tr||V_V,fr|),
    |lse_g - lse| <= eps + c u (1 + |lse|)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as att
from position_invariant_kv_kamera_amd import binding as kb

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


def _bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Case:
    def __init__(self, n_kv, D, R, layout, theta, specs, spans, G, seed, n_layers=2,
                 inv_freq=None, pair_section=None):
        self.n_kv, self.D, self.R, self.layout, self.theta = n_kv, D, R, layout, theta
        self.specs, self.spans, self.G, self.n_layers = specs, spans, G, n_layers
        self.inv_freq, self.pair_section = inv_freq, pair_section
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        row = n_kv * D
        self.chunks = []
        for (T, delta, mk, mv, *sec) in specs:
            c = {"T": T, "delta": delta, "sec": tuple(sec[0]) if sec else (delta, delta)}
            c["K"] = torch.randn((n_layers, T, row), generator=gen, device="cuda").to(torch.bfloat16)
            c["V"] = torch.randn((n_layers, T, row), generator=gen, device="cuda").to(torch.bfloat16)
            for name, m in (("k", mk), ("v", mv)):
                c["m" + name] = m
                if m:
                    c["U" + name] = (0.1 * torch.randn((n_layers, n_kv, T, m), generator=gen,
                                                       device="cuda")).to(torch.bfloat16)
                    c["W" + name] = (0.1 * torch.randn((n_layers, n_kv, D, m), generator=gen,
                                                       device="cuda")).to(torch.bfloat16)
            self.chunks.append(c)
        kw = {}
        if inv_freq is not None:
            kw["inv_freq"] = inv_freq
        if pair_section is not None:
            kw["pair_section"] = pair_section
        self.model = kb.make_model("gqa", "bf16", n_layers, n_kv, D, R, layout, theta, **kw)

    def items(self):
        out = []
        for c in self.chunks:
            T = c["T"]
            row = self.n_kv * self.D
            it = {"n_tokens": T, "delta": c["delta"], "delta_sections": c["sec"],
                  "src": [(c["K"].data_ptr(), T * row, row), (c["V"].data_ptr(), T * row, row)],
                  "patch": [None, None]}
            for ch, name in enumerate(("k", "v")):
                m = c["m" + name]
                if m:
                    U, W = c["U" + name], c["W" + name]
                    it["patch"][ch] = (m, U.data_ptr(), U.stride(0), U.stride(1), W.data_ptr(),
                                       W.stride(0), W.stride(1))
            out.append(it)
        return out

    def oracle_chunks(self, layer, h):
        D = self.D
        res = []
        for c in self.chunks:
            d = {"K": _bits(c["K"][layer, :, h * D:(h + 1) * D]),
                 "V": _bits(c["V"][layer, :, h * D:(h + 1) * D]), "delta": c["delta"],
                 "section_delta": np.array([c["delta"], *c["sec"]], np.int64)}
            for name in ("k", "v"):
                if c["m" + name]:
                    d["U" + name] = _bits(c["U" + name][layer, h])
                    d["V" + name] = _bits(c["W" + name][layer, h])
            res.append(d)
        return res


def _rope_kw(case):
    kw = dict(layout=case.layout, theta=case.theta, rot_dim=case.R)
    if case.inv_freq is not None:
        kw["inv_freq"] = case.inv_freq
    if case.pair_section is not None:
        kw["pair_section"] = case.pair_section
    return kw


def _partner_mag(q, R, layout):
    """|q_d| + |q_partner(d)| on rotated features, |q_d| elsewhere (rows of q)."""
    a = np.abs(q).copy()
    idx = np.arange(q.shape[1])
    if layout == oracle.HALF_SPLIT:
        part = np.where(idx < R // 2, idx + R // 2, idx - R // 2)
    else:
        part = idx ^ 1
    rot = idx < R
    a[:, rot] += np.abs(q[:, part[rot]])
    return a


def _check(case, layer, q, scale, out, lse):
    D, G = case.D, case.G
    q64 = _f64(_bits(q))
    kw = _rope_kw(case)
    worst = 0.0
    for j, (first, count) in enumerate(case.spans):
        for h in range(case.n_kv):
            qh = q64[j, h * G:(h + 1) * G]
            chunks = case.oracle_chunks(layer, h)[first:first + count]
            o, l = att.chunk_attention(qh, chunks, scale, **kw)
            og, lg = out[j, h * G:(h + 1) * G], lse[j, h * G:(h + 1) * G]
            if not chunks or sum(c["K"].shape[0] for c in chunks) == 0:
                assert np.all(og == 0) and np.all(np.isneginf(lg)), (j, h)
                continue
            # bounds of the score terms and of the values, per token
            qt = _partner_mag(qh, case.R, case.layout)
            B, Vabs, S, tiles, mv = [], [], [], 0, 0
            for c in chunks:
                K, V = _f64(c["K"]), _f64(c["V"])
                b = qt @ np.abs(K).T
                va = np.abs(V)
                if "Uk" in c:
                    Wt = np.abs(qh) @ np.abs(_f64(c["Vk"]))
                    b = b + Wt @ np.abs(_f64(c["Uk"])).T
                if "Uv" in c:
                    va = va + np.abs(_f64(c["Uv"])) @ np.abs(_f64(c["Vv"])).T
                    mv = max(mv, c["Uv"].shape[1])
                kp, vp = att.chunk_keys_values(c, **kw)
                S.append(scale * qh @ kp.T)
                B.append(abs(scale) * b)
                Vabs.append(va)
                tiles += -(-K.shape[0] // 16)
            S, B, Vabs = np.concatenate(S, 1), np.concatenate(B, 1), np.concatenate(Vabs, 0)
            w = np.exp(S - S.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            eps = 2.0 ** -13 * B.max(axis=1)
            c_u = (64 + tiles + mv) * U32
            otol = (2 * eps + c_u)[:, None] * (w @ Vabs)
            ltol = eps + c_u * (1 + np.abs(l))
            err = np.abs(og - o)
            assert np.all(err <= otol + 1e-30), (j, h, float((err / (otol + 1e-30)).max()))
            lerr = np.abs(lg - l)
            assert np.all(lerr <= ltol), (j, h, float((lerr / ltol).max()))
            worst = max(worst, float((err / (otol + 1e-30)).max()), float((lerr / ltol).max()))
    print(f"[chunk-attn] worst error / tolerance {worst:.3g}", flush=True)


def _run(case, layer, scale, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    n_q = case.n_kv * case.G
    q = torch.randn((len(case.spans), n_q, case.D), generator=gen, device="cuda").to(torch.bfloat16)
    print(f"[chunk-attn] D={case.D} R={case.R} layout={case.layout} G={case.G} "
          f"chunks={[s[:4] for s in case.specs]} spans={case.spans} layer={layer}", flush=True)
    out, lse = kb.run_chunk_attention(case.model, layer, case.items(), case.spans, q, scale)
    torch.cuda.synchronize()
    _check(case, layer, q, scale, out.cpu().numpy().astype(np.float64),
           lse.cpu().numpy().astype(np.float64))


def test_half_split_rank16_chunks_with_an_empty_one_and_a_long_one():
    specs = [(300, 1234, 16, 16), (17, -50, 16, 16), (0, 5, 16, 16), (2100, 30000, 16, 16)]
    case = Case(4, 128, 128, oracle.HALF_SPLIT, 1e6, specs,
                [(0, 4), (1, 1), (3, 1), (2, 1), (0, 0)], G=7, seed=1)
    _run(case, 1, 1 / math.sqrt(128), seed=2)


def test_head64_interleaved_mixed_and_unaligned_ranks():
    specs = [(257, 100, 0, 32), (64, -3000, 64, 0), (33, 7, 12, 20), (16, 0, 8, 8)]
    case = Case(2, 64, 64, oracle.INTERLEAVED, 1e4, specs, [(0, 4), (2, 2), (0, 1)], G=8,
                seed=3)
    _run(case, 0, 0.125, seed=4)


def test_partial_rotary_mha_rank_zero_and_rank64():
    specs = [(500, 65536, 0, 0), (123, -65536, 64, 64)]
    case = Case(8, 128, 64, oracle.HALF_SPLIT, 1e4, specs, [(0, 2), (1, 1)], G=1, seed=5)
    _run(case, 1, 1 / math.sqrt(128), seed=6)


def test_whole_row_blocks_head64_interleaved_unaligned_ranks():
    """Four KV heads (one whole-row block per segment) at head_dim 64 with ranks that are not
    multiples of 8 (the U rows and factors go through the 2-byte paths)."""
    specs = [(257, 100, 0, 32), (33, 7, 12, 20), (16, 0, 8, 8), (400, -2000, 32, 5)]
    case = Case(4, 64, 64, oracle.INTERLEAVED, 1e4, specs, [(0, 4), (1, 2), (3, 1)], G=3,
                seed=11)
    _run(case, 0, 0.125, seed=12)


def test_whole_row_blocks_eight_heads_rank32_partial_rotary():
    """Eight KV heads (two whole-row blocks per segment), rank-32 class, partial rotary."""
    specs = [(500, 65536, 32, 24), (123, -65536, 1, 32), (1100, 4096, 17, 0)]
    case = Case(8, 128, 64, oracle.HALF_SPLIT, 1e4, specs, [(0, 2), (1, 1), (2, 1)], G=2,
                seed=13)
    _run(case, 1, 1 / math.sqrt(128), seed=14)


def test_whole_row_blocks_twelve_heads_full_groups_interleaved():
    """Three quads of KV heads, 16 query heads per KV head, rank-16 class with odd ranks."""
    specs = [(130, 777, 16, 3), (47, -9, 5, 16), (260, 1 << 20, 0, 11)]
    case = Case(12, 64, 64, oracle.INTERLEAVED, 1e4, specs, [(0, 3), (1, 1), (2, 1)], G=16,
                seed=15)
    _run(case, 0, 0.125, seed=16)


def test_frequency_table_and_sections():
    sec = np.repeat(np.array([0, 1, 2], np.uint8), [16, 24, 24])
    table = np.sort(10.0 ** np.random.default_rng(3).uniform(-6, 0, 64))[::-1].copy()
    specs = [(200, 1500, 16, 16, (-20, 333)), (90, -7, 16, 0, (5, 4000))]
    case = Case(4, 128, 128, oracle.HALF_SPLIT, 1e6, specs, [(0, 2), (1, 1)], G=4, seed=7,
                inv_freq=table, pair_section=sec)
    _run(case, 0, 0.09, seed=8)


def test_rank_zero_shift_zero_matches_decode_attention_over_the_same_rows():
    """With every delta 0 and no patch the read is plain attention over the rows: the same
    numbers kamera_decode_attention gives over a dense cache holding them (both GPU paths,
    each within its tolerance of the oracle, are compared to each other loosely)."""
    specs = [(688, 0, 0, 0)]
    case = Case(4, 128, 128, oracle.HALF_SPLIT, 1e6, specs, [(0, 1)], G=7, seed=9, n_layers=1)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(10)
    q = torch.randn((1, 28, 128), generator=gen, device="cuda").to(torch.bfloat16)
    out, lse = kb.run_chunk_attention(case.model, 0, case.items(), case.spans, q, 0.088)
    c = kb.KameraCache()
    K, V = case.chunks[0]["K"], case.chunks[0]["V"]
    c.pool[0], c.pool[1] = K.data_ptr(), V.data_ptr()
    c.layer_stride = K.stride(0)
    c.token_stride = K.stride(1)
    c.page_table = None
    c.n_logical_pages = 688 // 16
    c.page_size = 16
    c.n_pages = 688 // 16
    # the dense pool is the canonical rows themselves (43 pages of 16 tokens)
    out2, lse2 = kb.run_decode_attention(case.model, c, 0, q, [(0, 688)], 0.088)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), out2.cpu().numpy(), rtol=0, atol=2e-3)
    np.testing.assert_allclose(lse.cpu().numpy(), lse2.cpu().numpy(), rtol=0, atol=2e-3)
