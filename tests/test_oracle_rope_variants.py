"""Oracle pins for the RoPE variants of real backbones (relocation of keys that carry them).

Each pin applies a library's own RoPE to random keys at canonical positions and at shifted
positions, with cos/sin formed in 50-digit arithmetic (mpmath) from the library's frequencies,
and requires the oracle's relocation of the canonical keys to land on the shifted ones:
  * multimodal 3-D positions, contiguous sections (transformers' Qwen2-VL
    apply_multimodal_rotary_pos_emb, mrope_section [16, 24, 24]), with a different shift per
    position component;
  * multimodal 3-D positions, interleaved sections (the pair -> component map read off
    transformers' Qwen3-VL apply_interleaved_mrope, mrope_section [24, 20, 20]);
  * partial rotary (transformers' GPT-NeoX apply_rotary_pos_emb: only the first rotary_dim
    features turn);
  * scaled frequency tables (transformers' llama3 and yarn initialisers; yarn's attention
    factor scales cos and sin alike, so relocation is still a pure rotation).
Relocation by one shift on every component must equal plain RoPE relocation exactly.
"""
import mpmath
import numpy as np
import pytest
import torch

import oracle

mpmath.mp.dps = 50


def _cos_sin(pos: np.ndarray, inv_freq: np.ndarray):
    """cos/sin of pos[t] * inv_freq[i] in 50-digit arithmetic, as fp64 arrays [T, P]."""
    c = np.empty((len(pos), len(inv_freq)))
    s = np.empty_like(c)
    for t, p in enumerate(pos):
        for i, f in enumerate(inv_freq):
            a = mpmath.mpf(int(p)) * mpmath.mpf(float(f))
            c[t, i] = float(mpmath.cos(a))
            s[t, i] = float(mpmath.sin(a))
    return c, s


def _torch_cs(c, s):
    """[T, P] halves -> [T, 2P] cos/sin as the rotate_half libraries build them."""
    return (torch.from_numpy(np.concatenate([c, c], axis=-1)),
            torch.from_numpy(np.concatenate([s, s], axis=-1)))


def _ladder(theta, dim):
    return oracle.inv_freq(theta, dim)


def _mrope_grid(T, offset):
    """3-D positions of T vision tokens on a grid, t = offset, (h, w) = offset + (row, col)."""
    side = int(np.ceil(np.sqrt(T)))
    r = np.arange(T) // side
    c = np.arange(T) % side
    return np.stack([np.full(T, offset), offset + r, offset + c])


# ---- Qwen2-VL: contiguous sections ------------------------------------------------------

@pytest.mark.parametrize("shifts", [(500, 500, 500), (1200, -37, 9001), (0, 64, -64)])
def test_qwen2vl_mrope_relocation(shifts):
    from transformers.models.qwen2_vl.modeling_qwen2_vl import apply_multimodal_rotary_pos_emb
    D, T, theta = 128, 24, 1e6
    section = [16, 24, 24]
    inv = _ladder(theta, D)
    rng = np.random.default_rng(7)
    raw = rng.standard_normal((T, D))
    pos0 = _mrope_grid(T, 3)
    pos1 = pos0 + np.asarray(shifts)[:, None]

    def embed(pos):
        cs = [_torch_cs(*_cos_sin(pos[k], inv)) for k in range(3)]
        cos = torch.stack([a for a, _ in cs])[:, None]           # [3, 1, T, D]
        sin = torch.stack([b for _, b in cs])[:, None]
        k = torch.from_numpy(raw)[None, None]                       # [1, 1, T, D]
        q, kk = apply_multimodal_rotary_pos_emb(k, k, cos, sin, section)
        return kk[0, 0].numpy()

    canonical, target = embed(pos0), embed(pos1)
    pair_section = np.repeat([0, 1, 2], section)
    got, _ = oracle.segment(canonical, rotate=True, layout=oracle.HALF_SPLIT, theta=theta,
                            pair_delta=oracle.pair_deltas(pair_section, shifts))
    np.testing.assert_allclose(got, target, rtol=0, atol=2e-12)
    if len(set(shifts)) == 1:
        plain, _ = oracle.segment(canonical, rotate=True, layout=oracle.HALF_SPLIT,
                                  theta=theta, delta=shifts[0])
        assert np.array_equal(got, plain)


def test_qwen2vl_sections_matter():
    """Using one shift for all pairs where the components moved differently is wrong."""
    from transformers.models.qwen2_vl.modeling_qwen2_vl import apply_multimodal_rotary_pos_emb
    D, T, theta = 128, 8, 1e6
    section = [16, 24, 24]
    inv = _ladder(theta, D)
    raw = np.random.default_rng(8).standard_normal((T, D))
    pos0 = _mrope_grid(T, 0)
    shifts = (100, 0, 0)
    pos1 = pos0 + np.asarray(shifts)[:, None]
    outs = []
    for pos in (pos0, pos1):
        cs = [_torch_cs(*_cos_sin(pos[k], inv)) for k in range(3)]
        cos = torch.stack([a for a, _ in cs])[:, None]
        sin = torch.stack([b for _, b in cs])[:, None]
        k = torch.from_numpy(raw)[None, None]
        outs.append(apply_multimodal_rotary_pos_emb(k, k, cos, sin, section)[1][0, 0].numpy())
    wrong, _ = oracle.segment(outs[0], rotate=True, theta=theta, delta=100)
    assert np.max(np.abs(wrong - outs[1])) > 0.1


# ---- Qwen3-VL: interleaved sections -----------------------------------------------------

def _qwen3vl_pair_section(section, pairs):
    from transformers.models.qwen3_vl.modeling_qwen3_vl import Qwen3VLTextRotaryEmbedding
    probe = torch.arange(3, dtype=torch.float64).view(3, 1, 1, 1).expand(3, 1, 1, pairs)
    out = Qwen3VLTextRotaryEmbedding.apply_interleaved_mrope(None, probe.clone(), section)
    return out.reshape(-1).round().long().numpy()


def test_qwen3vl_interleaved_mrope_relocation():
    from transformers.models.qwen3_vl.modeling_qwen3_vl import apply_rotary_pos_emb
    D, T, theta = 128, 16, 5e6
    section = [24, 20, 20]
    pair_section = _qwen3vl_pair_section(section, D // 2)
    assert sorted(np.bincount(pair_section, minlength=3)) == sorted(section)
    assert len(set(pair_section[:6])) == 3        # interleaved, not contiguous
    inv = _ladder(theta, D)
    raw = np.random.default_rng(9).standard_normal((T, D))
    pos0 = _mrope_grid(T, 11)
    shifts = (4096, -3, 250)
    pos1 = pos0 + np.asarray(shifts)[:, None]

    def embed(pos):
        # each pair takes the angle of its own position component
        ang_c = np.empty((T, D // 2))
        ang_s = np.empty((T, D // 2))
        for comp in range(3):
            c, s = _cos_sin(pos[comp], inv)
            sel = pair_section == comp
            ang_c[:, sel] = c[:, sel]
            ang_s[:, sel] = s[:, sel]
        cos, sin = _torch_cs(ang_c, ang_s)
        k = torch.from_numpy(raw)[None, None]
        return apply_rotary_pos_emb(k, k, cos[None], sin[None])[1][0, 0].numpy()

    got, _ = oracle.segment(embed(pos0), rotate=True, theta=theta,
                            pair_delta=oracle.pair_deltas(pair_section, shifts))
    np.testing.assert_allclose(got, embed(pos1), rtol=0, atol=2e-12)


# ---- partial rotary (GPT-NeoX) ------------------------------------------------------------

@pytest.mark.parametrize("rot_dim", [32, 64])
def test_partial_rotary_relocation(rot_dim):
    from transformers.models.gpt_neox.modeling_gpt_neox import apply_rotary_pos_emb
    D, T, theta, delta = 128, 12, 1e4, 3333
    inv = _ladder(theta, rot_dim)
    raw = np.random.default_rng(10).standard_normal((T, D))
    pos = np.arange(T) + 5

    def embed(p):
        cos, sin = _torch_cs(*_cos_sin(p, inv))
        k = torch.from_numpy(raw)[None, None]
        return apply_rotary_pos_emb(k, k, cos[None], sin[None])[1][0, 0].numpy()

    canonical, target = embed(pos), embed(pos + delta)
    assert np.array_equal(canonical[:, rot_dim:], raw[:, rot_dim:])   # pass-through features
    got, _ = oracle.segment(canonical, rotate=True, rot_dim=rot_dim, theta=theta, delta=delta)
    np.testing.assert_allclose(got, target, rtol=0, atol=2e-12)
    assert np.array_equal(got[:, rot_dim:], canonical[:, rot_dim:])


# ---- scaled frequency tables ---------------------------------------------------------------

def _scaled_inv_freq(kind):
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    if kind == "llama3":
        scaling = {"rope_type": "llama3", "factor": 8.0, "low_freq_factor": 1.0,
                   "high_freq_factor": 4.0, "original_max_position_embeddings": 8192}
        theta = 500000.0
    else:
        scaling = {"rope_type": "yarn", "factor": 4.0, "original_max_position_embeddings": 32768}
        theta = 1e6
    cfg = LlamaConfig(hidden_size=1024, num_attention_heads=8, head_dim=128, rope_theta=theta,
                      max_position_embeddings=131072, rope_scaling=scaling)
    inv, factor = ROPE_INIT_FUNCTIONS[kind](cfg, "cpu")
    return inv.double().numpy(), float(factor), theta


@pytest.mark.parametrize("kind", ["llama3", "yarn"])
def test_scaled_frequency_table_relocation(kind):
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    inv, factor, theta = _scaled_inv_freq(kind)
    assert not np.allclose(inv, _ladder(theta, 128))        # the table differs from the ladder
    D, T, delta = 128, 10, 70000
    raw = np.random.default_rng(11).standard_normal((T, D))
    pos = np.arange(T) * 3

    def embed(p):
        c, s = _cos_sin(p, inv)
        cos, sin = _torch_cs(c * factor, s * factor)
        k = torch.from_numpy(raw)[None, None]
        return apply_rotary_pos_emb(k, k, cos[None], sin[None])[1][0, 0].numpy()

    canonical, target = embed(pos), embed(pos + delta)
    got, _ = oracle.segment(canonical, rotate=True, theta=theta, inv_freq=inv, delta=delta)
    np.testing.assert_allclose(got, target, rtol=0, atol=4e-12)
    ladder, _ = oracle.segment(canonical, rotate=True, theta=theta, delta=delta)
    assert np.max(np.abs(ladder - target)) > 1e-3           # the ladder would be wrong here


def test_table_equal_to_ladder_is_the_plain_operator():
    theta, D = 1e4, 64
    x = np.random.default_rng(12).standard_normal((5, D))
    a, _ = oracle.segment(x, rotate=True, theta=theta, delta=77)
    b, _ = oracle.segment(x, rotate=True, theta=theta, delta=77, inv_freq=_ladder(theta, D),
                          pair_delta=np.full(D // 2, 77))
    assert np.array_equal(a, b)


def test_variant_arguments_are_checked():
    x = np.zeros((2, 64))
    with pytest.raises(ValueError):
        oracle.segment(x, rotate=True, rot_dim=32, inv_freq=np.ones(32))
    with pytest.raises(ValueError):
        oracle.segment(x, rotate=True, rot_dim=96)
