"""Decode attention and the state merge at the C-ABI boundary, without a GPU: exports,
sizing and host validation. Every call is rejected before anything is enqueued (a NULL
workspace is the backstop for the attention call; the merge calls here all fail earlier)."""
import ctypes
import math

import pytest

from position_invariant_kv_kamera_amd import binding as kb

FAKE = 0x7F0000000000
GiB = 1 << 30


def _model(**kw):
    d = dict(family="gqa", dtype="bf16", n_layers=4, n_kv_heads=4, head_dim=128, rope_dim=128,
             rope_layout="half_split", theta=1e6)
    d.update(kw)
    return kb.make_model(**d)


def _cache(model):
    c = kb.KameraCache()
    row = model.n_kv_heads * model.head_dim
    c.pool[0] = FAKE
    c.pool[1] = FAKE + 8 * GiB
    c.layer_stride = 1000 * 16 * row
    c.token_stride = row
    c.page_table = None
    c.n_logical_pages = 1000
    c.page_size = 16
    c.n_pages = 1000
    return c


def _call(model=None, cache=None, layer=0, n_q_heads=28, ranges=((0, 100),), scale=0.088,
          q=FAKE + 20 * GiB, out=FAKE + 21 * GiB, lse=FAKE + 22 * GiB):
    model = model or _model()
    cache = cache or _cache(model)
    qs = kb.attn_queries_of(ranges)
    return kb.kamera_decode_attention(model, cache, layer, q, n_q_heads, qs, len(ranges), scale,
                                      out, lse, None, 0, None)


def test_exports_and_layout():
    names = set(kb.header_functions())
    assert {"kamera_decode_attention", "kamera_state_merge",
            "kamera_attention_workspace_bytes"} <= names
    assert ctypes.sizeof(kb.KameraAttnQuery) == 8


def test_well_formed_call_reaches_the_workspace_check():
    assert _call() == kb.KAMERA_ERR_WORKSPACE
    assert _call(_model(head_dim=64, rope_dim=64), n_q_heads=16) == kb.KAMERA_ERR_WORKSPACE
    mla = _model(family="mla", n_kv_heads=1, head_dim=512, rope_dim=64)
    assert _call(mla, n_q_heads=16) == kb.KAMERA_ERR_WORKSPACE
    # MLA query rows are 576 wide: q overlapping out by its true extent is caught
    rows = 16
    assert _call(mla, n_q_heads=16, q=FAKE + 21 * GiB - rows * 576 * 2 + 64) == kb.KAMERA_ERR_OVERLAP


def test_workspace_bytes():
    m = _model()
    qs = kb.attn_queries_of([(0, 1000), (5, 0), (0, 512)])
    need = kb.kamera_attention_workspace_bytes(m, 28, qs, 3)
    segs = 2 + 0 + 1
    assert need >= segs * 28 * 128 * 4 + segs * 28 * 4
    assert need % 256 == 0
    assert kb.kamera_attention_workspace_bytes(m, 27, qs, 3) == 0       # not a multiple of 4


@pytest.mark.parametrize("kw,status", [
    (dict(model=_model(family="mla", n_kv_heads=1, head_dim=512, rope_dim=64)), kb.KAMERA_ERR_UNSUPPORTED),   # 28 heads > 16
    (dict(model=_model(family="mla", n_kv_heads=1, head_dim=256, rope_dim=64), n_q_heads=16), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(model=_model(family="mla", n_kv_heads=1, head_dim=512, rope_dim=32), n_q_heads=16), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(model=_model(dtype="f32")), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(model=_model(head_dim=96, rope_dim=96)), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(n_q_heads=30), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(n_q_heads=68), kb.KAMERA_ERR_UNSUPPORTED),                  # 17 per KV head
    (dict(layer=4), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(layer=-1), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(ranges=((-1, 10),)), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(ranges=((0, -1),)), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(ranges=((15990, 11),)), kb.KAMERA_ERR_INVALID_ARGUMENT),    # past 16000 tokens
    (dict(scale=math.inf), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(scale=3e38), kb.KAMERA_ERR_INVALID_ARGUMENT),     # times log2(e) overflows fp32
    (dict(q=None), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 20 * GiB + 2), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(lse=FAKE + 21 * GiB + 64), kb.KAMERA_ERR_OVERLAP),          # lse inside out
])
def test_validation(kw, status):
    assert _call(**kw) == status
    assert kb.kamera_last_error()


def test_zero_queries_and_empty_ranges_are_valid():
    assert _call(ranges=()) == kb.KAMERA_ERR_WORKSPACE
    assert _call(ranges=((7, 0),)) == kb.KAMERA_ERR_WORKSPACE


def test_state_merge_validation():
    P, O, L, R = FAKE, FAKE + GiB, FAKE + 2 * GiB, FAKE + 3 * GiB
    assert kb.kamera_state_merge(-1, 4, 128, P, L, O, R, None) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert kb.kamera_state_merge(2, 4, 0, P, L, O, R, None) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert kb.kamera_state_merge(2, 4, 2048, P, L, O, R, None) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert kb.kamera_state_merge(2, 4, 128, None, L, O, R, None) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert kb.kamera_state_merge(2, 4, 128, P, L, P + 64, R, None) == kb.KAMERA_ERR_OVERLAP
    assert kb.kamera_state_merge(2, 0, 128, None, None, None, None, None) == kb.KAMERA_OK


# ---- attention over chunks read in place --------------------------------------------------

def _view(n_tokens=300, m=(16, 16), delta=500, row=512, aligned=True):
    base = FAKE + (0 if aligned else 2)
    patch = [None, None]
    for ch in range(2):
        if m[ch]:
            patch[ch] = (m[ch], FAKE + (30 + ch) * GiB, 4 * 2000 * m[ch], 2000 * m[ch],
                         FAKE + (32 + ch) * GiB, 4 * 128 * m[ch], 128 * m[ch])
    return {"n_tokens": n_tokens, "delta": delta,
            "src": [(base, 2000 * row, row), (base + 4 * GiB, 2000 * row, row)],
            "patch": patch}


def _chunk_call(model=None, views=None, spans=((0, 2),), n_q_heads=28, layer=0, scale=0.088,
                q=FAKE + 20 * GiB, out=FAKE + 21 * GiB, lse=FAKE + 22 * GiB):
    model = model or _model()
    views = views if views is not None else [_view(), _view(40, (0, 8), -7)]
    ch = kb.attn_chunks_of(views)
    qs = kb.chunk_queries_of(spans)
    return kb.kamera_chunk_attention(model, layer, ch, len(views), qs, len(spans), q, n_q_heads,
                                     scale, out, lse, None, 0, None)


def test_chunk_attention_exports_and_layout():
    names = set(kb.header_functions())
    assert {"kamera_chunk_attention", "kamera_chunk_attention_workspace_bytes"} <= names
    assert ctypes.sizeof(kb.KameraAttnChunk) == ctypes.sizeof(kb.KameraChunk) == 192
    assert ctypes.sizeof(kb.KameraChunkQuery) == 8


def test_chunk_attention_well_formed_call_reaches_the_workspace_check():
    assert _chunk_call() == kb.KAMERA_ERR_WORKSPACE
    m64 = _model(head_dim=64, rope_dim=32, rope_layout="interleaved")
    views = [_view(row=256), _view(5, (64, 0), 3, row=256)]
    assert _chunk_call(m64, views, n_q_heads=16) == kb.KAMERA_ERR_WORKSPACE


def test_chunk_attention_workspace_bytes_grow_with_segments():
    m = _model()
    views = [_view(3000), _view(0), _view(700)]
    small = kb.kamera_chunk_attention_workspace_bytes(m, 28, kb.attn_chunks_of(views[:1]), 1,
                                                      kb.chunk_queries_of([(0, 1)]), 1)
    big = kb.kamera_chunk_attention_workspace_bytes(m, 28, kb.attn_chunks_of(views), 3,
                                                    kb.chunk_queries_of([(0, 3), (1, 2)]), 2)
    assert 0 < small < big and small % 256 == 0 and big % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(model=_model(family="mla", head_dim=512, rope_dim=64, n_kv_heads=1)), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(model=_model(dtype="f32")), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(model=_model(head_dim=96, rope_dim=96)), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(n_q_heads=30), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(n_q_heads=4 * 17), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(views=[_view(m=(65, 0))], spans=((0, 1),)), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(views=[_view(m=(-1, 0))], spans=((0, 1),)), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(views=[_view(n_tokens=-1)], spans=((0, 1),)), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(views=[_view(aligned=False)], spans=((0, 1),)), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(spans=((1, 2),)), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(spans=((-1, 1),)), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(layer=4), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.inf), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(scale=3e38), kb.KAMERA_ERR_INVALID_ARGUMENT),     # times log2(e) overflows fp32
    (dict(q=None), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 20 * GiB + 2), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(out=FAKE + 20 * GiB), kb.KAMERA_ERR_OVERLAP),
])
def test_chunk_attention_rejects(kw, status):
    assert _chunk_call(**kw) == status
    assert kb.kamera_last_error()


def test_chunk_attention_rejects_a_patch_without_factors():
    v = _view(m=(0, 0))
    v["patch"] = [(8, None, 0, 0, None, 0, 0), None]
    assert _chunk_call(views=[v], spans=((0, 1),)) == kb.KAMERA_ERR_INVALID_ARGUMENT
