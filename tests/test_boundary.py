"""The C-ABI boundary without a GPU: exports, helpers, and host-side validation.

Every compute call here is built to be rejected by host validation. As a backstop each one
also passes a NULL workspace (validation checks the workspace after every other argument),
so no call in this file can reach a HIP launch, on any machine.
"""
import ctypes
import math

import pytest

from position_invariant_kv_kamera_amd import binding as kb
from position_invariant_kv_kamera_amd import workloads as wl

FAKE = 0x7F0000000000      # never dereferenced: every call below fails validation first


def lib():
    return kb.load_library()


def test_every_header_function_is_exported():
    names = kb.header_functions()
    assert {"kamera_reuse_batch", "kamera_relocate", "kamera_patch", "kamera_workspace_bytes",
            "kamera_status_string", "kamera_last_error", "kamera_version",
            "kamera_patch_bytes", "kamera_kv_bytes", "kamera_read_fault_count"} <= set(names)
    so = lib()
    for n in names:
        assert hasattr(so, n), n


def test_version_and_status_strings():
    assert kb.kamera_version() == 10300
    for st in range(7):
        assert kb.kamera_status_string(st) not in ("", "unknown status")
    assert kb.kamera_status_string(99) == "unknown status"


def test_workspace_bytes():
    assert kb.kamera_workspace_bytes(-1) == 0
    a, b = kb.kamera_workspace_bytes(0), kb.kamera_workspace_bytes(100)
    assert a >= 256 and a % 256 == 0 and b % 256 == 0 and b > a


def _model(**kw):
    d = dict(family=0, dtype=1, n_layers=28, n_kv_heads=4, head_dim=128, rope_dim=128,
             rope_layout=0, n_sections=0, rope_theta=1e6)
    d.update(kw)
    return kb.KameraModel(**d)


def test_kv_and_patch_bytes_closed_form():
    """Patch footprint (technical summary §4, memory): U is tokens x m and V features x m per
    head, per channel, per layer."""
    m = _model()
    L = 1296
    assert kb.kamera_kv_bytes(m, L) == 2 * 28 * L * 4 * 128 * 2
    assert kb.kamera_patch_bytes(m, L, 16) == 2 * 28 * 4 * (L + 128) * 16 * 2
    mla = _model(family=1, n_kv_heads=1, head_dim=512, rope_dim=64, n_layers=27, rope_theta=1e4)
    assert kb.kamera_kv_bytes(mla, 2048) == 27 * 2048 * 576 * 2
    assert kb.kamera_patch_bytes(mla, 2048, 32) == 27 * ((2048 + 64) + (2048 + 512)) * 32 * 2
    assert kb.kamera_patch_bytes(_model(n_layers=0), 10, 4) == 0


def _cache(**kw):
    c = kb.KameraCache()
    c.pool[0] = FAKE
    c.pool[1] = FAKE + (1 << 36)
    c.layer_stride = 1000 * 16 * 512
    c.token_stride = 512
    c.page_table = None
    c.n_logical_pages = 1000
    c.page_size = 16
    c.n_pages = 1000
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _chunks(n=1, **kw):
    arr = (kb.KameraChunk * n)()
    for i in range(n):
        k = arr[i]
        k.n_tokens = 100
        k.dst_token_offset = 100 * i
        k.delta = 5
        for ch in range(2):
            k.src[ch] = kb.KameraSrc(FAKE + (1 << 38) + (ch << 30), 100 * 512, 512)
        for key, v in kw.items():
            setattr(k, key, v)
    return arr


def call(model=None, cache=None, chunks=None, n=1, ws=None, ws_bytes=0, fn="kamera_reuse_batch"):
    model = _model() if model is None else model
    cache = _cache() if cache is None else cache
    chunks = _chunks(n) if chunks is None else chunks
    st = getattr(kb, fn)(model, cache, chunks, n, ws, ws_bytes, None)
    return st, kb.kamera_last_error()


@pytest.mark.parametrize("fn", ["kamera_reuse_batch", "kamera_relocate", "kamera_patch"])
def test_null_workspace_is_the_last_check(fn):
    st, msg = call(fn=fn)
    assert st == kb.KAMERA_ERR_WORKSPACE and "workspace" in msg


def test_workspace_misaligned_and_too_small():
    need = kb.kamera_workspace_bytes(1)
    st, _ = call(ws=FAKE + 8, ws_bytes=need)
    assert st == kb.KAMERA_ERR_WORKSPACE
    st, msg = call(ws=FAKE, ws_bytes=need - 1)
    assert st == kb.KAMERA_ERR_WORKSPACE and "needs" in msg


@pytest.mark.parametrize("kw,status", [
    (dict(family=7), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(dtype=9), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(n_layers=0), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(rope_layout=3), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(rope_theta=math.inf), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(rope_theta=math.nan), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(rope_theta=1.0), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(head_dim=127, rope_dim=127), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(rope_dim=130), kb.KAMERA_ERR_INVALID_ARGUMENT),      # rotary part wider than the head
    (dict(n_sections=4), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(n_sections=3), kb.KAMERA_ERR_INVALID_ARGUMENT),      # sections without a pair map
    (dict(head_dim=2048, rope_dim=2048), kb.KAMERA_ERR_UNSUPPORTED),
    (dict(n_kv_heads=0), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(family=1, n_kv_heads=2, head_dim=512, rope_dim=64), kb.KAMERA_ERR_INVALID_ARGUMENT),
])
def test_model_validation(kw, status):
    st, msg = call(model=_model(**kw))
    assert st == status, msg
    assert msg


def test_rope_variant_tables_are_validated():
    import numpy as np
    ok = kb.make_model("gqa", "bf16", 28, 4, 128, 128, "half_split", 1e6,
                       inv_freq=np.linspace(1.0, 1e-6, 64),
                       pair_section=np.repeat([0, 1, 2], [16, 24, 24]))
    st, msg = call(model=ok)
    assert st == kb.KAMERA_ERR_WORKSPACE, msg                 # valid up to the workspace
    bad = kb.make_model("gqa", "bf16", 28, 4, 128, 128, "half_split", 1e6,
                        inv_freq=np.r_[np.ones(63), np.nan])
    assert call(model=bad)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    bad = kb.make_model("gqa", "bf16", 28, 4, 128, 128, "half_split", 1e6,
                        inv_freq=np.r_[np.ones(63), -1.0])
    assert call(model=bad)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    bad = kb.make_model("gqa", "bf16", 28, 4, 128, 128, "half_split", 1e6,
                        pair_section=np.repeat([0, 1, 2], [16, 24, 24]))
    bad.n_sections = 2                                        # entry 2 is not below 2
    assert call(model=bad)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    part = kb.make_model("gqa", "bf16", 28, 4, 128, 64, "half_split", 1e6)
    assert call(model=part)[0] == kb.KAMERA_ERR_WORKSPACE     # partial rotary is accepted


def test_section_shifts_are_range_checked():
    import numpy as np
    m = kb.make_model("gqa", "bf16", 28, 4, 128, 128, "half_split", 1e6,
                      pair_section=np.repeat([0, 1, 2], [16, 24, 24]))
    ch = _chunks(1)
    ch[0].delta_sections[1] = 1 << 31
    st, msg = call(model=m, chunks=ch)
    assert st == kb.KAMERA_ERR_INVALID_ARGUMENT and "delta_sections" in msg
    plain = _model()                                           # no sections: not read
    assert call(model=plain, chunks=ch)[0] == kb.KAMERA_ERR_WORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=0), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(n_pages=0), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(n_logical_pages=0), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(n_logical_pages=1001), kb.KAMERA_ERR_INVALID_ARGUMENT),  # identity table too short
    (dict(token_stride=256), kb.KAMERA_ERR_INVALID_ARGUMENT),      # row of 4x128 does not fit
    (dict(layer_stride=10), kb.KAMERA_ERR_INVALID_ARGUMENT),
])
def test_cache_validation(kw, status):
    st, msg = call(cache=_cache(**kw))
    assert st == status, msg


def test_cache_pool_null_and_overlapping_pools():
    c = _cache()
    c.pool[1] = None
    assert call(cache=c)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    c = _cache()
    c.pool[1] = FAKE + 64          # second pool overlaps the first one's rows
    assert call(cache=c)[0] == kb.KAMERA_ERR_OVERLAP


def test_mla_pools_sharing_rows_are_accepted_until_the_workspace_check():
    """MLA stores c_KV and k_rope in one row: pool[1] = base, pool[0] = base + 512 elements."""
    model = _model(family=1, n_kv_heads=1, head_dim=512, rope_dim=64, n_layers=27,
                   rope_theta=1e4)
    c = _cache(token_stride=576, layer_stride=1000 * 16 * 576)
    c.pool[1] = FAKE
    c.pool[0] = FAKE + 512 * 2
    st, msg = call(model=model, cache=c)
    assert st == kb.KAMERA_ERR_WORKSPACE, msg


def test_chunk_validation():
    assert call(chunks=_chunks(1, n_tokens=-1))[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert call(chunks=_chunks(1, dst_token_offset=-3))[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    # past the cache's 16000 logical tokens
    assert call(chunks=_chunks(1, dst_token_offset=15950))[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert call(chunks=_chunks(1, delta=1 << 31))[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert call(chunks=_chunks(1, delta=-(1 << 31)))[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    st, msg = call(chunks=_chunks(1), n=-1)
    assert st == kb.KAMERA_ERR_INVALID_ARGUMENT
    st, msg = call(chunks=_chunks(1), n=0)   # zero chunks is valid: reaches the workspace check
    assert st == kb.KAMERA_ERR_WORKSPACE


def test_chunk_src_problems():
    ch = _chunks(1)
    ch[0].src[1] = kb.KameraSrc(None, 0, 512)
    assert call(chunks=ch)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(1)
    ch[0].src[0] = kb.KameraSrc(FAKE + (1 << 38), 100 * 512, 100)     # row of 512 does not fit
    assert call(chunks=ch)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(1)
    ch[0].src[0] = kb.KameraSrc(FAKE + 4096, 100 * 512, 512)          # inside the K pool
    assert call(chunks=ch)[0] == kb.KAMERA_ERR_OVERLAP


def test_patch_problems():
    ch = _chunks(1)
    ch[0].patch[0] = kb.KameraPatchRef(-1)
    assert call(chunks=ch)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(1)
    ch[0].patch[0] = kb.KameraPatchRef(kb.MAX_RANK + 1, 0, FAKE, 0, 0, FAKE, 0, 0)
    assert call(chunks=ch)[0] == kb.KAMERA_ERR_UNSUPPORTED
    ch = _chunks(1)
    ch[0].patch[1] = kb.KameraPatchRef(8, 0, None, 0, 0, FAKE + (1 << 40), 0, 0)
    assert call(chunks=ch)[0] == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(1)
    ch[0].patch[1] = kb.KameraPatchRef(8, 0, FAKE + 100, 0, 0, FAKE + (1 << 40), 0, 0)
    assert call(chunks=ch)[0] == kb.KAMERA_ERR_OVERLAP                # U inside the K pool
    # relocate ignores the patch fields entirely
    ch = _chunks(1)
    ch[0].patch[0] = kb.KameraPatchRef(-1)
    assert call(chunks=ch, fn="kamera_relocate")[0] == kb.KAMERA_ERR_WORKSPACE


def test_patch_mode_ignores_src():
    ch = _chunks(1)
    ch[0].src[0] = kb.KameraSrc(None, 0, 0)
    assert call(chunks=ch, fn="kamera_patch")[0] == kb.KAMERA_ERR_WORKSPACE


def test_two_chunks_writing_one_token_are_rejected():
    ch = _chunks(2)
    ch[1].dst_token_offset = 50
    st, msg = call(chunks=ch, n=2)
    assert st == kb.KAMERA_ERR_INVALID_ARGUMENT and "token" in msg


def test_last_error_is_cleared_by_a_later_call_and_is_per_thread():
    import threading
    call(model=_model(family=7))
    assert "family" in kb.kamera_last_error()
    seen = []
    t = threading.Thread(target=lambda: seen.append(kb.kamera_last_error()))
    t.start()
    t.join()
    assert seen == [""]
    call()
    assert "workspace" in kb.kamera_last_error()


def test_workloads_plans_are_consistent():
    """The seeded plans: destinations disjoint and inside the cache, table a partial
    permutation, shapes as described."""
    import numpy as np
    for name in wl.PLANS:
        p = wl.plan(name)
        spans = sorted((o, o + n) for o, n in zip(p.dst_offsets, p.chunk_tokens))
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert spans[-1][1] <= p.n_logical_pages * p.page_size
        if p.page_table is not None:
            assert len(np.unique(p.page_table)) == p.n_logical_pages
            assert p.page_table.max() < p.n_pages
    w = wl.plan("qwen3vl_window_bf16")
    assert sum(m > 0 for m in w.m_rot) == 64 and len(w.m_rot) == 256
    k = w.notes["slide_k"]
    for d, m in zip(w.deltas, w.m_rot):
        assert (d == -k * 256) if m == 0 else (d >= 0 and d % 256 == 0)
    r = wl.plan("mha7b_reorder_bf16")
    assert sorted(r.dst_offsets) == [4096 * i for i in range(16)] and r.deltas == r.dst_offsets
    q = wl.plan("qwen25vl_gqa_bf16")
    assert all(-32768 <= d <= 32768 for d in q.deltas)
    assert wl.plan("qwen25vl_gqa_bf16").deltas == q.deltas          # seeded


def test_a_batch_past_the_grid_limit_is_rejected_before_any_device_call():
    """One fp32 chunk of 2^30 tokens would need more than 2^23 blocks of the VALU kernel (64
    tokens each): the plan refuses it (UNSUPPORTED) instead of launching an oversized grid."""
    model = _model(dtype=0, n_layers=1, n_kv_heads=1, head_dim=128, rope_dim=128)
    n = 1 << 30
    cache = _cache(layer_stride=n * 128, token_stride=128, n_logical_pages=n // 16,
                   n_pages=n // 16, pool=(ctypes.c_void_p * 2)(FAKE, FAKE + (1 << 42)))
    ch = (kb.KameraChunk * 1)()
    ch[0].n_tokens = n
    ch[0].delta = 3
    for c in range(2):
        ch[0].src[c] = kb.KameraSrc(FAKE + (1 << 43) + (c << 41), n * 128, 128)
    need = kb.kamera_workspace_bytes(1)
    st, msg = call(model, cache, ch, 1, ws=FAKE + (1 << 44), ws_bytes=need)
    assert st == kb.KAMERA_ERR_UNSUPPORTED and "2^23" in msg
