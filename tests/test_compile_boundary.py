"""kamera_patch_compile at the C-ABI boundary, without a GPU: sizing and host validation.

Every compile call here is rejected by host validation before anything is enqueued; each
also passes a NULL workspace as a backstop (the workspace is checked after every other
argument), so no call in this file can reach a HIP launch.
"""
import ctypes

import pytest

from position_invariant_kv_kamera_amd import binding as kb

FAKE = 0x7F0000000000       # never dereferenced
GiB = 1 << 30


def _model(**kw):
    d = dict(family=0, dtype=1, n_layers=2, n_kv_heads=2, head_dim=128, rope_dim=128,
             rope_layout=0, n_sections=0, rope_theta=1e6)
    d.update(kw)
    return kb.KameraModel(**d)


def _mla(**kw):
    d = dict(family=1, n_kv_heads=1, head_dim=512, rope_dim=64, rope_theta=1e4)
    d.update(kw)
    return _model(**d)


def _row(model, ch):
    if model.family == 1:
        return model.rope_dim if ch == 0 else model.head_dim
    return model.n_kv_heads * model.head_dim


def _width(model, ch):
    if model.family == 1:
        return model.rope_dim if ch == 0 else model.head_dim
    return model.head_dim


def _chunks(model, n=1, n_tokens=300, m=16, delta=100):
    """n well-formed chunks: every tensor in its own 1 GiB slot of a fake address space."""
    arr = (kb.KameraCompileChunk * max(1, n))()
    heads = model.n_kv_heads if model.family == 0 else 1
    slot = 0

    def addr():
        nonlocal slot
        slot += 1
        return FAKE + slot * GiB

    for i in range(n):
        k = arr[i]
        k.n_tokens, k.m, k.delta = n_tokens, m, delta
        for ch in range(2):
            row = _row(model, ch)
            k.canonical[ch] = kb.KameraSrc(addr(), n_tokens * row, row)
            k.conditioned[ch] = kb.KameraSrc(addr(), n_tokens * row, row)
            w = _width(model, ch)
            k.out[ch] = kb.KameraFactorsOut(addr(), heads * n_tokens * m, n_tokens * m,
                                            addr(), heads * w * m, w * m)
    return arr


def _compile(model, chunks, n=1, n_iter=8, ws=None, nbytes=0):
    return kb.kamera_patch_compile(model, chunks, n, n_iter, ws, nbytes, None)


def test_compile_functions_are_exported():
    names = set(kb.header_functions())
    assert {"kamera_patch_compile", "kamera_compile_workspace_bytes"} <= names


def test_struct_sizes_match_the_header_layout():
    assert ctypes.sizeof(kb.KameraFactorsOut) == 48
    assert ctypes.sizeof(kb.KameraCompileChunk) == 32 + 2 * 24 + 2 * 24 + 2 * 48
    assert ctypes.sizeof(kb.KameraModel) == 56
    assert ctypes.sizeof(kb.KameraChunk) == 32 + 2 * 24 + 2 * 56


def test_well_formed_call_reaches_the_workspace_check():
    m = _model()
    ch = _chunks(m)
    assert _compile(m, ch) == kb.KAMERA_ERR_WORKSPACE
    need = kb.kamera_compile_workspace_bytes(m, ch, 1)
    assert need > 0 and need % 256 == 0
    assert _compile(m, ch, ws=FAKE + 8, nbytes=need) == kb.KAMERA_ERR_WORKSPACE   # misaligned
    assert _compile(m, ch, ws=None, nbytes=need) == kb.KAMERA_ERR_WORKSPACE
    mla = _mla()
    assert _compile(mla, _chunks(mla, m=32)) == kb.KAMERA_ERR_WORKSPACE


def test_workspace_bytes_closed_form():
    """Sizing depends on geometry only: partial Gram tiles per token split, the assembled G
    where there is more than one partial, and the fp32 basis (width x mp) per layer and head.
    Jobs with 64 or more Gram tiles do not split their tokens."""
    m = _model(n_layers=28, n_kv_heads=4)
    one = _chunks(m, n_tokens=1296, m=16)
    need = kb.kamera_compile_workspace_bytes(m, one, 1)
    units = 28 * 4
    per_ch = units * (128 * 128 + 128 * 16)                     # one split, one tile pair
    data = 2 * per_ch * 4
    assert data < need < data + 64 * 1024
    # 2 layers x 2 heads = 4 tiles per job: split into ceil(3000 / 1024) = 3 partials
    small = _model()
    ch3 = _chunks(small, n_tokens=3000, m=16)
    units = 2 * 2
    per_ch = units * (3 * 128 * 128 + 128 * 128 + 128 * 16)
    data = 2 * per_ch * 4
    got = kb.kamera_compile_workspace_bytes(small, ch3, 1)
    assert data < got < data + 64 * 1024
    two = _chunks(m, n=2, n_tokens=1296, m=16)
    assert kb.kamera_compile_workspace_bytes(m, two, 2) > need
    empty = _chunks(m, n_tokens=0)
    base = kb.kamera_compile_workspace_bytes(m, None, 0)      # the frequency / section tables
    assert 4096 < base <= 8192 and base % 256 == 0
    assert kb.kamera_compile_workspace_bytes(m, empty, 1) == base
    assert kb.kamera_compile_workspace_bytes(m, None, -1) == 0
    assert kb.kamera_compile_workspace_bytes(None, one, 1) == 0


@pytest.mark.parametrize("n_iter", [0, -1, 101])
def test_n_iter_range(n_iter):
    m = _model()
    assert _compile(m, _chunks(m), n_iter=n_iter) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert "n_iter" in kb.kamera_last_error()


@pytest.mark.parametrize("kw,chunk_kw,status", [
    ({}, dict(m=0), kb.KAMERA_ERR_INVALID_ARGUMENT),
    ({}, dict(m=-3), kb.KAMERA_ERR_INVALID_ARGUMENT),
    ({}, dict(m=65), kb.KAMERA_ERR_UNSUPPORTED),
    ({}, dict(n_tokens=-1), kb.KAMERA_ERR_INVALID_ARGUMENT),
    ({}, dict(delta=1 << 31), kb.KAMERA_ERR_INVALID_ARGUMENT),
    ({}, dict(delta=-(1 << 31)), kb.KAMERA_ERR_INVALID_ARGUMENT),
    (dict(head_dim=48, rope_dim=48), {}, kb.KAMERA_ERR_UNSUPPORTED),      # not a multiple of 32
    (dict(head_dim=256, rope_dim=256), {}, kb.KAMERA_ERR_UNSUPPORTED),    # rotated width > 128
    (dict(head_dim=32, rope_dim=32), dict(m=33), kb.KAMERA_ERR_INVALID_ARGUMENT),  # m > width
    (dict(head_dim=128, rope_dim=40), {}, kb.KAMERA_ERR_UNSUPPORTED),     # partial, 40 % 16
    (dict(head_dim=128, rope_dim=124), {}, kb.KAMERA_ERR_UNSUPPORTED),    # pass-through 4 wide
])
def test_geometry_validation(kw, chunk_kw, status):
    m = _model(**kw)
    args = dict(n_tokens=300, m=16, delta=100)
    args.update(chunk_kw)
    assert _compile(m, _chunks(m, **args)) == status
    assert kb.kamera_last_error()


def test_mla_latent_width_and_rank_limits():
    assert _compile(_mla(), _chunks(_mla(), m=33)) == kb.KAMERA_ERR_UNSUPPORTED   # 512 wide, m > 32
    assert _compile(_mla(head_dim=384), _chunks(_mla(head_dim=384))) == kb.KAMERA_ERR_WORKSPACE
    assert _compile(_mla(head_dim=320), _chunks(_mla(head_dim=320))) == kb.KAMERA_ERR_UNSUPPORTED
    assert _compile(_mla(head_dim=640), _chunks(_mla(head_dim=640))) == kb.KAMERA_ERR_UNSUPPORTED


def test_invalid_model_is_rejected_first():
    assert _compile(None, _chunks(_model())) == kb.KAMERA_ERR_INVALID_ARGUMENT
    bad = _model(rope_theta=0.5)
    assert _compile(bad, _chunks(bad)) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert _compile(_model(), None, n=1) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert _compile(_model(), None, n=-1) == kb.KAMERA_ERR_INVALID_ARGUMENT


def test_pointer_problems():
    m = _model()
    ch = _chunks(m)
    ch[0].canonical[1].ptr = None
    assert _compile(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(m)
    ch[0].out[0].V = None
    assert _compile(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(m)
    ch[0].conditioned[0].token_stride = 100          # shorter than the 256-element row
    assert _compile(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(m)
    ch[0].conditioned[0].ptr += 2                     # not on a 16-byte boundary
    assert _compile(m, ch) == kb.KAMERA_ERR_UNSUPPORTED
    ch = _chunks(m)
    ch[0].canonical[0].token_stride = 260             # 520 bytes: rows misaligned
    assert _compile(m, ch) == kb.KAMERA_ERR_UNSUPPORTED
    ch = _chunks(m)
    ch[0].out[1].u_head_stride = -1
    assert _compile(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT


def test_factor_strides_that_overlap_heads_or_layers():
    m = _model()
    ch = _chunks(m)
    ch[0].out[0].u_head_stride = 300 * 16 - 1         # heads overlap
    assert _compile(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(m)
    ch[0].out[0].v_layer_stride = 128 * 16            # layer 1 lands on head 1 of layer 0
    assert _compile(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _chunks(m)                                   # heads outer, layers inner: disjoint
    ch[0].out[0].u_layer_stride = 300 * 16
    ch[0].out[0].u_head_stride = 2 * 300 * 16
    assert _compile(m, ch) == kb.KAMERA_ERR_WORKSPACE


def test_outputs_overlapping_inputs_or_each_other():
    m = _model()
    ch = _chunks(m, n=2)
    ch[1].out[0].U = ch[0].conditioned[1].ptr + 64    # writes into another chunk's input
    assert _compile(m, ch, n=2) == kb.KAMERA_ERR_OVERLAP
    ch = _chunks(m, n=2)
    ch[1].out[1].V = ch[0].out[0].U                   # two outputs share memory
    assert _compile(m, ch, n=2) == kb.KAMERA_ERR_OVERLAP
    ch = _chunks(m, n=2)
    ch[0].out[0].V = ch[0].canonical[0].ptr           # in place is not supported
    assert _compile(m, ch, n=2) == kb.KAMERA_ERR_OVERLAP
    ch = _chunks(m, n=2)                              # inputs may alias each other
    ch[1].canonical[0].ptr = ch[0].canonical[0].ptr
    ch[1].conditioned[1].ptr = ch[0].canonical[0].ptr
    assert _compile(m, ch, n=2) == kb.KAMERA_ERR_WORKSPACE


def test_zero_token_chunks_are_skipped():
    m = _model()
    ch = _chunks(m, n=2)
    ch[1].n_tokens = 0
    ch[1].m = 999                                     # ignored: the chunk is skipped
    ch[1].out[0].U = None
    assert _compile(m, ch, n=2) == kb.KAMERA_ERR_WORKSPACE
    assert kb.kamera_compile_workspace_bytes(m, ch, 2) == kb.kamera_compile_workspace_bytes(
        m, _chunks(m), 1)


# ---- orbit compile -------------------------------------------------------------------------

def _orbit(model, n=1, n_members=3, n_tokens=300, m=16):
    """n well-formed orbit chunks in the fake address space, each with n_members orderings."""
    plain = _chunks(model, n=n, n_tokens=n_tokens, m=m)
    arr = (kb.KameraOrbitChunk * max(1, n))()
    keep = []
    slot = 10_000
    for i in range(n):
        k = arr[i]
        k.n_tokens, k.m, k.n_members = n_tokens, m, n_members
        mem = (kb.KameraOrbitMember * max(1, n_members))()
        for q in range(n_members):
            mem[q].delta = 10 * q
            for ch in range(2):
                slot += 1
                row = _row(model, ch)
                mem[q].conditioned[ch] = kb.KameraSrc(FAKE + slot * GiB, n_tokens * row, row)
        keep.append(mem)
        k.members = ctypes.cast(mem, ctypes.POINTER(kb.KameraOrbitMember))
        for ch in range(2):
            k.canonical[ch] = plain[i].canonical[ch]
            k.out[ch] = plain[i].out[ch]
    arr._keep = (keep, plain)
    return arr


def _orbit_call(model, chunks, n=1, n_iter=8):
    return kb.kamera_patch_compile_orbit(model, chunks, n, n_iter, None, 0, None)


def test_orbit_struct_layout():
    assert ctypes.sizeof(kb.KameraOrbitMember) == 8 + 16 + 2 * 24
    assert ctypes.sizeof(kb.KameraOrbitChunk) == 16 + 8 + 2 * 24 + 2 * 48


def test_orbit_well_formed_call_reaches_the_workspace_check():
    m = _model()
    assert _orbit_call(m, _orbit(m)) == kb.KAMERA_ERR_WORKSPACE
    mla = _mla()
    assert _orbit_call(mla, _orbit(mla, m=32)) == kb.KAMERA_ERR_WORKSPACE


def test_orbit_of_one_ordering_sizes_like_the_compile():
    m = _model()
    one = _orbit(m, n_members=1)
    plain = _chunks(m)
    assert kb.kamera_orbit_compile_workspace_bytes(m, one, 1) == \
        kb.kamera_compile_workspace_bytes(m, plain, 1)
    more = _orbit(m, n_members=6)
    # only the member table grows (48 bytes per ordering and channel), rounded to 256
    assert 0 <= kb.kamera_orbit_compile_workspace_bytes(m, more, 1) - \
        kb.kamera_compile_workspace_bytes(m, plain, 1) <= 1024


@pytest.mark.parametrize("n_members", [0, -1, 65])
def test_orbit_member_count(n_members):
    m = _model()
    ch = _orbit(m, n_members=3)
    ch[0].n_members = n_members
    assert _orbit_call(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    assert "n_members" in kb.kamera_last_error()


def test_orbit_member_problems():
    m = _model()
    ch = _orbit(m)
    ch[0].members = None
    assert _orbit_call(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _orbit(m)
    ch[0].members[1].conditioned[1].ptr = None
    assert _orbit_call(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _orbit(m)
    ch[0].members[2].conditioned[0].ptr += 4               # misaligned rows
    assert _orbit_call(m, ch) == kb.KAMERA_ERR_UNSUPPORTED
    ch = _orbit(m)
    ch[0].members[2].delta = 1 << 31
    assert _orbit_call(m, ch) == kb.KAMERA_ERR_INVALID_ARGUMENT
    ch = _orbit(m)
    ch[0].out[1].U = ch[0].members[1].conditioned[0].ptr   # output on a member's input
    assert _orbit_call(m, ch) == kb.KAMERA_ERR_OVERLAP
    ch = _orbit(m)
    ch[0].n_tokens = 0                                      # skipped: members not read
    ch[0].members = None
    assert _orbit_call(m, ch) == kb.KAMERA_ERR_WORKSPACE
    assert _orbit_call(m, ch, n_iter=0) == kb.KAMERA_ERR_INVALID_ARGUMENT
