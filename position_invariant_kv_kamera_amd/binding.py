"""ctypes binding of libkamera.so (include/kamera.h): argument marshalling only.

The functions keep the C names. Every step of the operator runs in the library's HIP kernels;
PyTorch is used only for device memory and streams. If libkamera.so is missing this module
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import re
from pathlib import Path

PKG = Path(__file__).resolve().parent
# KAMERA_LIBRARY selects another build of the same library (e.g. one built with different
# tuning macros); the default is the in-tree build.
LIB_PATH = Path(os.environ.get("KAMERA_LIBRARY", PKG / "libkamera.so"))
HEADER = PKG.parent / "include" / "kamera.h"

KAMERA_OK = 0
KAMERA_ERR_INVALID_ARGUMENT = 1
KAMERA_ERR_UNSUPPORTED = 2
KAMERA_ERR_OVERLAP = 3
KAMERA_ERR_WORKSPACE = 4
KAMERA_ERR_HIP = 5
KAMERA_ERR_BUSY = 6

FAMILY = {"gqa": 0, "mla": 1}
DTYPE = {"f32": 0, "bf16": 1}
LAYOUT = {"half_split": 0, "interleaved": 1}
MAX_RANK = 256

c_i32, c_i64, c_dbl, c_vp, c_size = (ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                      ctypes.c_void_p, ctypes.c_size_t)


class KameraModel(ctypes.Structure):
    _fields_ = [("family", c_i32), ("dtype", c_i32), ("n_layers", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("rope_dim", c_i32), ("rope_layout", c_i32),
                ("n_sections", c_i32), ("rope_theta", c_dbl), ("inv_freq", c_vp),
                ("pair_section", c_vp)]


class KameraCache(ctypes.Structure):
    _fields_ = [("pool", c_vp * 2), ("layer_stride", c_i64), ("token_stride", c_i64),
                ("page_table", c_vp), ("n_logical_pages", c_i32), ("page_size", c_i32),
                ("n_pages", c_i32), ("reserved0", c_i32)]


class KameraSrc(ctypes.Structure):
    _fields_ = [("ptr", c_vp), ("layer_stride", c_i64), ("token_stride", c_i64)]


class KameraPatchRef(ctypes.Structure):
    _fields_ = [("m", c_i32), ("reserved0", c_i32), ("U", c_vp), ("u_layer_stride", c_i64),
                ("u_head_stride", c_i64), ("V", c_vp), ("v_layer_stride", c_i64),
                ("v_head_stride", c_i64)]


class KameraChunk(ctypes.Structure):
    _fields_ = [("n_tokens", c_i32), ("dst_token_offset", c_i32), ("delta", c_i64),
                ("delta_sections", c_i64 * 2), ("src", KameraSrc * 2),
                ("patch", KameraPatchRef * 2)]


class KameraFactorsOut(ctypes.Structure):
    _fields_ = [("U", c_vp), ("u_layer_stride", c_i64), ("u_head_stride", c_i64),
                ("V", c_vp), ("v_layer_stride", c_i64), ("v_head_stride", c_i64)]


class KameraCompileChunk(ctypes.Structure):
    _fields_ = [("n_tokens", c_i32), ("m", c_i32), ("delta", c_i64),
                ("delta_sections", c_i64 * 2),
                ("canonical", KameraSrc * 2), ("conditioned", KameraSrc * 2),
                ("out", KameraFactorsOut * 2)]


COMPILE_MAX_RANK = 64
ORBIT_MAX_MEMBERS = 64
ATTN_SEGMENT = 512


class KameraAttnQuery(ctypes.Structure):
    _fields_ = [("kv_start", c_i32), ("kv_len", c_i32)]


class KameraAttnChunk(ctypes.Structure):
    _fields_ = [("n_tokens", c_i32), ("reserved0", c_i32), ("delta", c_i64),
                ("delta_sections", c_i64 * 2), ("src", KameraSrc * 2),
                ("patch", KameraPatchRef * 2)]


class KameraChunkQuery(ctypes.Structure):
    _fields_ = [("first_chunk", c_i32), ("n_chunks", c_i32)]


class KameraOrbitMember(ctypes.Structure):
    _fields_ = [("delta", c_i64), ("delta_sections", c_i64 * 2), ("conditioned", KameraSrc * 2)]


class KameraOrbitChunk(ctypes.Structure):
    _fields_ = [("n_tokens", c_i32), ("m", c_i32), ("n_members", c_i32), ("reserved0", c_i32),
                ("members", ctypes.POINTER(KameraOrbitMember)), ("canonical", KameraSrc * 2),
                ("out", KameraFactorsOut * 2)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libkamera.so from the package directory; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m position_invariant_kv_kamera_amd.build` (there is no "
                           "fallback path)")
    lib = ctypes.CDLL(str(LIB_PATH))
    compute = [ctypes.POINTER(KameraModel), ctypes.POINTER(KameraCache),
               ctypes.POINTER(KameraChunk), c_i32, c_vp, c_size, c_vp]
    for name in ("kamera_reuse_batch", "kamera_relocate", "kamera_patch"):
        fn = getattr(lib, name)
        fn.argtypes = compute
        fn.restype = ctypes.c_int
    lib.kamera_reuse_batch_noalloc.argtypes = [ctypes.POINTER(KameraModel),
                                                ctypes.POINTER(KameraCache),
                                                ctypes.POINTER(KameraChunk), c_i32, c_vp]
    lib.kamera_reuse_batch_noalloc.restype = ctypes.c_int
    lib.kamera_init.argtypes = []
    lib.kamera_init.restype = ctypes.c_int
    lib.kamera_workspace_bytes.argtypes = [c_i32]
    lib.kamera_workspace_bytes.restype = c_size
    lib.kamera_read_fault_count.argtypes = [c_vp, c_vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.kamera_read_fault_count.restype = ctypes.c_int
    lib.kamera_patch_bytes.argtypes = [ctypes.POINTER(KameraModel), c_i32, c_i32]
    lib.kamera_patch_bytes.restype = c_size
    lib.kamera_kv_bytes.argtypes = [ctypes.POINTER(KameraModel), c_i32]
    lib.kamera_kv_bytes.restype = c_size
    lib.kamera_status_string.argtypes = [ctypes.c_int]
    lib.kamera_status_string.restype = ctypes.c_char_p
    lib.kamera_last_error.argtypes = []
    lib.kamera_last_error.restype = ctypes.c_char_p
    lib.kamera_version.argtypes = []
    lib.kamera_version.restype = c_i32
    lib.kamera_compile_workspace_bytes.argtypes = [ctypes.POINTER(KameraModel),
                                                   ctypes.POINTER(KameraCompileChunk), c_i32]
    lib.kamera_compile_workspace_bytes.restype = c_size
    lib.kamera_patch_compile.argtypes = [ctypes.POINTER(KameraModel),
                                         ctypes.POINTER(KameraCompileChunk), c_i32, c_i32, c_vp,
                                         c_size, c_vp]
    lib.kamera_patch_compile.restype = ctypes.c_int
    lib.kamera_orbit_compile_workspace_bytes.argtypes = [ctypes.POINTER(KameraModel),
                                                         ctypes.POINTER(KameraOrbitChunk), c_i32]
    lib.kamera_orbit_compile_workspace_bytes.restype = c_size
    lib.kamera_patch_compile_orbit.argtypes = [ctypes.POINTER(KameraModel),
                                               ctypes.POINTER(KameraOrbitChunk), c_i32, c_i32,
                                               c_vp, c_size, c_vp]
    lib.kamera_patch_compile_orbit.restype = ctypes.c_int
    lib.kamera_attention_workspace_bytes.argtypes = [ctypes.POINTER(KameraModel), c_i32,
                                                     ctypes.POINTER(KameraAttnQuery), c_i32]
    lib.kamera_attention_workspace_bytes.restype = c_size
    lib.kamera_decode_attention.argtypes = [ctypes.POINTER(KameraModel),
                                            ctypes.POINTER(KameraCache), c_i32, c_vp, c_i32,
                                            ctypes.POINTER(KameraAttnQuery), c_i32,
                                            ctypes.c_float, c_vp, c_vp, c_vp, c_size, c_vp]
    lib.kamera_decode_attention.restype = ctypes.c_int
    lib.kamera_state_merge.argtypes = [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.kamera_state_merge.restype = ctypes.c_int
    lib.kamera_chunk_attention_workspace_bytes.argtypes = [
        ctypes.POINTER(KameraModel), c_i32, ctypes.POINTER(KameraAttnChunk), c_i32,
        ctypes.POINTER(KameraChunkQuery), c_i32]
    lib.kamera_chunk_attention_workspace_bytes.restype = c_size
    lib.kamera_chunk_attention.argtypes = [
        ctypes.POINTER(KameraModel), c_i32, ctypes.POINTER(KameraAttnChunk), c_i32,
        ctypes.POINTER(KameraChunkQuery), c_i32, c_vp, c_i32, ctypes.c_float, c_vp, c_vp, c_vp,
        c_size, c_vp]
    lib.kamera_chunk_attention.restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/kamera.h declares."""
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(kamera_[a-z_]+)\s*\(",
                                 text, re.M)))


class KameraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kamera status {status}: {message}")
        self.status = status


# ---- the C calls, same names -----------------------------------------------------------

def kamera_init() -> int:
    return int(load_library().kamera_init())


def kamera_workspace_bytes(n_chunks: int) -> int:
    return int(load_library().kamera_workspace_bytes(n_chunks))


def _compute(name, model, cache, chunks, n_chunks, workspace, workspace_bytes, stream):
    fn = getattr(load_library(), name)
    return int(fn(ctypes.byref(model) if model is not None else None,
                  ctypes.byref(cache) if cache is not None else None,
                  chunks, int(n_chunks), workspace, int(workspace_bytes), stream))


def kamera_reuse_batch(model, cache, chunks, n_chunks, workspace, workspace_bytes, stream):
    return _compute("kamera_reuse_batch", model, cache, chunks, n_chunks, workspace,
                    workspace_bytes, stream)


def kamera_reuse_batch_noalloc(model, cache, chunks, n_chunks, stream):
    return int(load_library().kamera_reuse_batch_noalloc(
        ctypes.byref(model) if model is not None else None,
        ctypes.byref(cache) if cache is not None else None, chunks, int(n_chunks), stream))


def kamera_relocate(model, cache, chunks, n_chunks, workspace, workspace_bytes, stream):
    return _compute("kamera_relocate", model, cache, chunks, n_chunks, workspace,
                    workspace_bytes, stream)


def kamera_patch(model, cache, chunks, n_chunks, workspace, workspace_bytes, stream):
    return _compute("kamera_patch", model, cache, chunks, n_chunks, workspace,
                    workspace_bytes, stream)


def kamera_read_fault_count(workspace, stream) -> tuple[int, int]:
    out = ctypes.c_uint32(0)
    st = int(load_library().kamera_read_fault_count(workspace, stream, ctypes.byref(out)))
    return st, int(out.value)


def kamera_patch_bytes(model, n_tokens, m) -> int:
    return int(load_library().kamera_patch_bytes(ctypes.byref(model), n_tokens, m))


def kamera_kv_bytes(model, n_tokens) -> int:
    return int(load_library().kamera_kv_bytes(ctypes.byref(model), n_tokens))


def kamera_status_string(status: int) -> str:
    return load_library().kamera_status_string(status).decode()


def kamera_last_error() -> str:
    return load_library().kamera_last_error().decode()


def kamera_version() -> int:
    return int(load_library().kamera_version())


def kamera_compile_workspace_bytes(model, chunks, n_chunks) -> int:
    return int(load_library().kamera_compile_workspace_bytes(
        ctypes.byref(model) if model is not None else None, chunks, int(n_chunks)))


def kamera_patch_compile(model, chunks, n_chunks, n_iter, workspace, workspace_bytes, stream):
    return int(load_library().kamera_patch_compile(
        ctypes.byref(model) if model is not None else None, chunks, int(n_chunks), int(n_iter),
        workspace, int(workspace_bytes), stream))


def kamera_orbit_compile_workspace_bytes(model, chunks, n_chunks) -> int:
    return int(load_library().kamera_orbit_compile_workspace_bytes(
        ctypes.byref(model) if model is not None else None, chunks, int(n_chunks)))


def kamera_patch_compile_orbit(model, chunks, n_chunks, n_iter, workspace, workspace_bytes,
                               stream):
    return int(load_library().kamera_patch_compile_orbit(
        ctypes.byref(model) if model is not None else None, chunks, int(n_chunks), int(n_iter),
        workspace, int(workspace_bytes), stream))


def kamera_attention_workspace_bytes(model, n_q_heads, queries, n_queries) -> int:
    return int(load_library().kamera_attention_workspace_bytes(
        ctypes.byref(model) if model is not None else None, int(n_q_heads), queries,
        int(n_queries)))


def kamera_decode_attention(model, cache, layer, q, n_q_heads, queries, n_queries, scale, out,
                            lse, workspace, workspace_bytes, stream):
    return int(load_library().kamera_decode_attention(
        ctypes.byref(model) if model is not None else None,
        ctypes.byref(cache) if cache is not None else None, int(layer), q, int(n_q_heads),
        queries, int(n_queries), float(scale), out, lse, workspace, int(workspace_bytes), stream))


def kamera_state_merge(n_parts, n_rows, head_dim, part_out, part_lse, out, lse, stream):
    return int(load_library().kamera_state_merge(int(n_parts), int(n_rows), int(head_dim),
                                                 part_out, part_lse, out, lse, stream))


# ---- marshalling of torch tensors (workloads.Batch) into descriptors --------------------

def make_model(family, dtype, n_layers, n_kv_heads, head_dim, rope_dim, rope_layout, theta, *,
               inv_freq=None, pair_section=None) -> KameraModel:
    """A KameraModel; the optional host tables are copied and kept alive by the struct."""
    import numpy as np
    m = KameraModel(FAMILY.get(family, family), DTYPE.get(dtype, dtype), n_layers, n_kv_heads,
                    head_dim, rope_dim, LAYOUT.get(rope_layout, rope_layout), 0, float(theta),
                    None, None)
    if inv_freq is not None:
        m._inv_freq = np.ascontiguousarray(inv_freq, np.float64)
        m.inv_freq = m._inv_freq.ctypes.data
    if pair_section is not None:
        m._pair_section = np.ascontiguousarray(pair_section, np.uint8)
        m.pair_section = m._pair_section.ctypes.data
        m.n_sections = int(m._pair_section.max()) + 1 if m._pair_section.size else 0
    return m


def model_of(plan) -> KameraModel:
    m = make_model(plan.family, plan.dtype, plan.n_layers, plan.n_kv_heads, plan.head_dim,
                   plan.rope_dim, plan.rope_layout, plan.theta,
                   inv_freq=getattr(plan, "inv_freq", None),
                   pair_section=getattr(plan, "pair_section", None))
    if getattr(plan, "n_sections", None):
        m.n_sections = int(plan.n_sections)
    return m


def cache_of(batch) -> KameraCache:
    p = batch.plan
    pools = batch.pools
    c = KameraCache()
    c.pool[0] = pools[0].data_ptr()
    c.pool[1] = pools[1].data_ptr()
    c.layer_stride = pools[0].stride(0)
    c.token_stride = pools[0].stride(2)
    c.page_table = None if batch.page_table is None else batch.page_table.data_ptr()
    c.n_logical_pages = p.n_logical_pages
    c.page_size = p.page_size
    c.n_pages = p.n_pages
    return c


def chunks_of(batch, m_override: int | None = None):
    """One KameraChunk per chunk of the batch (ctypes array)."""
    p = batch.plan
    arr = (KameraChunk * max(1, p.n_chunks))()
    for c, ct in enumerate(batch.chunks):
        k = arr[c]
        k.n_tokens = p.chunk_tokens[c]
        k.dst_token_offset = p.dst_offsets[c]
        k.delta = p.deltas[c]
        ds = getattr(p, "delta_sections", None)
        if ds is not None:
            k.delta_sections[0], k.delta_sections[1] = int(ds[c][0]), int(ds[c][1])
        for ch in range(2):
            s = ct.src[ch]
            k.src[ch] = KameraSrc(s.data_ptr(), s.stride(0), s.stride(1))
            U, V = ct.U[ch], ct.V[ch]
            if U is not None and m_override != 0:
                k.patch[ch] = KameraPatchRef(U.shape[-1], 0, U.data_ptr(), U.stride(0),
                                             U.stride(1), V.data_ptr(), V.stride(0), V.stride(1))
            else:
                k.patch[ch] = KameraPatchRef()
    return arr


class Workspace:
    """Device workspace for up to `n_chunks` chunks (torch uint8 tensor, 256-byte aligned), or
    of `nbytes` bytes when given."""

    def __init__(self, n_chunks: int = 0, device="cuda", *, nbytes: int | None = None):
        import torch
        self.nbytes = kamera_workspace_bytes(n_chunks) if nbytes is None else int(nbytes)
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        base = self._buf.data_ptr()
        self.ptr = (base + 255) // 256 * 256


def current_stream_ptr():
    import torch
    return torch.cuda.current_stream().cuda_stream


def check(status: int):
    if status != KAMERA_OK:
        raise KameraError(status, f"{kamera_status_string(status)}: {kamera_last_error()}")


def run_batch(op: str, batch, workspace: Workspace | None = None, stream=None, *,
              m_override: int | None = None):
    """Describe `batch` and run one of "reuse", "relocate", "patch" on it (asynchronous)."""
    model = model_of(batch.plan)
    cache = cache_of(batch)
    chunks = chunks_of(batch, m_override)
    ws = workspace or Workspace(batch.plan.n_chunks)
    s = current_stream_ptr() if stream is None else stream
    fn = {"reuse": kamera_reuse_batch, "relocate": kamera_relocate, "patch": kamera_patch}[op]
    check(fn(model, cache, chunks, batch.plan.n_chunks, ws.ptr, ws.nbytes, s))
    return ws


# ---- patch compile ------------------------------------------------------------------------

class CompileItem:
    """Tensors of one chunk to compile. Per channel c: canonical[c] and conditioned[c] are
    [layers, tokens, heads*width] views (unit inner stride); U[c] is [layers, heads, tokens, m]
    and V[c] [layers, heads, width, m], written by the call."""

    def __init__(self, n_tokens, m, delta, canonical, conditioned, U, V, delta_sections=(0, 0)):
        self.n_tokens, self.m, self.delta = int(n_tokens), int(m), int(delta)
        self.delta_sections = tuple(int(d) for d in delta_sections)
        self.canonical, self.conditioned, self.U, self.V = canonical, conditioned, U, V


def compile_chunks_of(items):
    arr = (KameraCompileChunk * max(1, len(items)))()
    for i, it in enumerate(items):
        k = arr[i]
        k.n_tokens, k.m, k.delta = it.n_tokens, it.m, it.delta
        k.delta_sections[0], k.delta_sections[1] = it.delta_sections
        for ch in range(2):
            a, b = it.canonical[ch], it.conditioned[ch]
            k.canonical[ch] = KameraSrc(a.data_ptr(), a.stride(0), a.stride(1))
            k.conditioned[ch] = KameraSrc(b.data_ptr(), b.stride(0), b.stride(1))
            U, V = it.U[ch], it.V[ch]
            k.out[ch] = KameraFactorsOut(U.data_ptr(), U.stride(0), U.stride(1), V.data_ptr(),
                                         V.stride(0), V.stride(1))
    return arr


def run_compile(model: KameraModel, items, *, n_iter: int = 8, workspace: Workspace | None = None,
                stream=None) -> Workspace:
    """kamera_patch_compile over `items` (asynchronous on the stream); returns the workspace."""
    chunks = compile_chunks_of(items)
    need = kamera_compile_workspace_bytes(model, chunks, len(items))
    if need == 0:
        raise KameraError(KAMERA_ERR_INVALID_ARGUMENT, kamera_last_error())
    ws = workspace if workspace is not None and workspace.nbytes >= need else Workspace(nbytes=need)
    s = current_stream_ptr() if stream is None else stream
    check(kamera_patch_compile(model, chunks, len(items), n_iter, ws.ptr, ws.nbytes, s))
    return ws


class OrbitItem:
    """One chunk of an orbit compile: canonical[c] as in CompileItem, `members` a list of
    (delta, conditioned) or (delta, conditioned, delta_sections) per ordering, conditioned a
    per-channel list of [layers, tokens, heads*width] views; U, V outputs as in CompileItem."""

    def __init__(self, n_tokens, m, canonical, members, U, V):
        self.n_tokens, self.m = int(n_tokens), int(m)
        self.canonical, self.members, self.U, self.V = canonical, members, U, V


def orbit_chunks_of(items):
    arr = (KameraOrbitChunk * max(1, len(items)))()
    keep = []
    for i, it in enumerate(items):
        k = arr[i]
        k.n_tokens, k.m, k.n_members = it.n_tokens, it.m, len(it.members)
        mem = (KameraOrbitMember * max(1, len(it.members)))()
        for q, entry in enumerate(it.members):
            delta, cond = entry[0], entry[1]
            ds = entry[2] if len(entry) > 2 else (delta, delta)
            mem[q].delta = int(delta)
            mem[q].delta_sections[0], mem[q].delta_sections[1] = int(ds[0]), int(ds[1])
            for ch in range(2):
                mem[q].conditioned[ch] = KameraSrc(cond[ch].data_ptr(), cond[ch].stride(0),
                                                   cond[ch].stride(1))
        keep.append(mem)
        k.members = ctypes.cast(mem, ctypes.POINTER(KameraOrbitMember))
        for ch in range(2):
            a = it.canonical[ch]
            k.canonical[ch] = KameraSrc(a.data_ptr(), a.stride(0), a.stride(1))
            U, V = it.U[ch], it.V[ch]
            k.out[ch] = KameraFactorsOut(U.data_ptr(), U.stride(0), U.stride(1), V.data_ptr(),
                                         V.stride(0), V.stride(1))
    arr._keep = keep
    return arr


def run_orbit_compile(model: KameraModel, items, *, n_iter: int = 8,
                      workspace: Workspace | None = None, stream=None) -> Workspace:
    """kamera_patch_compile_orbit over `items` (asynchronous on the stream)."""
    chunks = orbit_chunks_of(items)
    need = kamera_orbit_compile_workspace_bytes(model, chunks, len(items))
    if need == 0:
        raise KameraError(KAMERA_ERR_INVALID_ARGUMENT, kamera_last_error())
    ws = workspace if workspace is not None and workspace.nbytes >= need else Workspace(nbytes=need)
    s = current_stream_ptr() if stream is None else stream
    check(kamera_patch_compile_orbit(model, chunks, len(items), n_iter, ws.ptr, ws.nbytes, s))
    return ws


# ---- consumer side ---------------------------------------------------------------------------

def kamera_chunk_attention_workspace_bytes(model, n_q_heads, chunks, n_chunks, queries,
                                           n_queries) -> int:
    return int(load_library().kamera_chunk_attention_workspace_bytes(
        ctypes.byref(model) if model is not None else None, int(n_q_heads), chunks,
        int(n_chunks), queries, int(n_queries)))


def kamera_chunk_attention(model, layer, chunks, n_chunks, queries, n_queries, q, n_q_heads,
                           scale, out, lse, workspace, workspace_bytes, stream):
    return int(load_library().kamera_chunk_attention(
        ctypes.byref(model) if model is not None else None, int(layer), chunks, int(n_chunks),
        queries, int(n_queries), q, int(n_q_heads), float(scale), out, lse, workspace,
        int(workspace_bytes), stream))


def attn_chunks_of(items):
    """A KameraAttnChunk array from dicts: 'n_tokens', 'delta', optional 'delta_sections',
    'src' (two (ptr, layer_stride, token_stride)), optional 'patch' (two
    (m, U ptr, u_layer_stride, u_head_stride, V ptr, v_layer_stride, v_head_stride) or None)."""
    arr = (KameraAttnChunk * max(1, len(items)))()
    for i, it in enumerate(items):
        c = KameraAttnChunk()
        c.n_tokens = int(it["n_tokens"])
        c.delta = int(it["delta"])
        ds = it.get("delta_sections", (it["delta"], it["delta"]))
        c.delta_sections[0], c.delta_sections[1] = int(ds[0]), int(ds[1])
        for ch in range(2):
            ptr, ls, ts = it["src"][ch]
            c.src[ch] = KameraSrc(ptr, int(ls), int(ts))
            pr = (it.get("patch") or (None, None))[ch]
            if pr is not None:
                m, U, uls, uhs, V, vls, vhs = pr
                c.patch[ch] = KameraPatchRef(int(m), 0, U, int(uls), int(uhs), V, int(vls),
                                             int(vhs))
        arr[i] = c
    return arr


def chunk_queries_of(spans):
    """A KameraChunkQuery array from (first_chunk, n_chunks) pairs."""
    arr = (KameraChunkQuery * max(1, len(spans)))()
    for i, (a, n) in enumerate(spans):
        arr[i] = KameraChunkQuery(int(a), int(n))
    return arr


def run_chunk_attention(model: KameraModel, layer: int, chunk_items, spans, q, scale, *,
                        stream=None):
    """kamera_chunk_attention of q ([n_queries, n_q_heads, head_dim] bf16 device tensor), query j
    over chunks spans[j] = (first, count) of chunk_items; returns (out fp32, lse)."""
    import torch
    n, heads, D = q.shape
    chunks = attn_chunks_of(chunk_items)
    queries = chunk_queries_of(spans)
    need = kamera_chunk_attention_workspace_bytes(model, heads, chunks, len(chunk_items), queries, n)
    if need == 0:
        raise KameraError(KAMERA_ERR_INVALID_ARGUMENT, kamera_last_error())
    ws = Workspace(nbytes=need, device=q.device)
    out = torch.empty((n, heads, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((n, heads), dtype=torch.float32, device=q.device)
    s = current_stream_ptr() if stream is None else stream
    check(kamera_chunk_attention(model, layer, chunks, len(chunk_items), queries, n,
                                 q.data_ptr(), heads, scale, out.data_ptr(), lse.data_ptr(),
                                 ws.ptr, ws.nbytes, s))
    out._kamera_ws = ws
    return out, lse


def attn_queries_of(ranges):
    """A KameraAttnQuery array from (kv_start, kv_len) pairs."""
    arr = (KameraAttnQuery * max(1, len(ranges)))()
    for i, (a, n) in enumerate(ranges):
        arr[i] = KameraAttnQuery(int(a), int(n))
    return arr


def run_decode_attention(model: KameraModel, cache: KameraCache, layer: int, q, ranges, scale,
                         *, stream=None):
    """kamera_decode_attention of q ([n_queries, n_q_heads, head_dim] bf16 device tensor; MLA:
    [.., 576] = [q_c | q_r]) over the given (kv_start, kv_len) ranges; returns
    (out [n, heads, head_dim] fp32, lse [n, heads])."""
    import torch
    n, heads, _ = q.shape
    D = model.head_dim                 # out rows: head_dim (MLA: the 512-wide latent)
    queries = attn_queries_of(ranges)
    need = kamera_attention_workspace_bytes(model, heads, queries, n)
    if need == 0:
        raise KameraError(KAMERA_ERR_INVALID_ARGUMENT, kamera_last_error())
    ws = Workspace(nbytes=need, device=q.device)
    out = torch.empty((n, heads, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((n, heads), dtype=torch.float32, device=q.device)
    s = current_stream_ptr() if stream is None else stream
    check(kamera_decode_attention(model, cache, layer, q.data_ptr(), heads, queries, n, scale,
                                  out.data_ptr(), lse.data_ptr(), ws.ptr, ws.nbytes, s))
    out._kamera_ws = ws                # keep the workspace alive until the caller syncs
    return out, lse
