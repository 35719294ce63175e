"""Plain fp64 CPU oracle of the Kamera reuse operator (ctypes over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg are
the only callers. Nothing in the product path imports this package, and this package imports
nothing from the product path.

The arithmetic lives in ``kamera_oracle.c`` (plain C, fp64, one term at a time). This module
marshals numpy arrays to it. See that file for the definition being computed: the reuse
equation of the Kamera technical summary, §2 Methodology, KV^(B|A) = R(delta) KV(B|empty) +
U_m V_m^T, with the rotation applied first and the patch added unrotated.

Element types: numpy float32 ("f32"), float64 ("f64", used by the pins), and uint16 holding
bf16 bit patterns ("bf16").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "kamera_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"

_DTYPE_CODE = {"f32": 0, "bf16": 1, "f64": 2}
_NP_DTYPE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}
HALF_SPLIT = 0
INTERLEAVED = 1

_lib = None


def build(force: bool = False) -> Path:
    """Compile liboracle.so with gcc (OpenMP, no fast-math, no FMA contraction)."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_suffix(f".so.tmp{os.getpid()}")
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        build()
    lib = ctypes.CDLL(str(_LIB_PATH))
    c_i32, c_i64, c_dbl, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.kamera_oracle_threads.restype = ctypes.c_int
    lib.kamera_oracle_inv_freq.argtypes = [c_dbl, c_i32, c_vp]
    lib.kamera_oracle_phase.argtypes = [c_i64, c_dbl, c_i32, c_vp, c_vp]
    lib.kamera_oracle_segment.argtypes = [c_i32, c_vp, c_i64, c_i32, c_i32, c_i32, c_i32, c_i64,
                                          c_dbl, c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp]
    lib.kamera_oracle_segment.restype = ctypes.c_int
    lib.kamera_oracle_segment_ex.argtypes = [c_i32, c_vp, c_i64, c_i32, c_i32, c_i32, c_i32,
                                             c_i32, c_vp, c_vp, c_i64, c_dbl, c_i32, c_vp,
                                             c_i64, c_vp, c_i64, c_vp, c_vp]
    lib.kamera_oracle_segment_ex.restype = ctypes.c_int
    lib.kamera_oracle_to_f32.argtypes = [c_vp, c_i64, c_vp]
    lib.kamera_oracle_to_bf16.argtypes = [c_vp, c_i64, c_vp]
    lib.kamera_oracle_slots.argtypes = [c_vp, c_i32, c_i32, c_i64, c_i32, c_vp]
    lib.kamera_oracle_slots.restype = ctypes.c_int
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().kamera_oracle_threads())


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def dtype_of(a: np.ndarray) -> str:
    for name, npd in _NP_DTYPE.items():
        if a.dtype == npd:
            return name
    raise TypeError(f"oracle: unsupported element type {a.dtype}")


def inv_freq(theta: float, rot_dim: int) -> np.ndarray:
    """theta_i = theta^(-2i/rot_dim) for every pair i (fp64)."""
    out = np.empty(rot_dim // 2, np.float64)
    _load().kamera_oracle_inv_freq(float(theta), int(rot_dim), _ptr(out))
    return out


def phase(delta: int, theta: float, rot_dim: int) -> tuple[np.ndarray, np.ndarray]:
    """cos and sin of delta * theta_i for every pair i (fp64)."""
    c = np.empty(rot_dim // 2, np.float64)
    s = np.empty(rot_dim // 2, np.float64)
    _load().kamera_oracle_phase(int(delta), float(theta), int(rot_dim), _ptr(c), _ptr(s))
    return c, s


def _rows(a: np.ndarray, name: str) -> tuple[np.ndarray, int]:
    """A 2-D view with unit inner stride; returns (array, row stride in elements)."""
    if a.ndim != 2:
        raise ValueError(f"oracle: {name} must be 2-D, got shape {a.shape}")
    if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        a = np.ascontiguousarray(a)
    return a, a.strides[0] // a.itemsize


def pair_deltas(pair_section, section_delta) -> np.ndarray:
    """Per-pair shift of a multimodal (sectioned) RoPE: pair i turns by the shift of the
    position component it encodes."""
    sec = np.asarray(pair_section, np.int64)
    return np.asarray(section_delta, np.int64)[sec]


def segment(src: np.ndarray, *, rotate: bool, layout: int = HALF_SPLIT, delta: int = 0,
            theta: float = 1e4, U: np.ndarray | None = None,
            V: np.ndarray | None = None, rot_dim: int | None = None,
            inv_freq: np.ndarray | None = None,
            pair_delta: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """One head: src (tokens x width) -> (out, abs_sum), both fp64 (tokens x width).

    out = R src + U V^T, R applied to the pairs (of ``layout``) of the first ``rot_dim``
    features (default: all) when ``rotate``; pair i turns by pair_delta[i] (default: delta)
    times inv_freq[i] (default: theta^(-2i/rot_dim)). U is tokens x m and V width x m, in the
    element type of src.
    """
    dt = dtype_of(src)
    src, src_stride = _rows(src, "src")
    n_tokens, width = src.shape
    m = 0
    u_stride = v_stride = 0
    if U is not None and U.shape[-1] > 0:
        if dtype_of(U) != dt or dtype_of(V) != dt:
            raise TypeError("oracle: U, V must share the element type of src")
        U, u_stride = _rows(U, "U")
        V, v_stride = _rows(V, "V")
        m = U.shape[1]
        if U.shape[0] != n_tokens or V.shape != (width, m):
            raise ValueError(f"oracle: U {U.shape} / V {V.shape} do not fit src {src.shape}")
    else:
        U = V = None
    out = np.empty((n_tokens, width), np.float64)
    mag = np.empty((n_tokens, width), np.float64)
    rd = width if rot_dim is None else int(rot_dim)
    freq = None if inv_freq is None else np.ascontiguousarray(inv_freq, np.float64)
    pdel = None if pair_delta is None else np.ascontiguousarray(pair_delta, np.int64)
    for name, arr in (("inv_freq", freq), ("pair_delta", pdel)):
        if arr is not None and arr.shape != (rd // 2,):
            raise ValueError(f"oracle: {name} needs {rd // 2} entries, got {arr.shape}")
    rc = _load().kamera_oracle_segment_ex(_DTYPE_CODE[dt], _ptr(src), src_stride, n_tokens,
                                          width, int(bool(rotate)), int(layout), rd,
                                          _ptr(freq), _ptr(pdel), int(delta), float(theta),
                                          m, _ptr(U), u_stride, _ptr(V), v_stride, _ptr(out),
                                          _ptr(mag))
    if rc != 0:
        raise ValueError("oracle: kamera_oracle_segment rejected its arguments")
    return out, mag


def to_f32(z: np.ndarray) -> np.ndarray:
    """fp64 -> binary32, round to nearest even."""
    z = np.ascontiguousarray(z, np.float64)
    out = np.empty(z.shape, np.float32)
    _load().kamera_oracle_to_f32(_ptr(z), z.size, _ptr(out))
    return out


def to_bf16(z: np.ndarray) -> np.ndarray:
    """fp64 -> binary32 (RNE) -> bf16 (RNE); returns uint16 bit patterns."""
    z = np.ascontiguousarray(z, np.float64)
    out = np.empty(z.shape, np.uint16)
    _load().kamera_oracle_to_bf16(_ptr(z), z.size, _ptr(out))
    return out


def slots(page_table: np.ndarray | None, page_size: int, dst_offset: int,
          n_tokens: int) -> np.ndarray:
    """Physical cache slot of each token of a chunk placed at logical token dst_offset."""
    out = np.empty(n_tokens, np.int64)
    if page_table is None:
        rc = _load().kamera_oracle_slots(None, 0, int(page_size), int(dst_offset), int(n_tokens),
                                         _ptr(out))
    else:
        table = np.ascontiguousarray(page_table, np.int32)
        rc = _load().kamera_oracle_slots(_ptr(table), table.size, int(page_size),
                                         int(dst_offset), int(n_tokens), _ptr(out))
    if rc != 0:
        raise ValueError("oracle: slots() ran past the page table")
    return out


def expected_head(src: np.ndarray, *, rotate: bool, layout: int, delta: int, theta: float,
                  U: np.ndarray | None, V: np.ndarray | None, **rope) -> dict:
    """What the operator must produce for one head of one chunk/layer/channel.

    Returns a dict with ``copy`` (True when the channel is unrotated and unpatched, so the
    output must be the input bits), and otherwise ``z`` (fp64 result) and ``S`` (sum of
    absolute terms).
    """
    m = 0 if U is None else U.shape[-1]
    if not rotate and m == 0:
        return {"copy": True, "bits": src}
    z, S = segment(src, rotate=rotate, layout=layout, delta=delta, theta=theta, U=U, V=V, **rope)
    return {"copy": False, "z": z, "S": S}


# ----------------------------------------------------------------------------------------
# patch compile (technical summary §1: the deficit Delta = KV(B|A) - KV(B|empty), taken in
# the target frame; §2: the patch is the top-m SVD factors of one conditioned pass)
# ----------------------------------------------------------------------------------------

def values(x: np.ndarray) -> np.ndarray:
    """Exact fp64 values of an f32 / f64 / bf16-bits array."""
    z, _ = segment(np.ascontiguousarray(x).reshape(-1, x.shape[-1]), rotate=False)
    return z.reshape(x.shape)


def deficit(conditioned: np.ndarray, canonical: np.ndarray, *, rotate: bool, layout: int = HALF_SPLIT,
            delta: int = 0, theta: float = 1e4, **rope) -> np.ndarray:
    """Delta = KV(B|A) - R(delta) KV(B|empty) for one head (tokens x features), fp64."""
    reloc, _ = segment(canonical, rotate=rotate, layout=layout, delta=delta, theta=theta, **rope)
    return values(conditioned) - reloc


def compile_patch(conditioned: np.ndarray, canonical: np.ndarray, *, m: int, rotate: bool,
                  layout: int = HALF_SPLIT, delta: int = 0, theta: float = 1e4, **rope) -> dict:
    """Top-m SVD factors of the deficit of one head (LAPACK through numpy).

    Returns U (tokens x m) = left singular vectors times the singular values, V (features x m)
    = right singular vectors, the product UV (= the best rank-m approximation of Delta,
    Eckart-Young), all singular values `s`, and Delta itself."""
    d = deficit(conditioned, canonical, rotate=rotate, layout=layout, delta=delta, theta=theta,
                **rope)
    u, s, vt = np.linalg.svd(d, full_matrices=False)
    U = u[:, :m] * s[:m]
    V = vt[:m].T.copy()
    return {"U": U, "V": V, "UV": U @ V.T, "s": s, "delta": d}


def orbit_patch(members: list, canonical: np.ndarray, *, m: int, rotate: bool,
                layout: int = HALF_SPLIT, theta: float = 1e4, **rope) -> dict:
    """The orbit patch of one head (technical summary §3, item 1: one patch, averaged over the
    orderings of a cached set, serves every ordering): the deficits of the chunk in each
    ordering, each in its own frame, are averaged and the mean is reduced to its top-m SVD
    factors. `members` lists (conditioned, delta) or (conditioned, delta, pair_delta) per
    ordering; `rope` holds the model's variant arguments shared by all members (rot_dim,
    inv_freq)."""
    total = None
    for mem in members:
        cond, delta = mem[0], mem[1]
        kw = dict(rope)
        if len(mem) > 2 and mem[2] is not None:
            kw["pair_delta"] = mem[2]
        d = deficit(cond, canonical, rotate=rotate, layout=layout, delta=delta, theta=theta, **kw)
        total = d if total is None else total + d
    mean = total / len(members)
    u, s, vt = np.linalg.svd(mean, full_matrices=False)
    U = u[:, :m] * s[:m]
    V = vt[:m].T.copy()
    return {"U": U, "V": V, "UV": U @ V.T, "s": s, "delta": mean}
