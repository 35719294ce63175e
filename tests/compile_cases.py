"""Inputs and checks for the patch-compile tests (test helper, not a test file).

A case is a model geometry plus chunks. Per chunk and channel:
  * canonical KV: seeded Gaussian rows (scale 1), stored in the model's element type;
  * a planted deficit per layer and head: sum_r s_r a_r b_r^T with orthonormal a_r (tokens)
    and b_r (features), rank `rank`, singular values falling geometrically from s_1 to
    s_1 / spread, s_1 = `level` * sqrt(tokens * width / rank) (so the deficit's Frobenius norm
    is about `level` times the KV's);
  * conditioned KV = element type(R(delta) canonical + planted), the rotation done by the
    oracle (fp64), one rounding. For bf16 that rounding adds full-rank noise of about 2^-9 of
    each element, far below s_rank.
Expectations: oracle.compile_patch on the stored canonical and conditioned values (the exact
deficit of what the GPU reads, then LAPACK SVD).

Tolerance of the GPU factors (u = 2^-8 for bf16 factors, 2^-24 for fp32):
  * subspace: the GPU forms G = Delta^T Delta in fp32. A perturbation of G of norm e moves the
    top-m subspace by sin(theta) <= e / (s_m^2 - s_(m+1)^2) (Davis-Kahan). With e bounded by
    8 sqrt(n) 2^-24 ||Delta||_F^2 (fp32 accumulation of n terms, probabilistic sqrt(n) growth,
    factor 8 for Delta's own fp32 formation and the power iteration's arithmetic):
        eps_sub = 8 sqrt(n) 2^-24 sum_i s_i^2 / (s_m^2 - s_(m+1)^2).
    Convergence of n_iter rounds adds (s_(m+1)/s_m)^(2 n_iter) times the start's tangent; the
    cases keep s_(m+1)/s_m <= 0.05, so that term is below 1e-18 and left out.
  * stored factors: rounding U and V to the element type changes sum_r U_tr V_fr by at most
    2u sum_r |U_tr||V_fr| <= 2u ||U_t|| ||V_f|| (Cauchy-Schwarz) with ||U_t|| = ||(Delta_m)_t||
    and ||V_f|| = sqrt(P_ff), P = V V^T the oracle's projector (both basis-free).
  * patch:      |U V^T - Delta_m|_tf <= 2u(1+2^-6) ||(Delta_m)_t|| sqrt(P_ff)
                                        + 2 eps_sub ||Delta_t|| + 1e-6 ||Delta_t||
  * projector:  |V V^T - P|_fg      <= 2u(1+2^-6) sqrt(P_ff P_gg) + 2 eps_sub + 1e-6
  * columns:    |V^T V - I|          <= 2u(1+2^-6) + 2^-20  (the GPU basis itself)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import oracle


@dataclass
class ChunkSpec:
    n_tokens: int
    m: int
    delta: int
    rank: int | None = None        # planted rank (default m); 0 plants nothing
    spread: float = 2.0
    level: float = 0.15
    same_as_canonical: bool = False   # conditioned = canonical bits (delta should be 0)
    delta_sections: tuple | None = None   # shifts of sections 1, 2 (default: delta)


@dataclass
class Case:
    name: str
    family: str                    # "gqa" | "mla"
    dtype: str                     # "bf16" | "f32"
    n_layers: int
    n_kv_heads: int
    head_dim: int
    rope_dim: int
    layout: int                    # oracle.HALF_SPLIT | oracle.INTERLEAVED
    theta: float
    chunks: list = field(default_factory=list)
    seed: int = 0
    n_iter: int = 8
    mla_shared_rows: bool = False  # MLA channels as views of one [c_KV | k_rope] row

    def geometry(self, ch: int) -> tuple[int, int, bool]:
        """(heads, width, rotated) of channel ch."""
        if self.family == "mla":
            return (1, self.rope_dim, True) if ch == 0 else (1, self.head_dim, False)
        return self.n_kv_heads, self.head_dim, ch == 0


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return oracle.to_bf16(x) if dtype == "bf16" else oracle.to_f32(x)


def _orthonormal(rng, rows: int, cols: int) -> np.ndarray:
    q, _ = np.linalg.qr(rng.standard_normal((rows, cols)))
    return q


def oracle_rope(case: Case, spec: ChunkSpec, ch: int, rope: dict | None) -> dict:
    """Oracle arguments of the RoPE variant `rope` ({"inv_freq", "pair_section"}, optional)
    for channel ch; a GQA case with rope_dim < head_dim is partially rotary."""
    if ch != 0:
        return {}
    rope = rope or {}
    kw = {}
    if case.family == "gqa" and case.rope_dim < case.head_dim:
        kw["rot_dim"] = case.rope_dim
    if rope.get("inv_freq") is not None:
        kw["inv_freq"] = rope["inv_freq"]
    if rope.get("pair_section") is not None:
        s1, s2 = spec.delta_sections or (spec.delta, spec.delta)
        kw["pair_delta"] = oracle.pair_deltas(rope["pair_section"], (spec.delta, s1, s2))
    return kw


def build(case: Case, rope: dict | None = None) -> list[dict]:
    """Per chunk: {"canonical": [ch] array [L, T, H*W], "conditioned": same}; the arrays hold
    element bits (uint16 for bf16, float32 for fp32)."""
    rng = np.random.default_rng(case.seed)
    out = []
    for spec in case.chunks:
        T = spec.n_tokens
        item = {"canonical": [], "conditioned": []}
        for ch in range(2):
            H, W, rot = case.geometry(ch)
            L = case.n_layers
            canon = _store(rng.standard_normal((L, T, H * W)), case.dtype)
            rank = spec.m if spec.rank is None else spec.rank
            cond = np.empty_like(canon)
            for l in range(L):
                for h in range(H):
                    head = canon[l, :, h * W:(h + 1) * W]
                    if spec.same_as_canonical:
                        cond[l, :, h * W:(h + 1) * W] = head
                        continue
                    r = min(rank, T, W)
                    planted = np.zeros((T, W))
                    if r > 0:
                        s1 = spec.level * math.sqrt(T * W / r)
                        s = s1 * spec.spread ** (-np.arange(r) / max(1, r - 1))
                        planted = (_orthonormal(rng, T, r) * s) @ _orthonormal(rng, W, r).T
                    moved, _ = oracle.segment(head, rotate=rot, layout=case.layout,
                                              delta=spec.delta, theta=case.theta,
                                              **oracle_rope(case, spec, ch, rope))
                    cond[l, :, h * W:(h + 1) * W] = _store(moved + planted, case.dtype)
            item["canonical"].append(canon)
            item["conditioned"].append(cond)
        out.append(item)
    return out


def expected(case: Case, inputs: list[dict], c: int, ch: int, layer: int, head: int,
             rope: dict | None = None) -> dict:
    """oracle.compile_patch for one head (with the tolerance terms that depend on it)."""
    spec = case.chunks[c]
    H, W, rot = case.geometry(ch)
    sl = slice(head * W, (head + 1) * W)
    cond = inputs[c]["conditioned"][ch][layer, :, sl]
    canon = inputs[c]["canonical"][ch][layer, :, sl]
    e = oracle.compile_patch(cond, canon, m=spec.m, rotate=rot, layout=case.layout,
                             delta=spec.delta, theta=case.theta,
                             **oracle_rope(case, spec, ch, rope))
    s2 = e["s"] ** 2
    m_eff = min(spec.m, len(s2))
    gap = s2[m_eff - 1] - (s2[m_eff] if m_eff < len(s2) else 0.0)
    n = spec.n_tokens
    e["eps_sub"] = (8 * math.sqrt(n) * 2.0 ** -24 * s2.sum() / gap) if gap > 0 else math.inf
    e["full_rank"] = spec.m <= len(s2) and gap > 0 and s2[m_eff - 1] > 0
    return e


# ---- orbit patch ---------------------------------------------------------------------------
# Orbit inputs: one chunk seen in K orderings at shifts delta_k; ordering k's conditioned KV is
# element type(R(delta_k) canonical + shared + own_k) with `shared` the planted rank-m deficit
# of the chunk spec and own_k a rank-2 ordering-specific part with singular values
# own_level * s_m. The GPU forms the mean deficit from K fp32 sums, so its formation error
# grows with K and with |KV| / |Delta_bar|: the subspace budget adds
# 4 (K + 2) (||KV||_F / ||Delta_bar||_F) 2^-24 to the 8 sqrt(n) 2^-24 factor.

def build_orbit(case: Case, deltas, own_level: float = 0.01, rope: dict | None = None) -> dict:
    rng = np.random.default_rng(case.seed)
    spec = case.chunks[0]
    T = spec.n_tokens
    out = {"canonical": [], "conditioned": [[] for _ in deltas], "deltas": list(deltas)}
    for ch in range(2):
        H, W, rot = case.geometry(ch)
        L = case.n_layers
        canon = _store(rng.standard_normal((L, T, H * W)), case.dtype)
        conds = [np.empty_like(canon) for _ in deltas]
        r = min(spec.m, T, W)
        for l in range(L):
            for h in range(H):
                head = canon[l, :, h * W:(h + 1) * W]
                s1 = spec.level * math.sqrt(T * W / r)
                sv = s1 * spec.spread ** (-np.arange(r) / max(1, r - 1))
                shared = (_orthonormal(rng, T, r) * sv) @ _orthonormal(rng, W, r).T
                for k, d in enumerate(deltas):
                    own = (_orthonormal(rng, T, 2) * (own_level * sv[-1])) @ _orthonormal(rng, W, 2).T
                    sk = ChunkSpec(T, spec.m, d)
                    moved, _ = oracle.segment(head, rotate=rot, layout=case.layout, delta=d,
                                              theta=case.theta, **oracle_rope(case, sk, ch, rope))
                    conds[k][l, :, h * W:(h + 1) * W] = _store(moved + shared + own, case.dtype)
        out["canonical"].append(canon)
        for k in range(len(deltas)):
            out["conditioned"][k].append(conds[k])
    return out


def expected_orbit(case: Case, inp: dict, ch: int, layer: int, head: int,
                   rope: dict | None = None) -> dict:
    spec = case.chunks[0]
    H, W, rot = case.geometry(ch)
    sl = slice(head * W, (head + 1) * W)
    canon = inp["canonical"][ch][layer, :, sl]
    members = []
    shared_kw = {}
    for k, d in enumerate(inp["deltas"]):
        kw = oracle_rope(case, ChunkSpec(spec.n_tokens, spec.m, d), ch, rope)
        members.append((inp["conditioned"][k][ch][layer, :, sl], d, kw.pop("pair_delta", None)))
        shared_kw = kw
    e = oracle.orbit_patch(members, canon, m=spec.m, rotate=rot, layout=case.layout,
                           theta=case.theta, **shared_kw)
    s2 = e["s"] ** 2
    m_eff = min(spec.m, len(s2))
    gap = s2[m_eff - 1] - (s2[m_eff] if m_eff < len(s2) else 0.0)
    K = len(members)
    ratio = np.linalg.norm(oracle.values(canon)) / max(np.linalg.norm(e["delta"]), 1e-300)
    fac = 8 * math.sqrt(spec.n_tokens) + 4 * (K + 2) * ratio
    e["eps_sub"] = fac * 2.0 ** -24 * s2.sum() / gap if gap > 0 else math.inf
    e["full_rank"] = spec.m <= len(s2) and gap > 0 and s2[m_eff - 1] > 0
    return e


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.astype(np.float64)


@dataclass
class HeadCheck:
    patch_excess: float      # max |UV^T - Delta_m| / tol (<= 1 passes)
    proj_excess: float       # max |VV^T - P| / tol, or 0 when not checked
    orth_err: float          # max |V^T V - I|
    orth_tol: float

    @property
    def ok(self) -> bool:
        return self.patch_excess <= 1.0 and self.proj_excess <= 1.0 and self.orth_err <= self.orth_tol


def check_head(U: np.ndarray, V: np.ndarray, e: dict, dtype: str) -> HeadCheck:
    """U (n x m) and V (width x m) from the GPU, decoded to fp64, against the oracle's e."""
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    r = 2 * u * (1 + 2.0 ** -6)
    eps = e["eps_sub"]
    Vo = e["V"]
    P = Vo @ Vo.T
    pf = np.sqrt(np.clip(np.diag(P), 0.0, None))
    dm_rows = np.linalg.norm(e["UV"], axis=1)
    d_rows = np.linalg.norm(e["delta"], axis=1)
    tol = r * np.outer(dm_rows, pf) + (2 * eps + 1e-6) * d_rows[:, None]
    err = np.abs(U @ V.T - e["UV"])
    patch_excess = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    proj_excess = 0.0
    if e["full_rank"]:
        tolp = r * np.outer(pf, pf) + 2 * eps + 1e-6
        proj_excess = float(np.max(np.abs(V @ V.T - P) / tolp))
    g = V.T @ V
    orth_err = float(np.max(np.abs(g - np.eye(g.shape[0]))))
    return HeadCheck(patch_excess, proj_excess, orth_err, r + 2.0 ** -20)


# ---- the cases ------------------------------------------------------------------------------

def small_cases() -> list[Case]:
    HS, IL = oracle.HALF_SPLIT, oracle.INTERLEAVED
    return [
        Case("gqa_bf16_d128", "gqa", "bf16", 2, 2, 128, 128, HS, 1e6,
             [ChunkSpec(300, 16, 1234)], seed=1),
        Case("gqa_f32_d128", "gqa", "f32", 2, 2, 128, 128, HS, 1e6,
             [ChunkSpec(300, 16, -4321)], seed=2),
        Case("gqa_bf16_d64_interleaved", "gqa", "bf16", 1, 3, 64, 64, IL, 1e4,
             [ChunkSpec(77, 8, 50000)], seed=3),
        Case("mla_bf16", "mla", "bf16", 2, 1, 512, 64, HS, 1e4,
             [ChunkSpec(300, 32, 777)], seed=4, mla_shared_rows=True),
        Case("gqa_bf16_rank64", "gqa", "bf16", 1, 2, 128, 128, HS, 1e6,
             [ChunkSpec(500, 64, 99)], seed=5),
        Case("gqa_f32_d96_rank48", "gqa", "f32", 1, 1, 96, 96, HS, 1e4,
             [ChunkSpec(200, 48, 31)], seed=6),
        Case("gqa_f32_d32_full_width", "gqa", "f32", 1, 2, 32, 32, IL, 1e4,
             [ChunkSpec(64, 32, -7)], seed=7),
        Case("mla_f32_latent128", "mla", "f32", 1, 1, 128, 32, HS, 1e4,
             [ChunkSpec(130, 16, 4096)], seed=8),
        # rank class 64 below its width (columns m..63 empty), and the fp32 rank-64 path
        Case("gqa_bf16_rank56_interleaved", "gqa", "bf16", 1, 2, 128, 128, IL, 1e4,
             [ChunkSpec(260, 56, 321)], seed=12),
        Case("gqa_f32_rank64", "gqa", "f32", 1, 1, 128, 128, HS, 1e6,
             [ChunkSpec(200, 64, -77)], seed=13),
        # 512-wide latent heads: the rank-16 class, and ranks 12 and 32 in one launch (the
        # rank-12 heads then run in the rank-32 class with 20 empty columns)
        Case("mla_bf16_rank16", "mla", "bf16", 1, 1, 512, 64, HS, 1e4,
             [ChunkSpec(200, 16, 42)], seed=16, mla_shared_rows=True),
        Case("mla_bf16_ranks_12_and_32", "mla", "bf16", 1, 1, 512, 64, HS, 1e4,
             [ChunkSpec(260, 12, 555), ChunkSpec(180, 32, -90)], seed=17),
    ]


def degenerate_cases() -> list[Case]:
    HS = oracle.HALF_SPLIT
    return [
        # no context: conditioned == canonical and delta == 0, so Delta == 0 exactly
        Case("zero_deficit", "gqa", "bf16", 1, 2, 128, 128, HS, 1e6,
             [ChunkSpec(100, 16, 0, same_as_canonical=True)], seed=9),
        # fewer tokens than m: Delta has rank 5, the rank-16 truncation is Delta itself
        Case("tokens_below_rank", "gqa", "f32", 1, 2, 64, 64, HS, 1e4,
             [ChunkSpec(5, 16, 12)], seed=10),
        # the same at rank 64: 40 tokens leave 24 collapsed columns
        Case("tokens_below_rank64", "gqa", "bf16", 1, 2, 128, 128, HS, 1e6,
             [ChunkSpec(40, 64, 5)], seed=14),
        # and on 512-wide latent heads at rank 32: 20 tokens leave 12 collapsed columns
        Case("mla_tokens_below_rank32", "mla", "bf16", 1, 1, 512, 64, HS, 1e4,
             [ChunkSpec(20, 32, 3)], seed=18),
    ]


def full_case() -> Case:
    """One chunk at the full Qwen2.5-VL-like geometry (28 layers, 4 KV heads, 128 wide, 1296
    tokens, rank 16)."""
    return Case("qwen25vl_chunk", "gqa", "bf16", 28, 4, 128, 128, oracle.HALF_SPLIT, 1e6,
                [ChunkSpec(1296, 16, 20000)], seed=11)


def full_mla_case() -> Case:
    """One chunk at the full DeepSeek-V2-Lite-like MLA geometry (27 layers, rows of a 512-wide
    latent and a 64-wide rotary part, 2048 tokens, rank 32)."""
    return Case("dsv2lite_mla_chunk", "mla", "bf16", 27, 1, 512, 64, oracle.HALF_SPLIT, 1e4,
                [ChunkSpec(2048, 32, 40000)], seed=12, mla_shared_rows=True)


def full_rank64_case() -> Case:
    """The 7B-like MHA reorder geometry at rank 64 (32 heads x 128, interleaved RoPE, 4096
    tokens), on 4 of its 32 layers: the per-head shapes of the full compile."""
    return Case("mha7b_chunk_rank64", "gqa", "bf16", 4, 32, 128, 128, oracle.INTERLEAVED, 1e4,
                [ChunkSpec(4096, 64, 12288)], seed=13)
