"""Comparison of the GPU operator's output with the oracle (test helper, not a test file).

Rules (all elementwise):
  * copy channels (unrotated, m = 0): output bits == input bits.
  * fp32:  |g - z| <= 1e-5 * S, z the fp64 oracle value and S the sum of the absolute values of
    its terms (S >= |z|, so this is relative error except where the terms cancel).
  * bf16 (the pass/fail rule):  |g - o| <= 2 ulp_bf16(max(|o|, 2^-14 S)), with
    o = bf16(fp32(z)) (the fp32 oracle rounded to bf16) and ulp_bf16(v) = 2^(floor(log2 v) - 7).
    The floor 2^-14 S only acts where the terms cancel and |o| is tiny. Reported next to it:
      - floor_active: elements whose tolerance the floor raised above 2 ulp(|o|);
      - unfloored_fail: elements outside 2 ulp(|o|) (they pass only because of the floor);
      - max_ulp: the largest |g - o| / ulp(|o|);
      - chain_fail: elements outside the fp32 operation-chain bound
        2 ulp(|o|) + 2 (m + 4) 2^-24 S of the GPU's arithmetic (a diagnostic, not the rule).
  * placement: every chunk token is read back from page_table[p / page_size], slot
    p % page_size; every slot no chunk addresses still holds the sentinel bits.

Every report a test builds is also kept in REPORTS, so the test session prints one line per
test with these counts (tests/conftest.py).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
from position_invariant_kv_kamera_amd import workloads as wl

U32 = 2.0 ** -24


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (normal range: 2^(floor(log2 |v|) - 7))."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Element bits of a device/host tensor (uint16 for bf16, float32 for fp32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


REPORTS: list = []   # (test id, Report) of every comparison made in this process


@dataclass
class Report:
    elements: int = 0
    copies: int = 0
    copy_mismatches: int = 0
    float_fail: int = 0          # outside the pass/fail rule (bf16: C2; fp32: 1e-5 S)
    floor_active: int = 0        # bf16: the 2^-14 S floor raised the tolerance
    unfloored_fail: int = 0      # bf16: outside 2 ulp(|o|)
    chain_fail: int = 0          # bf16: outside the fp32 operation-chain bound (diagnostic)
    max_ulp: float = 0.0         # bf16: max |g - o| / ulp(|o|)
    max_rel_s: float = 0.0       # fp32: max |g - z| / S
    sentinel_bad: int = 0
    details: list = field(default_factory=list)

    def line(self) -> str:
        return (f"elements={self.elements} copies={self.copies} "
                f"copy_mismatch={self.copy_mismatches} fail={self.float_fail} "
                f"floor_active={self.floor_active} unfloored_fail={self.unfloored_fail} "
                f"chain_fail={self.chain_fail} max_ulp={self.max_ulp:.3f} "
                f"max_err/S={self.max_rel_s:.2e} sentinel_bad={self.sentinel_bad}")

    @property
    def ok(self) -> bool:
        return self.copy_mismatches == 0 and self.float_fail == 0 and self.sentinel_bad == 0

    def merge(self, o: "Report"):
        self.elements += o.elements
        self.copies += o.copies
        self.copy_mismatches += o.copy_mismatches
        self.float_fail += o.float_fail
        self.floor_active += o.floor_active
        self.unfloored_fail += o.unfloored_fail
        self.chain_fail += o.chain_fail
        self.max_ulp = max(self.max_ulp, o.max_ulp)
        self.max_rel_s = max(self.max_rel_s, o.max_rel_s)
        self.sentinel_bad += o.sentinel_bad
        self.details.extend(o.details[:5])


def record(rep: "Report", what: str = "") -> "Report":
    """Keep a finished report for the session summary, under the running test's id."""
    import os
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" (")[0] or "(outside pytest)"
    REPORTS.append((test + (f" [{what}]" if what else ""), rep))
    return rep


def compare_head(exp: dict, got: np.ndarray, dtype: str, m: int, where: str) -> Report:
    r = Report(elements=got.size)
    if exp["copy"]:
        r.copies = got.size
        same = np.array_equal(np.ascontiguousarray(got).view(np.uint8),
                              np.ascontiguousarray(exp["bits"]).view(np.uint8))
        if not same:
            r.copy_mismatches = int(np.sum(got.view(np.uint16 if dtype == "bf16" else np.uint32)
                                           != exp["bits"].view(got.dtype)))
            r.details.append(f"{where}: copy differs in {r.copy_mismatches} elements")
        return r
    z, S = exp["z"], exp["S"]
    if dtype == "f32":
        g = got.astype(np.float64)
        err = np.abs(g - z)
        bad = ~(err <= 1e-5 * S)
        r.float_fail = int(bad.sum())
        with np.errstate(invalid="ignore", divide="ignore"):
            r.max_rel_s = float(np.nanmax(np.where(S > 0, err / S, 0.0)))
    else:
        o_bits = oracle.to_bf16(z)
        o = bf16_bits_to_f64(o_bits)
        g = bf16_bits_to_f64(got)
        err = np.abs(g - o)
        u = ulp_bf16(o)
        u_floor = ulp_bf16(np.maximum(np.abs(o), 2.0 ** -14 * S))
        bad = ~(err <= 2 * u_floor)
        r.float_fail = int(bad.sum())
        r.floor_active = int((u_floor > u).sum())
        r.unfloored_fail = int((~(err <= 2 * u)).sum())
        r.chain_fail = int((~(err <= 2 * u + 2 * (m + 4) * U32 * S)).sum())
        r.max_ulp = float(np.max(err / u)) if err.size else 0.0
    if r.float_fail:
        idx = np.argwhere(bad)[:3]
        r.details.append(f"{where}: {r.float_fail} out of tolerance, e.g. at {idx.tolist()}")
    return r


def _pool_rows(pool_l: torch.Tensor) -> torch.Tensor:
    """[n_pages, page_size, row] view -> [n_pages * page_size, row]."""
    return pool_l.view(pool_l.shape[0] * pool_l.shape[1], pool_l.shape[2])


def rope_kwargs(p: wl.Plan, c: int, ch: int, op: str = "reuse") -> dict:
    """The oracle's RoPE-variant arguments for chunk c, channel ch of plan p: the rotary part
    of a partially rotary key head, the model's frequency table, and per-pair shifts from the
    multimodal sections."""
    if ch != 0 or op == "patch":
        return {}
    kw = {}
    if p.family == wl.GQA and p.rope_dim < p.head_dim:
        kw["rot_dim"] = p.rope_dim
    if p.inv_freq is not None:
        kw["inv_freq"] = p.inv_freq
    if p.pair_section is not None:
        d1, d2 = p.delta_sections[c] if p.delta_sections else (p.deltas[c], p.deltas[c])
        kw["pair_delta"] = oracle.pair_deltas(p.pair_section, (p.deltas[c], d1, d2))
    return kw


def compare_batch(batch: wl.Batch, op: str = "reuse", layers=None, chunks=None,
                  check_sentinel: bool = True, patch_inputs=None) -> Report:
    """Compare every element of the chosen chunks/layers (all by default).

    op: "reuse" (R(delta) + patch), "relocate" (R(delta) only), "patch" (patch only, the
    input being `patch_inputs[c][ch]` — per chunk and channel a host array [layers, L, row]
    of what the pool held before the call).
    """
    p = batch.plan
    rep = Report()
    layers = range(p.n_layers) if layers is None else layers
    chunks = range(p.n_chunks) if chunks is None else chunks
    table = p.page_table
    for c in chunks:
        L = p.chunk_tokens[c]
        if L == 0:
            continue
        slots = torch.from_numpy(oracle.slots(table, p.page_size, p.dst_offsets[c], L))
        ct = batch.chunks[c]
        for l in layers:
            for ch in range(2):
                W, H = p.width(ch), p.heads(ch)
                got_rows = to_numpy_bits(_pool_rows(batch.pools[ch][l]).index_select(
                    0, slots.to(batch.pools[ch].device)))
                if op == "patch":
                    src_rows = patch_inputs[c][ch][l]
                else:
                    src_rows = to_numpy_bits(ct.src[ch][l])
                m = 0 if op == "relocate" or ct.U[ch] is None else ct.U[ch].shape[-1]
                if op == "patch" and m == 0:
                    continue
                Uh = to_numpy_bits(ct.U[ch][l]) if m else None
                Vh = to_numpy_bits(ct.V[ch][l]) if m else None
                for h in range(H):
                    exp = oracle.expected_head(
                        np.ascontiguousarray(src_rows[:, h * W:(h + 1) * W]),
                        rotate=(ch == 0 and op != "patch"),
                        layout=0 if p.rope_layout == wl.HALF_SPLIT else 1,
                        delta=p.deltas[c], theta=p.theta,
                        U=None if not m else np.ascontiguousarray(Uh[h]),
                        V=None if not m else np.ascontiguousarray(Vh[h]),
                        **rope_kwargs(p, c, ch, op))
                    got = np.ascontiguousarray(got_rows[:, h * W:(h + 1) * W])
                    rep.merge(compare_head(exp, got, p.dtype, m, f"chunk {c} layer {l} ch {ch} head {h}"))
    if check_sentinel:
        rep.sentinel_bad = count_sentinel_damage(batch, layers)
    return record(rep, f"{p.name} {op}")


def count_sentinel_damage(batch: wl.Batch, layers=None) -> int:
    """Slots no chunk addresses must still hold the sentinel in every layer and channel."""
    p = batch.plan
    layers = range(p.n_layers) if layers is None else layers
    n_slots = p.n_pages * p.page_size
    written = np.zeros(n_slots, bool)
    for c in range(p.n_chunks):
        if p.chunk_tokens[c]:
            written[oracle.slots(p.page_table, p.page_size, p.dst_offsets[c],
                                 p.chunk_tokens[c])] = True
    free = torch.from_numpy(np.nonzero(~written)[0]).to(batch.pools[0].device)
    if free.numel() == 0:
        return 0
    bad = 0
    for ch in range(2):
        for l in layers:
            rows = _pool_rows(batch.pools[ch][l]).index_select(0, free)
            if rows.dtype == torch.bfloat16:
                bad += int((rows.view(torch.int16) != wl.SENTINEL_BF16).sum().item())
            else:
                bad += int((rows.view(torch.int32) != wl.SENTINEL_F32).sum().item())
    return bad


def sample_rows(batch: wl.Batch, n_rows: int, seed: int = 0, op: str = "reuse") -> Report:
    """Oracle check of n_rows random (chunk, layer, channel, head, token) rows of a batch of
    any size: the oracle computes just those rows."""
    p = batch.plan
    rng = np.random.default_rng(seed)
    rep = Report()
    for _ in range(n_rows):
        c = int(rng.integers(p.n_chunks))
        L = p.chunk_tokens[c]
        if L == 0:
            continue
        l, ch = int(rng.integers(p.n_layers)), int(rng.integers(2))
        h, t = int(rng.integers(p.heads(ch))), int(rng.integers(L))
        W = p.width(ch)
        ct = batch.chunks[c]
        slot = int(oracle.slots(p.page_table, p.page_size, p.dst_offsets[c] + t, 1)[0])
        got = to_numpy_bits(_pool_rows(batch.pools[ch][l])[slot, h * W:(h + 1) * W])[None]
        src = to_numpy_bits(ct.src[ch][l, t, h * W:(h + 1) * W])[None]
        m = 0 if op == "relocate" or ct.U[ch] is None else ct.U[ch].shape[-1]
        U = to_numpy_bits(ct.U[ch][l, h, t:t + 1]) if m else None
        V = to_numpy_bits(ct.V[ch][l, h]) if m else None
        exp = oracle.expected_head(src, rotate=(ch == 0 and op != "patch"), delta=p.deltas[c],
                                   theta=p.theta,
                                   layout=0 if p.rope_layout == wl.HALF_SPLIT else 1, U=U, V=V,
                                   **rope_kwargs(p, c, ch, op))
        rep.merge(compare_head(exp, got, p.dtype, m, f"chunk {c} layer {l} ch {ch} head {h} token {t}"))
    return record(rep, f"{p.name} {op} sampled")
