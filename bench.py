"""Benchmark of the Kamera reuse operator on one MI355X.

One step = one kamera_reuse_batch call over the whole batch: work decomposition, fp64 phase
generation, streaming of the canonical KV, rotation, the rank-m patch, and the page-table
scatter, for every chunk, layer, channel and head. Inputs are resident in HBM before timing.
The headline workload is the largest that fits one GPU: the 7B-like MHA reorder batch (32
layers, 32 heads x 128, 16 chunks of 4096 tokens, rank-64 patches, paged), 86.4 GB moved per
step.

Prints one JSON line (metric: relocated + patched KV tokens/s and achieved HBM GB/s), which
also carries:
  "configs": a compact record per other workload (the Qwen2.5-VL-like GQA batch, the
    DeepSeek-V2-Lite-like MLA batch, the Qwen3-VL-like sliding window, and the tiny fp32 case
    as a latency), each timed on its own;
  "cpu_baseline": the fp64 oracle on a bounded sample of the headline batch, host cores;
  "patch_compile": kamera_patch_compile (deficit, Gram, subspace iteration, projection) on a
    few chunks of the headline batch, next to one reuse pass over the same chunks, with the
    orbit compile over 3 orderings;
  "decode_attention" / "decode_attention_mla": the consumer-side decode attention (with its
    state merge) on a 64-sequence x 16K-token paged cache, GQA and MLA;
  "chunk_attention": the same decode read from 16 canonical chunks per sequence in place.
    python bench.py [--steps K] [--warmup W] [--workload NAME] [--configs A,B|none]
                    [--no-cpu-baseline] [--compile-steps N] [--compile-chunks N]
                    [--attention-steps N] [--chunk-attention-steps N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
# the largest workload that fits one GPU (86.4 GB moved per step)
DEFAULT_WORKLOAD = "mha7b_reorder_bf16"
# the other workloads, each timed after the headline into a compact record (the fp32 one is
# latency bound and reported in microseconds)
OTHER_CONFIGS = ["qwen25vl_gqa_bf16", "dsv2lite_mla_bf16", "qwen3vl_window_bf16", "tiny_gqa_f32"]
METRIC = "relocated+patched KV tokens/s and achieved HBM GB/s (% of peak), 1 GPU"
CALIB_BYTES = 2 << 30
KERNEL_SOURCES = ["position_invariant_kv_kamera_amd/csrc/kamera_kernels.hip",
                  "position_invariant_kv_kamera_amd/csrc/kamera_api.cpp",
                  "position_invariant_kv_kamera_amd/csrc/kamera_internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()[:16]


def algorithmic_bytes(p) -> dict:
    """What the method itself must move: canonical KV read once, output written once, patch
    factors read once, page table read once."""
    es = p.elem_bytes
    kv = 0
    patch = 0
    for c, L in enumerate(p.chunk_tokens):
        for ch, m in ((0, p.m_rot[c]), (1, p.m_plain[c])):
            H, W = p.heads(ch), p.width(ch)
            kv += p.n_layers * L * H * W * es
            patch += p.n_layers * H * (L + W) * m * es
    table = 0 if p.page_table is None else p.page_table.size * 4
    return {"read_kv": kv, "write_kv": kv, "patch": patch, "page_table": table,
            "total": 2 * kv + patch + table}


def patch_flops(p) -> float:
    f = 0.0
    for c, L in enumerate(p.chunk_tokens):
        for ch, m in ((0, p.m_rot[c]), (1, p.m_plain[c])):
            f += 2.0 * m * p.n_layers * L * p.heads(ch) * p.width(ch)
    return f


def traffic_from_profile(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources."""
    f = ROOT / "profiles" / f"traffic_{workload}.json"
    if not f.exists():
        return None, None
    d = json.loads(f.read_text())
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None, "stale"
    return d.get("traffic_bytes"), d.get("kernel")


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, budget_s: float) -> dict:
    """The oracle, as it is, on (chunk, layer) units of the same batch in order (every channel
    and head of the layer; chunk by chunk, starting over when the batch is done) until about
    `budget_s` seconds of CPU work. A token counts once all its layers are done, so the rate is
    (layer-token units / n_layers) per second, comparable with the GPU's tokens/s. Host copies
    of the inputs are made per unit and are not timed."""
    import numpy as np
    import torch
    import oracle

    p = batch.plan
    layout = 0 if p.rope_layout == "half_split" else 1

    def host(t):
        if t is None:
            return None
        t = t.detach().contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    busy = 0.0
    layer_tokens = 0
    units = 0
    while busy < budget_s:
        c = (units // p.n_layers) % p.n_chunks
        l = units % p.n_layers
        ct = batch.chunks[c]
        srcs = [host(ct.src[ch][l]) for ch in range(2)]
        Us = [host(ct.U[ch][l]) if ct.U[ch] is not None else None for ch in range(2)]
        Vs = [host(ct.V[ch][l]) if ct.V[ch] is not None else None for ch in range(2)]
        t0 = time.perf_counter()
        for ch in range(2):
            W = p.width(ch)
            for h in range(p.heads(ch)):
                x = np.ascontiguousarray(srcs[ch][:, h * W:(h + 1) * W])
                U = None if Us[ch] is None else Us[ch][h]
                V = None if Vs[ch] is None else Vs[ch][h]
                e = oracle.expected_head(x, rotate=(ch == 0), layout=layout,
                                         delta=p.deltas[c], theta=p.theta, U=U, V=V)
                if not e["copy"]:
                    oracle.to_bf16(e["z"]) if p.dtype == "bf16" else oracle.to_f32(e["z"])
        busy += time.perf_counter() - t0
        layer_tokens += p.chunk_tokens[c]
        units += 1
    return {"value": layer_tokens / p.n_layers / busy, "unit": "tokens/s",
            "cores": oracle.threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{units} (chunk, layer) units of {p.name} in batch order "
                      f"({units / (p.n_chunks * p.n_layers):.4f} of the batch; "
                      f"{layer_tokens} token-layers, every channel and head), "
                      f"{busy:.1f} s of oracle time on {oracle.threads()} OpenMP threads"}


FP32_PEAK_TFLOPS = 157.3       # dense fp32 (MFMA and vector alike)


def compile_leg(p, batch, steps: int, stream, orbit_steps: int = 2,
                max_chunks: int | None = None) -> dict:
    """Time kamera_patch_compile over the first `max_chunks` chunks of the batch (all when
    None; one step = those chunks' patches at the workload's largest rank), next to one reuse
    pass over the same chunks. The conditioned KV is the canonical KV plus Gaussian noise; the
    compile does the same work whatever the values."""
    import torch
    from position_invariant_kv_kamera_amd import binding as kb

    n_sub = p.n_chunks if max_chunks is None else min(p.n_chunks, max_chunks)
    # one reuse pass over the same chunks, for the compile / reuse cost ratio
    model0, cache0 = kb.model_of(p), kb.cache_of(batch)
    chunks0 = kb.chunks_of(batch)
    ws0 = kb.Workspace(n_sub)
    sp = stream.cuda_stream
    for _ in range(3):
        kb.check(kb.kamera_reuse_batch(model0, cache0, chunks0, n_sub, ws0.ptr, ws0.nbytes, sp))
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(10):
        kb.check(kb.kamera_reuse_batch(model0, cache0, chunks0, n_sub, ws0.ptr, ws0.nbytes, sp))
    r1.record(stream)
    torch.cuda.synchronize()
    reuse_ms = r0.elapsed_time(r1) / 10

    m = max(p.m_rot + p.m_plain) or 16
    n_iter = 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    items = []
    es = p.elem_bytes
    io_bytes = in_bytes = gram_flops = proj_flops = 0
    for c, ct in enumerate(batch.chunks[:n_sub]):
        T = p.chunk_tokens[c]
        cond, U, V = [], [], []
        for ch in range(2):
            src = ct.src[ch]
            noise = torch.randn(src.shape, generator=gen, device="cuda", dtype=torch.float32)
            cond.append((src.float() + 0.05 * noise).to(src.dtype))
            H, W = p.heads(ch), p.width(ch)
            U.append(torch.empty((p.n_layers, H, T, m), dtype=src.dtype, device="cuda"))
            V.append(torch.empty((p.n_layers, H, W, m), dtype=src.dtype, device="cuda"))
            units = p.n_layers * H
            in_bytes += 2 * units * T * W * es
            io_bytes += 2 * 2 * units * T * W * es + units * (T + W) * m * es
            gram_flops += 1.0 * units * T * W * (W + 1)   # distinct entries of G (symmetric)
            proj_flops += 2.0 * units * T * W * m
        items.append(kb.CompileItem(T, m, p.deltas[c], list(ct.src), cond, U, V))
    model = kb.model_of(p)
    ws = kb.run_compile(model, items, n_iter=n_iter)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        kb.run_compile(model, items, n_iter=n_iter, workspace=ws, stream=stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # bf16 rows: the Gram and the projection run on bf16 MFMA (high/low parts), whose rate is
    # not the binding limit, so the floor is the HBM time of the bytes; fp32 rows: the fp32
    # MFMA rate as well
    bf16_rows = p.dtype == "bf16"
    hbm_ms = io_bytes / (HBM_PEAK_GBPS * 1e9) * 1e3
    floor_ms = hbm_ms if bf16_rows else max(
        hbm_ms, (gram_flops + proj_flops) / (FP32_PEAK_TFLOPS * 1e12) * 1e3)
    floor_text = ("bytes / 8 TB/s (bf16 rows: Gram and projection on bf16 MFMA)" if bf16_rows else
                  "max(bytes / 8 TB/s, (Gram + projection flops) / 157.3 TFLOP/s fp32)")

    result = {"chunks": f"{n_sub} of the {p.n_chunks} chunks of {p.name}",
              "ms_per_batch": round(ms, 3), "steps": steps, "rank": m, "n_iter": n_iter,
              "input_bytes": in_bytes, "reuse_ms_per_batch": round(reuse_ms, 4),
              "compile_over_reuse": round(ms / reuse_ms, 2), "io_bytes": io_bytes,
              "gram_flops": gram_flops, "project_flops": proj_flops,
              "floor_ms": round(floor_ms, 3), "frac_of_floor": round(floor_ms / ms, 4),
              "floor": floor_text,
              "timed_with": "hip events on the launch stream"}
    if orbit_steps <= 0:
        return result
    # orbit patch over 3 orderings per chunk (each ordering's conditioned rows are one more
    # input per streaming pass)
    K = 3
    orbit_items = []
    for c, it in enumerate(items):
        members = [(it.delta, it.conditioned)]
        for k in range(1, K):
            cond = []
            for ch in range(2):
                noise = torch.randn(it.canonical[ch].shape, generator=gen, device="cuda")
                cond.append((it.canonical[ch].float() + 0.05 * noise).to(it.canonical[ch].dtype))
            members.append((it.delta + 1000 * k, cond))
        orbit_items.append(kb.OrbitItem(it.n_tokens, m, it.canonical, members, it.U, it.V))
    ows = kb.run_orbit_compile(model, orbit_items, n_iter=n_iter)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(orbit_steps):
        kb.run_orbit_compile(model, orbit_items, n_iter=n_iter, workspace=ows,
                             stream=stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    orbit_ms = e0.elapsed_time(e1) / orbit_steps
    orbit_io = io_bytes + 2 * (K - 1) * in_bytes // 2
    del orbit_items, ows
    result["orbit"] = {"orderings": K, "ms_per_batch": round(orbit_ms, 3), "io_bytes": orbit_io,
                       "ms_over_compile": round(orbit_ms / ms, 3), "steps": orbit_steps}
    return result


def attention_leg(steps: int, stream) -> dict:
    """Decode attention on one layer of a Qwen2.5-VL-7B-like cache (4 KV heads x 128, 28 query
    heads): 64 sequences x 16384 tokens each, paged 16 with a shuffled page table, one query
    token per sequence. Bytes = every K and V row read once."""
    import numpy as np
    import torch
    from position_invariant_kv_kamera_amd import binding as kb

    n_seq, ctx, n_kv, D, n_q, ps = 64, 16384, 4, 128, 28, 16
    n_pages = n_seq * ctx // ps
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    row = n_kv * D
    pools = [torch.randn((1, n_pages, ps, row), generator=g, device="cuda").to(torch.bfloat16)
             for _ in range(2)]
    table = torch.from_numpy(np.random.default_rng(77).permutation(n_pages).astype(np.int32)).cuda()
    model = kb.make_model("gqa", "bf16", 1, n_kv, D, D, "half_split", 1e6)
    cache = kb.KameraCache()
    cache.pool[0], cache.pool[1] = pools[0].data_ptr(), pools[1].data_ptr()
    cache.layer_stride = pools[0].stride(0)
    cache.token_stride = row
    cache.page_table = table.data_ptr()
    cache.n_logical_pages = n_pages
    cache.page_size = ps
    cache.n_pages = n_pages
    q = torch.randn((n_seq, n_q, D), generator=g, device="cuda").to(torch.bfloat16)
    ranges = [(i * ctx, ctx) for i in range(n_seq)]
    queries = kb.attn_queries_of(ranges)
    need = kb.kamera_attention_workspace_bytes(model, n_q, queries, n_seq)
    ws = kb.Workspace(nbytes=need)
    out = torch.empty((n_seq, n_q, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_seq, n_q), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream

    def call():
        kb.check(kb.kamera_decode_attention(model, cache, 0, q.data_ptr(), n_q, queries, n_seq,
                                            1.0 / D ** 0.5, out.data_ptr(), lse.data_ptr(),
                                            ws.ptr, ws.nbytes, sp))

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kv_bytes = 2 * n_seq * ctx * row * 2
    gbps = kv_bytes / (ms * 1e-3) / 1e9
    del pools, table, q, out, lse, ws
    return {"shape": f"{n_seq} sequences x {ctx} tokens, {n_kv} KV heads x {D}, {n_q} query heads, "
                     f"paged {ps} shuffled, one layer",
            "ms_per_call": round(ms, 4), "kv_bytes": kv_bytes, "achieved_gbps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "steps": steps,
            "timed_with": "hip events on the launch stream (segment + merge kernels)"}


def mla_attention_leg(steps: int, stream) -> dict:
    """Decode attention over one layer of a DeepSeek-V2-Lite-like MLA cache (rows [c_KV 512 |
    k_rope 64], 16 query heads reading the one latent row): 64 sequences x 16384 tokens, paged
    16 with a shuffled page table. Bytes = every latent and k_rope row read once."""
    import numpy as np
    import torch
    from position_invariant_kv_kamera_amd import binding as kb

    n_seq, ctx, n_q, ps = 64, 16384, 16, 16
    n_pages = n_seq * ctx // ps
    g = torch.Generator(device="cuda")
    g.manual_seed(79)
    rows = torch.randn((1, n_pages, ps, 576), generator=g, device="cuda").to(torch.bfloat16)
    table = torch.from_numpy(np.random.default_rng(79).permutation(n_pages).astype(np.int32)).cuda()
    model = kb.make_model("mla", "bf16", 1, 1, 512, 64, "half_split", 1e4)
    cache = kb.KameraCache()
    cache.pool[1], cache.pool[0] = rows.data_ptr(), rows.data_ptr() + 512 * 2
    cache.layer_stride = rows.stride(0)
    cache.token_stride = 576
    cache.page_table = table.data_ptr()
    cache.n_logical_pages = n_pages
    cache.page_size = ps
    cache.n_pages = n_pages
    q = torch.randn((n_seq, n_q, 576), generator=g, device="cuda").to(torch.bfloat16)
    queries = kb.attn_queries_of([(i * ctx, ctx) for i in range(n_seq)])
    need = kb.kamera_attention_workspace_bytes(model, n_q, queries, n_seq)
    ws = kb.Workspace(nbytes=need)
    out = torch.empty((n_seq, n_q, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_seq, n_q), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream

    def call():
        kb.check(kb.kamera_decode_attention(model, cache, 0, q.data_ptr(), n_q, queries, n_seq,
                                            1.0 / 192 ** 0.5, out.data_ptr(), lse.data_ptr(),
                                            ws.ptr, ws.nbytes, sp))

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kv_bytes = n_seq * ctx * 576 * 2
    gbps = kv_bytes / (ms * 1e-3) / 1e9
    del rows, table, q, out, lse, ws
    return {"shape": f"{n_seq} sequences x {ctx} tokens, MLA rows c_KV 512 + k_rope 64, "
                     f"{n_q} query heads, paged {ps} shuffled, one layer",
            "ms_per_call": round(ms, 4), "kv_bytes": kv_bytes, "achieved_gbps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "steps": steps,
            "timed_with": "hip events on the launch stream (segment + merge kernels)"}


def chunk_attention_leg(steps: int, stream) -> dict:
    """Attention over chunks read in place, shaped like the decode leg: 64 sequences x 16
    canonical chunks of 1024 tokens, 4 KV heads x 128, 28 query heads, one layer, each chunk
    with its own shift (uniform in [0, 65536)) and rank-16 patches on K and V. Bytes = every
    canonical K and V row, every U_K and U_V row, and each chunk's V_K and V_V once."""
    import numpy as np
    import torch
    from position_invariant_kv_kamera_amd import binding as kb

    n_seq, n_ck, T, n_kv, D, n_q, m = 64, 16, 1024, 4, 128, 28, 16
    n_chunks = n_seq * n_ck
    row = n_kv * D
    g = torch.Generator(device="cuda")
    g.manual_seed(78)
    K = torch.randn((n_chunks, T, row), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((n_chunks, T, row), generator=g, device="cuda").to(torch.bfloat16)
    UK, UV = [(0.05 * torch.randn((n_chunks, n_kv, T, m), generator=g, device="cuda")).to(torch.bfloat16)
              for _ in range(2)]
    VK, VV = [(0.05 * torch.randn((n_chunks, n_kv, D, m), generator=g, device="cuda")).to(torch.bfloat16)
              for _ in range(2)]
    deltas = np.random.default_rng(78).integers(0, 65536, n_chunks)
    es = 2
    items = []
    for c in range(n_chunks):
        items.append({"n_tokens": T, "delta": int(deltas[c]),
                      "src": [(K.data_ptr() + c * K.stride(0) * es, K.stride(0), row),
                              (V.data_ptr() + c * V.stride(0) * es, V.stride(0), row)],
                      "patch": [(m, UK.data_ptr() + c * UK.stride(0) * es, UK.stride(0), UK.stride(1),
                                 VK.data_ptr() + c * VK.stride(0) * es, VK.stride(0), VK.stride(1)),
                                (m, UV.data_ptr() + c * UV.stride(0) * es, UV.stride(0), UV.stride(1),
                                 VV.data_ptr() + c * VV.stride(0) * es, VV.stride(0), VV.stride(1))]})
    chunks = kb.attn_chunks_of(items)
    queries = kb.chunk_queries_of([(s * n_ck, n_ck) for s in range(n_seq)])
    model = kb.make_model("gqa", "bf16", 1, n_kv, D, D, "half_split", 1e6)
    q = torch.randn((n_seq, n_q, D), generator=g, device="cuda").to(torch.bfloat16)
    need = kb.kamera_chunk_attention_workspace_bytes(model, n_q, chunks, n_chunks, queries, n_seq)
    ws = kb.Workspace(nbytes=need)
    out = torch.empty((n_seq, n_q, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_seq, n_q), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream

    def call():
        kb.check(kb.kamera_chunk_attention(model, 0, chunks, n_chunks, queries, n_seq,
                                           q.data_ptr(), n_q, 1.0 / D ** 0.5, out.data_ptr(),
                                           lse.data_ptr(), ws.ptr, ws.nbytes, sp))

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kv_bytes = 2 * n_chunks * T * row * es
    patch_bytes = 2 * n_chunks * n_kv * (T + D) * m * es
    gbps = (kv_bytes + patch_bytes) / (ms * 1e-3) / 1e9
    del K, V, UK, UV, VK, VV, q, out, lse, ws
    return {"shape": f"{n_seq} sequences x {n_ck} chunks x {T} tokens, {n_kv} KV heads x {D}, "
                     f"{n_q} query heads, rank {m} patches on K and V, one layer",
            "ms_per_call": round(ms, 4), "bytes": kv_bytes + patch_bytes,
            "achieved_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "steps": steps,
            "timed_with": "hip events on the launch stream (chunk + merge kernels)"}


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_profile(prof_dir: str, workload: str, command: str, bench_log: str = "") -> None:
    """Turn rocprofv3 CSV output (a kernel-trace --stats run named `kt`, and --pmc runs named
    `fetch` (FETCH_SIZE) and `write` (WRITE_SIZE), all on `bench.py --workload <workload>`) into
    the committed summaries under profiles/."""
    d = Path(prof_dir)
    p = __import__("position_invariant_kv_kamera_amd.workloads", fromlist=["plan"]).plan(workload)
    ab = algorithmic_bytes(p)["total"]
    lines = [f"# kamera_mfma_kernel on {workload}", "",
             "Commands (R = repository root on the machine that ran them):", ""]
    lines += [f"    {c.strip()}" for c in command.split(";") if c.strip()] + [""]
    stats = sorted(d.glob("**/kt_kernel_stats.csv"))
    avg_ns = None
    n_inst = 0
    if stats:
        rows = _read_csv(stats[0])
        lines += ["## rocprofv3 --kernel-trace --stats", "",
                  "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
        for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0)))[:8]:
            name = r["Name"][:70].replace("|", "/")
            lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                         f"{float(r['Percentage']):.1f} |")
        # a step launches each instantiation in use once (one per window width), so the
        # step's kernel time is the sum of their averages
        kam = [r for r in rows if "kamera_mfma_kernel" in r["Name"]]
        if kam:
            n_inst = len(kam)
            avg_ns = sum(float(r["AverageNs"]) for r in kam)
        if avg_ns:
            what = ("kamera_mfma_kernel average" if n_inst == 1 else
                    f"kamera_mfma_kernel, sum of the averages of its {n_inst} instantiations "
                    f"(one launch each per step):")
            lines += ["", f"{what} {avg_ns / 1e3:.1f} us; algorithmic bytes "
                          f"per step {ab} -> {ab / avg_ns:.1f} GB/s "
                          f"({ab / avg_ns / HBM_PEAK_GBPS:.3f} of 8 TB/s)."]
        if avg_ns and bench_log and Path(bench_log).exists():
            rec = [json.loads(l) for l in Path(bench_log).read_text().splitlines()
                   if l.startswith("{") and '"metric"' in l]
            if rec:
                ev = rec[-1]["kernel_ms"]["mean"] * 1e6
                lines += [f"The benchmark's own HIP-event mean in this profiled run: {ev / 1e3:.1f} us "
                          f"per step (the event pair also brackets the job-table upload); "
                          f"rocprofv3 / events = {avg_ns / ev:.3f}."]
    counters = {}
    for tag, cname in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        files = sorted(d.glob(f"**/{tag}_counter_collection.csv"))
        if not files:
            continue
        per = {}
        for r in _read_csv(files[0]):
            if r.get("Counter_Name") != cname:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        counters[cname] = per
    traffic = None
    if counters:
        lines += ["", "## rocprofv3 --pmc (KiB per step: per dispatch, averaged over dispatches, "
                      "summed over the kernel's instantiations)", "",
                  "| kernel | counter | dispatches | KiB / step |", "|---|---|---|---|"]

        def pick(per, key):
            # per step: the average per dispatch of every matching kernel name, summed over
            # names (each instantiation is dispatched once per step)
            names = [k for k in per if key(k)]
            if not names:
                return None, 0
            return (sum(sum(per[k]) / len(per[k]) for k in names),
                    sum(len(per[k]) for k in names))

        copy_key = lambda k: "bitwise_not" in k.lower()
        kam_key = lambda k: "kamera_mfma_kernel" in k
        fig = {}
        for cname, per in counters.items():
            for label, key in (("kamera_mfma_kernel", kam_key), ("stream kernel (calibration)", copy_key)):
                v, n = pick(per, key)
                if v is not None:
                    lines.append(f"| {label} | {cname} | {n} | {v:.0f} |")
                    fig[(label, cname)] = v
        copy_bytes = CALIB_BYTES   # the calibration kernel reads 2 GiB and writes 2 GiB
        kf = fig.get(("kamera_mfma_kernel", "FETCH_SIZE"))
        kw = fig.get(("kamera_mfma_kernel", "WRITE_SIZE"))
        cf = fig.get(("stream kernel (calibration)", "FETCH_SIZE"))
        cw = fig.get(("stream kernel (calibration)", "WRITE_SIZE"))
        if None not in (kf, kw, cf, cw):
            sf, sw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
            traffic = kf * 1024 * sf + kw * 1024 * sw
            lines += ["", f"Calibration: a 2 GiB elementwise stream (bitwise_not) reads {cf * 1024 / copy_bytes:.3f}x "
                          f"and writes {cw * 1024 / copy_bytes:.3f}x its size by these counters; "
                          f"scale factors {sf:.3f} (fetch), {sw:.3f} (write).",
                      f"kamera_mfma_kernel HBM traffic per step: {traffic / 1e9:.3f} GB "
                      f"(fetch {kf * 1024 * sf / 1e9:.3f} + write {kw * 1024 * sw / 1e9:.3f}) "
                      f"vs algorithmic {ab / 1e9:.3f} GB: ratio {traffic / ab:.3f}."]
    out_md = ROOT / "profiles" / f"kamera_mfma_kernel_{workload}.md"
    out_md.write_text("\n".join(lines) + "\n")
    if traffic is not None:
        (ROOT / "profiles" / f"traffic_{workload}.json").write_text(json.dumps(
            {"kernel": "kamera_mfma_kernel", "workload": workload,
             "kernel_source_sha": kernel_source_hash(), "traffic_bytes": int(traffic),
             "algorithmic_bytes": ab, "command": command}, indent=1) + "\n")
    print(out_md.read_text())


def summarize_compile_profile(prof_dir: str, workload: str, command: str, bench_log: str) -> None:
    """profiles/patch_compile_<workload>.md from a rocprofv3 --kernel-trace --stats run (named
    `kt`) of bench.py and that run's JSON line (per-step bytes and flops of the compile)."""
    d = Path(prof_dir)
    rec = [json.loads(l) for l in Path(bench_log).read_text().splitlines()
           if l.startswith("{") and '"metric"' in l][-1]
    pc = rec["patch_compile"]
    calls = pc["steps"] + 1                     # one untimed call, then the timed ones
    rows = _read_csv(sorted(d.glob("**/kt_kernel_stats.csv"))[0])
    kinds = {"gram": [], "subspace": [], "project": []}
    for r in rows:
        for k in kinds:
            if k in r["Name"]:
                kinds[k].append(r)
    io = pc["io_bytes"]
    lines = [f"# patch compile on {workload}", "",
             "Commands (R = repository root on the machine that ran them):", ""]
    lines += [f"    {c.strip()}" for c in command.split(";") if c.strip()] + [""]
    lines += [f"Per compile call: rank {pc['rank']}, {pc['n_iter']} subspace rounds; "
              f"{pc['ms_per_batch']} ms by HIP events in this run "
              f"(one reuse pass over the same batch: {pc['reuse_ms_per_batch']} ms).", "",
              "| kernel | launches | us per call | bound | achieved | of peak |",
              "|---|---|---|---|---|---|"]
    gram_f, proj_f = pc["gram_flops"], pc["project_flops"]
    read2 = pc["input_bytes"]      # canonical + conditioned, read once by each streaming pass
    for k, rs in kinds.items():
        if not rs:
            continue
        tot_ns = sum(float(r["TotalDurationNs"]) for r in rs)
        n = sum(int(r["Calls"]) for r in rs)
        per_call_us = tot_ns / calls / 1e3
        if k == "gram":
            tf = gram_f / (per_call_us * 1e-6) / 1e12
            if rec.get("dtype") == "bf16":
                # bf16 rows: the Gram runs on bf16 MFMA over high/low parts of Delta, far from
                # that unit's peak; it is bounded by reading its inputs
                gbps = read2 / (per_call_us * 1e-6) / 1e9
                lines.append(f"| gram (Delta^T Delta, bf16 MFMA on split parts; {tf:.0f} TFLOP/s of "
                             f"distinct entries) | {n} | {per_call_us:.1f} | hbm | "
                             f"{gbps:.0f} GB/s | {gbps / HBM_PEAK_GBPS:.3f} |")
            else:
                lines.append(f"| gram (Delta^T Delta, fp32 MFMA) | {n} | {per_call_us:.1f} | mfma fp32 | "
                             f"{tf:.1f} TFLOP/s | {tf / FP32_PEAK_TFLOPS:.3f} |")
        elif k == "project":
            gbps = read2 / (per_call_us * 1e-6) / 1e9
            lines.append(f"| project (U = Delta V) | {n} | {per_call_us:.1f} | hbm | "
                         f"{gbps:.0f} GB/s | {gbps / HBM_PEAK_GBPS:.3f} |")
        else:
            lines.append(f"| subspace iteration | {n} | {per_call_us:.1f} | issue (MFMA products, fp64 factorisation chains) | - | - |")
    lines += ["", "Gram flops per call: n D (D + 1) per head (the distinct entries of the "
              "symmetric product) = "
              f"{gram_f / 1e9:.1f} GFLOP; Gram and projection bytes per call: both inputs once = "
              f"{read2 / 1e9:.3f} GB.", "",
              "## rocprofv3 --kernel-trace --stats (top kernels)", "",
              "| kernel | calls | avg us | total % |", "|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0)))[:8]:
        lines.append(f"| `{r['Name'][:70].replace('|', '/')}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    out_md = ROOT / "profiles" / f"patch_compile_{workload}.md"
    out_md.write_text("\n".join(lines) + "\n")
    print(out_md.read_text())


def summarize_attention_profile(prof_dir: str, command: str, bench_log: str) -> None:
    """profiles/decode_attention.md from a rocprofv3 --kernel-trace --stats run (named `kt`)
    of bench.py and that run's JSON line."""
    d = Path(prof_dir)
    rec = [json.loads(l) for l in Path(bench_log).read_text().splitlines()
           if l.startswith("{") and '"metric"' in l][-1]
    da = rec["decode_attention"]
    rows = _read_csv(sorted(d.glob("**/kt_kernel_stats.csv"))[0])
    seg = [r for r in rows if "attn_segment_kernel" in r["Name"] or "attn_rows_kernel" in r["Name"]]
    mrg = [r for r in rows if "attn_merge_kernel" in r["Name"]]
    chk = [r for r in rows if "chunk_attn_kernel" in r["Name"] or "chunk_rows_kernel" in r["Name"]]
    mla = [r for r in rows if "mla_segment_kernel" in r["Name"]]
    ca = rec.get("chunk_attention")
    dm = rec.get("decode_attention_mla")
    lines = ["# decode attention (consumer side)", "", "Commands (R = repository root on the machine that ran them):", ""]
    lines += [f"    {c.strip()}" for c in command.split(";") if c.strip()] + [""]
    lines += [f"Shape: {da['shape']}. Bytes per call: K and V once = {da['kv_bytes'] / 1e9:.3f} GB.",
              f"HIP events in this run: {da['ms_per_call']} ms per call (both kernels) = "
              f"{da['achieved_gbps']} GB/s ({da['hbm_frac']} of 8 TB/s).", "",
              "| kernel | calls | avg us | GB/s (K+V bytes / avg) | of 8 TB/s |", "|---|---|---|---|---|"]
    for r in seg + mrg:
        avg = float(r["AverageNs"])
        gb = da["kv_bytes"] / avg if "merge" not in r["Name"] else float("nan")
        lines.append(f"| `{r['Name'][:60]}` | {r['Calls']} | {avg / 1e3:.1f} | "
                     f"{gb:.0f} | {gb / HBM_PEAK_GBPS:.3f} |")
    if dm and mla:
        lines += ["", f"MLA cache: {dm['shape']}. Bytes per call: latent and k_rope rows once = "
                  f"{dm['kv_bytes'] / 1e9:.3f} GB. HIP events: {dm['ms_per_call']} ms per call "
                  f"(segment + merge kernels) = {dm['achieved_gbps']} GB/s ({dm['hbm_frac']} of 8 TB/s).",
                  "", "| kernel | calls | avg us | GB/s (bytes / avg) | of 8 TB/s |",
                  "|---|---|---|---|---|"]
        for r in mla:
            avg = float(r["AverageNs"])
            gb = dm["kv_bytes"] / avg
            lines.append(f"| `{r['Name'][:60]}` | {r['Calls']} | {avg / 1e3:.1f} | "
                         f"{gb:.0f} | {gb / HBM_PEAK_GBPS:.3f} |")
    if ca and chk:
        lines += ["", f"Attention over chunks read in place: {ca['shape']}. Bytes per call: "
                  f"canonical K and V, U_K and U_V rows and each chunk's V_K, V_V once = "
                  f"{ca['bytes'] / 1e9:.3f} GB. HIP events: {ca['ms_per_call']} ms per call "
                  f"(chunk + merge kernels) = {ca['achieved_gbps']} GB/s ({ca['hbm_frac']} of "
                  f"8 TB/s). The merge kernel's launches are counted with the decode ones above.",
                  "", "| kernel | calls | avg us | GB/s (bytes / avg) | of 8 TB/s |",
                  "|---|---|---|---|---|"]
        for r in chk:
            avg = float(r["AverageNs"])
            gb = ca["bytes"] / avg
            lines.append(f"| `{r['Name'][:60]}` | {r['Calls']} | {avg / 1e3:.1f} | "
                         f"{gb:.0f} | {gb / HBM_PEAK_GBPS:.3f} |")
    out_md = ROOT / "profiles" / "decode_attention.md"
    out_md.write_text("\n".join(lines) + "\n")
    print(out_md.read_text())


def config_of(p) -> dict:
    return {"workload": p.name, "family": p.family, "layers": p.n_layers,
            "kv_heads": p.n_kv_heads, "head_dim": p.head_dim, "rope_dim": p.rope_dim,
            "rope_layout": p.rope_layout, "chunks": p.n_chunks,
            "chunk_tokens": p.chunk_tokens[0], "rank": max(p.m_rot + p.m_plain),
            "cache": "dense" if p.page_table is None else f"paged{p.page_size}",
            "parallelism": "none (1 GPU)"}


def time_reuse(p, batch, steps: int, warmup: int, stream) -> dict:
    """`warmup` untimed kamera_reuse_batch calls over the whole batch, then `steps` timed ones:
    HIP events around every call on the launch stream, and the wall clock around them all
    (bracketed by device synchronisation)."""
    import torch
    from position_invariant_kv_kamera_amd import binding as kb

    ws = kb.Workspace(p.n_chunks)
    model, cache, chunks = kb.model_of(p), kb.cache_of(batch), kb.chunks_of(batch)
    sptr = stream.cuda_stream

    def step():
        kb.check(kb.kamera_reuse_batch(model, cache, chunks, p.n_chunks, ws.ptr, ws.nbytes, sptr))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    mean = sum(ev) / len(ev)
    return {"ev_mean": mean, "wall_ms": wall * 1e3 / steps,
            "kernel_ms": {"mean": round(mean, 4), "p10": round(ev[len(ev) // 10], 4),
                          "p50": round(ev[len(ev) // 2], 4),
                          "p90": round(ev[(9 * len(ev)) // 10], 4)}}


def config_record(name: str, steps: int, warmup: int, stream) -> dict:
    """One workload timed on its own (materialized, timed, freed): kernel time by HIP events,
    tokens/s, algorithmic GB/s and its fraction of 8 TB/s, and the HBM traffic of the
    committed counter summary when it was taken on the current kernel sources."""
    import torch
    from position_invariant_kv_kamera_amd import workloads as wl

    p = wl.plan(name)
    batch = wl.materialize(p, "cuda")
    t = time_reuse(p, batch, steps, warmup, stream)
    del batch
    ab = algorithmic_bytes(p)["total"]
    ms = t["ev_mean"]
    gbps = ab / (ms * 1e-3) / 1e9
    traffic, tinfo = traffic_from_profile(name)
    rec = {"kernel_ms": t["kernel_ms"], "tokens_per_s": round(p.total_tokens / (ms * 1e-3), 1),
           "algorithmic_bytes": ab, "achieved_gbps": round(gbps, 1),
           "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
           "traffic_over_algorithmic": round(traffic / ab, 4) if traffic else None,
           "steps": steps, "dtype": p.dtype, "config": config_of(p)}
    if tinfo == "stale":
        rec["traffic_note"] = "counters were taken on older kernel sources"
    if p.dtype == "f32":   # latency bound: the figure is the call's duration
        rec["latency_us"] = {k: round(v * 1e3, 2) for k, v in t["kernel_ms"].items()}
    torch.cuda.synchronize()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 CSV output in DIR and exit")
    ap.add_argument("--summarize-attention-profile", metavar="DIR",
                    help="write the decode-attention summary from rocprofv3 CSV output in DIR and exit")
    ap.add_argument("--summarize-compile-profile", metavar="DIR",
                    help="write the patch-compile summary from rocprofv3 CSV output in DIR and exit")
    ap.add_argument("--profile-command", default="", help="commands recorded in the summary (';'-separated)")
    ap.add_argument("--profile-bench-log", default="", help="stdout of the profiled kernel-trace run")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--compile-steps", type=int, default=5,
                    help="timed kamera_patch_compile calls over the same batch (0: skip)")
    ap.add_argument("--orbit-steps", type=int, default=2,
                    help="timed orbit compiles (3 orderings) in the compile leg (0: skip)")
    ap.add_argument("--attention-steps", type=int, default=20,
                    help="timed kamera_decode_attention calls on a 64 x 16K decode (0: skip)")
    ap.add_argument("--chunk-attention-steps", type=int, default=20,
                    help="timed kamera_chunk_attention calls on 64 x 16 chunks of 1024 (0: skip)")
    ap.add_argument("--compile-chunks", type=int, default=4,
                    help="chunks of the batch the compile leg forms patches for (0: all)")
    ap.add_argument("--configs", default=",".join(OTHER_CONFIGS),
                    help="workloads timed after the headline, one compact record each "
                         "('none': skip)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed reuse calls per additional workload")
    args = ap.parse_args()
    if args.summarize_attention_profile:
        summarize_attention_profile(args.summarize_attention_profile, args.profile_command,
                                    args.profile_bench_log)
        return
    if args.summarize_compile_profile:
        summarize_compile_profile(args.summarize_compile_profile, args.workload,
                                  args.profile_command, args.profile_bench_log)
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload, args.profile_command,
                          args.profile_bench_log)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the operator has no cross-GPU step and this "
              "build runs on a single MI355X (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from position_invariant_kv_kamera_amd import binding as kb
    from position_invariant_kv_kamera_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kb.load_library()   # raises if the HIP library is missing

    kb.check(kb.kamera_init())   # the staging ring: set up before anything is timed
    stream = torch.cuda.current_stream()

    p = wl.plan(args.workload)
    print(f"[bench] materializing {args.workload} on cuda:0", file=sys.stderr, flush=True)
    batch = wl.materialize(p, "cuda")
    print(f"[bench] timing {args.steps} reuse steps on {args.workload}", file=sys.stderr, flush=True)
    t = time_reuse(p, batch, args.steps, args.warmup, stream)
    ev_avg, ms_per_step = t["ev_mean"], t["wall_ms"]

    ab = algorithmic_bytes(p)
    gbps = ab["total"] / (ev_avg * 1e-3) / 1e9
    value = p.total_tokens / (ms_per_step * 1e-3)
    traffic, tinfo = traffic_from_profile(args.workload)
    flops = patch_flops(p)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": config_of(p),
        "achieved_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "kernel_ms": t["kernel_ms"],
        "mfma_util": round(flops / (ev_avg * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 5),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": ab["total"],
                     "kernel": "kamera_mfma_kernel" if p.dtype == "bf16" else "kamera_valu_kernel",
                     "timed_with": "hip events on the launch stream"},
        "kernel_source_sha": kernel_source_hash(),
    }
    if tinfo == "stale":
        out["roofline"]["traffic_note"] = "counters were taken on older kernel sources"
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(batch, args.cpu_budget)
    if args.compile_steps > 0:
        print("[bench] timing the patch compile", file=sys.stderr, flush=True)
        out["patch_compile"] = compile_leg(p, batch, args.compile_steps, stream, args.orbit_steps,
                                           args.compile_chunks or None)
    del batch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # context: the runtime's device-to-device copy, and a plain elementwise stream kernel
    # (bitwise_not over 2 GiB of int32: 2 GiB read, 2 GiB written; it also calibrates the
    # rocprofv3 byte counters)
    buf = torch.zeros(CALIB_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(buf)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return reps * 2 * CALIB_BYTES / (e0.elapsed_time(e1) * 1e-3) / 1e9

    copy_gbps = timed(lambda: dst.copy_(buf))
    stream_gbps = timed(lambda: torch.bitwise_not(buf, out=dst))
    del buf, dst
    out["device_copy_gbps"] = round(copy_gbps, 1)
    out["stream_kernel_gbps"] = round(stream_gbps, 1)
    out["frac_of_stream_kernel"] = round(gbps / stream_gbps, 4)

    configs = [c for c in args.configs.split(",") if c and c != "none" and c != args.workload]
    if configs:
        out["configs"] = {}
    for name in configs:
        print(f"[bench] per-config record: {name}", file=sys.stderr, flush=True)
        out["configs"][name] = config_record(name, args.config_steps, args.warmup, stream)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.attention_steps > 0:
        print("[bench] timing decode attention", file=sys.stderr, flush=True)
        out["decode_attention"] = attention_leg(args.attention_steps, stream)
        print("[bench] timing decode attention over an MLA cache", file=sys.stderr, flush=True)
        out["decode_attention_mla"] = mla_attention_leg(args.attention_steps, stream)
    if args.chunk_attention_steps > 0:
        print("[bench] timing attention over chunks read in place", file=sys.stderr, flush=True)
        out["chunk_attention"] = chunk_attention_leg(args.chunk_attention_steps, stream)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
