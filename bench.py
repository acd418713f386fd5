"""Benchmark of one gated layer of TokenGate's pruned prefill on one MI355X.

One step = tg_gate_score -> tg_topk_select -> tg_gather_kept -> tg_attn_prepare
-> tg_attn_forward (the two halves of tg_keybias_attn_prefill) on one batch of
seeded synthetic input, all resident in HBM before the timed region.  Q/K/V are synthetic stand-ins for the host
model's projections of the kept residuals (sized by the kept count); the
projections themselves are outside the gated layer.

Prints one JSON line: ms per gated layer at 128k (headline: steps bracketed by
synchronisations, no events inside), per-stage times from a second pass with
HIP events recorded on the launch stream between the calls, the attention
kernel's roofline against
the bf16 MFMA peak, top-K + gather bandwidth against HBM, one decode step over
the kept-only cache against HBM, the same attention over all 131072 tokens (the
full-prefill comparator), the 32k budget sweep, and the CPU oracle timed on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from learned_token_pruning_05_amd import _lib as tg  # noqa: E402

METRIC = "ms/gated layer + key-bias attn TFLOP/s (frac bf16 peak) at 32k/128k, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILE_PMC = os.path.join(ROOT, "profiles", "gated_layer_hbm_counters.md")
COPY_BYTES = 256 << 20         # --calibrate-copy: bytes read (and written) per copy


def attn_flops(cu_kept, hq, d):
    m = np.diff(np.asarray(cu_kept, dtype=np.int64))
    return float(2 * d * hq * np.sum(m * (m + 1)))


class Layer:
    """Device-resident inputs, outputs and workspace of one gated layer."""

    def __init__(self, w: workloads.Workload):
        dev = torch.device("cuda:0")
        self.w = w
        g = w.gate_inputs()
        self.x = g["x"].to(dev)
        self.w1 = g["w1"].to(dev)
        self.w2 = g["w2"].to(dev)
        self.b2 = g["b2"]
        i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(dev)
        self.cu = i32(w.cu_seqlens)
        self.db, self.de, self.kd = i32(w.doc_begin), i32(w.doc_end), i32(w.k_doc_arr)
        self.ck_h = tg.tg_kept_counts(w.cu_seqlens, w.doc_begin, w.doc_end, w.k_doc_arr)
        self.ck = i32(self.ck_h)
        self.m = int(self.ck_h[-1])
        self.max_seq = int(max(w.seqlens))
        self.max_kept = int(np.diff(self.ck_h).max())
        q, k, v = w.qkv(self.m)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        gain, self.tau = w.attn_params()
        self.gain = torch.from_numpy(gain).to(dev)
        n = w.n_tokens
        self.scores = torch.empty(n, dtype=torch.float32, device=dev)
        self.kept = torch.empty(self.m, dtype=torch.int32, device=dev)
        self.xk = torch.empty((self.m, w.d_model), dtype=self.x.dtype, device=dev)
        self.sk = torch.empty(self.m, dtype=torch.float32, device=dev)
        self.pk = torch.empty(self.m, dtype=torch.int32, device=dev)
        self.out = torch.empty((self.m, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.n_q_heads, self.m), dtype=torch.float32, device=dev)
        self.ws_topk = torch.empty(tg.tg_topk_workspace_bytes(w.n_seqs, n, self.max_seq), dtype=torch.uint8,
                                   device=dev)
        self.ws = torch.empty(tg.tg_attn_workspace_bytes(w.n_seqs, self.m, w.n_kv_heads, w.head_dim),
                              dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    STAGES = ("gate", "topk", "gather", "attn_prep", "attn_fwd")

    def step(self, ev=None):
        """One gated layer; ev = 6 events recorded between the stages, or None."""
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        tg.tg_gate_score(self.x, self.w1, None, self.w2, self.b2, scores=self.scores)
        rec(1)
        tg.tg_topk_select(self.scores, self.cu, self.db, self.de, self.kd, self.ck, self.m, self.max_seq,
                          kept_idx=self.kept, workspace=self.ws_topk)
        rec(2)
        tg.tg_gather_kept(self.x, self.scores, self.kept, self.cu, self.ck, x_kept=self.xk,
                          scores_kept=self.sk, pos_kept=self.pk)
        rec(3)
        # tg_keybias_attn_prefill in its two halves, so the attention kernel can be timed alone
        tg.tg_attn_prepare(self.k, self.v, self.sk, self.pk, self.ck, rope_base=self.w.rope_base,
                           workspace=self.ws)
        rec(4)
        tg.tg_attn_forward(self.q, self.gain, self.tau, self.ck, self.max_kept, self.w.n_kv_heads, self.ws,
                           rope_base=self.w.rope_base, out=self.out, lse=self.lse)
        rec(5)

    def step_fused(self):
        """The same layer through tg_gated_select (gate -> top-K -> gather in one call)."""
        tg.tg_gated_select(self.x, self.w1, None, self.w2, self.b2, self.cu, self.db, self.de, self.kd, self.ck,
                           self.m, self.max_seq, scores=self.scores, kept_idx=self.kept, x_kept=self.xk,
                           scores_kept=self.sk, pos_kept=self.pk, workspace=self.ws_topk)
        tg.tg_attn_prepare(self.k, self.v, self.sk, self.pk, self.ck, rope_base=self.w.rope_base,
                           workspace=self.ws)
        tg.tg_attn_forward(self.q, self.gain, self.tau, self.ck, self.max_kept, self.w.n_kv_heads, self.ws,
                           rope_base=self.w.rope_base, out=self.out, lse=self.lse)

    def measure_graph(self, steps):
        """The layer captured once into a HIP graph (the front half through
        tg_gated_select), then `steps` replays back to back between two
        synchronisations: one host launch per layer."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step_fused()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step_fused()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        del graph
        return {"ms_per_gated_layer": round(ms, 4), "launches_per_layer": 1,
                "calls": "tg_gated_select + tg_attn_prepare + tg_attn_forward, captured into one HIP graph"}

    def measure(self, steps, warmup):
        """Headline: `steps` back-to-back layers bracketed by synchronisations, no
        events between stages.  Breakdown: a second pass with an event between
        every stage (HIP events on the launch stream)."""
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps * 1e3
        gpu = e0.elapsed_time(e1) / steps
        n = len(self.STAGES)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(n)] for e in evs])   # ms
        return dict(wall_ms=wall, gpu_ms=gpu, stage_ms=st.mean(axis=0), stage_med=np.median(st, axis=0),
                    stage_p10=np.percentile(st, 10, axis=0), stage_p90=np.percentile(st, 90, axis=0))

    def measure_cold(self, steps):
        """Per-stage times with cold caches: before every layer (outside the
        events) a 512 MiB buffer is written, which evicts the 256 MB Infinity
        Cache and the L2s, so the gate, top-K and gather read their inputs
        from HBM.  Median and p10/p90 per stage."""
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=self.x.device)
        n = len(self.STAGES)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
        for i in range(steps):
            scratch.fill_(i & 255)
            self.step(evs[i])
        torch.cuda.synchronize()
        del scratch
        st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(n)] for e in evs]) * 1e3   # us
        return {"stage_us_median": {k: round(float(v), 2) for k, v in zip(self.STAGES, np.median(st, axis=0))},
                "stage_us_p10_p90": {k: [round(float(a), 1), round(float(b), 1)] for k, a, b in
                                     zip(self.STAGES, np.percentile(st, 10, axis=0), np.percentile(st, 90, axis=0))},
                "steps": steps}

    # algorithmic work per launch
    def gate_work(self):
        w = self.w
        n, d, dh = w.n_tokens, w.d_model, w.d_hid
        e = self.x.element_size()
        return 2.0 * n * d * dh, float(n * d * e + dh * d * e + 4 * n)

    def topk_gather_bytes(self):
        """Algorithmic bytes of top-K + gather: the scores read, the kept indices
        written, and per kept row its residual read and written plus index,
        score and position."""
        n, m, d = self.w.n_tokens, self.m, self.w.d_model
        e = self.x.element_size()
        return float(4 * n + 4 * m + m * (2 * d * e + 12) + 4 * m)

    def attn_work(self):
        return attn_flops(self.ck_h, self.w.n_q_heads, self.w.head_dim)


def measure_decode(layer: Layer, steps=50, warmup=5):
    """One decode step (tg_attn_decode: one new query per sequence) over the
    kept-only cache the layer's tg_attn_prepare left in its workspace; HBM-bound
    by the cache read (K' (D+16) x 2 B + V^T D x 2 B per kept key and kv head)."""
    w = layer.w
    dev = layer.q.device
    g = torch.Generator(device="cpu").manual_seed(11)
    qn = torch.randn(w.n_seqs, w.n_q_heads, w.head_dim, generator=g).to(torch.bfloat16).to(dev)
    q_pos = torch.from_numpy(np.asarray(w.seqlens, dtype=np.int32)).to(dev)   # past every kept position
    out = torch.empty((w.n_seqs, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.n_q_heads, w.n_seqs), dtype=torch.float32, device=dev)
    wsd = torch.empty(max(1, tg.tg_attn_decode_workspace_bytes(w.n_seqs, layer.max_kept, w.n_q_heads,
                                                                w.head_dim)), dtype=torch.uint8, device=dev)
    f = lambda: tg.tg_attn_decode(qn, q_pos, layer.gain, layer.tau, layer.pk, layer.ck, layer.max_kept,
                                  w.n_kv_heads, layer.ws, rope_base=w.rope_base, out=out, lse=lse, workspace=wsd)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    ref = out.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        f()
    e1.record()
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) / steps * 1e3
    # A serving loop replays captured decode steps: `steps` calls in one HIP
    # graph run back to back on the GPU, without the host's per-call cost
    # (argument checks and two launches, about 20 us here) between them.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            f()
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    if not torch.equal(out, ref):
        raise RuntimeError("decode: graph replay differs from the eager call")
    del graph
    cache = float(layer.m * w.n_kv_heads * (4 * w.head_dim + 32))
    return {"us_per_step": round(us, 2), "us_per_call_eager": round(us_eager, 2), "cache_bytes": cache,
            "gbs": round(cache / us / 1e3, 1), "frac_hbm": round(cache / us / 1e3 / PEAK_HBM_GBS, 4),
            "queries": w.n_seqs, "timing": f"{steps} steps captured in one HIP graph, one replay timed with events",
            "kernels": "attn_decode_split_kernel + attn_decode_combine_kernel (tg_attn_decode)"}


def measure_gate_grads(layer: Layer, steps=10, warmup=3):
    """Gate-side gradients (tg_attn_gate_grads: dL/ds_j, dL/dg_h, dL/dtau) of the
    layer's attention for a synthetic dL/dO, over the cache and the forward
    output and LSE the layer left.  Algorithmic work: the two products of every
    causal pair and q head, q.k and dO.v, 4 D flops per pair (the same count
    as the forward)."""
    w = layer.w
    dev = layer.q.device
    d_out = w.d_out(layer.m).to(dev)
    dsc = torch.empty(layer.m, dtype=torch.float32, device=dev)
    dg = torch.empty(w.n_q_heads, dtype=torch.float32, device=dev)
    dt = torch.empty(1, dtype=torch.float32, device=dev)
    wsg = torch.empty(tg.tg_attn_gate_grads_workspace_bytes(w.n_seqs, layer.m, layer.max_kept, w.n_q_heads,
                                                            w.head_dim), dtype=torch.uint8, device=dev)
    f = lambda: tg.tg_attn_gate_grads(layer.q, layer.v, layer.sk, layer.gain, layer.tau, layer.ck, layer.max_kept,
                                      layer.out, layer.lse, d_out, layer.ws, rope_base=w.rope_base, d_score=dsc,
                                      d_gain=dg, d_tau=dt, workspace=wsg)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        f()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    fl = layer.attn_work()
    return {"us_per_step": round(us, 1), "flops": fl, "tflops": round(fl / us / 1e6, 1),
            "frac_bf16_peak": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4),
            "kernels": "bwd_prep_kernel + bwd_main_kernel + bwd_reduce_kernel (tg_attn_gate_grads)"}


def measure_random_k(layer: Layer, steps=50, warmup=5):
    """The random-K selector mode (tg_random_k_select: SplitMix64 scores for every
    token, then the top-K passes) on the layer's sequence layout, a new seed per
    call.  Bytes as the top-K's: the scores written and read, the kept indices."""
    w = layer.w
    dev = layer.x.device
    n = w.n_tokens
    kept = torch.empty(layer.m, dtype=torch.int32, device=dev)
    wsr = torch.empty(tg.tg_random_k_workspace_bytes(w.n_seqs, n, layer.max_seq), dtype=torch.uint8, device=dev)
    f = lambda seed: tg.tg_random_k_select(seed, layer.cu, layer.db, layer.de, layer.kd, layer.ck, n, layer.m,
                                           layer.max_seq, kept_idx=kept, workspace=wsr)
    for i in range(warmup):
        f(1000 + i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        f(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    return {"us_per_call": round(us, 2), "tokens": n, "kept": layer.m,
            "kernels": "random_scores_kernel + the four top-K kernels (tg_random_k_select)"}


def measure_full_prefill(w: workloads.Workload, pruned_layer_ms: float, reps=3):
    """The same attention at K = n_doc (every token kept, no gate/select/gather):
    tg_attn_prepare + tg_attn_forward over all N tokens, beside the pruned layer,
    as a per-layer analogue of the pages' full-vs-pruned prefill comparison."""
    dev = torch.device("cuda:0")
    n = w.n_tokens
    ck = np.array([0, n], dtype=np.int32)
    g = torch.Generator(device="cpu").manual_seed(4)
    q = (torch.randn(n, w.n_q_heads, w.head_dim, generator=g)).to(torch.bfloat16).to(dev)
    k = (torch.randn(n, w.n_kv_heads, w.head_dim, generator=g)).to(torch.bfloat16).to(dev)
    v = (torch.randn(n, w.n_kv_heads, w.head_dim, generator=g)).to(torch.bfloat16).to(dev)
    sk = torch.randn(n, generator=g).to(dev)
    gain, tau = w.attn_params()
    gain = torch.from_numpy(gain).to(dev)
    pos = torch.arange(n, dtype=torch.int32, device=dev)
    ckd = torch.from_numpy(ck).to(dev)
    ws = torch.empty(tg.tg_attn_workspace_bytes(1, n, w.n_kv_heads, w.head_dim), dtype=torch.uint8, device=dev)
    out = torch.empty((n, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.n_q_heads, n), dtype=torch.float32, device=dev)
    prep = lambda: tg.tg_attn_prepare(k, v, sk, pos, ckd, rope_base=w.rope_base, workspace=ws)
    fwd = lambda: tg.tg_attn_forward(q, gain, tau, ckd, n, w.n_kv_heads, ws, rope_base=w.rope_base, out=out, lse=lse)
    prep(); fwd()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_prep, t_fwd = [], []
    for _ in range(reps):
        e[0].record(); prep(); e[1].record(); fwd(); e[2].record()
        torch.cuda.synchronize()
        t_prep.append(e[0].elapsed_time(e[1]))
        t_fwd.append(e[1].elapsed_time(e[2]))
    fl = attn_flops(ck, w.n_q_heads, w.head_dim)
    fwd_ms, prep_ms = float(np.median(t_fwd)), float(np.median(t_prep))
    del q, k, v, ws, out, lse
    torch.cuda.empty_cache()
    return {"tokens": n, "attn_prep_ms": round(prep_ms, 3), "attn_fwd_ms": round(fwd_ms, 3),
            "attn_fwd_tflops": round(fl / fwd_ms / 1e9, 2),
            "attn_fwd_frac_bf16_peak": round(fl / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "full_over_pruned_layer": round((prep_ms + fwd_ms) / pruned_layer_ms, 2)}


def pmc_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source (else None)."""
    if not os.path.exists(PROFILE_PMC):
        return None
    import hashlib
    src = os.path.join(ROOT, "learned_token_pruning_05_amd", "csrc", "tg_attn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    vals = {}
    for line in open(PROFILE_PMC):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().split()[0]
    if vals.get("kernel_source_sha256_16") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w: workloads.Workload):
    """The fp64 oracle, as it stands, over one whole gated layer of the same
    workload (about 10 s on the host's CPU threads, so no extrapolation)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    g = w.gate_inputs()
    n = w.n_tokens
    t = time.perf_counter()
    oracle.gate_score(g["x_f"], g["w1_f"], g["b1_f"], g["w2_f"], g["b2"])
    gate_ms = (time.perf_counter() - t) * 1e3
    s32 = w.topk_scores()                   # seeded selector input of this workload's shape
    t = time.perf_counter()
    kept, ck = oracle.topk_select(s32, w.cu_seqlens, w.doc_begin, w.doc_end, w.k_doc_arr)
    topk_ms = (time.perf_counter() - t) * 1e3
    t = time.perf_counter()
    _, sk, pk = oracle.gather_kept(g["x_f"], s32, kept, w.cu_seqlens, ck)
    gather_ms = (time.perf_counter() - t) * 1e3
    m = int(ck[-1])
    q, k, v = (t_.float().numpy() for t_ in w.qkv(m))
    gain, tau = w.attn_params()
    t = time.perf_counter()
    oracle.keybias_attention(q, k, v, sk, gain, tau, pk, ck, rope_base=w.rope_base)
    attn_ms = (time.perf_counter() - t) * 1e3
    total = gate_ms + topk_ms + gather_ms + attn_ms
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(total, 3), "unit": "ms/gated layer", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "os_cpu_count": os.cpu_count(),
            "sample": f"{w.name}: the whole gated layer ({n} tokens, {m} kept, all heads), no extrapolation; "
                      f"per stage ms: gate {gate_ms:.0f}, topk {topk_ms:.0f}, gather {gather_ms:.0f}, "
                      f"attn {attn_ms:.0f}"}


def machine_context():
    """Context for the peaks: a plain device copy's GB/s and a plain bf16 GEMM's
    TFLOP/s (vendor library) on this GPU, and the amdgpu kernel driver's current clock levels."""
    dev = torch.device("cuda:0")
    x = torch.ones(256 << 20, dtype=torch.bfloat16, device=dev)   # 512 MiB
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * x.numel() * 2 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del x, y
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(copy_gbs, 1), "copy_frac_hbm": round(copy_gbs / PEAK_HBM_GBS, 4),
            "bf16_gemm_8192_tflops": round(gemm_tflops, 1),
            "bf16_gemm_frac_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
            "dpm_clock_levels": dpm_clock_levels()}


def dpm_clock_levels():
    """The current shader and memory clock levels the amdgpu driver lists in sysfs
    for this device (the entry marked '*'), read from files rather than through a
    child process, so that a profiler's preload never reaches another program."""
    try:
        pr = torch.cuda.get_device_properties(0)
        d = f"/sys/bus/pci/devices/{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        out = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            with open(os.path.join(d, name)) as f:
                cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
            out[name[-4:]] = cur[0] if cur else None
        return out
    except Exception:
        return None


def summarize(layer: Layer, r):
    stage_s = dict(zip(Layer.STAGES, (x * 1e-3 for x in r["stage_ms"])))
    gf, gb = layer.gate_work()
    tb = layer.topk_gather_bytes()
    af = layer.attn_work()
    tg_s = stage_s["topk"] + stage_s["gather"]
    return {
        "ms_per_gated_layer": round(r["wall_ms"], 4),
        "gpu_ms_per_gated_layer": round(r["gpu_ms"], 4),
        "stage_us": {k: round(v * 1e6, 2) for k, v in stage_s.items()},
        "stage_us_median": {k: round(float(v) * 1e3, 2) for k, v in zip(Layer.STAGES, r["stage_med"])},
        "stage_us_p10_p90": {k: [round(a * 1e3, 1), round(b * 1e3, 1)]
                             for k, a, b in zip(Layer.STAGES, r["stage_p10"], r["stage_p90"])},
        "attn_fwd_tflops": round(af / stage_s["attn_fwd"] / 1e12, 2),
        "attn_fwd_frac_bf16_peak": round(af / stage_s["attn_fwd"] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "attn_prep_plus_fwd_tflops": round(af / (stage_s["attn_prep"] + stage_s["attn_fwd"]) / 1e12, 2),
        "topk_gather_gbs": round(tb / tg_s / 1e9, 1),
        "topk_gather_frac_hbm": round(tb / tg_s / 1e9 / PEAK_HBM_GBS, 4),
        "gate_tflops": round(gf / stage_s["gate"] / 1e12, 2), "gate_gbs": round(gb / stage_s["gate"] / 1e9, 1),
        "gate_frac_hbm": round(gb / stage_s["gate"] / 1e9 / PEAK_HBM_GBS, 4),
        "kept": layer.m,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true", help="skip the 32k budget sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 3 plain device copies of 256 MiB, the reference kernel for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    tg.load()
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t_start = time.perf_counter()

    def progress(what):
        print(f"[bench] {what} done ({time.perf_counter() - t_start:.1f} s)", file=sys.stderr, flush=True)

    w = workloads.long128k()
    layer = Layer(w)
    r = layer.measure(args.steps, args.warmup)
    progress("128k gated layer")
    head = summarize(layer, r)
    af = layer.attn_work()
    attn_s = r["stage_ms"][Layer.STAGES.index("attn_fwd")] * 1e-3
    achieved = af / attn_s / 1e12
    cold = layer.measure_cold(args.steps)
    graph = layer.measure_graph(args.steps)
    decode = measure_decode(layer)
    grads = measure_gate_grads(layer)
    random_k = measure_random_k(layer)
    del layer
    torch.cuda.empty_cache()
    full = measure_full_prefill(w, r["wall_ms"])
    progress("128k cold cache, graph, decode, gate gradients, random-K, full prefill")

    # the other two configurations' layers: 16k (one sequence) and varlen (8 packed sequences)
    others = {}
    for wo in (workloads.qwen16k(), workloads.varlen()):
        lo = Layer(wo)
        ro = lo.measure(args.steps, args.warmup)
        others[wo.name] = summarize(lo, ro)
        others[wo.name]["cold_cache_stage_us_median"] = lo.measure_cold(args.steps)["stage_us_median"]
        others[wo.name]["decode"] = measure_decode(lo)
        others[wo.name]["gate_grads"] = measure_gate_grads(lo)
        others[wo.name]["random_k"] = measure_random_k(lo)
        del lo
        torch.cuda.empty_cache()
        progress(f"{wo.name} gated layer")

    sweep = {}
    if not args.no_sweep:
        for pct in workloads.BUDGET_PCTS:
            ws = workloads.sweep32k(pct)
            ls = Layer(ws)
            rs = ls.measure(max(5, args.steps // 2), 2)
            sweep[ws.name] = summarize(ls, rs)
            sweep[ws.name]["cold_cache_stage_us_median"] = ls.measure_cold(max(5, args.steps // 2))["stage_us_median"]
            del ls
            torch.cuda.empty_cache()
            progress(ws.name)

    context = machine_context()
    cpu = None
    cpu_others = {}
    if not args.no_cpu:
        cpu = cpu_baseline(w)
        progress("CPU oracle 128k")
        for wo in (workloads.qwen16k(), workloads.varlen()):
            cpu_others[wo.name] = cpu_baseline(wo)
            progress(f"CPU oracle {wo.name}")

    line = {
        "metric": METRIC,
        "value": round(r["wall_ms"], 4),
        "unit": "ms/gated layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Qwen3-1.7B-shaped gated layer, stands in for the pages' NIAH/QA workloads)",
        "config": {"workload": "128k: 1 sequence, N=131072 (130816 document + 256 question), keep 8192 "
                               "document tokens (M=8448), d_model 2048 bf16, gate 2048->256->1, 16 q / 8 kv "
                               "heads, head_dim 128, RoPE 1e6, causal key-bias attention over kept tokens",
                   "global_batch": 1, "seq_len": w.n_tokens, "kept": head["kept"], "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "attn_fwd_kernel (tg_attn_forward)",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": pmc_traffic()},
        "gated_layer_128k": head,
        "cold_cache_128k": cold,
        "graph_128k": graph,
        "decode_128k": decode,
        "gate_grads_128k": grads,
        "random_k_128k": random_k,
        "full_prefill_128k": full,
        "gated_layer_16k": others.get("16k"),
        "gated_layer_varlen": others.get("varlen"),
        "sweep_32k": sweep,
        "machine_context": context,
        "cpu_baseline": cpu,
        "cpu_baseline_16k": cpu_others.get("16k"),
        "cpu_baseline_varlen": cpu_others.get("varlen"),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
