#!/usr/bin/env python3
"""Throughput of absorbed-MLA decode on one MI355X, against its roofline.

One step = the whole decode path for one batch: absorbed query
(mla_absorb_q), then attention over the paged latent cache, the split merge
and the W_UV up-projection (mla_decode_upproj: one launch for up to 64 heads
and 32 sequences, else mla_decode_partial followed by the merge and
up-projection kernels).  Inputs are synthetic with the workload's
shapes and distributions and are resident in HBM before timing starts.  To
keep the 256 MB last-level cache from serving repeated reads, the step
rotates over enough replicas of its inputs (cache, weights, queries) to
exceed 600 MB.  Consecutive steps are captured together in HIP graphs of up
to 10 steps (as a model's layers share one graph per decode step), so that a
graph launch is not charged to every step; --graph-steps 1 times one graph
per step.

With --layer the step starts from hidden states instead: the query path
(mla_q_project: c^Q, q^C, q^R), the new token's cache append
(mla_kv_append: c^KV and the rotated k^R), the same decode path, and the
output projection (mla_output_proj: u = W^O [o_1..o_H]), with synthetic
bf16 weights at model width --d-model; each projection is also timed alone
against its HBM roofline.

Prints one JSON line: value = cached tokens per second over the whole step
(median, p10 and p90 of the per-step times beside the mean), the decode
kernel's achieved HBM bandwidth and matrix-core rate against MI355X's
published peaks and against ceilings measured in the same run (streaming
HBM read, bf16 matrix-core loop, LDS reads: include/mla_ceilings.h), and the
CPU oracle timed on a bounded sample.  The default workload is the largest
one that fits one GPU, decode_h128 (B = 64 sequences, 128 heads, lengths
U[8192, 32768]); with the default --config the line also carries, under
"workloads", one record per other workload (decode_h16, long_bf16, long_fp8,
prefill_h128) measured the same way with fewer steps.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode cached-tokens/s + TB/s & TFLOP/s as % of MI355X roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 matrix cores
PEAK_F32_TFLOPS = 157.3        # fp32 matrix
FLOP_PER_TOKEN_HEAD = 2 * 576 + 2 * 512   # score + latent accumulation
REPLICA_TARGET_BYTES = 600 << 20
HEADLINE = "decode_h128"
SUB_WORKLOADS = ("decode_h16", "long_bf16", "long_fp8", "prefill_h128")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=HEADLINE,
                    choices=["decode_h16", "decode_h128", "long_bf16", "long_fp8", "tiny_f32", "prefill_h128"])
    ap.add_argument("--splits", type=int, default=-1, help="num_splits (-1: the workload's own, 0: automatic)")
    ap.add_argument("--replicas", type=int, default=0, help="input replicas (0: enough for 600 MB)")
    ap.add_argument("--no-graph", action="store_true", help="launch the step eagerly instead of as a HIP graph")
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="decode steps per HIP graph (0: the largest divisor of --steps up to 10; "
                         "1: a graph per step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layer", action="store_true",
                    help="step from hidden states to u: query path, cache append, decode, output projection")
    ap.add_argument("--d-model", type=int, default=7168, help="model width d for --layer (not fixed by the pages)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (multi-token decode, mla_decode_multi); decode workloads only")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-workload sub-records of the default run")
    ap.add_argument("--sub-steps", type=int, default=20, help="timed steps of each sub-record")
    ap.add_argument("--sub-cpu-seconds", type=float, default=3.0, help="CPU oracle budget of each sub-record")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling kernels")
    return ap.parse_args()


def _pct(xs, q):
    """q-th percentile (linear interpolation) of a list of floats."""
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def decode_kernel_name(dtype: str, heads: int) -> str:
    """The attention kernel the library launches for a cache dtype and a
    (query tokens x heads) count: the fp32 kernel, the four-wave kernel for
    65..128 heads over a bf16 or fp8 cache, else the eight-wave kernel."""
    if dtype == "f32":
        return "decode_f32_kernel"
    return "decode_wide_kernel" if heads > 64 else "decode_mfma_kernel"


def step_stats(step_ms):
    return {"median": _pct(step_ms, 50), "p10": _pct(step_ms, 10), "p90": _pct(step_ms, 90), "n": len(step_ms)}


def blas_info():
    """The NumPy build and the BLAS library and thread count the oracle runs on."""
    import numpy as np
    try:
        import threadpoolctl
        info = [{k: d.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    except Exception as e:  # threadpoolctl missing: record that
        info = [{"error": str(e)}]
    return {"numpy": np.__version__, "blas": info}


def measure_ceilings(dev):
    """Streaming HBM read (2 GiB), bf16 matrix-core loops (both shapes the
    kernels issue) and LDS reads (16-byte and transposing), each the median
    of five timed launches."""
    import torch

    import mla_latent_kv_30_amd as mla
    from mla_latent_kv_30_amd import _lib as L

    sink = L.ceiling_sink(dev)
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)

    def timed(launch, reps=5):
        launch()
        torch.cuda.synchronize()
        ms = []
        work = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            work = launch()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        return work, ms[len(ms) // 2]

    out = {}
    w, ms = timed(lambda: L.ceiling_hbm_read(buf, sink))
    out["hbm_read_GBps"] = w / (ms * 1e-3) / 1e9
    del buf
    for name, shape in (("mfma_bf16_32x32x16_TFLOPs", L.CEILING_MFMA_32X32X16),
                        ("mfma_bf16_16x16x32_TFLOPs", L.CEILING_MFMA_16X16X32)):
        w, ms = timed(lambda: L.ceiling_mfma_bf16(shape, 20000, sink))
        out[name] = w / (ms * 1e-3) / 1e12
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for name, kind in (("lds_read_b128_B_per_clk_cu", L.CEILING_LDS_B128),
                       ("lds_read_tr_b64_B_per_clk_cu", L.CEILING_LDS_TR_B64)):
        w, ms = timed(lambda: L.ceiling_lds_read(kind, 4000, sink))
        out[name] = w / (ms * 1e-3) / cus / 2.4e9
    out["note"] = ("medians of 5 launches; LDS bytes per clock per compute unit at the 2.4 GHz nominal clock; "
                   f"{cus} compute units")
    torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, host, budget_s):
    """The oracle as it stands, on whole sequences until the time budget is
    used: sequences in order, over the workload again when it is done before
    the budget (a small workload takes well under a second per pass).  Every
    head for up to 16 heads, else the first 8 (heads are independent)."""
    from oracle import mla_oracle as orc

    cores = len(os.sched_getaffinity(0))
    off = host["offsets"]
    heads = list(range(wl.H)) if wl.H <= 16 else list(range(8))
    tokens = 0
    seqs = 0
    t0 = time.perf_counter()
    while seqs == 0 or time.perf_counter() - t0 <= budget_s:
        b = seqs % wl.B
        orc.decode_sequence(host["q_c"][b][heads], host["q_r"][b][heads], host["c_kv"][off[b]:off[b + 1]],
                            host["k_r"][off[b]:off[b + 1]], host["w_uk"][heads], host["w_uv"][heads])
        tokens += int(wl.lens[b])
        seqs += 1
    dt = time.perf_counter() - t0
    # cached tokens per second with all of the workload's heads
    rate = tokens * len(heads) / wl.H / dt
    passes = f"{seqs / wl.B:.1f} passes over the {wl.B} sequences" if seqs > wl.B else f"{seqs} of {wl.B} sequences"
    return {"value": rate, "unit": "cached-tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{passes} ({tokens} cached tokens) x {len(heads)} of {wl.H} heads, "
                      f"fp64 NumPy, {dt:.1f} s; rate scaled to all {wl.H} heads",
            "extrapolated_full_step_s": wl.total_tokens / rate, "build": blas_info()}


def cpu_baseline_prefill(wl, host, budget_s, seed=0):
    """The oracle's causal prefill on 8 heads, one query row at a time (row
    T-1, row 0, then random rows) until the time budget is used; rate in the
    method's algorithmic TFLOP/s (causal pairs x heads x 2176 FLOP)."""
    import numpy as np

    from oracle import mla_oracle as orc

    cores = len(os.sched_getaffinity(0))
    T = int(wl.lens[0])
    heads = list(range(min(8, wl.H)))
    rng = np.random.default_rng(seed)
    order = [T - 1, 0] + [int(x) for x in rng.permutation(np.arange(1, T - 1))]
    q_c, q_r = host["q_c"][:, heads], host["q_r"][:, heads]
    w_uk, w_uv = host["w_uk"][heads], host["w_uv"][heads]
    pairs = 0
    rows = 0
    t0 = time.perf_counter()
    while rows == 0 or (time.perf_counter() - t0 <= budget_s and rows < len(order)):
        t = order[rows]
        orc.prefill_causal(q_c, q_r, host["c_kv"], host["k_r"], w_uk, w_uv, rows=[t])
        pairs += t + 1
        rows += 1
    dt = time.perf_counter() - t0
    rate = pairs * len(heads) * FLOP_PER_TOKEN_HEAD / dt / 1e12
    full = T * (T + 1) // 2 * wl.H * FLOP_PER_TOKEN_HEAD / (rate * 1e12)
    return {"value": rate, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} query rows (row {T - 1}, row 0, then random; {pairs} causal pairs) x {len(heads)} of "
                      f"{wl.H} heads, fp64 NumPy, {dt:.1f} s",
            "extrapolated_full_step_s": full, "build": blas_info()}


def _timed_steps(run, n, group):
    """Run `run(i)` for i < n between events: the total and one time per call
    (each call runs `group` steps), in ms."""
    import torch

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(n):
        run(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) / group for i in range(n) for _ in range(group)]
    return evs[0].elapsed_time(evs[n]), per, wall


def _timed_batches(call, K, R):
    """The kernel alone: K back-to-back launches between two events on the
    stream it runs on, three times (sorted ms per launch); a GPU sleep first
    lets the host enqueue every launch ahead of the device, so no host
    latency lands inside the timed batch."""
    import torch

    out_ms = []
    for _rep in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(int(2.4e9 * (0.002 + 40e-6 * K)))
        except Exception:  # no device sleep available: host latency may inflate the kernel time
            pass
        e0.record()
        for k in range(K):
            call(k % R)
        e1.record()
        torch.cuda.synchronize()
        out_ms.append(e0.elapsed_time(e1) / K)
    out_ms.sort()
    return out_ms


def run_prefill(args, wl, dev, steps, warmup, cpu_seconds):
    """Causal prefill of one sequence: absorb_q + prefill_causal (cache append and
    causal attention) + upproj_v over all T rows; value = algorithmic TFLOP/s."""
    import numpy as np
    import torch

    import mla_latent_kv_30_amd as mla
    from mla_latent_kv_30_amd import workload as W

    T, H = int(wl.lens[0]), wl.H
    w_uk, w_uv = W.weights(wl)
    q_c, q_r = W.queries(wl)
    c, k = W.sequence_latents(wl, 0)
    host = {"q_c": q_c, "q_r": q_r, "w_uk": w_uk, "w_uv": w_uv, "c_kv": c, "k_r": k}
    td = lambda x: torch.from_numpy(x).to(dev, torch.bfloat16)
    w_uk, w_uv, q_c, q_r, c, k = (td(x) for x in (w_uk, w_uv, q_c, q_r, c, k))
    npg = (T + 63) // 64
    cache = mla.PagedCache(npg, torch.bfloat16, dev)
    perm = np.random.default_rng(args.seed).permutation(npg).astype(np.int32)
    bt = torch.from_numpy(perm).to(dev)
    pos = torch.arange(T, dtype=torch.int32, device=dev)
    q_abs = torch.empty((T, H, 576), dtype=torch.bfloat16, device=dev)
    z = torch.empty((T, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    o = torch.empty((T, H, 128), dtype=torch.float32, device=dev)

    LAYER = args.layer
    if LAYER:
        D = args.d_model
        lw = {kk: td(v) for kk, v in W.projection_weights(wl, d=D).items()}
        h = td(W.hidden_states(wl, 0, D))
        dcq = lw["w_dq"].shape[0]
        ws_q = torch.empty(max(1, mla.q_project_workspace_size(T, D, dcq, H)), dtype=torch.uint8, device=dev)
        ws_kv = torch.empty(max(1, mla.linear_workspace_size(T, 576, D)), dtype=torch.uint8, device=dev)
        ws_o = torch.empty(max(1, mla.linear_workspace_size(T, D, H * 128)), dtype=torch.uint8, device=dev)
        o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
        u = torch.empty((T, D), dtype=torch.float32, device=dev)

    def q_proj():
        mla.q_project(h, lw["w_dq"], lw["w_uq"], lw["w_qr"], H, workspace=ws_q, q_c=q_c, q_r=q_r)

    def kv_proj():
        c2, k2 = mla.linear(h, lw["w_dkv"], lw["w_kr"], workspace=ws_kv)
        c.copy_(c2)
        k.copy_(k2)

    def out_proj():
        mla.output_proj(o.view(T, H * 128), lw["w_o"], workspace=ws_o, out=u)

    def step(_i=0):
        if LAYER:
            q_proj()
            kv_proj()
        mla.absorb_q(q_c, q_r, pos, w_uk, out=q_abs)
        mla.prefill_causal(q_abs, c, k, cache, bt, z=z, lse=lse)
        mla.upproj_v(z, w_uv, out=o, out_dtype=o.dtype)
        if LAYER:
            out_proj()

    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    K = steps
    total_ms, per_step, wall = _timed_steps(step, K, 1)
    ms_per_step = total_ms / K
    kern_ms = _timed_batches(lambda _r: mla.prefill_causal(q_abs, c, k, cache, bt, z=z, lse=lse), K, 1)
    kern_avg_ms = kern_ms[1]
    pairs = T * (T + 1) // 2
    attn_flops = pairs * H * FLOP_PER_TOKEN_HEAD
    proj_flops = 2 * T * H * 2 * 128 * 512
    tflops_kernel = attn_flops / (kern_avg_ms * 1e-3) / 1e12
    # the step's other parts alone
    parts = {}
    for name, call in (("absorb_q", lambda _r: mla.absorb_q(q_c, q_r, pos, w_uk, out=q_abs)),
                       ("upproj_v", lambda _r: mla.upproj_v(z, w_uv, out=o, out_dtype=o.dtype))):
        parts[name] = {"us": _timed_batches(call, K, 1)[1] * 1e3}
    layer = None
    if LAYER:
        flops = {"q_project": 2 * T * (D * dcq + dcq * H * 192), "kv_projection": 2 * T * D * 576,
                 "output_proj": 2 * T * H * 128 * D}
        layer = {"d_model": D, "d_cq": dcq}
        for name, call in (("q_project", q_proj), ("kv_projection", kv_proj), ("output_proj", out_proj)):
            ms = _timed_batches(lambda _r: call(), K, 1)[1]
            tf = flops[name] / (ms * 1e-3) / 1e12
            layer[name] = {"us": ms * 1e3, "alg_flops": flops[name], "TFLOP/s": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS}
        proj_flops += sum(flops.values())
    from mla_latent_kv_30_amd import traffic as TR
    mc = TR.load(decode_kernel_name(wl.dtype, H), wl.name, os.path.join(ROOT, "profiles"), "mfma")
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(wl, host, cpu_seconds, args.seed)
    return {
        "metric": "MLA causal prefill TFLOP/s (absorbed attention + absorb + up-projection)",
        "value": (attn_flops + proj_flops) / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": warmup, "ms_per_step": ms_per_step,
        "step_ms": step_stats(per_step),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + (f"+layer(d={D})" if LAYER else ""), "tokens": T, "heads": H,
                   "causal_pairs": pairs,
                   "step": ("q_project + kv projection + " if LAYER else "") +
                           "absorb_q + prefill_causal (cache append + causal attention) + upproj_v" +
                           (" + output_proj" if LAYER else "")},
        "layer": layer, "parts": parts,
        "roofline": {
            "bound": "mfma", "achieved": tflops_kernel, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops_kernel / PEAK_BF16_TFLOPS, "traffic": None, "kernel": "prefill attention (mla_prefill_causal)",
            "kernel_avg_us": kern_avg_ms * 1e3, "kernel_batches_us": [x * 1e3 for x in kern_ms],
            "alg_flops_per_launch": attn_flops,
            "mfma_counters": None if mc is None else {
                "issued_tflops": mc["issued_tflops"], "busy_frac": mc["busy_frac"],
                "issued_over_algorithmic": mc["mfma_flops_issued"] / attn_flops},
        },
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }


def run_decode(args, wl, dev, steps, warmup, cpu_seconds):
    import numpy as np
    import torch

    import mla_latent_kv_30_amd as mla
    from mla_latent_kv_30_amd import device_inputs as DI
    from mla_latent_kv_30_amd import workload as W

    splits = wl.splits if args.splits < 0 else args.splits
    t_setup = time.perf_counter()
    dd = DI.decode_inputs(wl, dev, keep_host=not args.no_cpu_baseline)
    torch.cuda.synchronize()
    B, H, total = wl.B, wl.H, wl.total_tokens
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    # ---- replicas of everything a step reads
    per_rep = dd.cache.nbytes() + sum(t.numel() * t.element_size() for t in (dd.q_c, dd.q_r, dd.w_uk, dd.w_uv))
    QL = max(1, args.q_len)
    if QL * H > 128:
        sys.exit(f"--q-len {QL} with {H} heads: multi-token decode takes q_len * H <= 128")
    LAYER = args.layer
    lw0 = None
    if LAYER:
        if QL > 1 or wl.dtype == "f32":
            sys.exit("--layer: one-token decode over a bf16 or fp8 cache only")
        D = args.d_model
        lw0 = {k: torch.from_numpy(v).to(dev, torch.bfloat16) for k, v in W.projection_weights(wl, d=D).items()}
        lw0["h"] = torch.from_numpy(W.new_token_hidden(wl, D)).to(dev, torch.bfloat16)
        per_rep += sum(t.numel() * t.element_size() for t in lw0.values())
        last = (wl.lens - 1).astype(np.int64)
        slot_new = torch.from_numpy((dd.layout.block_table[np.arange(B), last // 64].astype(np.int64) * 64
                                     + last % 64).astype(np.int32)).to(dev)
        dcq = lw0["w_dq"].shape[0]
        ws_qkv = torch.empty(max(1, mla.qkv_project_workspace_size(B, D, dcq, H, dd.cache.code)), dtype=torch.uint8,
                             device=dev)
        ws_q = torch.empty(max(1, mla.q_project_workspace_size(B, D, dcq, H)), dtype=torch.uint8, device=dev)
        ws_kv = torch.empty(max(1, mla.kv_append_workspace_size(B, D, dd.cache.code)), dtype=torch.uint8,
                            device=dev)
        ws_o = torch.empty(max(1, mla.linear_workspace_size(B, D, H * 128)), dtype=torch.uint8, device=dev)
        u = torch.empty((B, D), dtype=torch.float32, device=dev)
    R = args.replicas or max(1, min(16, math.ceil(REPLICA_TARGET_BYTES / per_rep)))
    if QL > 1:  # q_len new tokens per sequence at positions L - q_len + t
        q_c0, q_r0, pos_q, _, _ = DI.multi_query_inputs(dd, QL)
    else:
        q_c0, q_r0, pos_q = dd.q_c, dd.q_r, dd.pos
    reps = [(dd.cache, q_c0, q_r0, dd.w_uk, dd.w_uv, lw0)]
    for _ in range(R - 1):
        c = mla.PagedCache.__new__(mla.PagedCache)
        c.__dict__.update(dd.cache.__dict__)
        for name in ("rows", "ckv", "scale", "kr"):
            t = getattr(dd.cache, name)
            setattr(c, name, None if t is None else t.clone())
        lw = None if lw0 is None else {k: v.clone() for k, v in lw0.items()}
        reps.append((c, q_c0.clone(), q_r0.clone(), dd.w_uk.clone(), dd.w_uv.clone(), lw))
    q_abs = torch.empty((B * QL, H, 576), dtype=dt, device=dev)
    z = torch.empty((B * QL, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B * QL, H), dtype=torch.float32, device=dev)
    o = torch.empty((B * QL, H, 128), dtype=torch.bfloat16 if LAYER else torch.float32, device=dev)
    ws = mla.decode_workspace(B, QL * H, splits, dev)
    # one token per sequence: decode, merge and W_UV in one call, a single
    # launch where the library can (the decode kernel runs the merge jobs)
    ws_up = mla.decode_upproj_workspace(B, H, splits, dev) if QL == 1 else None
    one_launch = QL == 1 and mla.decode_upproj_launches(B, H, splits, dd.cache.code) == 1
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def q_proj(r):
        _, q_c, q_r, _, _, lw = reps[r]
        mla.q_project(lw["h"], lw["w_dq"], lw["w_uq"], lw["w_qr"], H, workspace=ws_q, q_c=q_c, q_r=q_r)

    def kv_app(r):
        cache, *_, lw = reps[r]
        mla.kv_append(cache, lw["h"], lw["w_dkv"], lw["w_kr"], pos_q, slot_new, workspace=ws_kv)

    def qkv_proj(r):
        cache, q_c, q_r, *_, lw = reps[r]
        mla.qkv_project(cache, lw["h"], lw["w_dq"], lw["w_dkv"], lw["w_kr"], lw["w_uq"], lw["w_qr"], pos_q, slot_new,
                        H, workspace=ws_qkv, q_c=q_c, q_r=q_r)

    def out_proj(r):
        lw = reps[r][-1]
        mla.output_proj(o, lw["w_o"], workspace=ws_o, out=u)

    def step(r):
        cache, q_c, q_r, w_uk, w_uv, lw = reps[r]
        if LAYER:
            qkv_proj(r)
        mla.absorb_q(q_c, q_r, pos_q, w_uk, out=q_abs)
        if QL > 1:
            mla.decode_multi_upproj(q_abs.view(B, QL, H, 576), cache, dd.block_table, dd.seq_lens, w_uv,
                                    num_splits=splits, workspace=ws, z=z.view(B, QL, H, 512),
                                    lse=lse.view(B, QL, H), out=o.view(B, QL, H, 128))
        else:
            mla.decode_upproj(q_abs, cache, dd.block_table, dd.seq_lens, w_uv, num_splits=splits, workspace=ws_up,
                              z=z, lse=lse, out=o, out_dtype=o.dtype)
        if LAYER:
            out_proj(r)

    for k in range(max(1, warmup)):
        step(k % R)
    torch.cuda.synchronize()

    # Graphs of G consecutive steps, as the layers of a model share one graph
    # per decode step.  G divides K, so the timed loop replays whole graphs;
    # graph j runs steps jG .. jG+G-1 (modulo R) and the graphs rotate, so
    # step k always reads replica k % R, as with a graph per step.
    K = steps
    graphs = None
    G = 1
    multis = []
    if not args.no_graph:
        try:
            graphs = []
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for r in range(R):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side):
                        step(r)
                    graphs.append(g)
            want = args.graph_steps if args.graph_steps > 0 else 10
            G = max(d for d in range(1, want + 1) if K % d == 0)
            if G > 1:
                with torch.cuda.stream(side):
                    for j in range(R // math.gcd(G, R)):
                        g = torch.cuda.CUDAGraph()
                        with torch.cuda.graph(g, stream=side):
                            for i in range(G):
                                step((j * G + i) % R)
                        multis.append(g)
            torch.cuda.current_stream().wait_stream(side)
            for g in multis:
                g.replay()
            for k in range(max(1, warmup)):
                graphs[k % R].replay()
            torch.cuda.synchronize()
        except Exception as e:  # capture not available: fall back to eager launches
            print(f"note: graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graphs = None
            G = 1

    # ---- timed region: exactly `steps` steps between two synchronisations,
    # an event after every graph (G steps) for the per-step distribution
    if graphs is not None and G > 1:
        total_ms, per_step, wall = _timed_steps(lambda t: multis[t % len(multis)].replay(), K // G, G)
    elif graphs is not None:
        total_ms, per_step, wall = _timed_steps(lambda k: graphs[k % R].replay(), K, 1)
    else:
        total_ms, per_step, wall = _timed_steps(lambda k: step(k % R), K, 1)
    ms_per_step = total_ms / K

    # ---- the decode kernel alone (mla_decode_partial; in the one-launch form
    # the kernel also merges and up-projects, so it is timed as that call)
    def decode_only(r):
        cache = reps[r][0]
        if QL > 1:  # the multi-token entry point is decode + merge
            mla.decode_multi(q_abs.view(B, QL, H, 576), cache, dd.block_table, dd.seq_lens, num_splits=splits,
                             workspace=ws, z=z.view(B, QL, H, 512), lse=lse.view(B, QL, H))
        elif one_launch:
            mla.decode_upproj(q_abs, cache, dd.block_table, dd.seq_lens, reps[r][4], num_splits=splits,
                              workspace=ws_up, z=z, lse=lse, out=o, out_dtype=o.dtype)
        else:
            mla.decode_partial(q_abs, cache, dd.block_table, dd.seq_lens, ws, z, lse, num_splits=splits)

    kern_ms = _timed_batches(decode_only, K, R)
    kern_avg_ms = kern_ms[1]  # median of the three batches
    # in the one-launch form, the same kernel without the merge jobs as well
    # (mla_decode_partial: decode and piece stores only)
    alone_ms = None
    if one_launch:
        alone_ms = _timed_batches(lambda r: mla.decode_partial(q_abs, reps[r][0], dd.block_table, dd.seq_lens, ws, z,
                                                               lse, num_splits=splits), K, R)[1]
    parts = None
    if QL == 1 and not LAYER:
        parts = {
            "absorb_q": {"us": _timed_batches(lambda r: mla.absorb_q(reps[r][1], reps[r][2], pos_q, reps[r][3],
                                                                     out=q_abs), K, R)[1] * 1e3},
        }
        if one_launch:
            parts["decode_upproj (one launch)"] = {"us": kern_avg_ms * 1e3}
        else:
            # mla_decode_upproj's second launch, after decode_partial
            parts["decode_merge_upproj"] = {"us": _timed_batches(
                lambda r: mla.decode_merge_upproj(dd.seq_lens, H, ws_up, z, reps[r][4], lse=lse, num_splits=splits,
                                                  out=o, out_dtype=o.dtype), K, R)[1] * 1e3}

    layer = None
    if LAYER:
        # each projection alone, against the bytes it must move (weights,
        # activations in and out, intermediates written and read once)
        tok_b = {"bf16": 1152, "fp8": 656}[wl.dtype]
        nbytes = {
            "qkv_project": 2 * ((dcq + 576) * D + H * 192 * dcq + B * D + 2 * B * dcq + B * H * 192) + B * tok_b,
            "q_project": 2 * (dcq * D + H * 192 * dcq + B * D + 2 * B * dcq + B * H * 192),
            "kv_append": 2 * (576 * D + B * D + 2 * B * 576) + B * tok_b,
            "output_proj": 2 * (D * H * 128 + B * H * 128) + 4 * B * D,
        }
        layer = {"d_model": D, "d_cq": dcq}
        for name, call in (("qkv_project", qkv_proj), ("q_project", q_proj), ("kv_append", kv_app),
                           ("output_proj", out_proj)):
            ms = _timed_batches(call, K, R)[1]
            gbs_p = nbytes[name] / (ms * 1e-3) / 1e9
            layer[name] = {"us": ms * 1e3, "alg_bytes": nbytes[name], "GB/s": gbs_p, "hbm_frac": gbs_p / PEAK_HBM_GBS}

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # ---- roofline of the decode kernel (algorithmic bytes / FLOPs per launch)
    tok_bytes = {"f32": 2304, "bf16": 1152, "fp8": 656}[wl.dtype]
    q_bytes = B * QL * H * 576 * (4 if wl.dtype == "f32" else 2)
    out_bytes = B * QL * H * (512 + 1) * 4
    alg_bytes = total * tok_bytes + q_bytes + out_bytes
    decode_alg_bytes = alg_bytes
    # query token t of a sequence of L cached tokens sees L - q_len + t + 1 of them
    seen = int(sum(QL * int(L) - QL * (QL - 1) // 2 for L in wl.lens))
    alg_flops = seen * H * FLOP_PER_TOKEN_HEAD
    if one_launch:  # W_UV read once and o written, o = W_UV z per (sequence, head)
        alg_bytes += H * 128 * 512 * 2 + B * H * 128 * o.element_size()
        alg_flops += B * H * 128 * 512 * 2
    gbs = alg_bytes / (kern_avg_ms * 1e-3) / 1e9
    tflops = alg_flops / (kern_avg_ms * 1e-3) / 1e12
    mfma_peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
    # the bound at MI355X's ridge (matrix-core peak / HBM peak, FLOP per byte)
    mfma_bound = alg_flops / alg_bytes > mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9)

    cpu = None
    if not args.no_cpu_baseline and QL == 1:
        cpu = cpu_baseline(wl, dd.host, cpu_seconds)

    # HBM bytes per launch from the stored counter runs, if they were taken on
    # the current kernel sources
    from mla_latent_kv_30_amd import traffic as TR
    kname = decode_kernel_name(wl.dtype, wl.H * QL)
    tr = TR.load(kname, wl.name, os.path.join(ROOT, "profiles")) if QL == 1 else None
    mc = TR.load(kname, wl.name, os.path.join(ROOT, "profiles"), "mfma") if QL == 1 else None
    if QL > 1:
        kname += " + merge_kernel"
    elif one_launch:
        kname += " (decode + split merge + W_UV up-projection in one launch)"

    roof = {
        "bound": "mfma" if mfma_bound else "hbm",
        "achieved": tflops if mfma_bound else gbs,
        "peak": mfma_peak if mfma_bound else PEAK_HBM_GBS,
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "frac": tflops / mfma_peak if mfma_bound else gbs / PEAK_HBM_GBS,
        "traffic": None if tr is None else tr["traffic_bytes"], "kernel": kname,
        "traffic_fetch_bytes": None if tr is None else tr["fetch_bytes"],
        "traffic_write_bytes": None if tr is None else tr["write_bytes"],
        "kernel_avg_us": kern_avg_ms * 1e3, "kernel_batches_us": [x * 1e3 for x in kern_ms],
        "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops,
        "hbm_GBps": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
        "tflops": tflops, "mfma_peak_tflops": mfma_peak, "mfma_frac": tflops / mfma_peak,
        "decode_without_merge": None if alone_ms is None else {
            "us": alone_ms * 1e3, "alg_bytes": decode_alg_bytes,
            "hbm_frac": decode_alg_bytes / (alone_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        # matrix-core counters of the same kernel (stored run on the current sources)
        "mfma_counters": None if mc is None else {
            "issued_tflops": mc["issued_tflops"], "busy_frac": mc["busy_frac"],
            "issued_over_algorithmic": mc["mfma_flops_issued"] / alg_flops},
    }
    del reps, dd
    return {
        "metric": METRIC,
        "value": total / (ms_per_step * 1e-3),
        "unit": "cached-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "step_ms": step_stats(per_step),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name + (f"+layer(d={D})" if LAYER else ""), "batch": B, "heads": H, "cached_tokens": total,
            "seq_len_min": int(wl.lens.min()), "seq_len_max": int(wl.lens.max()), "page_size": 64,
            "num_splits": splits if splits > 0 else "auto", "replicas": R, "graph": graphs is not None,
            "graph_steps": G if graphs is not None else 0,
            "step": ("qkv_project (cache append + query path) + absorb_q + decode_upproj + output_proj"
                     if LAYER else
                     ("absorb_q + decode_upproj (decode, split merge and W_UV up-projection in one launch)"
                      if one_launch else
                      "absorb_q + decode_upproj (decode_partial, then split merge + W_UV up-projection)") if QL == 1
                     else "absorb_q + decode_multi_upproj (decode, then split merge + W_UV up-projection)"),
            "q_len": QL, "query_tokens_per_s": B * QL / (ms_per_step * 1e-3),
        },
        "layer": layer, "parts": parts,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
        "setup_s": setup_s,
    }


def against_ceilings(rec, ceil):
    """Fractions of the measured ceilings beside those of the published peaks."""
    if not ceil or not rec or "roofline" not in rec:
        return
    rf = rec["roofline"]
    m16 = ceil.get("mfma_bf16_16x16x32_TFLOPs")
    if rf.get("hbm_GBps") is not None and ceil.get("hbm_read_GBps"):
        rf["hbm_frac_of_measured"] = rf["hbm_GBps"] / ceil["hbm_read_GBps"]
    tf = rf.get("tflops", rf["achieved"] if rf["unit"] == "TFLOP/s" else None)
    if tf is not None and m16 and rec.get("dtype") != "f32":
        rf["mfma_frac_of_measured"] = tf / m16


def run(args, name, dev, steps, warmup, cpu_seconds):
    from mla_latent_kv_30_amd import workload as W

    wl = W.make_workload(name, seed=args.seed)
    if wl.kind == "prefill":
        return run_prefill(args, wl, dev, steps, warmup, cpu_seconds)
    return run_decode(args, wl, dev, steps, warmup, cpu_seconds)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit(f"bench.py measures the decode path on one GPU only; --gpus {args.gpus} (WORLD_SIZE {world}) "
                 f"is not supported: sharding across GPUs is not part of this library.")

    import torch

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    out = run(args, args.config, dev, args.steps, args.warmup, args.cpu_seconds)
    torch.cuda.empty_cache()
    ceil = None
    if not args.no_ceilings:
        ceil = measure_ceilings(dev)
        against_ceilings(out, ceil)
    out["ceilings"] = ceil
    if (args.config == HEADLINE and not args.no_extra and not args.layer and args.q_len == 1
            and args.splits < 0):
        subs = {}
        for name in SUB_WORKLOADS:
            print(f"sub-record {name}", file=sys.stderr, flush=True)
            try:
                rec = run(args, name, dev, args.sub_steps, min(args.warmup, 3), args.sub_cpu_seconds)
                against_ceilings(rec, ceil)
            except Exception as e:  # a sub-record must not cost the headline line
                rec = {"error": f"{type(e).__name__}: {e}"}
            subs[name] = rec
            torch.cuda.empty_cache()
        out["workloads"] = subs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
