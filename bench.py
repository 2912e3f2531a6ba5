#!/usr/bin/env python
"""Benchmark of the absorbed MLA decode step on one MI355X.

One step = the whole path over one batch: absorb (q~ = W_UK^T q_nope) ->
latent attention over the paged cache (split-KV partials) -> log-sum-exp merge
and un-absorb (W_UV latent), in one kernel for bf16 partials and at most four
splits per sequence, else as two.  Workload: DeepSeek-V3 geometry, B=64 sequences of
L=4096 cached tokens, T=1, H=128, page size 64 with a seeded random page
permutation, synthetic N(0,1) bf16 inputs and N(0,1/512) weights.

Timing: untimed warm-up (at least W steps and 0.1 s of back-to-back work, so
that the clocks, which ramp up over the first ~20 ms after the set-up's idle
time, have settled), then K steps between two device synchronisations.
Three replicas of the cache and of the weights rotate from step to step so that
the 256 MB last-level cache cannot serve a step's reads from the previous one.
The decode kernel's own duration, from which the roofline fraction is computed,
is one pair of HIP events on its launch stream around K back-to-back decode
launches (replicas rotating), divided by K; event pairs around each launch of
K eager steps are reported beside it (they also span the packet processing
around the kernel).  The chain throughput (`value`) is the faster of two ways
of launching the same K steps: eager launches on one stream, and replays of the
step captured as a HIP graph (one graph per replica; `--no-graph` leaves the
graph out); `chain_launch` names the one taken and both times are reported.
The other workloads, the fp32-partials headline, the
FP8-row, sparse and sparse-FP8 kernels are timed the same way and reported
under ``detail``; so are a sustained clock/power sample of the headline decode
kernel and the practical-roof probes (``--roof-seconds``).

Prints one JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
ROW_BYTES = 1152                 # [c (512) || k_pe (64)] bf16
HEADLINE = "v3_b64_l4096"


def decode_algorithmic(case):
    """Algorithmic bytes and FLOPs of one decode launch: every visible cache row
    once (1152 B), the query (q~ 512 + q_pe 64, bf16), block table entries used,
    lengths, the bf16 latent output and the fp32 lse; FLOPs 2*H*(576+512) per
    visible (query, key) pair."""
    import numpy as np
    B, T, H, P = case.B, case.T, case.H, case.page_size
    L = case.seqlens.astype(np.int64)
    pairs = int(np.sum([T * (l - T) + T * (T + 1) // 2 for l in L]))   # visible (t, j) per sequence
    rows = int(L.sum())
    q_bytes = B * T * H * (512 + 64) * 2
    table_bytes = int(np.sum((L + P - 1) // P)) * 4
    out_bytes = B * T * H * 512 * 2 + B * T * H * 4
    nbytes = rows * ROW_BYTES + q_bytes + table_bytes + B * 4 + out_bytes
    flops = 2 * H * pairs * (576 + 512)
    return nbytes, flops


def chain_algorithmic(case, decode_bytes):
    B, T, H = case.B, case.T, case.H
    absorb = B * T * H * 128 * 2 + H * 128 * 512 * 2 + B * T * H * 512 * 2
    unabsorb = B * T * H * 512 * 2 + H * 128 * 512 * 2 + B * T * H * 128 * 4
    return decode_bytes + absorb + unabsorb


WARM_SECONDS = 0.1


def warm_up(fn, n_min, seconds=WARM_SECONDS):
    """Untimed warm-up: fn(i) for i = 0, 1, ... until at least n_min calls and
    `seconds` of back-to-back work have passed.  After the host-side set-up the
    GPU sits idle and its clocks ramp up again over the first ~20 ms of work (the
    first 50 steps of the headline chain take 1.7x the steady-state time), so a
    fixed small count would time part of the ramp."""
    import torch
    i = 0
    t0 = time.perf_counter()
    while i < n_min or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def sparse_algorithmic(sc, row_bytes=ROW_BYTES):
    """Algorithmic bytes and FLOPs of one sparse decode launch, counted as for the
    dense kernel: every valid selected row once with its index entry, the
    query, the bf16 latent output and the lse.  Split partials are overhead of
    the kernel, not useful traffic, so they are not counted."""
    import numpy as np
    B, T, H = sc.B, sc.T, sc.H
    n = sc.topk if sc.topk_length is None else np.minimum(sc.topk_length, sc.topk).astype(np.int64)
    keys = int(np.sum(n)) * T if sc.topk_length is not None else B * T * sc.topk
    q_bytes = B * T * H * (512 + 64) * 2
    out_bytes = B * T * H * (512 * 2 + 4)
    nbytes = keys * (row_bytes + 4) + q_bytes + out_bytes
    flops = 2 * H * keys * (576 + 512)
    return nbytes, flops


def bench_sparse(name, K, W, R, dev, fp8=False):
    """Time the sparse (top-k) decode kernel on its workload: HIP events around
    each launch on its stream, cache replicas rotating.  ``fp8``: the same
    selections over a pool of 656-byte FP8 rows (fields prefixed sparse_fp8_)."""
    import numpy as np
    import torch
    import mla_latent_kv_amd as mk
    import synth
    if fp8:
        f = synth.make_sparse_fp8(synth.SPARSE_WORKLOADS[name], synth.SPARSE_TOPK[name], poison=False)
        sc = f.sparse
    else:
        sc = synth.make_sparse(synth.SPARSE_WORKLOADS[name], synth.SPARSE_TOPK[name], poison=False)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    kv0 = torch.from_numpy(f.kv_fp8).to(dev) if fp8 else bf16(sc.kv_cache)
    decode = mk.mla_decode_sparse_fp8 if fp8 else mk.mla_decode_sparse
    kv = [kv0] + [kv0.clone() for _ in range(R - 1)]
    q_lat, q_pe = bf16(sc.q_lat), bf16(sc.q_pe)
    idx = torch.from_numpy(sc.indices).to(dev)
    tl = torch.from_numpy(sc.topk_length).to(dev)
    buf = mk.SparseBuffers(sc.B, sc.T, sc.H, sc.topk, 0, dev, part_dtype=torch.bfloat16)
    S = buf.num_splits
    lat = torch.empty((sc.B, sc.T, sc.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((sc.B, sc.T, sc.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    scale = mk.softmax_scale()
    BT = sc.B * sc.T

    def run(r, ev=None):
        if ev is not None:
            ev[0].record(stream)
        decode(q_lat, q_pe, kv[r], idx, tl, scale, buffers=buf, merge=False)
        if ev is not None:
            ev[1].record(stream)
        if S > 1:
            mk.mla_merge_splits(buf.part_out.view(BT * S, 1, sc.H, 512), buf.part_lse.view(BT * S, 1, sc.H),
                                buf.split_indptr, BT, out_latent=lat.view(BT, 1, sc.H, 512),
                                lse=lse.view(BT, 1, sc.H))

    warm_up(lambda i: run(i % R), W)
    t0 = time.perf_counter()      # decode + merge, launched eagerly
    for i in range(K):
        run(i % R)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        run(i % R, evs[i])
    torch.cuda.synchronize()
    us_pairs = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    # the kernel's duration: K launches back to back between one event pair
    eb = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    eb[0].record(stream)
    for i in range(K):
        decode(q_lat, q_pe, kv[i % R], idx, tl, scale, buffers=buf, merge=False)
    eb[1].record(stream)
    torch.cuda.synchronize()
    us = eb[0].elapsed_time(eb[1]) * 1e3 / K
    nbytes, flops = sparse_algorithmic(sc, 656 if fp8 else ROW_BYTES)
    del kv, kv0
    torch.cuda.empty_cache()
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "decode_sparse_fp8_hbm_traffic.json" if fp8 else
                         "decode_sparse_hbm_traffic.json")
    if os.path.exists(tpath):
        try:
            from mla_latent_kv_amd import _build
            rec = json.load(open(tpath))
            if rec.get("source_sha256") == _build.kernel_source_hash() and rec.get("workload") == name \
                    and int(rec.get("splits", -1)) == S:
                traffic = rec["bytes_per_launch"]
        except Exception:
            traffic = None
    pre = "sparse_fp8_" if fp8 else "sparse_"
    return {
        pre + "workload": name, pre + "topk": sc.topk, pre + "context": int(sc.seqlens.max()),
        pre + "splits": S,
        pre + "decode_us": us,
        pre + "decode_us_event_pairs_mean": us_pairs,
        pre + "step_us": (t1 - t0) * 1e6 / K,
        pre + "alg_bytes": nbytes,
        pre + "GBps": nbytes / (us * 1e-6) / 1e9,
        pre + "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        pre + "tflops": flops / (us * 1e-6) / 1e12,
        pre + "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        pre + "traffic": traffic,
    }


def bench_fp8(name, S, K, W, R, dev):
    """Time the decode kernel over FP8 rows on its workload (S uniform splits,
    bf16 partials, as the bf16 headline): HIP events around each launch on its
    stream, cache replicas rotating."""
    import numpy as np
    import torch
    import mla_latent_kv_amd as mk
    import synth
    f = synth.make_fp8_case(synth.FP8_WORKLOADS[name], poison=False)
    case = f.case

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    kv0 = torch.from_numpy(f.kv_fp8).to(dev)
    kv = [kv0] + [kv0.clone() for _ in range(R - 1)]
    q_lat = bf16(synth.normal_bf16(case.q_nope.shape[:3] + (512,), 9300, std=0.5))
    q_pe = bf16(case.q_pe)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seqlens).to(dev)
    buf = mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, S, dev,
                           part_dtype=torch.bfloat16)
    stream = torch.cuda.current_stream()
    scale = mk.softmax_scale()

    def run(r, ev=None):
        if ev is not None:
            ev[0].record(stream)
        mk.mla_decode_latent_fp8(q_lat, q_pe, kv[r], bt, sl, case.max_seqlen, scale, num_splits=S,
                                 buffers=buf, merge=False)
        if ev is not None:
            ev[1].record(stream)
        mk.mla_merge_splits(buf.part_out, buf.part_lse, buf.split_indptr, case.B)

    warm_up(lambda i: run(i % R), W)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        run(i % R, evs[i])
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    eb = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    eb[0].record(stream)
    for i in range(K):
        mk.mla_decode_latent_fp8(q_lat, q_pe, kv[i % R], bt, sl, case.max_seqlen, scale, num_splits=S,
                                 buffers=buf, merge=False)
    eb[1].record(stream)
    torch.cuda.synchronize()
    us = eb[0].elapsed_time(eb[1]) * 1e3 / K   # back to back, as the dense kernel
    bf16_bytes, flops = decode_algorithmic(case)
    rows = int(np.sum(case.seqlens))
    nbytes = bf16_bytes - rows * ROW_BYTES + rows * synth.FP8_ROW_BYTES
    del kv, kv0
    torch.cuda.empty_cache()
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "decode_fp8_hbm_traffic.json")
    if os.path.exists(tpath):
        try:
            from mla_latent_kv_amd import _build
            rec = json.load(open(tpath))
            if rec.get("source_sha256") == _build.kernel_source_hash() and rec.get("workload") == name \
                    and int(rec.get("splits", -1)) == S:
                traffic = rec["bytes_per_launch"]
        except Exception:
            traffic = None
    return {
        "fp8_workload": name, "fp8_splits": S, "fp8_traffic": traffic,
        "fp8_decode_us": us,
        "fp8_decode_us_event_pairs_mean": float(np.mean(ms)) * 1e3,
        "fp8_alg_bytes": nbytes,
        "fp8_GBps": nbytes / (us * 1e-6) / 1e9,
        "fp8_hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "fp8_tflops": flops / (us * 1e-6) / 1e12,
        "fp8_mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "fp8_tokens_per_s": case.B * case.T / (us * 1e-6),
    }


def crossover(Ts, S_ctx, B, K, W, dev):
    """Time the absorbed chain (absorb, latent attention with automatic splits,
    merge, un-absorb) and the Normal path (gather, up-projection GEMMs, MHA
    attention; one chunk) on the same seeded inputs for query blocks of T
    tokens over S_ctx cached tokens (causal over the block).  Returns one
    record per T and the model's MAC counts ("MLA in full detail", cost
    analysis: Normal S*512*128*256 + 128*T*S*320, absorbed T*128*128*512*2 +
    128*T*S*1088 multiply-adds per layer)."""
    import numpy as np
    import torch
    import mla_latent_kv_amd as mk
    import synth
    scale = mk.softmax_scale()
    rows = []

    def upload(case, dev):
        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return dict(q_nope=bf16(case.q_nope), q_pe=bf16(case.q_pe), w_uk=bf16(case.w_uk), w_uv=bf16(case.w_uv),
                    kv_cache=bf16(case.kv_cache), block_table=torch.from_numpy(case.block_table).to(dev),
                    seqlens=torch.from_numpy(case.seqlens).to(dev))

    for T in Ts:
        wl = synth.Workload(f"xover_t{T}", B=B, T=T, H=128, L=S_ctx, page_size=64, seed=3000 + T)
        case = synth.make_case(wl, poison=False)
        d = upload(case, dev)
        ws = torch.empty(max(mk.mla_normal_workspace_size(B, T, 128, S_ctx, S_ctx), 16), dtype=torch.uint8,
                         device=dev)
        n_out = torch.empty((B, T, 128, 128), dtype=torch.float32, device=dev)
        n_lse = torch.empty((B, T, 128), dtype=torch.float32, device=dev)
        buf = mk.DecodeBuffers(B, T, 128, S_ctx, 64, 0, dev, part_dtype=torch.bfloat16)

        def absorbed():
            return mk.absorbed_decode(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                      d["block_table"], d["seqlens"], S_ctx, num_splits=0, buffers=buf)

        def normal():
            return mk.mla_decode_normal(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                        d["block_table"], d["seqlens"], S_ctx, scale, chunk=S_ctx, workspace=ws,
                                        out=n_out, lse=n_lse)

        res = {}
        for name, fn in (("absorbed", absorbed), ("normal", normal)):
            for _ in range(W):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(K):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / K
        a_out, _ = absorbed()
        n_o, _ = normal()
        torch.cuda.synchronize()
        diff = float((a_out - n_o).abs().max())
        ref = float(n_o.abs().max())
        macs_normal = S_ctx * 512 * 128 * 256 + 128 * T * S_ctx * 320
        macs_absorbed = T * 128 * 128 * 512 * 2 + 128 * T * S_ctx * 1088
        rows.append({"T": T, "S": S_ctx, "B": B, "H": 128, "absorbed_ms": res["absorbed"],
                     "normal_ms": res["normal"], "normal_over_absorbed": res["normal"] / res["absorbed"],
                     "model_macs_normal_per_seq": macs_normal, "model_macs_absorbed_per_seq": macs_absorbed,
                     "max_abs_diff": diff, "max_abs_out": ref})
        del d, ws, n_out, n_lse, buf
        torch.cuda.empty_cache()
    return rows


class MetricsSampler:
    """Samples the GPU's firmware metrics table (amdsmi gpu_metrics: gfx clock,
    socket power, energy counter, throttle flags) from a thread every `period`
    seconds.  Reading the table does not touch the HIP runtime."""

    def __init__(self, period=0.005):
        import threading
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        self.error = None

    def start(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # no permission or no library: report, do not fail the bench
            self.error = f"{type(e).__name__}: {e}"
            return self
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            t = time.perf_counter()
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            row = {"t": t}
            for k, v in m.items():
                if isinstance(v, (int, float)) and not isinstance(v, bool):
                    row[k] = v
                elif isinstance(v, list) and v and all(isinstance(x, (int, float)) for x in v):
                    vals = [x for x in v if x not in (65535, 0xFFFFFFFF, 0xFFFFFFFFFFFFFFFF)]
                    if vals:
                        row[k + "_mean"] = sum(vals) / len(vals)
            self.samples.append(row)
            self._stop.wait(self.period)

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        try:
            self._smi.amdsmi_shut_down()
        except Exception:
            pass

    def summary(self, t0, t1, keys):
        import numpy as np
        rows = [r for r in self.samples if t0 <= r["t"] <= t1]
        out = {"samples": len(rows), "error": self.error}
        for k in keys:
            vals = [r[k] for r in rows if k in r]
            if vals:
                out[k] = {"median": float(np.median(vals)), "min": float(np.min(vals)),
                          "max": float(np.max(vals))}
        e = [(r["t"], r["energy_accumulator"]) for r in rows if "energy_accumulator" in r]
        if len(e) >= 2 and e[-1][0] > e[0][0]:
            # the accumulator counts in units of 15.259 uJ (firmware convention of this metrics table)
            out["energy_accumulator_W"] = (e[-1][1] - e[0][1]) * 15.259e-6 / (e[-1][0] - e[0][0])
        return out


def clock_sample(seconds, kind, dev):
    """Run one decode kernel of the headline geometry back to back for `seconds`
    (three cache replicas rotating, 4 uniform splits, bf16 partials) while the
    firmware metrics table is sampled; report the kernel's mean duration (HIP
    events on its stream), the gfx clock and power during the loop, and the
    cycles per 32-token step that the two imply."""
    import numpy as np
    import torch
    import mla_latent_kv_amd as mk
    import synth
    if kind == "fp8":
        f = synth.make_fp8_case(synth.FP8_WORKLOADS["v3_fp8_b64_l4096"], poison=False)
        case = f.case
        kv0 = torch.from_numpy(f.kv_fp8).to(dev)
        fn = mk.mla_decode_latent_fp8
    else:
        case = synth.make_case(synth.WORKLOADS[HEADLINE], poison=False)
        kv0 = torch.from_numpy(np.ascontiguousarray(case.kv_cache).view(np.int16)).view(torch.bfloat16).to(dev)
        fn = mk.mla_decode_latent
    kv = [kv0] + [kv0.clone() for _ in range(2)]
    q_lat = torch.from_numpy(synth.normal_bf16(case.q_nope.shape[:3] + (512,), 9300, std=0.5).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    q_pe = torch.from_numpy(np.ascontiguousarray(case.q_pe).view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seqlens).to(dev)
    S = 4
    buf = mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, S, dev,
                           part_dtype=torch.bfloat16)
    stream = torch.cuda.current_stream()
    scale = mk.softmax_scale()

    def launch(i):
        fn(q_lat, q_pe, kv[i % 3], bt, sl, case.max_seqlen, scale, num_splits=S, buffers=buf, merge=False)

    for i in range(20):
        launch(i)
    torch.cuda.synchronize()
    sampler = MetricsSampler().start()
    time.sleep(0.3)
    idle_t1 = time.perf_counter()
    batch = 64
    evs = []
    n = 0
    t0 = time.perf_counter()
    pending = []
    while time.perf_counter() - t0 < seconds:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            launch(n)
            n += 1
        e1.record(stream)
        evs.append((e0, e1))
        pending.append(e1)
        if len(pending) > 2:  # keep about two batches queued
            pending.pop(0).synchronize()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    time.sleep(0.2)
    sampler.stop()
    us = float(np.median([a.elapsed_time(b) for a, b in evs[1:]])) * 1e3 / batch
    keys = ["current_gfxclk", "average_gfxclk_frequency", "current_gfxclks_mean", "current_socket_power",
            "average_socket_power", "current_uclk", "average_uclk_frequency", "temperature_hotspot",
            "temperature_mem", "gfx_activity", "average_gfx_activity", "throttle_status",
            "indep_throttle_status"]
    busy = sampler.summary(t0 + 0.2, t1 - 0.05, keys)
    idle = sampler.summary(idle_t1 - 0.28, idle_t1, keys)
    steps_per_unit = (case.seqlens.max() // S + 31) // 32
    clk = None
    for k in ("current_gfxclks_mean", "current_gfxclk", "average_gfxclk_frequency"):
        if k in busy:
            clk = busy[k]["median"]
            break
    return {
        "clock_sample": kind, "workload": "v3_fp8_b64_l4096" if kind == "fp8" else HEADLINE,
        "splits": S, "launches": n, "seconds": t1 - t0,
        "kernel_us_median_of_batches": us,
        "steps_per_unit": int(steps_per_unit),
        "gfxclk_MHz_median": clk,
        "cycles_per_step_at_that_clock": (us * 1e-6 * clk * 1e6 / steps_per_unit) if clk else None,
        "busy": busy, "idle_before": idle,
        "sampler_error": sampler.error,
    }


def power_roof(seconds, dev):
    """Practical roofs under the power limit (context for the roofline line):
    the probe kernel of libmla_probe.so run back to back for `seconds` per
    mode -- MFMAs only, HBM stream only, both at the decode's FLOP/byte
    (one 1 KB load per 7 MFMAs of 32x32x16: 224 FLOP/B against the headline's
    228), and
    the same with one LDS operand read per MFMA -- each with the gfx clock and
    socket power it ran at."""
    import ctypes
    import numpy as np
    import torch
    from mla_latent_kv_amd import _build
    lib = ctypes.CDLL(_build.PROBE_LIB)
    lib.mla_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    grid, slice_ = 256, 4 << 20
    # random bf16 N(0,1) values: the LDS-fed modes then multiply changing data, as the decode does
    src = torch.randn(grid * slice_ // 2, dtype=torch.float32, device=dev).to(torch.bfloat16).view(torch.uint8)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    out = []
    for name, mode, ratio, iters in (("mfma_only_constant_operands", 0, 7, 16000),
                                     ("mfma_lds_fed_random_operands", 4, 7, 16000),
                                     ("hbm_stream_only", 1, 7, 6000),
                                     ("mfma_constant_operands_and_stream_224_flop_per_byte", 2, 7, 10000),
                                     ("mfma_lds_fed_random_operands_and_stream_224_flop_per_byte", 3, 7, 10000)):
        def launch():
            st = lib.mla_probe_launch(ctypes.c_void_p(src.data_ptr()), slice_, grid, iters, mode, ratio,
                                      ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"probe launch failed: hipError {st}")
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        sampler = MetricsSampler().start()
        time.sleep(0.2)
        evs = []
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(8):
                launch()
            e1.record(stream)
            evs.append((e0, e1))
            if len(evs) > 2:
                evs[-3][1].synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        sampler.stop()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs[1:]])) / 8
        waves = grid * 4
        flops = waves * 4 * iters * 32768 if mode != 1 else 0
        loads = iters if mode == 1 else (4 * iters) // ratio if mode in (2, 3) else 0
        nbytes = waves * loads * 1024
        summ = sampler.summary(t0 + 0.3, t1 - 0.05, ["current_gfxclks_mean", "current_socket_power"])
        clk = summ.get("current_gfxclks_mean", {}).get("median")
        out.append({"probe": name, "launch_ms": ms, "TFLOPs": flops / (ms * 1e-3) / 1e12,
                    "GBps": nbytes / (ms * 1e-3) / 1e9, "gfxclk_MHz": clk,
                    "socket_power_W": summ.get("current_socket_power", {}).get("median"),
                    "mfma_duty_at_that_clock": (flops / (ms * 1e-3)) / (256 * 4096 * clk * 1e6) if clk and flops
                    else None,
                    "sampler_error": sampler.error})
    del src
    torch.cuda.empty_cache()
    return out


def pipeline_roof(seconds, dev):
    """The decode kernel's data flow without its arithmetic, at the headline's
    shape (pipe_kernel of libmla_probe.so: 256 work units of 1024 tokens = 16
    randomly placed pages each, 36 KB tiles through a ring of four, a barrier
    per step), run back to back for `seconds` per variant with the gfx clock
    and socket power sampled: the stream alone, with the unit's 128 KB output
    block written at the end (plain and streaming stores), with the 68 MFMAs per
    wave and step fed from LDS, and with both; then the decode kernel itself
    (clock_sample).  Three page sets rotate, so the last-level cache cannot
    serve a launch from the previous one."""
    import ctypes
    import numpy as np
    import torch
    from mla_latent_kv_amd import _build
    lib = ctypes.CDLL(_build.PROBE_LIB)
    lib.mla_pipe_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]
    units, ppu, sets = 256, 16, 3
    page_bytes = 64 * 1152
    npages = sets * units * ppu
    pool = torch.randn(npages * page_bytes // 2, dtype=torch.float32, device=dev).to(torch.bfloat16)
    perm = np.random.default_rng(4242).permutation(npages).astype(np.int32).reshape(sets, units, ppu)
    assert 0 <= perm.min() and perm.max() < npages
    pages = [torch.from_numpy(perm[k].copy()).to(dev) for k in range(sets)]
    out = torch.empty(units * 131072, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    tile_bytes = units * 2 * ppu * 32 * 1152
    rows = []
    for name, flags in (("stream", 0), ("stream, output block written", 2),
                        ("stream, output block written with streaming stores", 6), ("stream and MFMAs", 1),
                        ("stream and MFMAs, output block written", 3),
                        ("stream and MFMAs, output block written with streaming stores", 7)):
        def launch(i):
            st = lib.mla_pipe_probe_launch(ctypes.c_void_p(pool.data_ptr()), npages,
                                           ctypes.c_void_p(pages[i % sets].data_ptr()), units, ppu, flags,
                                           ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                           ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"pipeline probe launch failed: hipError {st}")
        for i in range(6):
            launch(i)
        torch.cuda.synchronize()
        sampler = MetricsSampler().start()
        time.sleep(0.2)
        evs, n = [], 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(32):
                launch(n)
                n += 1
            e1.record(stream)
            evs.append((e0, e1))
            if len(evs) > 2:
                evs[-3][1].synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        sampler.stop()
        us = float(np.median([a.elapsed_time(b) for a, b in evs[1:]])) * 1e3 / 32
        summ = sampler.summary(t0 + 0.3, t1 - 0.05, ["current_gfxclks_mean", "current_socket_power", "current_uclk"])
        rows.append({"probe": name, "flags": flags, "launch_us": us, "tile_TBps": tile_bytes / (us * 1e-6) / 1e12,
                     "gfxclk_MHz": summ.get("current_gfxclks_mean", {}).get("median"),
                     "socket_power_W": summ.get("current_socket_power", {}).get("median"),
                     "uclk_MHz": summ.get("current_uclk", {}).get("median"),
                     "sampler_error": sampler.error})
    del pool, out
    torch.cuda.empty_cache()
    dec = clock_sample(seconds, "bf16", dev)
    dec["probe"] = "decode kernel (headline, 4 splits, bf16 partials)"
    rows.append(dec)
    return rows


def timeline(batches, dev):
    """Where a launch of the headline decode kernel goes, from inside it: the
    kernel of libmla_timeline.so (the same source built with
    MLA_DECODE_TIMELINE) stamps the 100 MHz real-time counter at eight points
    of every wave's work unit.  `batches` snapshots, each of the last of 300
    launches back to back (three cache replicas rotating, 4 uniform splits,
    bf16 partials).  The library must be the one loaded (main() loads it in
    place of libmla_latent.so for --timeline)."""
    import ctypes
    import numpy as np
    import torch
    import mla_latent_kv_amd as mk
    import synth
    lib = mk.load_library()
    lib.mla_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    case = synth.make_case(synth.WORKLOADS[HEADLINE], poison=False)
    kv0 = torch.from_numpy(np.ascontiguousarray(case.kv_cache).view(np.int16)).view(torch.bfloat16).to(dev)
    kv = [kv0] + [kv0.clone() for _ in range(2)]
    q_lat = torch.from_numpy(synth.normal_bf16(case.q_nope.shape[:3] + (512,), 9300, std=0.5).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    q_pe = torch.from_numpy(np.ascontiguousarray(case.q_pe).view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seqlens).to(dev)
    S, per_batch = 4, 300
    buf = mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, S, dev,
                           part_dtype=torch.bfloat16)
    scale = mk.softmax_scale()
    units = case.B * S   # one workgroup per unit (128 heads = one row group)
    host = np.zeros(units * 4 * 8, dtype=np.uint64)
    phases = ["set-up: length and block-table window read, query loads issued",
              "first tile loads issued, until the first tile has landed",
              "the 32 steps", "loop end to the final partial state", "normalisation and staging",
              "issuing the output stores", "the output stores' drain"]
    diffs, spans, skews, launch_us = [], [], [], []
    stream = torch.cuda.current_stream()
    for b in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(per_batch):
            mk.mla_decode_latent(q_lat, q_pe, kv[i % 3], bt, sl, case.max_seqlen, scale, num_splits=S, buffers=buf,
                                 merge=False)
        e1.record(stream)
        torch.cuda.synchronize()
        if lib.mla_timeline_read(host.ctypes.data, host.nbytes) != 0:
            raise RuntimeError("mla_timeline_read failed")
        if b == 0:
            continue   # the first batch follows the set-up's idle time (clock ramp)
        launch_us.append(e0.elapsed_time(e1) * 1e3 / per_batch)
        ts = host.reshape(units, 4, 8).astype(np.int64)
        rel = (ts - ts[:, :, 0].min()) / 100.0   # 100 MHz -> us, from the first unit's start
        diffs.append(np.diff(rel, axis=2).reshape(-1, 7))
        spans.append(float(rel[:, :, 7].max()))
        skews.append(float(rel[:, :, 0].max()))
    d = np.concatenate(diffs)
    return {"timeline": HEADLINE, "splits": S, "units": units, "snapshots": len(spans),
            "launch_us_median_of_batches": float(np.median(launch_us)),
            "phases_us": {n: {"median": float(np.median(d[:, k])), "p10": float(np.percentile(d[:, k], 10)),
                              "p90": float(np.percentile(d[:, k], 90))} for k, n in enumerate(phases)},
            "unit_start_skew_us_median": float(np.median(skews)),
            "first_start_to_last_store_done_us_median": float(np.median(spans))}


# decode kernel instantiation -> (workload, splits, partials, record file) in a
# run of `bench.py --no-cpu --no-workloads --roof-seconds 0 --copy-calibration`
TRAFFIC_RECORDS = {
    "void mla::decode_kernel<4, true, false, false, false>(mla::DecodeParams)":
        (HEADLINE, 4, "bf16", "decode_hbm_traffic.json"),
    "void mla::decode_kernel<3, true, false, false, true>(mla::DecodeParams)":
        ("v3_fp8_b64_l4096", 4, "bf16", "decode_fp8_hbm_traffic.json"),
    "void mla::decode_kernel<4, true, false, true, false>(mla::DecodeParams)":
        ("v3_sparse_b64_topk2048", 4, "bf16", "decode_sparse_hbm_traffic.json"),
    "void mla::decode_kernel<3, true, false, true, true>(mla::DecodeParams)":
        ("v3_sparse_b64_topk2048", 4, "bf16", "decode_sparse_fp8_hbm_traffic.json"),
}


def traffic_record(fetch_csv, write_csv):
    """HBM bytes per launch of each decode kernel from two rocprofv3 counter
    passes (FETCH_SIZE, then WRITE_SIZE; per-dispatch CSVs): the median over
    the kernel's dispatches, scaled by what the same counter reads for the
    benchmark's 1 GiB device-to-device copies (2^30 bytes read and written).  Writes
    one record per kernel under profiles/ (with the decode sources' hash, so
    the benchmark reports it only while the kernel is unchanged)."""
    import csv
    import statistics
    from mla_latent_kv_amd import _build

    def per_dispatch(path, counter):
        sums = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
        return sums

    fetch_d = per_dispatch(fetch_csv, "FETCH_SIZE")
    write_d = per_dispatch(write_csv, "WRITE_SIZE")
    # the 1 GiB device-to-device copies (the context measurement and the
    # calibration copy) are the copy dispatches that wrote exactly 2^20 KiB.  The
    # two passes make the same copies in the same order (the warm-up loops, whose
    # length depends on time, launch no copies), so a copy is matched across the
    # passes by its position among the copy dispatches
    def copies(d):
        return [v for (k, _), v in sorted(d.items(), key=lambda kv: kv[0][1]) if "copyBuffer" in k]
    fc, wc = copies(fetch_d), copies(write_d)
    cal = [i for i, v in enumerate(wc) if v == float(1 << 20)]
    if not cal or len(fc) != len(wc):
        raise SystemExit("no 1 GiB calibration copy in both counter passes (run bench.py with --copy-calibration)")
    fetch_factor = (1 << 30) / (statistics.median(fc[i] for i in cal) * 1024)   # bytes per counted KiB
    write_factor = (1 << 30) / (statistics.median(wc[i] for i in cal) * 1024)
    fetch, write = {}, {}
    for (k, _), v in fetch_d.items():
        fetch.setdefault(k, []).append(v)
    for (k, _), v in write_d.items():
        write.setdefault(k, []).append(v)
    out = []
    for kname, (workload, splits, partials, fname) in TRAFFIC_RECORDS.items():
        if kname not in fetch or kname not in write:
            continue
        rd = statistics.median(fetch[kname]) * 1024 * fetch_factor
        wr = statistics.median(write[kname]) * 1024 * write_factor
        rec = {"workload": workload, "kernel": kname, "source_sha256": _build.kernel_source_hash(),
               "bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
               "fetch_factor": fetch_factor, "write_factor": write_factor, "splits": splits, "partials": partials,
               "dispatches": len(fetch[kname])}
        with open(os.path.join(ROOT, "profiles", fname), "w") as fh:
            json.dump(rec, fh, indent=1)
        out.append(rec)
    # the step's other kernels in the same passes: printed, not recorded
    for kname in sorted(set(fetch) & set(write)):
        if kname in TRAFFIC_RECORDS or "copyBuffer" in kname:
            continue
        rd = statistics.median(fetch[kname]) * 1024 * fetch_factor
        wr = statistics.median(write[kname]) * 1024 * write_factor
        out.append({"kernel": kname, "context": True, "bytes_per_launch": rd + wr, "read_bytes": rd,
                    "write_bytes": wr, "dispatches": len(fetch[kname])})
    return out


def trace_segments(trace_csv, kernel=None):
    """Per-kernel durations from a rocprofv3 kernel-trace CSV: for each decode
    kernel, the mean over all its dispatches (what --stats reports) and the mean
    over its longest run of consecutive dispatches with no other kernel between
    them (the benchmark's back-to-back segment, which the roofline figure times),
    both as kernel durations and as the segment's span (first start to last end)
    per dispatch."""
    import csv
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    out = []
    for kname in sorted(set(names)):
        if "decode_kernel" not in kname or (kernel and kernel not in kname):
            continue
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in rows
                if r["Kernel_Name"] == kname]
        best, run = (0, 0), None
        for i, n in enumerate(names + [None]):
            if n == kname:
                run = i if run is None else run
            elif run is not None:
                if i - run > best[1] - best[0]:
                    best = (run, i)
                run = None
        seg = rows[best[0]:best[1]]
        seg_d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in seg]
        span = (int(seg[-1]["End_Timestamp"]) - int(seg[0]["Start_Timestamp"])) * 1e-3 / len(seg)
        out.append({"kernel": kname, "dispatches": len(durs), "mean_us": sum(durs) / len(durs),
                    "b2b_dispatches": len(seg), "b2b_mean_us": sum(seg_d) / len(seg_d),
                    "b2b_span_us_per_dispatch": span})
    return out


def cpu_baseline(case, pairs_n, threads, gpu_out=None, seed=123):
    """Time the CPU oracle (fp64 Normal path) on a seeded sample of (b, h) pairs
    and scale linearly to the whole batch (its cost is linear in pairs x keys).
    With ``gpu_out`` (the timed step's output), the oracle results also check
    it: the sampled pairs against the Normal path, every element against the
    absorbed mirror, to the product tolerance -- proof that the timed kernels
    computed the step."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(seed)
    B, H = case.B, case.H
    idx = rng.choice(B * H, size=min(pairs_n, B * H), replace=False)
    pairs = np.stack([idx // H, idx % H], axis=1).astype(np.int32)
    oracle.lib()
    t0 = time.perf_counter()
    ref_pairs, _ = oracle.normal_decode(case, pairs=pairs, nthreads=threads)
    dt = time.perf_counter() - t0
    keys_sample = float(np.sum(case.seqlens[pairs[:, 0]]))
    keys_all = float(np.sum(case.seqlens)) * H
    t_full = dt * keys_all / keys_sample
    # the fp64 absorbed mirror (absorb, latent attention, un-absorb) on the whole batch
    t0 = time.perf_counter()
    ql = oracle.absorb(case.q_nope, case.w_uk)
    lat, _ = oracle.latent_attention(case, ql, nthreads=threads)
    ref_all = oracle.unabsorb(lat, case.w_uv)
    t_mirror = time.perf_counter() - t0
    check = None
    if gpu_out is not None:
        sel = (pairs[:, 0], slice(None), pairs[:, 1])
        got_s, ref_s = gpu_out[sel], ref_pairs[sel]
        tol_s = 1e-2 * float(np.max(np.abs(ref_s))) + 1e-3
        err_s = float(np.max(np.abs(got_s - ref_s)))
        tol_a = 1e-2 * float(np.max(np.abs(ref_all))) + 1e-3
        err_a = float(np.max(np.abs(gpu_out - ref_all)))
        check = {"max_abs_err_vs_normal_sample": err_s, "tol_normal_sample": tol_s,
                 "max_abs_err_vs_absorbed_mirror": err_a, "tol_absorbed_mirror": tol_a,
                 "pass": bool(np.isfinite(gpu_out).all() and err_s <= tol_s and err_a <= tol_a)}
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": case.B * case.T / t_full,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 Normal-path oracle on {len(pairs)} of {B * H} (sequence, head) pairs "
                  f"({int(keys_sample)} keys, {dt:.1f} s on {threads} threads), scaled linearly "
                  f"to all {B * H} pairs; {cpu}, {os.cpu_count()} logical CPUs visible",
        "absorbed_mirror_value": case.B * case.T / t_mirror,
        "absorbed_mirror_sample": f"fp64 absorbed mirror (absorb, latent attention, un-absorb) on the whole "
                                  f"batch: {t_mirror:.1f} s on {threads} threads",
        "timed_output_check": check,
    }


def time_workload(wl, S, partials, K, W, R, dev, graph=True, warm=False):
    # merge and un-absorb in one kernel where that is the faster form: bf16
    # partials and at most four splits per sequence (measured A/B, interleaved,
    # on the headline: 104.8 against 109.6 us per step; with more splits per
    # row the fused kernel merges row by row and the two kernels are faster)
    """Time one workload's step (absorb -> decode -> merge -> un-absorb) on the
    GPU: R replicas of the cache and weights rotate from step to step.  The
    chain's time per step is the faster of K eager steps and K replays of the
    step captured as a HIP graph (one per replica); K further eager steps with
    HIP events around each decode launch, and K back-to-back decode launches
    between one event pair, give the decode kernel's own duration (with
    automatic splits it includes the one-workgroup plan kernel)."""
    import numpy as np
    import torch
    import mla_latent_kv_amd as mk
    import synth
    case = synth.make_case(wl, poison=False)
    B, T, H = case.B, case.T, case.H

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    kv0 = bf16(case.kv_cache)
    kv = [kv0] + [kv0.clone() for _ in range(R - 1)]
    wuk0, wuv0 = bf16(case.w_uk), bf16(case.w_uv)
    wuk = [wuk0] + [wuk0.clone() for _ in range(R - 1)]
    wuv = [wuv0] + [wuv0.clone() for _ in range(R - 1)]
    q_nope, q_pe = bf16(case.q_nope), bf16(case.q_pe)
    block_table = torch.from_numpy(case.block_table).to(dev)
    seqlens = torch.from_numpy(case.seqlens).to(dev)
    max_seqlen = case.max_seqlen
    scale = mk.softmax_scale()
    part_dtype = torch.bfloat16 if partials == "bf16" else torch.float32
    buf = mk.DecodeBuffers(B, T, H, max_seqlen, case.page_size, S, dev, part_dtype=part_dtype) \
        if S != 1 else None
    q_lat = torch.empty((B, T, H, 512), dtype=torch.bfloat16, device=dev)
    latent = torch.empty((B, T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    out = torch.empty((B, T, H, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    fused_ok = partials == "bf16" and 1 < S <= 4

    def step(r, ev=None, fused=fused_ok):
        mk.mla_absorb_q(q_nope, wuk[r], q_lat=q_lat)
        if ev is not None:
            ev[0].record(stream)
        if S == 1:
            mk.mla_decode_latent(q_lat, q_pe, kv[r], block_table, seqlens, max_seqlen, scale,
                                 num_splits=1, out_latent=latent, lse=lse)
        else:
            mk.mla_decode_latent(q_lat, q_pe, kv[r], block_table, seqlens, max_seqlen, scale,
                                 num_splits=S, buffers=buf, merge=False)
        if ev is not None:
            ev[1].record(stream)
        if S == 1:
            mk.mla_unabsorb_out(latent, wuv[r], out=out)
        elif fused:
            # merge and un-absorb in one kernel (the merged latent stays on chip)
            mk.mla_merge_unabsorb(buf.part_out, buf.part_lse, buf.split_indptr, wuv[r], B, out=out, lse=lse)
        else:
            mk.mla_merge_splits(buf.part_out, buf.part_lse, buf.split_indptr, B, out_latent=latent,
                                lse=lse)
            mk.mla_unabsorb_out(latent, wuv[r], out=out)

    warm_up(lambda i: step(i % R), W)
    # the chain launched eagerly: K steps between two synchronisations
    t0 = time.perf_counter()
    for i in range(K):
        step(i % R)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the same with the other form of the merge and un-absorb (context)
    alt_ms = None
    if S != 1:
        t0s = time.perf_counter()
        for i in range(K):
            step(i % R, fused=not fused_ok)
        torch.cuda.synchronize()
        alt_ms = (time.perf_counter() - t0s) * 1e3 / K
    # the same with an event pair around each decode launch (per-launch detail)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        step(i % R, evs[i])
    torch.cuda.synchronize()
    res = {"case": case, "kv": kv, "block_table": block_table, "seqlens": seqlens, "out": out,
           "dec_ms": [a.elapsed_time(b) for a, b in evs], "eager_ms_per_step": (t1 - t0) * 1e3 / K,
           "warm_ms": None, "graph_ms_per_step": None, "alt_merge_ms_per_step": alt_ms,
           "merge_unabsorb": "fused" if fused_ok else ("separate" if S != 1 else "none")}

    # the decode kernel's own duration: K launches back to back (replicas still
    # rotating) between one event pair, divided by K.  (An event pair around each
    # launch also spans the packet processing before and after the kernel.)
    def decode_only(r):
        if S == 1:
            mk.mla_decode_latent(q_lat, q_pe, kv[r], block_table, seqlens, max_seqlen, scale,
                                 num_splits=1, out_latent=latent, lse=lse)
        else:
            mk.mla_decode_latent(q_lat, q_pe, kv[r], block_table, seqlens, max_seqlen, scale,
                                 num_splits=S, buffers=buf, merge=False)
    warm_up(lambda i: decode_only(i % R), 3, seconds=0.02)
    eb = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    eb[0].record(stream)
    for i in range(K):
        decode_only(i % R)
    eb[1].record(stream)
    torch.cuda.synchronize()
    res["dec_b2b_ms"] = eb[0].elapsed_time(eb[1]) / K
    if warm:
        # the same with one cache replica (no rotation: the 256 MB last-level cache
        # may serve part of a step's reads from the previous step) -- context only
        wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i in range(K):
            step(0, wev[i])
        torch.cuda.synchronize()
        res["warm_ms"] = float(np.median([a.elapsed_time(b) for a, b in wev]))
    res["ms_per_step"] = res["eager_ms_per_step"]
    res["chain_launch"] = "eager"
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(R):
                step(r)
        torch.cuda.current_stream().wait_stream(side)
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        warm_up(lambda i: graphs[i % R].replay(), W)
        t0 = time.perf_counter()
        for i in range(K):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        res["graph_ms_per_step"] = (t1 - t0) * 1e3 / K
        res["graphs"] = graphs
        if res["graph_ms_per_step"] < res["ms_per_step"]:
            res["ms_per_step"] = res["graph_ms_per_step"]
            res["chain_launch"] = "hip_graph"
    return res


def workload_line(wl, S, partials, K, W, R, dev):
    """Timed figures of one workload (the other configurations beside the
    headline): decode kernel time and its algorithmic rates, chain time and
    query tokens per second."""
    import numpy as np
    import torch
    tw = time_workload(wl, S, partials, K, W, R, dev, graph=True)
    case = tw["case"]
    dec_ms = tw["dec_b2b_ms"]
    nbytes, flops = decode_algorithmic(case)
    rec = {
        "B": case.B, "T": case.T, "H": case.H, "L": wl.L, "context_tokens": int(np.sum(case.seqlens)),
        "page_size": case.page_size, "num_splits": S, "partials": partials, "cache_replicas": R, "steps": K,
        "decode_us": dec_ms * 1e3, "decode_us_event_pairs_mean": float(np.mean(tw["dec_ms"])) * 1e3,
        "decode_alg_bytes": nbytes, "decode_alg_flops": flops,
        "decode_GBps": nbytes / (dec_ms * 1e-3) / 1e9,
        "decode_hbm_frac": nbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "decode_tflops": flops / (dec_ms * 1e-3) / 1e12,
        "decode_mfma_frac": flops / (dec_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "chain_us_per_step": tw["ms_per_step"] * 1e3, "chain_launch": tw["chain_launch"],
        "chain_merge_unabsorb": tw["merge_unabsorb"],
        "tokens_per_s": case.B * case.T / (tw["ms_per_step"] * 1e-3),
        "chain_TBps": chain_algorithmic(case, nbytes) / (tw["ms_per_step"] * 1e-3) / 1e12,
    }
    del tw
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed warm-up steps before each timed region (at least; warm-up also lasts at "
                         "least 0.1 s of back-to-back work, for the clocks to settle)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--splits", type=int, default=4,
                    help="split-KV chunks per sequence (0 = automatic)")
    ap.add_argument("--partials", choices=["bf16", "f32"], default="bf16",
                    help="dtype of the split partial outputs")
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--cpu-pairs", type=int, default=640)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the decode over FP8 rows (detail fields fp8_*)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the chain with eager launches instead of replaying a captured HIP graph")
    ap.add_argument("--no-sparse", action="store_true",
                    help="skip the sparse (top-k) decode measurement reported under detail")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--crossover", action="store_true",
                    help="instead of the benchmark line: time the absorbed and the Normal path over query-block "
                         "lengths T (one JSON line per T)")
    ap.add_argument("--crossover-T", default="1,8,32,64,96,128,160,192,256,384,512")
    ap.add_argument("--crossover-S", type=int, default=4096)
    ap.add_argument("--crossover-B", type=int, default=4)
    ap.add_argument("--clock-sample", type=float, default=0.0,
                    help="instead of the benchmark line: run the headline decode kernel back to back for this "
                         "many seconds while sampling the gfx clock and power (one JSON line)")
    ap.add_argument("--clock-kernel", choices=["bf16", "fp8"], default="bf16")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the driver-timed lines of the other configurations (detail.workloads)")
    ap.add_argument("--roof-seconds", type=float, default=2.5,
                    help="seconds per practical-roof probe and half the seconds of the decode clock sample "
                         "reported under detail (0 skips them)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="instead of the benchmark line: write the decode kernels' HBM traffic records under "
                         "profiles/ from two rocprofv3 counter_collection CSVs (FETCH_SIZE pass, WRITE_SIZE pass)")
    ap.add_argument("--trace-segments", metavar="KERNEL_TRACE_CSV",
                    help="instead of the benchmark line: each decode kernel's mean duration over all dispatches and "
                         "over its back-to-back segment, from a rocprofv3 kernel-trace CSV")
    ap.add_argument("--timeline", type=int, default=0, metavar="BATCHES",
                    help="instead of the benchmark line: the headline decode kernel's phases timed from inside it "
                         "(libmla_timeline.so), over this many snapshots (one JSON line)")
    ap.add_argument("--pipeline-roof", type=float, default=0.0,
                    help="instead of the benchmark line: run the decode kernel's data flow without its arithmetic "
                         "(and the decode kernel) back to back for this many seconds each (one JSON line each)")
    ap.add_argument("--power-roof", type=float, default=0.0,
                    help="instead of the benchmark line: run the practical-roof probes for this many seconds each "
                         "(one JSON line per probe)")
    args = ap.parse_args()

    if args.traffic_record:
        for rec in traffic_record(*args.traffic_record):
            print(json.dumps(rec), flush=True)
        return
    if args.trace_segments:
        for rec in trace_segments(args.trace_segments):
            print(json.dumps(rec), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path does not shard across GPUs "
              "(one process, one device); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mla_latent_kv_amd as mk
    import synth

    if args.timeline > 0:
        from mla_latent_kv_amd import _build
        mk.LIB_PATH = _build.TIMELINE_LIB   # the instrumented build of the same source, in its place
    mk.load_library()
    dev = "cuda:0"
    if args.timeline > 0:
        print(json.dumps(timeline(args.timeline, dev)), flush=True)
        return
    if args.crossover:
        Ts = [int(x) for x in args.crossover_T.split(",")]
        for row in crossover(Ts, args.crossover_S, args.crossover_B, max(3, min(args.steps, 20)),
                             max(1, min(args.warmup, 3)), dev):
            print(json.dumps(row), flush=True)
        return
    if args.pipeline_roof > 0:
        for row in pipeline_roof(args.pipeline_roof, dev):
            print(json.dumps(row), flush=True)
        return
    if args.power_roof > 0:
        for row in power_roof(args.power_roof, dev):
            print(json.dumps(row), flush=True)
        return
    if args.clock_sample > 0:
        print(json.dumps(clock_sample(args.clock_sample, args.clock_kernel, dev)), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    K = args.steps
    R = max(1, args.replicas)
    S = args.splits
    tw = time_workload(wl, S, args.partials, K, args.warmup, R, dev, graph=not args.no_graph, warm=True)
    case, kv, block_table, seqlens, out = tw["case"], tw["kv"], tw["block_table"], tw["seqlens"], tw["out"]
    B, T, H = case.B, case.T, case.H
    stream = torch.cuda.current_stream()
    dec_ms = tw["dec_ms"]
    dec_ms_avg = tw["dec_b2b_ms"]   # the kernel's duration: back-to-back launches (see time_workload)
    eager_ms_per_step = tw["eager_ms_per_step"]
    warm_ms = tw["warm_ms"]
    ms_per_step = tw["ms_per_step"]

    # cache append of the step's new rows (written at position L - T + t of each
    # sequence; the timed cache's own rows there are overwritten, which changes
    # no timing)
    c_new = torch.randn((B, T, 512), device=dev).to(torch.bfloat16)
    kpe_new = torch.randn((B, T, 64), device=dev).to(torch.bfloat16)
    # (a few-microsecond kernel: one event pair around K back-to-back launches)
    app_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    warm_up(lambda i: mk.mla_append_cache(c_new, kpe_new, kv[i % R], block_table, seqlens), args.warmup,
            seconds=0.02)
    app_ev[0].record(stream)
    for i in range(K):
        mk.mla_append_cache(c_new, kpe_new, kv[i % R], block_table, seqlens)
    app_ev[1].record(stream)
    torch.cuda.synchronize()
    app_ms = app_ev[0].elapsed_time(app_ev[1]) / K
    app_bytes = 2 * B * T * (512 + 64) * 2 + 4 * B * 2   # rows read + written, seqlens, table entries

    # context line: the chip's practical streaming rate on a plain 1 GiB
    # device-to-device copy (read + written bytes over its duration)
    src_c = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst_c = torch.empty_like(src_c)
    src_c.fill_(1)
    for _ in range(2):
        dst_c.copy_(src_c)
    ce = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ce[0].record(stream)
    for _ in range(5):
        dst_c.copy_(src_c)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_GBps = 2 * (1 << 30) * 5 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del src_c, dst_c
    torch.cuda.empty_cache()

    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give the
        # factor that turns those counters into bytes for the decode kernel
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    dec_bytes, dec_flops = decode_algorithmic(case)
    achieved = dec_bytes / (dec_ms_avg * 1e-3) / 1e9
    value = B * T / (ms_per_step * 1e-3)

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "decode_hbm_traffic.json")
    if os.path.exists(tpath):
        try:
            from mla_latent_kv_amd import _build
            rec = json.load(open(tpath))
            if rec.get("source_sha256") == _build.kernel_source_hash() and rec.get("workload") == wl.name \
                    and int(rec.get("splits", -1)) == S and rec.get("partials") == args.partials:
                traffic = rec["bytes_per_launch"]
        except Exception:
            traffic = None

    result = {
        "metric": "MLA absorbed decode tokens/s + achieved HBM TB/s (% peak), H=128 B=64 L=4096",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "L": wl.L, "page_size": wl.page_size,
                   "kv_lora_rank": 512, "rope": 64, "num_splits": S, "partials": args.partials,
                   "cache_replicas": R},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "detail": {
            "kernel": "decode_kernel (latent attention, split-KV partials)",
            "decode_us": dec_ms_avg * 1e3,
            "decode_timing": "events around K back-to-back launches / K",
            "decode_us_event_pairs_mean": float(np.mean(dec_ms)) * 1e3,
            "decode_us_event_pairs_median": float(np.median(dec_ms)) * 1e3,
            "decode_us_event_pairs_p10": float(np.percentile(dec_ms, 10)) * 1e3,
            "decode_us_event_pairs_p90": float(np.percentile(dec_ms, 90)) * 1e3,
            "decode_us_warm_median": warm_ms * 1e3,
            "context_rows_per_s": float(np.sum(case.seqlens)) / (dec_ms_avg * 1e-3),
            "decode_us_event_pairs_min": float(np.min(dec_ms)) * 1e3,
            "hbm_copy_GBps": copy_GBps,
            "decode_alg_bytes": dec_bytes,
            "decode_alg_flops": dec_flops,
            "decode_tflops": dec_flops / (dec_ms_avg * 1e-3) / 1e12,
            "decode_mfma_frac": dec_flops / (dec_ms_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "chain_launch": tw["chain_launch"],
            "chain_eager_ms_per_step": eager_ms_per_step,
            "chain_graph_ms_per_step": tw["graph_ms_per_step"],
            "chain_merge_unabsorb": tw["merge_unabsorb"],
            "chain_eager_other_merge_unabsorb_ms_per_step": tw["alt_merge_ms_per_step"],
            "chain_alg_bytes": chain_algorithmic(case, dec_bytes),
            "chain_TBps": chain_algorithmic(case, dec_bytes) / (ms_per_step * 1e-3) / 1e12,
            "append_us": app_ms * 1e3,
            "append_alg_bytes": app_bytes,
            "append_GBps": app_bytes / (app_ms * 1e-3) / 1e9,
        },
    }
    if not args.no_workloads:
        # every other configuration, timed (fewer steps each), plus the
        # headline with fp32 partials (the partial dtype the scope table names)
        Kw, Ww = min(K, 30), min(args.warmup, 5)
        others = [("v2lite_tiny", "v2lite_tiny", 1, "bf16", 3),
                  ("v3_b64_l4096_f32_partials", HEADLINE, 4, "f32", 3),
                  ("v3_ragged_b128", "v3_ragged_b128", 0, "bf16", 2),
                  ("v3_long_b4_l131072", "v3_long_b4_l131072", 64, "bf16", 2),
                  # equal lengths: uniform splits (8 x 1024 tokens per sequence, 256 units)
                  # spare the automatic plan's extra kernel
                  ("v3_mtp_b32_t4_h32", "v3_mtp_b32_t4_h32", 8, "bf16", 3)]
        lines = {}
        for key, name, S_w, part, R_w in others:
            lines[key] = workload_line(synth.WORKLOADS[name], S_w, part, Kw, Ww, R_w, dev)
        result["detail"]["workloads"] = lines
    if args.roof_seconds > 0:
        result["detail"]["decode_clock_sample"] = clock_sample(args.roof_seconds * 2, "bf16", dev)
        result["detail"]["power_roof"] = power_roof(args.roof_seconds, dev)
    if not args.no_sparse:
        result["detail"].update(bench_sparse("v3_sparse_b64_topk2048", K, args.warmup, R, dev))
        if not args.no_fp8:
            result["detail"].update(bench_sparse("v3_sparse_b64_topk2048", K, args.warmup, R, dev, fp8=True))
    if not args.no_fp8:
        result["detail"].update(bench_fp8("v3_fp8_b64_l4096", 4, K, args.warmup, R, dev))
    if not args.no_cpu:
        try:
            threads = len(os.sched_getaffinity(0))   # every host core this process may run on
        except AttributeError:
            threads = os.cpu_count() or 1
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_pairs, threads,
                                              gpu_out=out.double().cpu().numpy())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
