#!/usr/bin/env python3
"""Mixed-batch attention throughput on one MI355X.

A step is one pass of the whole path over one packed batch: the host
decode-first budget split and work plan (cpa_build_metadata), one H2D copy of
the step metadata, the paged KV append (cpa_append_kv), then cpa_attention:
the split-KV decode kernel and the MFMA prefill-chunk kernel (one launch when
the chunk tiles fill a resident round) and one log-sum-exp merge launch for
the split pieces of both, all on one stream.  Inputs (q, new K/V, the paged
KV pool) are resident in HBM before timing.

Default workload, the largest of the configurations (heavy mixed step): 256
decode rows (contexts lognormal, median 1024, sigma 0.75, capped at 16384)
plus prefill chunks of 2048, 2048 and 3840 tokens at random prefixes in
[0, 16384], budget 8192, a 2 GiB KV pool; Hq=32, Hkv=8, D=128, bf16,
16-token pages.  Two instances of the recipe (two seeds), each with its own
pool, are rotated step by step, so no step finds its K/V in the 256 MB
last-level cache from the step before.  ``--config N`` picks another
configuration; the other configurations are also run briefly after the
headline and reported under ``other_configs``.

Prints ONE JSON line on stdout.  Per-kernel durations come from HIP events
recorded on the launch stream around each launch inside the timed region, on
whole rounds of instances (the first step of every instance, every
``--kernel-event-stride``-th round), which run each plan section as its own
launch (append, decode, chunk, decode merge, chunk merge) so each kernel has
its own span; the other steps make the one cpa_attention call and carry no
events (a marker costs a few microseconds of GPU time between two launches;
``empty_span_us`` is the span between two markers with no launch between, the
part of every kernel span that is not the kernel).  A plan section with no
entries launches nothing and is reported as ``{"launched": false}``.
The step rate is the wall clock over all timed steps.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, published
METRIC = "mixed-batch attention tokens/s; % HBM GB/s (decode) & % MFMA (chunk)"

WORKLOAD_TEXT = {
    1: "tiny: Hq=Hkv=4 D=64; 4 decode rows (context U[100,300]) + a 64-token chunk of a 256-token "
       "prompt, 4 chunk positions rotated; budget 68",
    2: "page1_defaults: 32 decode rows (context U[512,4096]) + a 480-token chunk of an 8192-token "
       "prompt at prefix 0/3840/7680 (3 instances rotated per step); Hq=32 Hkv=8 D=128 bf16, "
       "16-token pages, budget 512",
    3: "budget8192: 2 decode rows (context 1000, 3000) + a 2048-token chunk of an 8192-token prompt "
       "at prefix 0/2048/4096/6144 (4 instances rotated); cap 2048; Hq=32 Hkv=8 D=128",
    4: "long_context: final 1024-token chunk of a 32768-token prompt (prefix 31744) + 64 decode "
       "rows (context lognormal, median 2048, sigma 0.75, cap 32768); Hq=32 Hkv=8 D=128",
    5: "heavy_mixed: 256 decode rows (context lognormal, median 1024, sigma 0.75, cap 16384) + "
       "chunks of 2048, 2048 and 3840 tokens at random prefixes in [0,16384]; budget 8192; "
       "2 GiB KV pool; Hq=32 Hkv=8 D=128",
}

# kernels timed on their own in the sampled steps, in launch order
SPANS = ("append_kernel", "decode_kernel", "chunk_kernel", "decode_merge", "chunk_merge")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work of one step (what the method must move or compute)
# ---------------------------------------------------------------------------

def step_work(meta, Hq, Hkv, D):
    nd = meta["num_decodes"]
    seq = meta["seq_lens"]
    ctx = meta["context_lens"]
    nsch = meta["num_scheduled"]
    dec_keys = sum(int(seq[s]) for s in range(nd))
    dec_pages = sum(math.ceil(int(seq[s]) / 16) for s in range(nd))
    decode_bytes = dec_keys * Hkv * D * 2 * 2 + nd * Hq * D * 2 * 2 + dec_pages * 4
    chunk_flops = 0
    chunk_min_bytes = 0
    for s in range(nd, meta["num_seqs"]):
        n, c = int(nsch[s]), int(ctx[s])
        chunk_flops += 4 * D * Hq * (n * c + n * (n + 1) // 2)
        chunk_min_bytes += (c + n) * Hkv * D * 4 + 2 * n * Hq * D * 2
    T = meta["num_tokens"]
    append_bytes = T * Hkv * D * 2 * 2 * 2
    return {"decode_bytes": decode_bytes, "chunk_flops": chunk_flops,
            "chunk_min_bytes": chunk_min_bytes, "append_bytes": append_bytes, "tokens": T,
            "decode_keys": dec_keys}


# ---------------------------------------------------------------------------
# one resident instance with its per-step host work prepared
# ---------------------------------------------------------------------------

class Instance:
    def __init__(self, w, torch, cpa, DeviceStep):
        import numpy as np
        self.w = w
        self.torch = torch
        self.ds = ds = DeviceStep(w, validate=True, with_lse=False)
        lib = self.lib = cpa.load()
        m = ds.meta
        ns, words = ds.num_seqs, int(m["plan"].size)
        # packed metadata: [qsl | seq_lens | ctx | plan], each section 16-byte aligned
        def up4(x):
            return (x + 3) // 4 * 4
        self.off = off = {}
        at = 0
        for name, n in (("qsl", ns + 1), ("seq", ns), ("ctx", ns), ("plan", max(1, words))):
            off[name] = at
            at += up4(n)
        self.pinned = torch.zeros(at, dtype=torch.int32, pin_memory=True)
        self.dev = torch.zeros(at, dtype=torch.int32, device="cuda")
        pn = self.pinned.numpy()
        i32p = cpa.i32p
        self.reqs = (cpa.cpa_req_t * max(1, len(w.requests)))()
        for i, r in enumerate(w.requests):
            self.reqs[i] = cpa.cpa_req_t(r.id, r.num_computed, r.target_len, int(r.is_decode))
        self.nreq = len(w.requests)
        self.params = cpa.cpa_build_params_t(w.token_budget, w.long_prefill_cap, 16, w.num_q_heads,
                                             w.num_kv_heads, w.head_dim, 0, 0,
                                             cpa.CPA_POLICY_TRUNCATE, 0)
        self.scratch = {k: np.zeros(max(1, self.nreq), dtype=np.int32)
                        for k in ("order", "nsch", "newb")}
        meta = self.meta = cpa.cpa_meta_t()
        meta.max_seqs = max(1, self.nreq)
        meta.order = self.scratch["order"].ctypes.data_as(i32p)
        meta.num_scheduled = self.scratch["nsch"].ctypes.data_as(i32p)
        meta.new_blocks = self.scratch["newb"].ctypes.data_as(i32p)
        meta.query_start_loc = pn[off["qsl"]:].ctypes.data_as(i32p)
        meta.seq_lens = pn[off["seq"]:].ctypes.data_as(i32p)
        meta.context_lens = pn[off["ctx"]:].ctypes.data_as(i32p)
        meta.max_tokens = 0
        meta.slot_mapping = None
        meta.plan_capacity = max(1, words)
        meta.plan = pn[off["plan"]:].ctypes.data_as(i32p)
        self.build_host()  # fills the pinned buffer once
        self.host_build_s, self.host_builds = 0.0, 0  # host time of the per-step builds
        assert self.meta.num_tokens == ds.num_tokens and self.meta.plan_words == words
        # device tensors of the step now live in the packed buffer
        d = self.dev
        ds.query_start_loc = d[off["qsl"]:off["qsl"] + ns + 1]
        ds.seq_lens = d[off["seq"]:off["seq"] + ns]
        ds.context_lens = d[off["ctx"]:off["ctx"] + ns]
        ds.plan = d[off["plan"]:off["plan"] + max(1, words)]
        self.dev.copy_(self.pinned)
        torch.cuda.synchronize()
        self.copy_done = torch.cuda.Event()
        self.copy_done.record()
        self._prepare_calls(cpa)
        self.work = step_work(m, w.num_q_heads, w.num_kv_heads, w.head_dim)
        self.graph = None

    def build_host(self):
        st = self.lib.cpa_build_metadata(self.reqs, self.nreq, ctypes.byref(self.params), None, 0,
                                         0, ctypes.byref(self.meta))
        if st != 0:
            raise RuntimeError(f"cpa_build_metadata failed: {st}")

    def _prepare_calls(self, cpa):
        ds, w, torch = self.ds, self.w, self.torch
        vp = ctypes.c_void_p
        P = lambda t: vp(t.data_ptr()) if t is not None else None
        self.stream = vp(torch.cuda.current_stream().cuda_stream)
        c = ds.counts
        plan_base = ds.plan.data_ptr()
        off = cpa.section_offsets(c)
        tail = (ds.num_seqs, ds.num_decodes, ds.num_tokens, w.num_q_heads, w.num_kv_heads,
                w.head_dim, 16, ctypes.c_float(w.scale), P(ds.out), None, P(ds.workspace),
                ctypes.c_size_t(0 if ds.workspace is None else ds.workspace.numel()), self.stream)
        head = (P(ds.q), P(ds.k_cache), P(ds.v_cache), P(ds.block_table),
                int(ds.block_table.shape[1]), P(ds.query_start_loc), P(ds.seq_lens),
                P(ds.context_lens))
        zero = dict(num_decode_splits=0, num_decode_merges=0, num_chunk_tiles=0,
                    num_chunk_merges=0)
        # one plan section per call, so HIP events can bracket each launch; a
        # section with no entries launches nothing and has no span
        self.section_args = {}
        self.launches = {"append_kernel": ds.num_tokens > 0}
        self._keep = []
        for name, field, sec in (("decode_kernel", "num_decode_splits", "decode_splits"),
                                 ("chunk_kernel", "num_chunk_tiles", "chunk_tiles"),
                                 ("decode_merge", "num_decode_merges", "decode_merges"),
                                 ("chunk_merge", "num_chunk_merges", "chunk_merges")):
            counts = c.copy(**{**zero, field: getattr(c, field)})
            self.launches[name] = getattr(c, field) > 0
            self._keep.append(counts)
            self.section_args[name] = head + (vp(plan_base + 4 * off[sec]),
                                              ctypes.byref(counts)) + tail
        # the whole plan in one call, as a caller runs a step
        self.full_args = head + (vp(plan_base), ctypes.byref(c)) + tail
        self.append_args = (P(ds.k_new), P(ds.v_new), P(ds.query_start_loc), P(ds.context_lens),
                            P(ds.block_table), int(ds.block_table.shape[1]), ds.num_seqs,
                            ds.num_tokens, w.num_kv_heads, w.head_dim, 16, P(ds.k_cache),
                            P(ds.v_cache), self.stream)

    def capture(self):
        """Append + the whole attention call captured as one HIP graph on a
        capture stream; unsampled steps then replay it (the metadata copy stays
        outside the graph, before the replay on the same stream)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()  # default priority
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            st = self.lib.cpa_append_kv(*self.append_args[:-1], cs)
            st |= self.lib.cpa_attention(*self.full_args[:-1], cs)
        torch.cuda.current_stream().wait_stream(s)
        if st != 0:
            raise RuntimeError(f"launch failed during capture with status {st}")
        self.graph = g

    def step(self, events=None):
        """One full step.  With ``events`` (len(SPANS) + 3 HIP events) every
        launch runs on its own between two of them: events[0] before the
        metadata copy, events[1 + i] before span i, events[-2] after the
        last, and events[-1] right after events[-2] with nothing between
        (the cost of the markers themselves, which every span also holds);
        without, the step is one cpa_attention call (or the replay of the
        captured graph) and carries no events."""
        self.copy_done.synchronize()  # the previous copy out of the pinned buffer is done
        t0 = time.perf_counter()
        self.build_host()
        self.host_build_s += time.perf_counter() - t0
        self.host_builds += 1
        main = self.torch.cuda.current_stream()
        lib = self.lib
        if events is None:
            self.dev.copy_(self.pinned, non_blocking=True)
            self.copy_done.record()
            if self.graph is not None:
                self.graph.replay()
                return
            st = lib.cpa_append_kv(*self.append_args)
            st |= lib.cpa_attention(*self.full_args)
            if st != 0:
                raise RuntimeError(f"launch failed with status {st}")
            return
        events[0].record(main)
        self.dev.copy_(self.pinned, non_blocking=True)
        self.copy_done.record()
        st = 0
        for i, name in enumerate(SPANS):
            events[1 + i].record(main)
            if not self.launches[name]:
                continue
            if name == "append_kernel":
                st |= lib.cpa_append_kv(*self.append_args)
            else:
                st |= lib.cpa_attention(*self.section_args[name])
        events[-2].record(main)
        events[-1].record(main)
        if st != 0:
            raise RuntimeError(f"launch failed with status {st}")


def config_key(config: int) -> str:
    from chunked_prefill_mixed_amd import workloads
    return workloads.CONFIG_NAMES[config]


def traffic_for(kernel: str, config: int):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counter record, if it was taken on the current library sources."""
    from chunked_prefill_mixed_amd import counters
    rec = counters.traffic_record(kernel, config_key(config), os.path.join(ROOT, "profiles"))
    return None if rec is None else rec["traffic_bytes_per_launch"]


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * q
    lo, hi = math.floor(k), math.ceil(k)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def run_config(config, steps, warmup, stride, graph, torch, cpa, workloads, DeviceStep,
               kv_shard=1):
    """Warm up, then time ``steps`` steps of the configuration's instances,
    rotated; returns the measurements (see main)."""
    t_setup = time.perf_counter()
    ws = [workloads.make_workload(config, i, kv_shard)
          for i in range(workloads.num_instances(config))]
    insts = [Instance(w, torch, cpa, DeviceStep) for w in ws]
    log(f"config {config} setup {time.perf_counter() - t_setup:.1f}s: {len(insts)} instance(s), "
        f"{[i.ds.num_tokens for i in insts]} tokens/step")
    I = len(insts)
    NEV = len(SPANS) + 3
    # warm-up: each instance runs its sections once (the first launch of a
    # kernel on its own pays for loading it, which must not fall into a timed
    # span), then the one-call steps; a kernel trace of the run thus holds
    # one untimed launch per instance of each section kernel besides the
    # timed ones, in the same instance mix
    ev_w = [torch.cuda.Event(enable_timing=True) for _ in range(NEV)]
    for s in range(max(warmup, I)):
        insts[s % I].step(ev_w if s < I else None)
    torch.cuda.synchronize()
    if graph:
        for inst in insts:
            inst.capture()
        for inst in insts:  # one replay each before timing
            inst.step()
        torch.cuda.synchronize()
    # the first step of every instance in every stride-th round carries events
    order = [(warmup + s) % I for s in range(steps)]
    sampled = [s for s in range(steps) if (s // I) % max(1, stride) == 0]
    events = {s: [torch.cuda.Event(enable_timing=True) for _ in range(NEV)] for s in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        insts[order[s]].step(events.get(s))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    tokens = sum(insts[order[s]].work["tokens"] for s in range(steps))
    durs = {n: [] for n in SPANS}
    work = {n: [] for n in SPANS}
    wkey = {"append_kernel": "append_bytes", "decode_kernel": "decode_bytes",
            "chunk_kernel": "chunk_flops", "decode_merge": None, "chunk_merge": None}
    gpu_step, copy_us, gap_us = [], [], []
    span_steps = {n: [] for n in SPANS}  # the sampled steps in which span n launched
    for s in sampled:
        ev = events[s]
        copy_us.append(ev[0].elapsed_time(ev[1]) * 1e3)
        gpu_step.append(ev[1].elapsed_time(ev[-2]) * 1e3)
        gap_us.append(ev[-2].elapsed_time(ev[-1]) * 1e3)
        for i, n in enumerate(SPANS):
            if not insts[order[s]].launches[n]:
                continue
            span_steps[n].append(s)
            durs[n].append(ev[1 + i].elapsed_time(ev[2 + i]) * 1e3)  # us
            work[n].append(insts[order[s]].work[wkey[n]] if wkey[n] else 0)

    def stats(n):
        d = durs[n]
        if not d:
            return {"launched": False}
        by_inst = [[x for x, s in zip(d, span_steps[n]) if order[s] == k] for k in range(I)]
        return {"avg_us": sum(d) / len(d), "p10_us": percentile(d, 0.1),
                "p50_us": percentile(d, 0.5), "p90_us": percentile(d, 0.9),
                # instances in the order of config.instances (their work differs)
                "per_instance_avg_us": [sum(x) / len(x) if x else None for x in by_inst]}

    kernels = {n: stats(n) for n in SPANS}
    for n, unit, scale, peak in (("append_kernel", "GB/s", 1e9, HBM_PEAK_GBS),
                                 ("decode_kernel", "GB/s", 1e9, HBM_PEAK_GBS),
                                 ("chunk_kernel", "TFLOP/s", 1e12, MFMA_BF16_PEAK_TFS)):
        t = sum(durs[n]) * 1e-6
        v = sum(work[n]) / t / scale if t > 0 else None
        kernels[n][unit] = v
        kernels[n]["frac_of_peak"] = None if v is None else v / peak
        # the same rate at the median launch of each instance's launches
        kernels[n][unit + "_at_p50"] = (
            None if not durs[n] else
            percentile([w / d for w, d in zip(work[n], durs[n]) if d > 0], 0.5) * 1e6 / scale)
    # decode with its own merge counted (the pieces of a split row are not
    # attention output until merged)
    t_dm = (sum(durs["decode_kernel"]) + sum(durs["decode_merge"])) * 1e-6
    kernels["decode_kernel"]["frac_of_peak_with_decode_merge"] = (
        sum(work["decode_kernel"]) / t_dm / 1e9 / HBM_PEAK_GBS if t_dm > 0 else None)
    host_us = (sum(i.host_build_s for i in insts) / max(1, sum(i.host_builds for i in insts))
               * 1e6)
    res = {
        "value": tokens / elapsed,
        "ms_per_step": elapsed / steps * 1e3,
        "tokens_per_step": sorted({i.ds.num_tokens for i in insts}),
        "instances": [i.w.name for i in insts],
        "kernels": kernels,
        "gpu_step_us": sum(gpu_step) / len(gpu_step),
        # two markers back to back with no launch between: what every span
        # holds besides its kernel
        "empty_span_us": {"avg": sum(gap_us) / len(gap_us), "p50": percentile(gap_us, 0.5)},
        "metadata_upload_us": sum(copy_us) / len(copy_us),
        "host_build_us": host_us,
        "kernel_events": {"round_stride": stride, "sampled_steps": len(sampled),
                          "per_instance": [sum(1 for s in sampled if order[s] == k)
                                           for k in range(I)]},
        "work_per_step": {k: [i.work[k] for i in insts]
                          for k in ("decode_bytes", "chunk_flops", "append_bytes")},
    }
    res["workloads"] = ws
    del insts
    torch.cuda.empty_cache()
    return res


def measured_peaks(torch, build_lib):
    """What this machine sustains: a streaming read of 2 GiB, a streaming copy of
    2 GiB (bytes read + bytes written over time) and an MFMA-only loop of bf16
    32x32x16 chains at two workgroups per CU, each timed with HIP events over 5
    runs after 2 warm-up runs (libcpa_peaks.so)."""
    lib = ctypes.CDLL(build_lib.PEAKS_LIB)
    lib.cpa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_void_p]
    lib.cpa_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.cpa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    wgs, iters = 2 * 256, 4000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    rout = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")

    def timed(fn, reps=5):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    def copy():
        if lib.cpa_peak_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                             nbytes, stream) != 0:
            raise RuntimeError("peak copy launch failed")

    def read():
        if lib.cpa_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes,
                             ctypes.c_void_p(rout.data_ptr()), stream) != 0:
            raise RuntimeError("peak read launch failed")

    def mfma():
        if lib.cpa_peak_mfma(ctypes.c_void_p(out.data_ptr()), wgs, iters, stream) != 0:
            raise RuntimeError("peak MFMA launch failed")

    t_read = timed(read)
    t_copy = timed(copy)
    t_mfma = timed(mfma)
    del src, dst, out, rout
    torch.cuda.empty_cache()
    return {"hbm_read_GB/s": nbytes / t_read / 1e9,
            "hbm_copy_GB/s": 2 * nbytes / t_copy / 1e9,
            "mfma_bf16_TFLOP/s": wgs * 4 * iters * 8 * 32768 / t_mfma / 1e12,
            "method": "streaming non-temporal read of 2 GiB and copy of 2 GiB (read + write bytes), "
                      "one contiguous range per workgroup; MFMA-only loop on random bf16 operands "
                      "(8 operand sets rotated, 4 v_mfma_f32_32x32x16_bf16 chains per wave, 2 "
                      "workgroups of 4 waves per CU); HIP events, 5 runs after 2 warm-up"}


def cpu_baseline(workloads_list, seconds: float):
    """The fp64 oracle (as it stands) on the host cores, on a bounded sample of
    the same instances, round-robin until ``seconds`` of CPU work have run.
    Each sampled step runs the oracle's append of the whole step and its
    attention for every k-th packed token, k chosen so one step's sample is a
    few seconds of work; the attention time is scaled by the tokens left out,
    so the rate is whole steps per second of the oracle, extrapolated from the
    sample."""
    import numpy as np

    import oracle
    from chunked_prefill_mixed_amd import cpa
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max((i.get("num_threads", 1) for i in blas), default=1)
        blas_name = ",".join(sorted({f"{i.get('internal_api')}" for i in blas}))
    except Exception:  # pragma: no cover
        cores, blas_name = len(os.sched_getaffinity(0)), "unknown"
    t_app = t_att = spent = 0.0
    n_tok = n_sel = steps = 0
    k = 0
    while spent < seconds or steps == 0:
        w = workloads_list[k % len(workloads_list)]
        m = cpa.cpa_build_metadata(w.requests, token_budget=w.token_budget,
                                   long_prefill_cap=w.long_prefill_cap,
                                   num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                                   head_dim=w.head_dim)
        bt = w.block_table[m["order"]]
        T = m["num_tokens"]
        flops = step_work(m, w.num_q_heads, w.num_kv_heads, w.head_dim)["chunk_flops"]
        stride = max(1, int(math.ceil(flops / 30e9 / 3.0)))  # ~3 s at ~30 GFLOP/s fp64
        sel = np.arange(0, T, stride)
        t0 = time.perf_counter()
        kp, vp = oracle.append(w.k_pool, w.v_pool, w.k_new[:T], w.v_new[:T],
                               m["query_start_loc"], m["context_lens"], bt)
        t1 = time.perf_counter()
        oracle.attention(w.q[:T], kp, vp, m["query_start_loc"], m["context_lens"], bt,
                         w.num_kv_heads, w.scale, tokens=sel)
        t2 = time.perf_counter()
        spent += t2 - t0
        t_app += t1 - t0
        t_att += (t2 - t1) * T / sel.size
        n_tok += T
        n_sel += sel.size
        steps += 1
        k += 1
        del kp, vp
    return {"value": n_tok / (t_app + t_att), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{steps} step(s) of the same instances, round-robin, {spent:.1f} s of CPU "
                      f"work: the append of every "
                      f"token and the attention of {n_sel} of the {n_tok} packed tokens (every "
                      f"k-th token), the attention time scaled to all tokens; fp64 numpy "
                      f"({blas_name} BLAS)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--other-configs", default="2,3,4",
                    help="configurations run briefly after the headline and reported under "
                         "other_configs (comma list; empty for none)")
    ap.add_argument("--other-steps", type=int, default=24)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each instance's append + attention as one captured HIP graph on "
                         "the unsampled steps (the host metadata build and its copy still run "
                         "every step, outside the graph)")
    ap.add_argument("--kernel-event-stride", type=int, default=3,
                    help="record per-kernel HIP events on every n-th round of instances (each "
                         "instance's step of that round); the other steps carry no event")
    ap.add_argument("--kv-shard", type=int, default=1, choices=[1, 2, 4, 8],
                    help="time one GPU's share of each step split N ways by KV head (32/N query "
                         "heads on 8/N KV heads, the same rows and tokens); the default 1 is the "
                         "whole step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the attention step runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the path has no collectives or sharding.", file=sys.stderr)
        sys.exit(2)

    import torch
    from chunked_prefill_mixed_amd import build_lib, cpa, workloads
    from chunked_prefill_mixed_amd.step import DeviceStep

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (the HIP library has no CPU path)")
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 5}))
        return
    if not (os.path.exists(cpa.LIB_PATH) and os.path.exists(build_lib.PEAKS_LIB)):
        build_lib.build()
    cpa.load()

    K, W = args.steps, args.warmup
    head = run_config(args.config, K, W, args.kernel_event_stride, args.graph, torch, cpa,
                      workloads, DeviceStep, args.kv_shard)
    ws = head.pop("workloads")
    kernels = head["kernels"]
    # the dominant kernel of the step: the one with the largest time
    dominant = max(("decode_kernel", "chunk_kernel", "append_kernel"),
                   key=lambda n: kernels[n].get("avg_us", 0.0))
    if dominant == "chunk_kernel":
        ach = kernels[dominant]["TFLOP/s"]
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": ach,
                    "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s"}
    else:
        ach = kernels[dominant]["GB/s"]
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": ach, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s"}
    roofline["frac"] = ach / roofline["peak"]
    # the counter records are of the whole steps
    roofline["traffic"] = traffic_for(dominant, args.config) if args.kv_shard == 1 else None
    wk = {"chunk_kernel": "chunk_flops", "decode_kernel": "decode_bytes",
          "append_kernel": "append_bytes"}[dominant]
    roofline["algorithmic_per_launch"] = (sum(head["work_per_step"][wk])
                                          / len(head["work_per_step"][wk]))
    roofline["avg_launch_us"] = kernels[dominant]["avg_us"]

    others = {}
    for c in [int(x) for x in args.other_configs.split(",") if x.strip()]:
        if c == args.config:
            continue
        r = run_config(c, args.other_steps, 4, args.kernel_event_stride, False, torch, cpa,
                       workloads, DeviceStep, args.kv_shard)
        r.pop("workloads")
        others[config_key(c)] = {
            "value": r["value"], "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
            "tokens_per_step": r["tokens_per_step"],
            "kernels": {n: {k: v for k, v in d.items()} for n, d in r["kernels"].items()},
            "empty_span_us": r["empty_span_us"],
        }

    peaks = measured_peaks(torch, build_lib)
    for n, key, unit in (("append_kernel", "hbm_copy_GB/s", "GB/s"),
                         ("decode_kernel", "hbm_read_GB/s", "GB/s"),
                         ("chunk_kernel", "mfma_bf16_TFLOP/s", "TFLOP/s")):
        v = kernels[n].get(unit)
        kernels[n]["frac_of_measured"] = None if v is None else v / peaks[key]
    roofline["measured_peak"] = peaks[{"mfma": "mfma_bf16_TFLOP/s", "hbm": "hbm_read_GB/s"}
                                      [roofline["bound"]] if dominant != "append_kernel"
                                      else "hbm_copy_GB/s"]
    roofline["frac_of_measured"] = roofline["achieved"] / roofline["measured_peak"]

    config = {"workload": WORKLOAD_TEXT[args.config], "config": config_key(args.config),
              "tokens_per_step": head["tokens_per_step"], "instances": head["instances"]}
    if args.kv_shard != 1:
        config["workload"] += (f"; one GPU's share of a {args.kv_shard}-way split by KV head: "
                               f"Hq={32 // args.kv_shard} Hkv={8 // args.kv_shard}")
        config["kv_shard"] = args.kv_shard
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "kernels": kernels,
        "graph": bool(args.graph),
        "gpu_step_us": head["gpu_step_us"],
        "empty_span_us": head["empty_span_us"],
        "metadata_upload_us": head["metadata_upload_us"],
        "host_build_us": head["host_build_us"],
        "kernel_events": head["kernel_events"],
        "work_per_step": head["work_per_step"],
        "other_configs": others,
        "measured_peaks": peaks,
        "device": {"name": torch.cuda.get_device_name(0),
                   "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                   "hip": torch.version.hip, "torch": torch.__version__},
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host cores ...")
        result["cpu_baseline"] = cpu_baseline(ws, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
