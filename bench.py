#!/usr/bin/env python3
"""Mixed-batch attention throughput on one MI355X.

A step is one pass of the whole path over one packed batch: the host
decode-first budget split and work plan (cpa_build_metadata), one H2D copy of
the step metadata, the paged KV append (cpa_append_kv), then cpa_attention:
the split-KV decode kernel and the MFMA prefill-chunk kernel (one launch when
the chunk tiles fill a resident round) and one log-sum-exp merge launch for
the split pieces of both, all on one stream (``--two-streams`` runs the chunk
kernel on a second stream).
Inputs (q, new K/V, the paged KV pool) are resident in HBM before timing.

Default workload (Page-1 defaults of the chunked-prefill essay): 32 decode
rows with contexts uniform in [512, 4096] plus one 480-token chunk (budget
512) of an 8192-token prompt at prefix 0, 3840 and 7680; Hq=32, Hkv=8,
D=128, bf16, 16-token pages.  The three prefix instances have their own KV
pools and are rotated step by step, so no step finds its K/V in the 256 MB
last-level cache from the previous step.

Prints ONE JSON line on stdout.  Per-kernel durations come from HIP events
recorded on the launch stream around each launch inside the timed region, on
every eleventh timed step (``--kernel-event-stride``), which runs each plan
section as its own launch so each kernel has its own span; the other steps
make the one cpa_attention call and carry no events at all (each marker costs
a few microseconds of GPU time between two launches), and the step rate is
the wall clock over all timed steps.  ``host_build_us`` is the host time of
``cpa_build_metadata`` per step, which overlaps the GPU work of the step
before.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
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

KERNEL_SOURCES = {
    "decode_kernel": ["decode.hip", "decode_body.h", "device.h", "tiles.h"],
    "chunk_kernel": ["chunk.hip", "chunk_body.h", "device.h", "tiles.h"],
    "append_kernel": ["append.hip", "device.h", "tiles.h"],
    "merge_kernel": ["merge.hip", "device.h", "tiles.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "chunked_prefill_mixed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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
    def __init__(self, w, torch, cpa, DeviceStep, aux_stream=None):
        self.w = w
        self.aux_stream = aux_stream
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
        import numpy as np
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
        self._prepare_calls(torch, cpa)
        self.work = step_work(m, w.num_q_heads, w.num_kv_heads, w.head_dim)

    def build_host(self):
        st = self.lib.cpa_build_metadata(self.reqs, self.nreq, ctypes.byref(self.params), None, 0,
                                         0, ctypes.byref(self.meta))
        if st != 0:
            raise RuntimeError(f"cpa_build_metadata failed: {st}")

    def _prepare_calls(self, torch, cpa):
        ds, w = self.ds, self.w
        vp = ctypes.c_void_p
        P = lambda t: vp(t.data_ptr()) if t is not None else None
        self.stream = vp(torch.cuda.current_stream().cuda_stream)
        c = ds.counts
        plan_base = ds.plan.data_ptr()
        off = cpa.section_offsets(c)
        self.parts = []
        common_tail = (ds.num_seqs, ds.num_decodes, ds.num_tokens, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, 16, ctypes.c_float(w.scale), P(ds.out), None,
                       P(ds.workspace), ctypes.c_size_t(0 if ds.workspace is None
                                                        else ds.workspace.numel()),
                       self.stream)
        head = (P(ds.q), P(ds.k_cache), P(ds.v_cache), P(ds.block_table),
                int(ds.block_table.shape[1]), P(ds.query_start_loc), P(ds.seq_lens),
                P(ds.context_lens))
        zero = dict(num_decode_splits=0, num_decode_merges=0, num_chunk_tiles=0,
                    num_chunk_merges=0)
        # one launch per call, in the library's own order, so HIP events can
        # bracket each kernel (both merge sections are one launch)
        sections = [
            ("decode_kernel", ("num_decode_splits",), "decode_splits"),
            ("chunk_kernel", ("num_chunk_tiles",), "chunk_tiles"),
            ("merge_kernel", ("num_decode_merges", "num_chunk_merges"), "decode_merges"),
        ]
        for name, fields, sec in sections:
            counts = c.copy(**{**zero, **{f: getattr(c, f) for f in fields}})
            self.parts.append((name, counts, head + (vp(plan_base + 4 * off[sec]),
                                                     ctypes.byref(counts)) + common_tail))
        # the whole plan in one call, as a caller runs a step
        self.full_args = head + (vp(plan_base), ctypes.byref(c)) + common_tail
        self.torch = torch
        self.graph = None
        self.aux_parts = {}
        if self.aux_stream is not None:
            aux_tail = common_tail[:-1] + (vp(self.aux_stream.cuda_stream),)
            for name, counts, args in self.parts:
                self.aux_parts[name] = args[:len(head) + 2] + aux_tail
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

    def step(self, events, aux=None, per_kernel=True):
        """One full step.  events: 9 torch events.  With ``aux`` (a second
        stream) the chunk kernel runs on it, concurrently with the decode
        kernel on the main stream; both wait for the append, and the merge
        follows both on the main stream.  Without ``per_kernel`` only the
        step's first and last events are recorded (no markers between the
        launches), and the step is one cpa_attention call, or the replay of
        the captured graph with ``--graph``."""
        self.copy_done.synchronize()  # the previous copy out of the pinned buffer is done
        t0 = time.perf_counter()
        self.build_host()
        self.host_build_s += time.perf_counter() - t0
        self.host_builds += 1
        main = self.torch.cuda.current_stream()
        if per_kernel:
            events[8].record(main)  # before the metadata copy
        self.dev.copy_(self.pinned, non_blocking=True)
        self.copy_done.record()
        lib = self.lib
        parts = dict((name, args) for name, _, args in self.parts)
        st = 0
        if per_kernel:
            events[0].record(main)
        if self.graph is None or per_kernel or aux is not None:
            st |= lib.cpa_append_kv(*self.append_args)
        if aux is None and not per_kernel:
            if self.graph is not None:
                self.graph.replay()
            else:
                st |= lib.cpa_attention(*self.full_args)
            if st != 0:
                raise RuntimeError(f"launch failed with status {st}")
            return
        events[1].record(main)
        if aux is None:
            st |= lib.cpa_attention(*parts["decode_kernel"])
            events[2].record(main)
            events[5].record(main)
            st |= lib.cpa_attention(*parts["chunk_kernel"])
            events[6].record(main)
            events[3].record(main)
            st |= lib.cpa_attention(*parts["merge_kernel"])
            events[4].record(main)
            events[7].record(main)
        else:
            aux.wait_event(events[1])
            events[5].record(aux)
            st |= lib.cpa_attention(*self.aux_parts["chunk_kernel"])
            events[6].record(aux)
            st |= lib.cpa_attention(*parts["decode_kernel"])
            events[2].record(main)
            main.wait_event(events[6])
            events[3].record(main)
            st |= lib.cpa_attention(*parts["merge_kernel"])
            events[4].record(main)
            events[7].record(main)
        if st != 0:
            raise RuntimeError(f"launch failed with status {st}")


def traffic_for(kernel: str, config: int):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counter runs, if they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config_key(config)}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def config_key(config: int) -> str:
    from chunked_prefill_mixed_amd import workloads
    return workloads.CONFIG_NAMES[config]


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
    """The fp64 oracle (as it stands) on the host cores, whole steps of the
    same instances, round-robin until ``seconds`` of CPU work have run."""
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
    done_tokens, done_steps, t_total = 0, 0, 0.0
    k = 0
    while t_total < seconds or done_steps == 0:
        w = workloads_list[k % len(workloads_list)]
        m = cpa.cpa_build_metadata(w.requests, token_budget=w.token_budget,
                                   long_prefill_cap=w.long_prefill_cap,
                                   num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                                   head_dim=w.head_dim)
        bt = w.block_table[m["order"]]
        T = m["num_tokens"]
        t0 = time.perf_counter()
        kp, vp = oracle.append(w.k_pool, w.v_pool, w.k_new[:T], w.v_new[:T],
                               m["query_start_loc"], m["context_lens"], bt)
        oracle.attention(w.q[:T], kp, vp, m["query_start_loc"], m["context_lens"], bt,
                         w.num_kv_heads, w.scale)
        t_total += time.perf_counter() - t0
        done_tokens += T
        done_steps += 1
        k += 1
        del kp, vp
    return {"value": done_tokens / t_total, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done_steps} whole steps (append + attention of every token) of the same "
                      f"instances, round-robin, {t_total:.1f} s of fp64 numpy ({blas_name} BLAS)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=90)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-streams", action="store_true",
                    help="run the chunk kernel on a second stream, concurrently with the "
                         "decode kernel; the merge follows both (default: one stream, so each "
                         "kernel's HIP-event time is its own)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each instance's append + attention as one captured HIP graph on "
                         "the unsampled steps (the host metadata build and its copy still run "
                         "every step, outside the graph)")
    ap.add_argument("--kernel-event-stride", type=int, default=11,
                    help="record the per-kernel HIP events on every n-th timed step only (the "
                         "others carry just the step's start and end events, since a marker "
                         "between launches keeps a kernel from starting while the previous one "
                         "drains); per-kernel durations average the sampled steps.  Keep it "
                         "coprime to the number of rotated instances so each is sampled")
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

    t_setup = time.perf_counter()
    ws = [workloads.make_workload(args.config, i)
          for i in range(workloads.num_instances(args.config))]
    aux = torch.cuda.Stream() if args.two_streams else None  # default priority
    insts = [Instance(w, torch, cpa, DeviceStep, aux) for w in ws]
    log(f"setup {time.perf_counter() - t_setup:.1f}s: {len(insts)} instance(s), "
        f"{[i.ds.num_tokens for i in insts]} tokens/step")

    K, W = args.steps, args.warmup
    NEV = 9
    ev_w = [torch.cuda.Event(enable_timing=True) for _ in range(NEV)]
    for s in range(W):
        insts[s % len(insts)].step(ev_w, aux)
    torch.cuda.synchronize()
    if args.graph and aux is None:
        for inst in insts:
            inst.capture()
        for s in range(len(insts)):  # one replay each before timing
            insts[s].step(ev_w, None, per_kernel=False)
        torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(NEV)] for _ in range(K)]
    order = [(W + s) % len(insts) for s in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    stride = max(1, args.kernel_event_stride) if aux is None else 1
    sampled = [s for s in range(K) if s % stride == 0]
    for s in range(K):
        insts[order[s]].step(events[s], aux, per_kernel=(s % stride == 0))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # (kernel, start event, end event) on the stream the kernel ran on
    spans = {"append_kernel": (0, 1), "decode_kernel": (1, 2), "chunk_kernel": (5, 6),
             "merge_kernel": (3, 4)}
    names = list(spans)
    times = {n: 0.0 for n in names}
    gpu_step = 0.0
    work = {"decode_bytes": 0, "chunk_flops": 0, "append_bytes": 0, "tokens": 0}
    tokens = 0
    copy_us = 0.0
    for s in range(K):
        tokens += insts[order[s]].work["tokens"]
    for s in sampled:
        gpu_step += events[s][0].elapsed_time(events[s][7]) * 1e-3
        copy_us += events[s][8].elapsed_time(events[s][0]) * 1e3
    for s in sampled:  # per-kernel durations and work over the sampled steps
        ev = events[s]
        for n, (a, b) in spans.items():
            times[n] += ev[a].elapsed_time(ev[b]) * 1e-3
        wk = insts[order[s]].work
        for key in work:
            work[key] += wk[key]
    NS = len(sampled)
    value = tokens / elapsed

    def rate(n, amount, scale):
        return amount / times[n] / scale if times[n] > 0 else None

    kernels = {
        "append_kernel": {"avg_us": times["append_kernel"] / NS * 1e6,
                          "GB/s": rate("append_kernel", work["append_bytes"], 1e9)},
        "decode_kernel": {"avg_us": times["decode_kernel"] / NS * 1e6,
                          "GB/s": rate("decode_kernel", work["decode_bytes"], 1e9)},
        "merge_kernel": {"avg_us": times["merge_kernel"] / NS * 1e6},
        "chunk_kernel": {"avg_us": times["chunk_kernel"] / NS * 1e6,
                         "TFLOP/s": rate("chunk_kernel", work["chunk_flops"], 1e12)},
    }
    for n, peak, unit in (("append_kernel", HBM_PEAK_GBS, "GB/s"),
                          ("decode_kernel", HBM_PEAK_GBS, "GB/s"),
                          ("chunk_kernel", MFMA_BF16_PEAK_TFS, "TFLOP/s")):
        v = kernels[n].get(unit)
        kernels[n]["frac_of_peak"] = None if v is None else v / peak

    # the decode rate with the whole merge launch (decode and chunk merges
    # together) added to the decode kernel's time
    t_dm = times["decode_kernel"] + times["merge_kernel"]
    kernels["decode_kernel"]["frac_of_peak_with_merge_launch"] = (
        work["decode_bytes"] / t_dm / 1e9 / HBM_PEAK_GBS if t_dm > 0 else None)

    dominant = max(("decode_kernel", "chunk_kernel", "append_kernel"), key=lambda n: times[n])
    if dominant == "chunk_kernel":
        ach = kernels["chunk_kernel"]["TFLOP/s"]
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": ach,
                    "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFS}
    else:
        ach = kernels[dominant]["GB/s"]
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": ach, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": ach / HBM_PEAK_GBS}
    roofline["traffic"] = traffic_for(dominant, args.config)
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

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config], "config": config_key(args.config),
                   "tokens_per_step": sorted({i.ds.num_tokens for i in insts}),
                   "instances": len(insts)},
        "roofline": roofline,
        "kernels": kernels,
        "streams": ("decode and chunk on two streams, concurrently" if args.two_streams
                    else "one stream"),
        "graph": bool(args.graph and aux is None),
        # GPU time of a sampled step (append through merge, with the markers
        # between its launches) and of its metadata upload before it
        "gpu_step_us": gpu_step / NS * 1e6,
        "metadata_upload_us": copy_us / NS,
        # host wall time of cpa_build_metadata (budget split + work plan) per
        # step, every step run; it overlaps the GPU work of the step before
        "host_build_us": (sum(i.host_build_s for i in insts)
                          / max(1, sum(i.host_builds for i in insts)) * 1e6),
        "measured_peaks": peaks,
        "device": {"name": torch.cuda.get_device_name(0),
                   "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                   "hip": torch.version.hip, "torch": torch.__version__},
        "kernel_events": {"stride": stride, "sampled_steps": NS},
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host cores ...")
        result["cpu_baseline"] = cpu_baseline(ws, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
