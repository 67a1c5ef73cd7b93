"""Multi-step replay of a long prompt arriving among streaming requests, on
one MI355X, attention part only.

Three scenarios from the pages, each run over its own knob:

* ``budget`` -- "Chunked Prefill" (deepconcepts.dev), "Why a chunk can be
  nearly free" and "The budget points in two directions": 32 running decode
  streams and one 8192-token prompt that arrives at step 0, swept over the
  token budget B.  Decode-first gives every stream one token per step and the
  prompt B - 32 tokens per step (the page's 224-, 480- and 4064-token chunks
  at budgets 256, 512 and 4096; one pass at 8224).
* ``chunk`` -- "Chunked prefill" test on an M5 Max (the page's table of chunk
  size against time to first token and worst streaming pause): three
  streaming requests and one 8000-token prompt, swept over the chunk size C
  (budget 3 + C, so the prompt gets C tokens a step; 8003 = unchunked).

* ``knee`` -- one step, not a replay: the budget scenario's 32 streams plus
  one chunk of C tokens after a cached prefix (0, 1024, 4096), C swept from
  16 to 4096.  It gives the attention-only analogs of two of the pages'
  figures: the memory-to-compute knee ("How Chunked Prefill Stops Decode
  Starvation", "Why 512 is the sweet spot": on the A100 a kernel turns from
  memory- to compute-bound at a few hundred tokens) and the
  free-ride capacity ("Chunked Prefill", "Why a chunk can be nearly free":
  the prefill tokens whose compute fits in the time a decode pass spends
  reading memory).  ``knee_figures`` states how each is derived.

For every knob value the whole sequence of steps runs through the library
(cpa_build_metadata, cpa_append_kv, cpa_attention on one stream; the
streams' contexts grow by one token per step, the prompt's by its chunk) and
each step's append + attention is timed with HIP events.  Attention only: no
model layers, so the figures are the attention part of the pages' pass
times, not their whole passes.

Reported per knob value: chunk tokens, steps to finish the prompt, mean and
max step time, the decode-only step time at the same contexts (the streams
alone), and the replay's figures: time to first token of the prompt (the sum
of its steps: its first token comes from the last chunk's step), the worst
gap between two tokens of a stream while the prompt is prefilled (the longest
step), the stall above the undisturbed gap (longest step minus the
decode-only step), the tokens the streams receive meanwhile (streams x
steps) and the time to first token against the unchunked run.

    python -m chunked_prefill_mixed_amd.sweep [--scenario budget|chunk|knee]
                                              [--values ...] [--out FILE]

Inputs are seeded and synthetic (workloads.py recipe): stream contexts
uniform in [512, 4096] (budget scenario) or [128, 1024] (chunk scenario),
Hq=32, Hkv=8, D=128, bf16, 16-token pages.
"""

from __future__ import annotations

import argparse
import json
import math
import sys
from dataclasses import dataclass

import numpy as np

from . import cpa, workloads
from .step import caches_from_pools

HQ, HKV, D = 32, 8, 128
NUM_STREAMS = 32   # budget scenario
PROMPT = 8192


@dataclass(frozen=True)
class Scenario:
    name: str
    streams: int
    prompt: int
    ctx_lo: int
    ctx_hi: int
    seed: int
    values: tuple    # knob values: budgets, or chunk sizes
    knob: str        # "budget" or "chunk"

    def budget(self, value: int) -> int:
        return value if self.knob == "budget" else self.streams + value


SCENARIOS = {
    "budget": Scenario("budget", NUM_STREAMS, PROMPT, 512, 4096, 1002,
                       (64, 128, 256, 512, 1024, 2048, 4096, NUM_STREAMS + PROMPT), "budget"),
    "chunk": Scenario("chunk", 3, 8000, 128, 1024, 1003, (256, 512, 1024, 2048, 8000), "chunk"),
}
DEFAULT_BUDGETS = SCENARIOS["budget"].values


def stream_contexts(seed: int = 1002, n: int = NUM_STREAMS, lo: int = 512, hi: int = 4096) -> np.ndarray:
    """Initial cached lengths of the streams: uniform in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99]).spawn(1)[0]))
    return rng.integers(lo, hi, size=n, endpoint=True)


def _requests(contexts, k, done, prompt):
    n = len(contexts)
    reqs = [workloads.Req(i, int(c) + k, int(c) + k + 1, True) for i, c in enumerate(contexts)]
    reqs.append(workloads.Req(n, done, prompt, False))
    return reqs


def schedule(budget: int, contexts, prompt: int = PROMPT) -> list:
    """The steps of one run at this budget, host only: for each step the
    request list (queue order: streams, then the prompt) and the metadata
    cpa_build_metadata returns for it."""
    n = len(contexts)
    steps = []
    done = 0
    k = 0
    while done < prompt:
        reqs = _requests(contexts, k, done, prompt)
        meta = cpa.cpa_build_metadata(reqs, token_budget=budget, long_prefill_cap=0,
                                      num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)
        if meta["num_seqs"] <= n:  # budget leaves nothing for the prompt
            raise ValueError(f"budget {budget} cannot finish the prompt")
        steps.append((reqs, meta))
        done += int(meta["num_scheduled"][n])
        k += 1
    return steps


def _decode_only(contexts, k):
    reqs = [workloads.Req(i, int(c) + k, int(c) + k + 1, True) for i, c in enumerate(contexts)]
    meta = cpa.cpa_build_metadata(reqs, token_budget=len(contexts), long_prefill_cap=0,
                                  num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)
    return reqs, meta


def replay_figures(times, decode_only, streams, ttft_unchunked=None) -> dict:
    """The replay's figures from one run's step times (seconds) and the
    decode-only step time at the same contexts (seconds)."""
    t = np.asarray(times, dtype=np.float64)
    ttft = float(t.sum())
    fig = {"steps": int(t.size), "mean_step_us": float(t.mean() * 1e6),
           "max_step_us": float(t.max() * 1e6), "decode_only_step_us": float(decode_only * 1e6),
           "ttft_ms": ttft * 1e3, "worst_gap_us": float(t.max() * 1e6),
           "stall_us": float((t.max() - decode_only) * 1e6),
           "stream_tokens_during_prefill": int(streams * t.size),
           "mean_extra_us": float((t.mean() - decode_only) * 1e6)}
    if ttft_unchunked:
        fig["ttft_vs_unchunked"] = ttft / ttft_unchunked
    return fig


class _Gpu:
    """The run's pool and packed inputs in HBM, and one timed step."""

    def __init__(self, scn: Scenario, contexts, max_steps: int, max_budget: int,
                 prompt_cached: int = 0):
        import torch
        self.torch = torch
        n = len(contexts)
        reach = [int(c) + max_steps + 1 for c in contexts] + [scn.prompt]
        # the prompt's first prompt_cached positions hold values in the pool
        reqs = _requests(contexts, 0, prompt_cached, scn.prompt)
        st = workloads._streams(scn.seed, 99)
        w = workloads.build(f"replay_{scn.name}", scn.seed, 99, num_q_heads=HQ, num_kv_heads=HKV,
                            head_dim=D, token_budget=max_budget, long_prefill_cap=0,
                            requests=reqs, reach=reach, pool_blocks=None, streams=st)
        self.w = w
        self.n = n
        dev = "cuda"
        bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)
        self.k_cache0, self.v_cache0 = caches_from_pools(w.k_pool, w.v_pool, dev)
        self.k_cache = self.k_cache0.clone()
        self.v_cache = self.v_cache0.clone()
        self.q = bits(w.q)
        self.k_new = bits(w.k_new)
        self.v_new = bits(w.v_new)
        self.out = torch.empty((max_budget, HQ, D), dtype=torch.bfloat16, device=dev)
        self.block_table = torch.from_numpy(w.block_table.astype(np.int32)).to(dev)

    def reset(self):
        self.k_cache.copy_(self.k_cache0)
        self.v_cache.copy_(self.v_cache0)

    def step(self, meta) -> float:
        """Append + attention of one step; returns its GPU time in seconds."""
        torch = self.torch
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")
        T = meta["num_tokens"]
        bt = i32(self.w.block_table[meta["order"]])
        qsl, seq, ctx = i32(meta["query_start_loc"]), i32(meta["seq_lens"]), i32(meta["context_lens"])
        plan = i32(meta["plan"] if meta["plan"].size else np.zeros(1, dtype=np.int32))
        ws_bytes = cpa.cpa_workspace_size(meta["counts"], HQ, HKV, D)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda") if ws_bytes else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cpa.cpa_append_kv(self.k_new[:T], self.v_new[:T], qsl, ctx, bt, self.k_cache,
                          self.v_cache, num_seqs=meta["num_seqs"], num_tokens=T)
        cpa.cpa_attention(self.q[:T], self.k_cache, self.v_cache, bt, qsl, seq, ctx, plan,
                          meta["counts"], num_seqs=meta["num_seqs"],
                          num_decodes=meta["num_decodes"], num_tokens=T,
                          softmax_scale=self.w.scale, out=self.out[:T], workspace=ws)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3


def run(scenario: str = "budget", values=None, out_path=None) -> list:
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("the replay needs a GPU (the HIP library has no CPU path)")
    cpa.load()
    scn = SCENARIOS[scenario]
    values = sorted(values or scn.values)
    contexts = stream_contexts(scn.seed, scn.streams, scn.ctx_lo, scn.ctx_hi)
    plans = {v: schedule(scn.budget(v), contexts, scn.prompt) for v in values}
    max_steps = max(len(p) for p in plans.values())
    gpu = _Gpu(scn, contexts, max_steps, max(scn.budget(v) for v in values))
    n = scn.streams
    # warm-up: the first steps of every run and a decode-only step, so each
    # kernel the runs launch is loaded before a timed step; then reset the pool
    for v in values:
        for _, meta in plans[v][:3]:
            gpu.step(meta)
    gpu.step(_decode_only(contexts, 0)[1])
    runs = {}
    for v in values:
        gpu.reset()
        times, chunks = [], []
        for _, meta in plans[v]:
            times.append(gpu.step(meta))
            chunks.append(int(meta["num_scheduled"][n]))
        # decode-only steps at the first, middle and last contexts of the run
        # (own pool copy, so the run's cache contents are not disturbed)
        saved = gpu.k_cache.clone(), gpu.v_cache.clone()
        dec = [gpu.step(_decode_only(contexts, k)[1])
               for k in sorted({0, len(times) // 2, len(times) - 1})]
        gpu.k_cache.copy_(saved[0])
        gpu.v_cache.copy_(saved[1])
        runs[v] = (times, chunks, float(np.mean(dec)))
    unchunked = max(values, key=lambda v: scn.budget(v))
    ttft_unchunked = float(np.sum(runs[unchunked][0])) if len(plans[unchunked]) == 1 else None
    rows = []
    for v in values:
        times, chunks, d = runs[v]
        row = {"scenario": scn.name, scn.knob: v, "budget": scn.budget(v),
               "chunk_tokens": chunks[0]}
        row.update(replay_figures(times, d, n, ttft_unchunked))
        row["prompt_tokens_per_s"] = scn.prompt / (row["ttft_ms"] * 1e-3)
        row["stream_tokens_per_s"] = n / (row["mean_step_us"] * 1e-6)
        rows.append(row)
        print(json.dumps(row), flush=True)
    head = (f"{scn.knob:>6} chunk  steps  mean_us   max_us  decode_only_us  stall_us  ttft_ms"
            "  vs_unchunked  stream_tokens")
    lines = [f"scenario {scn.name}: {n} streams (contexts U[{scn.ctx_lo}, {scn.ctx_hi}]) + a "
             f"{scn.prompt}-token prompt; Hq={HQ} Hkv={HKV} D={D} bf16; append + attention per step",
             head]
    for r in rows:
        vs = f"{r['ttft_vs_unchunked']:12.2f}x" if "ttft_vs_unchunked" in r else f"{'-':>13}"
        lines.append(f"{r[scn.knob]:6d} {r['chunk_tokens']:5d} {r['steps']:6d} "
                     f"{r['mean_step_us']:8.1f} {r['max_step_us']:8.1f} "
                     f"{r['decode_only_step_us']:15.1f} {r['stall_us']:9.1f} {r['ttft_ms']:8.2f} "
                     f"{vs} {r['stream_tokens_during_prefill']:14d}")
    text = "\n".join(lines)
    print(text, file=sys.stderr)
    if out_path:
        with open(out_path, "w") as f:
            f.write(text + "\n")
    return rows


# ---------------------------------------------------------------------------
# Knee and free-ride figures: one step of 32 streams plus one chunk of C
# tokens at a fixed prefix, swept over C.
# ---------------------------------------------------------------------------

KNEE_SIZES = (16, 32, 64, 128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096)
KNEE_PREFIXES = (0, 1024, 4096)
HBM_PEAK = 8.0e12        # B/s, MI355X
MFMA_BF16_PEAK = 2.5e15  # dense bf16 FLOP/s, MI355X
FREE_RIDE_SLACK = 0.10   # "free": the step grows by at most this fraction


def chunk_flops(c: int, prefix: int, hq: int = HQ, d: int = D) -> float:
    """Attention flops of a chunk of c queries after `prefix` cached tokens:
    query j sees prefix + j + 1 keys, 2 d flops each for QK^T and for PV."""
    return 4.0 * d * hq * (c * prefix + c * (c + 1) / 2)


def decode_kv_bytes(contexts, hkv: int = HKV, d: int = D) -> float:
    """K and V bytes the decode rows read: (context + 1) keys and values each."""
    return float(sum((int(c) + 1) * hkv * d * 2 * 2 for c in contexts))


def tokens_for_flops(flops: float, prefix: int, hq: int = HQ, d: int = D) -> float:
    """The chunk size c (real) whose chunk_flops(c, prefix) equals flops."""
    a = 4.0 * d * hq
    # a (c prefix + c (c + 1) / 2) = flops  ->  c^2 / 2 + c (prefix + 1/2) - flops / a = 0
    b = prefix + 0.5
    return -b + math.sqrt(b * b + 2.0 * flops / a)


def knee_figures(sizes, step_s, decode_s, prefix: int, decode_bytes: float,
                 fit_from: int = 1024) -> dict:
    """Figures of one prefix's sweep.

    step_s[i]: time of the mixed step with a sizes[i]-token chunk; decode_s:
    the decode-only step at the same contexts.  The chunk's part of the step is
    x = step - decode.  Above fit_from tokens x is fitted as a + F / R (F the
    chunk's flops): a is the chunk's fixed cost per step, R its compute rate.
    The knee is the chunk size where the fitted compute time F / R equals a:
    below it the step is dominated by fixed costs, above it it grows linearly
    with the chunk's work.  Free ride, attention only (the pages' free-token
    estimate with the decode's KV read in place of the weights and the chunk's
    attention flops in place of 2 x params per token): the chunk tokens whose
    flops fit in the decode's HBM time decode_bytes / 8 TB/s at the bf16 MFMA
    peak, the same with the measured rate R and the measured decode-only step,
    and, as run (decode and chunk back to back), the largest chunk that keeps
    the step within FREE_RIDE_SLACK of the decode-only step."""
    sizes = np.asarray(sizes, dtype=np.int64)
    x = np.asarray(step_s, dtype=np.float64) - decode_s
    flops = np.array([chunk_flops(int(c), prefix) for c in sizes])
    sel = sizes >= fit_from
    if sel.sum() < 2:
        raise ValueError("need two chunk sizes at or above fit_from")
    slope, a = np.polyfit(flops[sel], x[sel], 1)
    rate = 1.0 / slope if slope > 0 else float("nan")  # no rate if time does not grow
    t_mem = decode_bytes / HBM_PEAK
    free_peak = tokens_for_flops(t_mem * MFMA_BF16_PEAK, prefix)
    if rate > 0:
        knee = tokens_for_flops(max(a, 0.0) * rate, prefix)
        free_rate = tokens_for_flops(decode_s * rate, prefix)
    else:
        knee = free_rate = float("nan")
    ok = sizes[np.asarray(step_s) <= (1.0 + FREE_RIDE_SLACK) * decode_s]
    return {"prefix": prefix, "fixed_us": a * 1e6, "rate_tflops": rate * 1e-12,
            "knee_tokens": knee, "decode_hbm_us": t_mem * 1e6,
            "free_ride_peak_tokens": free_peak, "free_ride_measured_rate_tokens": free_rate,
            "free_ride_as_run_tokens": int(ok.max()) if ok.size else 0}


def run_knee(sizes=KNEE_SIZES, prefixes=KNEE_PREFIXES, reps: int = 15, out_path=None) -> list:
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("the knee sweep needs a GPU (the HIP library has no CPU path)")
    cpa.load()
    sizes = sorted(sizes)
    prompt = max(prefixes) + max(sizes)
    scn = Scenario("knee", NUM_STREAMS, prompt, 512, 4096, 1004, tuple(sizes), "chunk")
    contexts = stream_contexts(scn.seed, scn.streams, scn.ctx_lo, scn.ctx_hi)
    gpu = _Gpu(scn, contexts, 1, NUM_STREAMS + max(sizes), prompt_cached=max(prefixes))
    n = scn.streams

    def meta_for(prefix, c):
        reqs = _requests(contexts, 0, prefix, prefix + c)
        return cpa.cpa_build_metadata(reqs, token_budget=n + c, long_prefill_cap=0,
                                      num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)

    def timed(meta):
        # the same step again: the append rewrites the same slots with the same bits
        for _ in range(3):
            gpu.step(meta)
        return float(np.median([gpu.step(meta) for _ in range(reps)]))

    dec = timed(_decode_only(contexts, 0)[1])
    dbytes = decode_kv_bytes(contexts)
    rows, figs = [], []
    for p in prefixes:
        times = [timed(meta_for(p, c)) for c in sizes]
        for c, t in zip(sizes, times):
            x = t - dec
            row = {"scenario": "knee", "prefix": p, "chunk_tokens": c, "step_us": t * 1e6,
                   "decode_only_us": dec * 1e6, "chunk_part_us": x * 1e6,
                   "chunk_gflop": chunk_flops(c, p) * 1e-9,
                   "chunk_part_tflops": chunk_flops(c, p) / x * 1e-12 if x > 0 else None}
            rows.append(row)
            print(json.dumps(row), flush=True)
        fig = knee_figures(sizes, times, dec, p, dbytes)
        figs.append(fig)
        print(json.dumps(fig), flush=True)
    lines = [f"scenario knee: {n} streams (contexts U[512, 4096], decode K/V read "
             f"{dbytes / 1e6:.1f} MB) + one chunk of C tokens after a cached prefix; Hq={HQ} "
             f"Hkv={HKV} D={D} bf16; append + attention per step, median of {reps}",
             f"decode-only step {dec * 1e6:.1f} us",
             "prefix  chunk   step_us  chunk_part_us  chunk_GFLOP  chunk_part_TFLOP/s"]
    for r in rows:
        tf = f"{r['chunk_part_tflops']:18.1f}" if r["chunk_part_tflops"] else f"{'-':>18}"
        lines.append(f"{r['prefix']:6d} {r['chunk_tokens']:6d} {r['step_us']:9.1f} "
                     f"{r['chunk_part_us']:14.1f} {r['chunk_gflop']:12.2f} {tf}")
    lines.append("")
    lines.append("prefix  fixed_us  rate_TFLOP/s  knee_tokens  decode_HBM_us  "
                 "free_ride@peak  free_ride@rate  free_ride_as_run(+10%)")
    for f in figs:
        lines.append(f"{f['prefix']:6d} {f['fixed_us']:9.1f} {f['rate_tflops']:13.1f} "
                     f"{f['knee_tokens']:12.0f} {f['decode_hbm_us']:14.1f} "
                     f"{f['free_ride_peak_tokens']:15.0f} {f['free_ride_measured_rate_tokens']:15.0f} "
                     f"{f['free_ride_as_run_tokens']:23d}")
    text = "\n".join(lines)
    print(text, file=sys.stderr)
    if out_path:
        with open(out_path, "w") as fh:
            fh.write(text + "\n")
    return rows + figs


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--scenario", choices=sorted(SCENARIOS) + ["knee"], default="budget")
    ap.add_argument("--values", type=int, nargs="+", default=None,
                    help="budgets (budget scenario) or chunk sizes (chunk scenario)")
    ap.add_argument("--budgets", type=int, nargs="+", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--out", default=None, help="also write the table to this file")
    args = ap.parse_args()
    if args.scenario == "knee":
        run_knee(args.values or KNEE_SIZES, out_path=args.out)
    else:
        run(args.scenario, args.values or args.budgets, args.out)


if __name__ == "__main__":
    main()
