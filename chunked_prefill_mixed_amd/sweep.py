"""Token-budget sweep of the attention step on one MI355X.

The scenario of "Chunked Prefill" (deepconcepts.dev), "Why a chunk can be
nearly free" and "The budget points in two directions": 32 running decode
streams and one 8192-token prompt that arrives at step 0.  With token budget
B the decode-first split gives every stream one token per step and the prompt
B - 32 tokens per step until it is prefilled (the pages' 224-, 480- and
4064-token chunks at budgets 256, 512 and 4096).  For each budget this runs
the whole sequence of steps through the library (cpa_build_metadata,
cpa_append_kv, cpa_attention on one stream; the streams' contexts grow by one
token per step, the prompt's by its chunk) and times each step's append +
attention with HIP events.  Attention only: no model layers, so the numbers
are the attention part of the pages' pass times, not their whole passes.

Reported per budget: chunk tokens per step, steps to finish the prompt, mean
and max step time, the decode-only step time at the same contexts (the same
32 streams with no prompt), the mean extra time a chunk adds to a step, the
prompt's prefill time (sum of its steps) and the rate at which the streams
and the prompt advance.

    python -m chunked_prefill_mixed_amd.sweep [--budgets 64 128 ...] [--out FILE]

Inputs are seeded and synthetic (workloads.py recipe): contexts uniform in
[512, 4096], Hq=32, Hkv=8, D=128, bf16, 16-token pages.
"""

from __future__ import annotations

import argparse
import json
import math
import sys

import numpy as np

from . import cpa, workloads

NUM_STREAMS = 32
PROMPT = 8192
HQ, HKV, D = 32, 8, 128
DEFAULT_BUDGETS = (64, 128, 256, 512, 1024, 2048, 4096, NUM_STREAMS + PROMPT)


def stream_contexts(seed: int = 1002) -> np.ndarray:
    """Initial cached lengths of the 32 streams: uniform in [512, 4096]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99]).spawn(1)[0]))
    return rng.integers(512, 4096, size=NUM_STREAMS, endpoint=True)


def schedule(budget: int, contexts) -> list:
    """The steps of one run at this budget, host only: for each step the
    request list (queue order: streams, then the prompt) and the metadata
    cpa_build_metadata returns for it."""
    steps = []
    done = 0
    k = 0
    while done < PROMPT:
        reqs = [workloads.Req(i, int(c) + k, int(c) + k + 1, True) for i, c in enumerate(contexts)]
        reqs.append(workloads.Req(NUM_STREAMS, done, PROMPT, False))
        meta = cpa.cpa_build_metadata(reqs, token_budget=budget, long_prefill_cap=0,
                                      num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)
        if meta["num_seqs"] <= NUM_STREAMS:  # budget leaves nothing for the prompt
            raise ValueError(f"budget {budget} cannot finish the prompt")
        steps.append((reqs, meta))
        done += int(meta["num_scheduled"][NUM_STREAMS])
        k += 1
    return steps


def _decode_only(contexts, k):
    reqs = [workloads.Req(i, int(c) + k, int(c) + k + 1, True) for i, c in enumerate(contexts)]
    meta = cpa.cpa_build_metadata(reqs, token_budget=NUM_STREAMS, long_prefill_cap=0,
                                  num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)
    return reqs, meta


class _Gpu:
    """The run's pool and packed inputs in HBM, and one timed step."""

    def __init__(self, contexts, max_steps: int, max_budget: int):
        import torch
        self.torch = torch
        reach = [int(c) + max_steps + 1 for c in contexts] + [PROMPT]
        reqs = [workloads.Req(i, int(c), int(c) + 1, True) for i, c in enumerate(contexts)]
        reqs.append(workloads.Req(NUM_STREAMS, 0, PROMPT, False))
        st = workloads._streams(1002, 99)
        w = workloads.build("budget_sweep", 1002, 99, num_q_heads=HQ, num_kv_heads=HKV,
                            head_dim=D, token_budget=max_budget, long_prefill_cap=0,
                            requests=reqs, reach=reach, pool_blocks=None, streams=st)
        self.w = w
        dev = "cuda"
        bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)
        self.k_cache0 = bits(w.k_pool)
        self.v_cache0 = bits(w.v_pool)
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


def run(budgets, out_path=None) -> list:
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("the sweep needs a GPU (the HIP library has no CPU path)")
    cpa.load()
    contexts = stream_contexts()
    plans = {b: schedule(b, contexts) for b in budgets}
    max_steps = max(len(p) for p in plans.values())
    gpu = _Gpu(contexts, max_steps, max(budgets))
    # warm-up: a few steps of the first budget, then reset the pool
    for _, meta in plans[budgets[0]][:3]:
        gpu.step(meta)
    rows = []
    for b in budgets:
        gpu.reset()
        times, decode_only, chunks = [], [], []
        for k, (_, meta) in enumerate(plans[b]):
            times.append(gpu.step(meta))
            chunks.append(int(meta["num_scheduled"][NUM_STREAMS]))
        # decode-only steps at the first, middle and last contexts of the run
        # (own pool copy, so the run's cache contents are not disturbed)
        saved = gpu.k_cache.clone(), gpu.v_cache.clone()
        for k in sorted({0, len(times) // 2, len(times) - 1}):
            decode_only.append(gpu.step(_decode_only(contexts, k)[1]))
        gpu.k_cache.copy_(saved[0])
        gpu.v_cache.copy_(saved[1])
        t = np.asarray(times)
        d = float(np.mean(decode_only))
        row = {"budget": b, "chunk_tokens": chunks[0], "steps": len(times),
               "mean_step_us": float(t.mean() * 1e6), "max_step_us": float(t.max() * 1e6),
               "decode_only_step_us": d * 1e6,
               "mean_extra_us": float((t.mean() - d) * 1e6),
               "prefill_ms": float(t.sum() * 1e3),
               "prompt_tokens_per_s": PROMPT / float(t.sum()),
               "stream_tokens_per_s": NUM_STREAMS / float(t.mean())}
        rows.append(row)
        print(json.dumps(row), flush=True)
    lines = ["budget  chunk  steps  mean_us   max_us  decode_only_us  extra_us  prefill_ms"
             "  prompt_tok/s  stream_tok/s"]
    for r in rows:
        lines.append(f"{r['budget']:6d} {r['chunk_tokens']:6d} {r['steps']:6d} "
                     f"{r['mean_step_us']:8.1f} {r['max_step_us']:8.1f} "
                     f"{r['decode_only_step_us']:15.1f} {r['mean_extra_us']:9.1f} "
                     f"{r['prefill_ms']:11.2f} {r['prompt_tokens_per_s']:13.0f} "
                     f"{r['stream_tokens_per_s']:13.0f}")
    text = "\n".join(lines)
    print(text, file=sys.stderr)
    if out_path:
        with open(out_path, "w") as f:
            f.write(text + "\n")
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--budgets", type=int, nargs="+", default=list(DEFAULT_BUDGETS))
    ap.add_argument("--out", default=None, help="also write the table to this file")
    args = ap.parse_args()
    run(sorted(args.budgets), args.out)


if __name__ == "__main__":
    main()
