"""fp64 oracle of one mixed decode + prefill-chunk attention step.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg, never by the
library.

Sources (cited by page title and section; the pages' own wording is not
reproduced here):

* P1  "Chunked Prefill" (deepconcepts.dev) -- token budget, decode-first split,
  chunk = budget minus running users, the budget floor.
* P2  "05. Chunked Prefill" (vLLM learning book) -- section 2 (slicing a
  prompt), section 3 (what a chunk attends to), section 4 (packed batch and
  its metadata), section 5 (decode-first hybrid policy), section 8 (K/V of
  the chunk is written before attention reads the cache).
* P3  "Chunked Prefill on an M5 Max ..." -- "Wiring it into the loop" (a
  chunk extends the cache; a finished prompt moves to the decode queue).
* P4  tbr8.org deep dive on chunked prefill -- 3.1 (decode tokens first, the
  rest of the budget to prefill), 3.3 (cached_prefix_len of a chunk), 4.1
  (a chunk sees earlier chunks and itself, never later ones), 4.2 (16-token
  KV pages, a request owns a list of pages).
* P5  "How Chunked Prefill Stops Decode Starvation" -- "The fix" (decodes
  first, a prefill that does not fit is chunked; causality across chunks),
  "The payoff" (chunking leaves attention's result and Theta(L^2) cost alone).

Readings where the pages are silent or disagree (each also listed in the
design notes):

* A decode row with context length c appends its own K/V at position c and
  attends to c + 1 keys.
* Key k of a row with context c is visible to chunk query j iff k <= c + j
  (every earlier chunk fully visible, causal inside the chunk).
* Query head h reads KV head h // (Hq / Hkv).
* A prefill that does not fit the remaining budget is truncated to it (P1 and
  P5), not deferred; several prefills may share a step, in FCFS order.
* Cache pages are logical: [num_blocks, Hkv, 16, D] for both K and V, one
  contiguous D-vector per (page, KV head, slot).  The pages fix only 16-token
  pages; how a library lays a page out in memory is its own choice, and the
  tests convert the library's pool to this form before comparing.
"""

from __future__ import annotations

import math
from typing import NamedTuple, Sequence

import numpy as np

BLOCK_SIZE = 16  # tokens per KV page (P4 section 4.2)


class BudgetError(ValueError):
    """Fewer budget tokens than running decodes (P1, "The budget points in two
    directions": the configuration can never finish a prompt)."""


class Request(NamedTuple):
    id: int
    num_computed: int  # tokens already in the KV cache (P4 3.3 cached_prefix_len)
    target_len: int  # prompt length for a prefill; ignored for a decode
    is_decode: bool


# --------------------------------------------------------------------------
# C1: decode-first token-budget split
# --------------------------------------------------------------------------

POLICIES = ("truncate", "defer", "quota")


# P4 7.1's queue-depth rule as rows of (decode count below which the row
# applies, multiplier, divisor); the first row whose bound exceeds the decode
# count scales the base chunk, and the last row (no bound) halves it.
ADAPTIVE_CHUNK_ROWS = ((1, 4, 1), (10, 2, 1), (50, 1, 1), (None, 1, 2))


def adaptive_chunk(base_chunk: int, num_decodes: int) -> int:
    """Per-request chunk size from the decode queue depth (P4 7.1), read off
    ADAPTIVE_CHUNK_ROWS; at least one token."""
    for bound, mul, div in ADAPTIVE_CHUNK_ROWS:
        if bound is None or num_decodes < bound:
            return max(1, base_chunk * mul // div)
    raise AssertionError("the last row has no bound")


def schedule(requests: Sequence[Request], token_budget: int, long_prefill_cap: int = 0,
             policy: str = "truncate", max_prefill_tokens: int = 0,
             adaptive: bool = False, block_aligned: bool = False) -> dict:
    """Split one step's token budget, decodes first (P2 section 5 hybrid
    policy; P4 3.1; P5 "The fix").

    * Every decode request gets one token.  More decodes than budget tokens
      is an error (P1, the budget floor).
    * ``policy="truncate"`` (the default reading): the remaining budget goes
      to prefill requests in queue order; each takes min(remaining prompt,
      per-request cap, remaining budget) tokens (P1 "Why a chunk can be nearly
      free": budget 512 with 32 users gives 480).
    * ``policy="defer"`` (P4 3.1 as printed): a prefill's chunk is
      min(remaining prompt, per-request cap); it is scheduled only if the
      remaining budget holds all of it, and the first one that does not fit
      ends the scan.
    * ``policy="quota"`` (P4 3.2): prefills share their own budget,
      ``max_prefill_tokens``, cut to token_budget - decodes when the decodes
      take more than 70% of token_budget; within it, prefills are taken as in
      "truncate".
    * ``adaptive``: the per-request cap is adaptive_chunk(long_prefill_cap,
      decodes) (P4 7.1); needs a positive cap.
    * ``block_aligned``: a chunk that stops before the end of its prompt
      stops on a page boundary instead, (c + n) rounded down to a multiple of
      BLOCK_SIZE, when that leaves it at least one token; the tokens given
      back stay in the budget for the prompts behind it.  Every page such a
      chunk writes is then complete, so a prefix cache can reuse it: P1's
      closing notes say a chunked prefill only reuses cached pages that sit on
      page boundaries, P4 6.1 that prefix caching and chunked prefill combine.
    * Rows come out decodes first (input order), then prefills (input order);
      a request given 0 tokens is left out.
    """
    if token_budget <= 0:
        raise ValueError("token budget must be positive")
    if long_prefill_cap < 0:
        raise ValueError("cap must be >= 0")
    if policy not in POLICIES:
        raise ValueError(f"unknown policy {policy}")
    if policy == "quota" and max_prefill_tokens <= 0:
        raise ValueError("the quota policy needs max_prefill_tokens > 0")
    if adaptive and long_prefill_cap <= 0:
        raise ValueError("adaptive chunking needs a base chunk (long_prefill_cap > 0)")
    for r in requests:
        if r.num_computed < 0:
            raise ValueError("negative num_computed")
        if not r.is_decode and r.target_len < r.num_computed:
            raise ValueError("target_len below num_computed")

    decodes = [i for i, r in enumerate(requests) if r.is_decode]
    prefills = [i for i, r in enumerate(requests) if not r.is_decode]
    if len(decodes) > token_budget:
        raise BudgetError(f"{len(decodes)} decodes exceed budget {token_budget}")
    cap = adaptive_chunk(long_prefill_cap, len(decodes)) if adaptive else long_prefill_cap

    rows: list[tuple[int, int]] = [(i, 1) for i in decodes]
    remaining = token_budget - len(decodes)
    if policy == "quota":
        remaining = max_prefill_tokens
        if 10 * len(decodes) > 7 * token_budget:  # decodes above 70% of the budget
            remaining = token_budget - len(decodes)
    for i in prefills:
        r = requests[i]
        want = r.target_len - r.num_computed
        if cap:
            want = min(want, cap)
        if policy == "defer":
            if want > remaining:
                break
            n = want
        else:
            if remaining == 0:
                break
            n = min(want, remaining)
        if block_aligned and 0 < n < r.target_len - r.num_computed:
            end = (r.num_computed + n) // BLOCK_SIZE * BLOCK_SIZE
            if end > r.num_computed:
                n = end - r.num_computed
        if n > 0:
            rows.append((i, n))
            remaining -= n

    order = [i for i, _ in rows]
    num_scheduled = [n for _, n in rows]
    context_lens = [requests[i].num_computed for i in order]
    seq_lens = [c + n for c, n in zip(context_lens, num_scheduled)]
    qsl = [0]
    for n in num_scheduled:
        qsl.append(qsl[-1] + n)
    new_blocks = [math.ceil(s / BLOCK_SIZE) - math.ceil(c / BLOCK_SIZE)
                  for s, c in zip(seq_lens, context_lens)]
    return {
        "order": order,
        "num_scheduled": num_scheduled,
        "query_start_loc": qsl,
        "seq_lens": seq_lens,
        "context_lens": context_lens,
        "new_blocks": new_blocks,
        "num_seqs": len(rows),
        "num_decodes": len(decodes),
        "num_tokens": qsl[-1],
    }


def advance(requests: Sequence[Request], sched: dict) -> list[Request]:
    """State of the queue after the step ``sched`` ran.

    Scheduled tokens are now cached.  A prefill whose cache reaches its
    prompt length becomes a decode in the next step (P2 section 2 step table;
    P3 "Wiring it into the loop"); its first output token comes from the last
    chunk row, so no extra attention row is added in the step that finishes it.
    """
    got = dict(zip(sched["order"], sched["num_scheduled"]))
    nxt = []
    for i, r in enumerate(requests):
        n = got.get(i, 0)
        done = r.num_computed + n
        is_dec = r.is_decode or done >= r.target_len
        nxt.append(Request(r.id, done, max(r.target_len, done), is_dec))
    return nxt


# --------------------------------------------------------------------------
# C2: paged KV append (bit copy)
# --------------------------------------------------------------------------

def _pages(block_table, s: int) -> np.ndarray:
    """Page ids of packed row s: its own block-table row (P4 4.2: a request
    owns a list of pages)."""
    return np.asarray(block_table[s])


def _context(context_lens, s: int) -> int:
    """Tokens of packed row s already cached before this step (P4 3.3)."""
    return int(context_lens[s])


def append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
           query_start_loc: Sequence[int], context_lens: Sequence[int],
           block_table: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Write every packed token's K/V into its page slot (P4 4.2; P3 "Wiring
    it into the loop": a chunk extends the cache).  Returns new pools.

    Token t of row s sits at position p = context_lens[s] + (t - qsl[s]);
    its page is block_table[s][p // 16] and its slot p % 16.
    """
    K = k_pool.copy()
    V = v_pool.copy()
    for s in range(len(context_lens)):
        pages = _pages(block_table, s)
        c = _context(context_lens, s)
        for t in range(query_start_loc[s], query_start_loc[s + 1]):
            p = c + (t - query_start_loc[s])
            b = int(pages[p // BLOCK_SIZE])
            o = p % BLOCK_SIZE
            K[b, :, o, :] = k_new[t]
            V[b, :, o, :] = v_new[t]
    return K, V


# --------------------------------------------------------------------------
# C3: attention, plain definition in fp64
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _visible(pos: np.ndarray, context_len: int, js: np.ndarray) -> np.ndarray:
    """[len(js), len(pos)] mask: key k is visible to chunk query j iff
    k <= context_len + j (earlier chunks fully, causal inside the chunk)."""
    return pos[None, :] <= (context_len + js)[:, None]


def _kv_head(h: int, group: int) -> int:
    """KV head read by query head h: consecutive query heads share one."""
    return h // group


def _row_keys(k_pool, v_pool, pages, g, length):
    """K and V of keys [0, length) of one row and KV head, as [length, D] fp64:
    key k sits in page pages[k // 16], slot k % 16."""
    pos = np.arange(length)
    blocks = np.asarray(pages)[pos // BLOCK_SIZE]
    offs = pos % BLOCK_SIZE
    Ks = bf16_bits_to_f64(k_pool[blocks, g, offs, :])
    Vs = bf16_bits_to_f64(v_pool[blocks, g, offs, :])
    return Ks, Vs


def softmax_weights(q, k_pool, block_table_row, context_len, q_row_start, j, h, num_kv_heads, scale):
    """Softmax weights of query j (chunk-local) and head h of one row over
    its visible keys [0, context_len + j]; returns a 1-D fp64 array."""
    Hq = q.shape[1]
    g = _kv_head(h, Hq // num_kv_heads)
    Ks, _ = _row_keys(k_pool, k_pool, block_table_row, g, context_len + j + 1)
    s = scale * (Ks @ bf16_bits_to_f64(q[q_row_start + j, h]))
    w = np.exp(s - s.max())
    return w / w.sum()


def attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
              query_start_loc: Sequence[int], context_lens: Sequence[int],
              block_table: np.ndarray, num_kv_heads: int, scale: float,
              tokens: np.ndarray | None = None, row_chunk: int = 256):
    """Attention output of every packed query against the (post-append) pool.

    For row s with context c, chunk query j (packed token t = qsl[s] + j,
    position c + j) and head h reading KV head g = h // (Hq/Hkv):
        score_k = scale * <q[t,h], K_s[k]>  for keys k <= c + j
        out[t,h] = sum_k softmax(score)_k V_s[k];  lse = max + log(sum exp)
    (P2 sections 3 and 8; P4 4.1; P5 "The fix").  Decode rows are rows with
    one query.  ``tokens`` restricts the work to a subset of packed tokens
    (others are left NaN); ``row_chunk`` only bounds memory, every query row
    is computed on its own.

    Returns (out [T,Hq,D] fp64, lse [T,Hq] fp64).
    """
    T, Hq, D = q.shape
    if Hq % num_kv_heads:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // num_kv_heads
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    for s in range(len(context_lens)):
        t0, t1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        js = np.nonzero(want[t0:t1])[0]
        if js.size == 0:
            continue
        c = _context(context_lens, s)
        pages = _pages(block_table, s)
        length = c + (t1 - t0)
        pos = np.arange(length)
        for g in range(num_kv_heads):
            Ks, Vs = _row_keys(k_pool, v_pool, pages, g, length)
            heads = [h for h in range(Hq) if _kv_head(h, G) == g]
            for a in range(0, js.size, row_chunk):
                jj = js[a:a + row_chunk]
                Q = bf16_bits_to_f64(q[t0 + jj][:, heads, :])         # [nj, G, D]
                S = scale * (Q @ Ks.T)                                 # [nj, G, L]
                visible = _visible(pos, c, jj)                         # [nj, L]
                S = np.where(visible[:, None, :], S, -np.inf)
                m = S.max(axis=-1, keepdims=True)
                W = np.exp(S - m)
                l = W.sum(axis=-1, keepdims=True)
                rows = (t0 + jj)[:, None]
                out[rows, heads, :] = (W @ Vs) / l
                lse[rows, heads] = (m + np.log(l))[..., 0]
    return out, lse
