"""Seeded synthetic inputs for one mixed decode + prefill-chunk step.

This module draws inputs only: request records, block tables, the initial KV
pool and the packed q / k_new / v_new tensors, all as bf16 bit patterns
(uint16).  It computes nothing the attention step computes; tests and the
bench feed the same arrays to the HIP library and to the CPU checker.

Recipe (all values N(0,1) drawn as fp32 by numpy's PCG64, rounded to bf16 by
round-to-nearest-even):

* Draw order per instance: context lengths -> prefix offsets -> extra prompt
  lengths -> block ids -> q -> k_new -> v_new -> cached K/V page contents.
  Each of these is its own child stream of ``SeedSequence([seed, instance])``
  so one stream's size never shifts another's values.
* Bulk draws are cut into fixed 4 Mi-element pieces, each with its own child
  seed, so they can be filled by several threads with identical results.
* q, k_new and v_new have ``token_budget`` rows (a step never schedules more);
  callers use the first ``num_tokens`` rows.
* Block ids: a random permutation of exactly the pages the instance needs, or
  a random sample of a fixed-size pool (the heavy mixed case).  Pages cover a
  request's whole prompt (prefill) or its context plus the steps it will run
  (decode).
* Page contents: random values at positions below ``num_computed``; every other
  slot, and every unused page, holds the sentinel 0xFFFF (a bf16 NaN) so a
  stray write or an unmasked read shows up.
* KV pools are logical: [num_blocks, Hkv, 16, D] for K and for V (one
  D-vector per page slot).  The library's own cache layout is made from them
  on the device (``step.py``).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
SENTINEL = np.uint16(0xFFFF)
_PIECE = 1 << 22


@dataclass
class Req:
    id: int
    num_computed: int
    target_len: int
    is_decode: bool


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    token_budget: int
    long_prefill_cap: int
    requests: list
    block_table: np.ndarray  # int32 [n_requests, max_blocks], queue order
    k_pool: np.ndarray  # uint16 [NB, Hkv, 16, D]
    v_pool: np.ndarray  # uint16 [NB, Hkv, 16, D]
    q: np.ndarray  # uint16 [budget, Hq, D]
    k_new: np.ndarray  # uint16 [budget, Hkv, D]
    v_new: np.ndarray  # uint16 [budget, Hkv, D]
    scale: float
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = x.view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def normal_bf16(seed_seq: np.random.SeedSequence, n: int) -> np.ndarray:
    """n N(0,1) values as bf16 bits; piecewise child streams, thread-parallel."""
    out = np.empty(n, dtype=np.uint16)
    pieces = [(a, min(n, a + _PIECE)) for a in range(0, n, _PIECE)]
    children = seed_seq.spawn(len(pieces)) if pieces else []

    def fill(k):
        a, b = pieces[k]
        rng = np.random.Generator(np.random.PCG64(children[k]))
        out[a:b] = _to_bf16_bits(rng.standard_normal(b - a, dtype=np.float32))

    if len(pieces) <= 1:
        for k in range(len(pieces)):
            fill(k)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(pieces))))
    return out


def softmax_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def build(name: str, seed: int, instance: int, *, num_q_heads: int, num_kv_heads: int,
          head_dim: int, token_budget: int, long_prefill_cap: int, requests: list,
          reach: list, pool_blocks: int | None, streams: dict) -> Workload:
    """Allocate pages, draw tensors and fill the pool for explicit requests.

    ``reach[i]`` is how many positions request i may ever occupy (pages are
    allocated for it); ``pool_blocks`` fixes the pool size (random sample of
    ids) or, if None, the pool is exactly the pages needed (random permutation).
    ``streams`` holds the remaining child SeedSequences: 'blocks', 'q', 'k',
    'v', 'pool'.
    """
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    pages_per_req = [math.ceil(r / BLOCK_SIZE) for r in reach]
    need = sum(pages_per_req)
    nb = need if pool_blocks is None else pool_blocks
    if need > nb:
        raise ValueError(f"{name}: needs {need} pages, pool has {nb}")
    rng_b = np.random.Generator(np.random.PCG64(streams["blocks"]))
    ids = rng_b.permutation(nb)[:need].astype(np.int32)
    max_pages = max(1, max(pages_per_req))
    bt = np.zeros((len(requests), max_pages), dtype=np.int32)
    at = 0
    for i, npg in enumerate(pages_per_req):
        bt[i, :npg] = ids[at:at + npg]
        at += npg

    q = normal_bf16(streams["q"], token_budget * Hq * D).reshape(token_budget, Hq, D)
    k_new = normal_bf16(streams["k"], token_budget * Hkv * D).reshape(token_budget, Hkv, D)
    v_new = normal_bf16(streams["v"], token_budget * Hkv * D).reshape(token_budget, Hkv, D)

    k_pool = np.full((nb, Hkv, BLOCK_SIZE, D), SENTINEL, dtype=np.uint16)
    v_pool = np.full((nb, Hkv, BLOCK_SIZE, D), SENTINEL, dtype=np.uint16)
    # pages holding at least one cached position, with their count of valid slots
    filled_ids, valid = [], []
    for i, r in enumerate(requests):
        c = r.num_computed
        for pg in range(math.ceil(c / BLOCK_SIZE)):
            filled_ids.append(bt[i, pg])
            valid.append(min(BLOCK_SIZE, c - pg * BLOCK_SIZE))
    if filled_ids:
        filled_ids = np.asarray(filled_ids, dtype=np.int64)
        valid = np.asarray(valid)
        page_elems = Hkv * BLOCK_SIZE * D
        kv_seq, = streams["pool"].spawn(1)
        ks, vs = kv_seq.spawn(2)
        kp = normal_bf16(ks, len(filled_ids) * page_elems).reshape(-1, Hkv, BLOCK_SIZE, D)
        vp = normal_bf16(vs, len(filled_ids) * page_elems).reshape(-1, Hkv, BLOCK_SIZE, D)
        slot = np.arange(BLOCK_SIZE)
        empty = slot[None, :] >= valid[:, None]  # [pages, 16]
        kp[np.broadcast_to(empty[:, None, :, None], kp.shape)] = SENTINEL
        vp[np.broadcast_to(empty[:, None, :, None], vp.shape)] = SENTINEL
        k_pool[filled_ids] = kp
        v_pool[filled_ids] = vp

    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    token_budget=token_budget, long_prefill_cap=long_prefill_cap,
                    requests=requests, block_table=bt, k_pool=k_pool, v_pool=v_pool,
                    q=q, k_new=k_new, v_new=v_new, scale=softmax_scale(D),
                    extra={"seed": seed, "instance": instance})


def _streams(seed: int, instance: int) -> dict:
    ss = np.random.SeedSequence([seed, instance])
    names = ["ctx", "prefix", "extra", "blocks", "q", "k", "v", "pool"]
    return dict(zip(names, ss.spawn(len(names))))


def _lognormal_lengths(ss, n, median, sigma, cap):
    rng = np.random.Generator(np.random.PCG64(ss))
    x = np.rint(np.exp(rng.normal(math.log(median), sigma, size=n))).astype(np.int64)
    return np.clip(x, 1, cap)


# ---------------------------------------------------------------------------
# The five measured configurations.  Sizes follow the pages' workloads:
# an 8B-class GQA model (Hq=32, Hkv=8, D=128), 16-token pages.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny",
    2: "page1_defaults",
    3: "budget8192",
    4: "long_context",
    5: "heavy_mixed",
}

PREFIXES = {2: (0, 3840, 7680), 3: (0, 2048, 4096, 6144)}


def num_instances(config: int) -> int:
    """Instances of a configuration: its prefix positions (configs 2 and 3),
    the steps of the tiny run, or two seeds of the same recipe (configs 4
    and 5), so that steps rotated over them never find their K/V in the
    256 MB last-level cache from the step before."""
    return {1: 4, 2: 3, 3: 4, 4: 2, 5: 2}[config]


def make_workload(config: int, instance: int = 0, kv_shard: int = 1) -> Workload:
    """Instance ``instance`` of measured configuration ``config`` (1..5).

    Config 1 instance i is step i of the tiny multi-step run with a fresh
    pool; use :func:`tiny_run` to carry the pool across steps.

    ``kv_shard`` = N (configs 2..5) gives one GPU's share of the step split N
    ways by KV head: the same rows, tokens and page ids, with 32/N query heads
    on 8/N KV heads (the pool's pages then hold 8/N heads each).
    """
    seed = 1000 + config
    st = _streams(seed, instance)
    if config == 1:
        if kv_shard != 1:
            raise ValueError("the tiny run is not split by KV head")
        run = tiny_run()
        return run.step_workload(instance, run.k_pool, run.v_pool)
    if kv_shard not in (1, 2, 4, 8):
        raise ValueError("kv_shard must divide the 8 KV heads")
    w = _measured_workload(config, instance, seed, st, 32 // kv_shard, 8 // kv_shard)
    if kv_shard != 1:
        w.name += f"/kvshard{kv_shard}"
    return w


def _measured_workload(config, instance, seed, st, hq, hkv):
    """Configurations 2..5 with hq query heads on hkv KV heads."""
    if config == 2:
        rng = np.random.Generator(np.random.PCG64(st["ctx"]))
        ctx = rng.integers(512, 4096, size=32, endpoint=True)
        prefix = PREFIXES[2][instance]
        reqs = [Req(i, int(c), int(c) + 1, True) for i, c in enumerate(ctx)]
        reqs.append(Req(32, prefix, 8192, False))
        reach = [int(c) + 1 for c in ctx] + [8192]
        return build(f"page1_defaults/prefix{prefix}", seed, instance, num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=128, token_budget=512, long_prefill_cap=0,
                     requests=reqs, reach=reach, pool_blocks=None, streams=st)
    if config == 3:
        prefix = PREFIXES[3][instance]
        ctx = [1000, 3000]
        reqs = [Req(0, 1000, 1001, True), Req(1, 3000, 3001, True), Req(2, prefix, 8192, False)]
        reach = [c + 1 for c in ctx] + [8192]
        return build(f"budget8192/prefix{prefix}", seed, instance, num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=128, token_budget=8192, long_prefill_cap=2048,
                     requests=reqs, reach=reach, pool_blocks=None, streams=st)
    if config == 4:
        ctx = _lognormal_lengths(st["ctx"], 64, 2048, 0.75, 32768)
        reqs = [Req(i, int(c), int(c) + 1, True) for i, c in enumerate(ctx)]
        reqs.append(Req(64, 31744, 32768, False))
        reach = [int(c) + 1 for c in ctx] + [32768]
        return build(f"long_context/prefix31744/seed{instance}", seed, instance, num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=128, token_budget=8192, long_prefill_cap=0,
                     requests=reqs, reach=reach, pool_blocks=None, streams=st)
    if config == 5:
        ctx = _lognormal_lengths(st["ctx"], 256, 1024, 0.75, 16384)
        rng_p = np.random.Generator(np.random.PCG64(st["prefix"]))
        offs = rng_p.integers(0, 16384, size=3, endpoint=True)
        rng_e = np.random.Generator(np.random.PCG64(st["extra"]))
        left3 = 3840 + int(rng_e.integers(1, 4096, endpoint=True))
        lefts = [2048, 2048, left3]
        reqs = [Req(i, int(c), int(c) + 1, True) for i, c in enumerate(ctx)]
        for k in range(3):
            reqs.append(Req(256 + k, int(offs[k]), int(offs[k]) + lefts[k], False))
        reach = [int(c) + 1 for c in ctx] + [int(offs[k]) + lefts[k] for k in range(3)]
        # 2 GiB of K+V: 32768 pages of 64 KiB (32 KiB K + 32 KiB V)
        return build(f"heavy_mixed/seed{instance}", seed, instance, num_q_heads=hq, num_kv_heads=hkv,
                     head_dim=128, token_budget=8192, long_prefill_cap=0, requests=reqs,
                     reach=reach, pool_blocks=32768, streams=st)
    raise ValueError(f"unknown config {config}")


# ---------------------------------------------------------------------------
# Tiny multi-step run: Hq=Hkv=4, D=64; a 256-token prompt in 4 chunks of 64
# plus 4 decode rows (contexts uniform in [100, 300]) growing by one per step.
# ---------------------------------------------------------------------------

@dataclass
class TinyRun:
    block_table: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    ctx: list
    steps: list  # per step: dict(q, k_new, v_new)
    seed: int = 1001

    def requests(self, step: int) -> list:
        reqs = [Req(i, c + step, c + step + 1, True) for i, c in enumerate(self.ctx)]
        reqs.append(Req(4, 64 * step, 256, False))
        return reqs

    def step_workload(self, step: int, k_pool, v_pool) -> Workload:
        d = self.steps[step]
        return Workload(name=f"tiny/step{step}", num_q_heads=4, num_kv_heads=4, head_dim=64,
                        token_budget=68, long_prefill_cap=0, requests=self.requests(step),
                        block_table=self.block_table, k_pool=k_pool, v_pool=v_pool,
                        q=d["q"], k_new=d["k"], v_new=d["v"], scale=softmax_scale(64),
                        extra={"seed": self.seed, "instance": step})


def tiny_run(num_steps: int = 4) -> TinyRun:
    seed = 1001
    st = _streams(seed, 0)
    rng = np.random.Generator(np.random.PCG64(st["ctx"]))
    ctx = [int(c) for c in rng.integers(100, 300, size=4, endpoint=True)]
    reqs = [Req(i, c, c + 1, True) for i, c in enumerate(ctx)] + [Req(4, 0, 256, False)]
    reach = [c + num_steps for c in ctx] + [256]
    w = build("tiny", seed, 0, num_q_heads=4, num_kv_heads=4, head_dim=64, token_budget=68,
              long_prefill_cap=0, requests=reqs, reach=reach, pool_blocks=None, streams=st)
    steps = [{"q": w.q, "k": w.k_new, "v": w.v_new}]
    for s in range(1, num_steps):
        sst = _streams(seed, s)
        steps.append({
            "q": normal_bf16(sst["q"], 68 * 4 * 64).reshape(68, 4, 64),
            "k": normal_bf16(sst["k"], 68 * 4 * 64).reshape(68, 4, 64),
            "v": normal_bf16(sst["v"], 68 * 4 * 64).reshape(68, 4, 64),
        })
    return TinyRun(block_table=w.block_table, k_pool=w.k_pool, v_pool=w.v_pool, ctx=ctx,
                   steps=steps, seed=seed)


def random_workload(seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    decode_ctx: list, chunks: list, token_budget: int | None = None,
                    long_prefill_cap: int = 0, pool_blocks: int | None = None) -> Workload:
    """Small explicit workload for parity tests.

    ``decode_ctx``: context length of each decode row.  ``chunks``: list of
    (num_computed, prompt_len) for prefill requests.  The budget defaults to
    exactly what everything needs.
    """
    st = _streams(seed, 0)
    reqs = [Req(i, int(c), int(c) + 1, True) for i, c in enumerate(decode_ctx)]
    reach = [int(c) + 1 for c in decode_ctx]
    for k, (c, L) in enumerate(chunks):
        reqs.append(Req(len(decode_ctx) + k, int(c), int(L), False))
        reach.append(int(L))
    if token_budget is None:
        token_budget = len(decode_ctx) + sum(L - c for c, L in chunks)
    token_budget = max(1, token_budget)
    return build(f"random/{seed}", seed, 0, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, token_budget=token_budget, long_prefill_cap=long_prefill_cap,
                 requests=reqs, reach=reach, pool_blocks=pool_blocks, streams=st)


# ---------------------------------------------------------------------------
# Score staircases: inputs whose attention scores climb in steps along a row
# ---------------------------------------------------------------------------

# Rises of a row's score level, in log2 units of the scaled score, at
# fractions of the row's key range: (fraction of the keys before the rise,
# rise).  Most rises are several times the 8-unit margin past which an
# online softmax has to move its running max; one is a fall.
STAIR_RISES = ((0.07, 9.5), (0.21, 12.0), (0.38, -6.0), (0.46, 17.0), (0.63, 10.5),
               (0.81, 21.0), (0.93, 9.0))
# and inside a chunk, at fractions of its new tokens (its causal diagonal)
STAIR_CHUNK_RISES = ((0.2, 11.0), (0.55, 14.0), (0.85, 9.25))


def stair_levels(context: int, new: int, is_chunk: bool) -> np.ndarray:
    """Score level (log2 units) of each key position [0, context + new) of a
    row: the sum of the rises at or before it."""
    L = context + new
    lv = np.zeros(L)
    for frac, up in STAIR_RISES:
        lv[int(frac * L):] += up
    if is_chunk:
        for frac, up in STAIR_CHUNK_RISES:
            lv[context + int(frac * new):] += up
    return lv


def staircase_workload(seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                       decode_ctx: list, chunks: list, noise: float = 0.25) -> Workload:
    """A random workload whose keys are re-drawn so that scores climb in steps.

    Per (request, KV head) a direction u ~ N(0,1)^D is drawn; every query of
    the request's G heads that share the KV head is u + noise * N(0,1), and
    key p of the request is a_p u + noise * N(0,1) with
    a_p = level(p) / (scale * log2(e) * |u|^2), so its scaled score against
    any of those queries is close to level(p) in log2 units (stair_levels).
    Values stay N(0,1).  Decode rows get the row-wide rises, chunks also rises
    inside their new tokens.
    """
    w = random_workload(seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, decode_ctx=decode_ctx, chunks=chunks)
    Hkv, D = num_kv_heads, head_dim
    G = num_q_heads // Hkv
    log2e = 1.4426950408889634
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    qsl = 0
    q = w.q.view(np.uint16)
    for i, r in enumerate(w.requests):
        c = r.num_computed
        n = 1 if r.is_decode else r.target_len - r.num_computed
        lv = stair_levels(c, n, not r.is_decode)
        pos = np.arange(c + n)
        blocks = w.block_table[i][pos // BLOCK_SIZE]
        offs = pos % BLOCK_SIZE
        for g in range(Hkv):
            u = _to_bf16_bits(rng.standard_normal(D, dtype=np.float32))
            uf = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            a = lv / (w.scale * log2e * float(uf @ uf))
            keys = a[:, None] * uf[None, :] + noise * rng.standard_normal((c + n, D))
            kb = _to_bf16_bits(keys.astype(np.float32))
            w.k_pool[blocks[:c], g, offs[:c], :] = kb[:c]
            w.k_new[qsl:qsl + n, g, :] = kb[c:]
            qs = uf[None, None, :] + noise * rng.standard_normal((n, G, D))
            q[qsl:qsl + n, g * G:(g + 1) * G, :] = _to_bf16_bits(qs.astype(np.float32))
        qsl += n
    w.name = f"staircase/{seed}"
    return w
