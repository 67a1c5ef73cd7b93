"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bar: the whole KV pool bit-identical to the oracle's after the append (it
starts from a sentinel-filled pool, so a stray write shows up); attention
outputs within max |err| <= 2e-2 of the fp64 oracle (bf16 inputs, fp32
accumulation, bf16 output); lse within 1e-2.
"""

import math

import numpy as np
import pytest

import oracle
from chunked_prefill_mixed_amd import cpa, workloads
from chunked_prefill_mixed_amd.step import DeviceStep, pools_from_caches

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2
LSE_TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu(lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def oracle_step(w, meta, tokens=None):
    """Oracle append + attention for the step the builder scheduled."""
    bt = w.block_table[meta["order"]]
    T = meta["num_tokens"]
    kp, vp = oracle.append(w.k_pool, w.v_pool, w.k_new[:T], w.v_new[:T], meta["query_start_loc"],
                           meta["context_lens"], bt)
    out, lse = oracle.attention(w.q[:T], kp, vp, meta["query_start_loc"], meta["context_lens"], bt,
                                w.num_kv_heads, w.scale, tokens=tokens)
    return kp, vp, out, lse


def sample_tokens(meta, rng, per_chunk=48):
    """All decode tokens plus, per chunk row, its first and last 16 tokens and
    random ones in between."""
    qsl, nd = meta["query_start_loc"], meta["num_decodes"]
    toks = list(range(qsl[nd]))
    for s in range(nd, meta["num_seqs"]):
        a, b = qsl[s], qsl[s + 1]
        toks += list(range(a, min(b, a + 16))) + list(range(max(a, b - 16), b))
        if b - a > 32:
            toks += list(rng.choice(np.arange(a + 16, b - 16), size=min(per_chunk, b - a - 32),
                                    replace=False))
    return np.unique(np.asarray(toks, dtype=np.int64))


def check_step(w, decode_split_tokens=0, tokens=None, label="", chunk_split_tokens=0):
    import torch
    ds = DeviceStep(w, decode_split_tokens=decode_split_tokens,
                    chunk_split_tokens=chunk_split_tokens)
    ds.run()
    torch.cuda.synchronize()
    kp, vp, out, lse = oracle_step(w, ds.meta, tokens)
    gk, gv = ds.pools_bits()
    assert np.array_equal(gk, kp), f"{label}: K pool differs at {np.argwhere(gk != kp)[:5]}"
    assert np.array_equal(gv, vp), f"{label}: V pool differs at {np.argwhere(gv != vp)[:5]}"
    got = ds.out_f64()
    sel = np.arange(ds.num_tokens) if tokens is None else np.asarray(tokens)
    err = np.max(np.abs(got[sel] - out[sel])) if sel.size else 0.0
    assert np.isfinite(got[sel]).all(), label
    assert err <= OUT_TOL, f"{label}: max |err| {err}"
    lerr = np.max(np.abs(ds.lse_f64()[sel] - lse[sel])) if sel.size else 0.0
    assert lerr <= LSE_TOL, f"{label}: lse err {lerr}"
    return ds, err


def test_tiny_four_steps_carry_the_pool():
    """Config 1: a 256-token prompt in 4 chunks of 64 beside 4 decode rows;
    the pool is carried from step to step on both sides."""
    import torch
    run = workloads.tiny_run()
    kp, vp = run.k_pool, run.v_pool
    gk, gv = kp, vp
    for step in range(4):
        w = run.step_workload(step, gk, gv)
        ds = DeviceStep(w)
        assert ds.num_tokens == 68 and ds.num_decodes == 4
        ds.run()
        torch.cuda.synchronize()
        wo = run.step_workload(step, kp, vp)
        kp, vp, out, lse = oracle_step(wo, ds.meta)
        gk, gv = ds.pools_bits()
        assert np.array_equal(gk, kp) and np.array_equal(gv, vp), step
        assert np.max(np.abs(ds.out_f64() - out)) <= OUT_TOL, step
        assert np.max(np.abs(ds.lse_f64() - lse)) <= LSE_TOL, step


SMALL = [
    # (Hq, Hkv, D, decode contexts, chunks as (num_computed, prompt_len), split)
    (4, 4, 64, [0, 1, 15, 16, 17, 250], [(0, 64), (64, 128)], 0),
    (8, 4, 64, [3, 200], [(17, 17 + 33), (0, 1), (5, 6)], 16),
    (16, 4, 128, [1000, 31, 77], [(100, 230), (0, 129)], 64),
    (32, 8, 128, [500, 1, 2048], [(1000, 1130), (3, 70)], 0),
    (32, 4, 128, [0, 300], [(511, 600), (0, 17)], 32),
    (8, 8, 128, [100, 64, 65], [(0, 200), (48, 49)], 16),
    (16, 2, 64, [40, 4000], [(2000, 2100)], 0),
    (8, 1, 128, [7, 129], [(70, 110)], 48),
]


WIDE = [
    # many KV heads: the append copies several 64-piece passes per token, and
    # G = 1 / 2 / 4 decode and chunk kernels at Hkv = 32 / 16 / 16
    (32, 32, 64, [0, 17, 700], [(33, 33 + 100)], 32),
    (32, 16, 128, [5, 1500], [(0, 77), (200, 300)], 0),
    (64, 16, 128, [256, 31], [(1000, 1100)], 64),
]


@pytest.mark.parametrize("case", range(len(WIDE)))
def test_wide_head_counts(case):
    Hq, Hkv, D, dec, chunks, split = WIDE[case]
    w = workloads.random_workload(600 + case, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  decode_ctx=dec, chunks=chunks)
    check_step(w, decode_split_tokens=split, label=f"wide{case}")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 3, 7, 29])
def test_chunk_tile_edges(G, D):
    """Chunks one token short of, exactly at and one past the query tile of
    256 (token, head) rows at head_dim 128 (128 at 64), i.e. floor(256/G)
    tokens, and one of two tiles plus a token, at the compiled head groupings
    and at three read at run time (3, 7, 29: tiles whose last rows hold no
    query; 29 also takes two decode waves per piece and KV head); one chunk
    after a 3000-token prefix, so the few tiles of the step are cut into key
    pieces and merged.  Every token of every row matches the oracle."""
    rows = 256 if D == 128 else 128
    T = rows // G
    chunks = [(0, max(1, T - 1)), (0, T), (3000, 3000 + T + 1), (5, 5 + 2 * T + 1)]
    w = workloads.random_workload(1500 + 10 * G + D, num_q_heads=2 * G, num_kv_heads=2,
                                  head_dim=D, decode_ctx=[10, 700], chunks=chunks)
    ds, _ = check_step(w, label=f"tile edges G{G} D{D}")
    assert ds.counts.num_chunk_merges > 0  # the prefixed chunk's tiles were split


def test_empty_step_touches_nothing():
    """num_tokens = 0: both device calls return CPA_OK without a launch, and
    the cache and the output buffer keep their bits."""
    import ctypes
    import torch
    w = workloads.random_workload(83, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                  decode_ctx=[40], chunks=[])
    ds = DeviceStep(w)
    ds.out.fill_(1.5)
    k0, v0, o0 = ds.k_cache.clone(), ds.v_cache.clone(), ds.out.clone()
    lib = cpa.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.cpa_append_kv(P(ds.k_new), P(ds.v_new), P(ds.query_start_loc), P(ds.context_lens),
                           P(ds.block_table), int(ds.block_table.shape[1]), ds.num_seqs, 0, 2, 64,
                           16, P(ds.k_cache), P(ds.v_cache), stream)
    assert st == cpa.CPA_OK
    counts = cpa.cpa_plan_counts_t()
    st = lib.cpa_attention(P(ds.q), P(ds.k_cache), P(ds.v_cache), P(ds.block_table),
                           int(ds.block_table.shape[1]), P(ds.query_start_loc), None,
                           P(ds.context_lens), P(ds.plan), ctypes.byref(counts), 0, 0, 0, 8, 2,
                           64, 16, ctypes.c_float(0.125), P(ds.out), None, None,
                           ctypes.c_size_t(0), stream)
    assert st == cpa.CPA_OK
    torch.cuda.synchronize()
    assert torch.equal(ds.k_cache.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(ds.v_cache.view(torch.int16), v0.view(torch.int16))
    assert torch.equal(ds.out, o0)


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_mixed_steps(case):
    Hq, Hkv, D, dec, chunks, split = SMALL[case]
    w = workloads.random_workload(500 + case, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  decode_ctx=dec, chunks=chunks)
    check_step(w, decode_split_tokens=split, label=f"small{case}")


def test_zero_query_gives_cumulative_mean():
    """q = 0: every visible key has the same weight; row j is the mean of V
    over keys 0..c+j (pins the visibility boundary key by key)."""
    w = workloads.random_workload(77, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                  decode_ctx=[33], chunks=[(21, 21 + 70)])
    w.q[:] = 0
    ds, _ = check_step(w, decode_split_tokens=16, label="q0")
    # and against the closed form directly
    out = ds.out_f64()
    bt = w.block_table[ds.meta["order"]]
    kp, vp = oracle.append(w.k_pool, w.v_pool, w.k_new[:ds.num_tokens], w.v_new[:ds.num_tokens],
                           ds.meta["query_start_loc"], ds.meta["context_lens"], bt)
    s = 1
    c = ds.meta["context_lens"][s]
    for j in (0, 1, 37, 69):
        t = ds.meta["query_start_loc"][s] + j
        keys = np.arange(c + j + 1)
        V = oracle.bf16_bits_to_f64(vp[bt[s][keys // 16], 0, keys % 16, :])
        assert np.max(np.abs(out[t, 0] - V.mean(axis=0))) <= OUT_TOL


def test_first_token_sees_only_itself():
    """Context 0, chunk starting at 0: token 0's output is its own V exactly."""
    w = workloads.random_workload(78, num_q_heads=4, num_kv_heads=4, head_dim=64, decode_ctx=[],
                                  chunks=[(0, 40)])
    ds, _ = check_step(w, label="self")
    v0 = oracle.bf16_bits_to_f64(w.v_new[0])  # [Hkv, D]
    assert np.array_equal(ds.out_f64()[0], v0)


def test_decode_row_equals_one_token_chunk_row():
    """The same query as a decode row (split-KV kernel) and as a one-token
    prefill row (MFMA kernel) gives the same output."""
    import torch
    w = workloads.random_workload(79, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                  decode_ctx=[700], chunks=[(700, 701)])
    # same query and new K/V for both rows, and identical cached context
    w.q[1] = w.q[0]
    w.k_new[1] = w.k_new[0]
    w.v_new[1] = w.v_new[0]
    pages = 701 // 16 + 1
    w.k_pool[w.block_table[1, :pages]] = w.k_pool[w.block_table[0, :pages]]
    w.v_pool[w.block_table[1, :pages]] = w.v_pool[w.block_table[0, :pages]]
    ds = DeviceStep(w, decode_split_tokens=0)
    assert ds.num_decodes == 1 and ds.num_seqs == 2 and ds.counts.num_chunk_tiles >= 1
    ds.run()
    torch.cuda.synchronize()
    out = ds.out_f64()
    assert np.max(np.abs(out[0] - out[1])) <= 1e-2
    _, _, ref, _ = oracle_step(w, ds.meta)
    assert np.max(np.abs(out - ref)) <= OUT_TOL


@pytest.mark.parametrize("split", [16, 32, 256, 1024])
def test_decode_split_count_does_not_change_result(split):
    w = workloads.random_workload(80, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                  decode_ctx=[4000, 1, 16, 17, 999], chunks=[])
    check_step(w, decode_split_tokens=split, label=f"split{split}")


@pytest.mark.parametrize("csplit", [64, 128, 320, 1 << 30])
def test_chunk_split_count_does_not_change_result(csplit):
    """Cutting chunk tiles' prefix keys into pieces (merged by log-sum-exp)
    gives the same outputs as one piece, for ragged chunks and every head
    grouping."""
    for case, (Hq, Hkv, D, chunks) in enumerate([(32, 8, 128, [(1000, 1130), (77, 300)]),
                                                  (8, 8, 64, [(640, 700)]),
                                                  (16, 2, 128, [(129, 129 + 17)])]):
        w = workloads.random_workload(90 + case, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                      decode_ctx=[50], chunks=chunks)
        ds, _ = check_step(w, chunk_split_tokens=csplit, label=f"csplit{csplit}/{case}")
        if csplit < 1 << 30 and case == 0:  # a 1000-key prefix is always cut here
            assert ds.counts.num_chunk_merges > 0


def test_two_streams_match_one_stream():
    """Decode sections on the main stream and chunk sections on a second
    stream, concurrently after the append, give the same bits as one stream."""
    import torch
    w = workloads.make_workload(2, 2)
    a = DeviceStep(w)
    a.run()
    b = DeviceStep(w)
    aux = torch.cuda.Stream()
    b.run_two_streams(aux)
    torch.cuda.synchronize()
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))


def _mixed_case(case):
    if case == "d64":
        # head_dim 64, G = 2: 192 tiles x 8 KV heads = 1536 chunk workgroups
        rng = np.random.default_rng(84)
        ctx = rng.integers(100, 3000, size=40).tolist()
        return workloads.random_workload(84, num_q_heads=16, num_kv_heads=8, head_dim=64,
                                         decode_ctx=ctx, chunks=[(0, 12288)])
    return workloads.make_workload(case, 0)


@pytest.mark.parametrize("case", [3, 4, 5, "d64"])
def test_one_launch_matches_separate_sections(case):
    """When the chunk tiles fill a resident round (256 8-wave workgroups at
    head_dim 128, 768 4-wave ones at 64), a step runs its decode pieces and
    chunk tiles as one launch: decode workgroups first when they fit one
    round (budget-8192, long-context and the head_dim-64 steps), chunk tiles
    first otherwise (heavy mixed).  The same plan run section by section, one
    launch each, gives the same bits."""
    import torch
    w = _mixed_case(case)
    a = DeviceStep(w, validate=False)
    c = a.counts
    slots = 256 * (1 if w.head_dim > 64 else 3)
    assert c.num_decode_splits > 0 and c.num_chunk_tiles * w.num_kv_heads >= slots
    a.run()
    b = DeviceStep(w, validate=False)
    b.append()
    for sec in ("decode_splits", "chunk_tiles", "decode_merges", "chunk_merges"):
        b._section_call(sec, None)
    torch.cuda.synchronize()
    for name in ("out", "lse"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), name


# (Hq, Hkv, D, decode contexts, chunks): groups the kernels read at run time.
# Decode pieces of up to 64 pages; a group above 16 takes ceil(G / 16) decode
# waves per piece and KV head.  The largest groups are one chunk tile's rows
# (one token per tile: 256 at head_dim 128, 128 at 64).
ANY_GROUP = [
    (6, 2, 128, [0, 15, 1500], [(0, 200), (2000, 2100)]),
    (10, 2, 64, [700, 5000], [(300, 420), (0, 1)]),
    (16, 1, 128, [64, 2047], [(900, 1000)]),
    (17, 1, 64, [3000, 1], [(0, 50), (600, 641)]),
    (96, 2, 128, [1200, 33], [(100, 140)]),
    (128, 1, 64, [2500], [(0, 9), (400, 403)]),
    (256, 1, 128, [900, 4100], [(1000, 1006)]),
]


@pytest.mark.parametrize("case", range(len(ANY_GROUP)))
def test_any_group_size(case):
    """Query heads per KV head outside the compiled 1, 2, 4 and 8: every
    token of every row against the oracle, at default and at fine splits."""
    Hq, Hkv, D, dec, chunks = ANY_GROUP[case]
    w = workloads.random_workload(2600 + case, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  decode_ctx=dec, chunks=chunks)
    check_step(w, label=f"G{Hq // Hkv} D{D}")
    check_step(w, decode_split_tokens=128, chunk_split_tokens=64, label=f"G{Hq // Hkv} D{D} split")


@pytest.mark.parametrize("Hq,Hkv,D,tokens", [(58, 2, 128, 1024), (28, 4, 64, 3456),
                                             (48, 1, 128, 1280)])
def test_any_group_one_launch(Hq, Hkv, D, tokens):
    """Run-time groups (29, 7, 48) with enough chunk tiles for the one-launch
    kernel: it matches the oracle on every token and gives the same bits as
    the plan run section by section."""
    import torch
    rng = np.random.default_rng(Hq + D)
    ctx = rng.integers(100, 3000, size=12).tolist()
    w = workloads.random_workload(2700 + Hq + D, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  decode_ctx=ctx, chunks=[(300, 300 + tokens)])
    a, _ = check_step(w, label=f"G{Hq // Hkv} D{D} one launch")
    c = a.counts
    assert c.num_decode_splits > 0
    assert c.num_chunk_tiles * Hkv >= 256 * (1 if D > 64 else 3)  # the one-launch path ran
    b = DeviceStep(w, validate=False)
    b.append()
    for sec in ("decode_splits", "chunk_tiles", "decode_merges", "chunk_merges"):
        b._section_call(sec, None)
    torch.cuda.synchronize()
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(a.lse, b.lse)


@pytest.mark.parametrize("rows", [449, 511, 512, 700])
def test_many_rows(rows):
    """Steps of 449 to 700 rows (one chunk, the rest decode rows with short
    contexts).  The append finds each token's row among fewer than 512 rows
    from registers (449 and 511 use all eight 64-row groups) and from memory
    at 512 rows and more; every row's K/V and outputs match the oracle."""
    rng = np.random.default_rng(rows)
    dec = rng.integers(0, 200, size=rows - 1).tolist()
    w = workloads.random_workload(1300 + rows, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                  decode_ctx=dec, chunks=[(40, 140)])
    ds, _ = check_step(w, label=f"rows{rows}")
    assert ds.num_seqs == rows


def test_128k_token_rows():
    """A decode row with 131071 cached tokens and a 100-token chunk after a
    100000-token prefix: 128 decode pieces and dozens of chunk prefix pieces
    per row go through the merge; K/V and outputs match the oracle."""
    w = workloads.random_workload(1400, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                  decode_ctx=[131071, 5], chunks=[(100000, 100100)])
    ds, _ = check_step(w, label="128k")
    c = ds.counts
    assert c.num_decode_merges >= 1 and c.num_chunk_merges >= 1
    assert c.num_decode_partials >= 128


# (Hq, Hkv, D, decode contexts, chunks): chunk tiles below a resident round
# (decode and chunk as separate launches), at one (one launch), head_dim 64
FAR_POOL = {
    "separate": (32, 8, 128, [700, 1500, 33], [(300, 800)]),
    "one_launch": (32, 8, 128, [900, 2100], [(1024, 3072)]),
    "d64": (16, 4, 64, [517, 60], [(250, 700)]),
}


@pytest.mark.parametrize("case", sorted(FAR_POOL))
def test_pages_past_4_gib_of_the_pool(case):
    """Every page of the step sits past the first 2^31 elements (4 GiB) of
    each cache, so every page address needs 64-bit arithmetic: the step's
    pages are moved to block ids offset by that much in a pool whose lower
    blocks hold the sentinel.  The moved pages match the oracle bit for bit,
    the lower blocks keep the sentinel, and the outputs match the oracle."""
    import torch
    Hq, Hkv, D, dec, chunks = FAR_POOL[case]
    w = workloads.random_workload(1200 + sorted(FAR_POOL).index(case), num_q_heads=Hq,
                                  num_kv_heads=Hkv, head_dim=D, decode_ctx=dec, chunks=chunks)
    ds = DeviceStep(w)
    off = (1 << 31) // (Hkv * 16 * D) + 3  # first moved block starts past element 2^31
    big = []
    for small in (ds.k_cache, ds.v_cache):
        t = torch.empty((off + small.shape[0],) + tuple(small.shape[1:]), dtype=small.dtype,
                        device=small.device)
        t[:off].view(torch.int16).fill_(-1)  # 0xFFFF sentinel
        t[off:] = small
        big.append(t)
    del small
    ds.k_cache, ds.v_cache = big
    ds.block_table += off
    ds.run()
    torch.cuda.synchronize()
    tokens = sample_tokens(ds.meta, np.random.default_rng(5))
    kp, vp, out, lse = oracle_step(w, ds.meta, tokens)
    gk, gv = pools_from_caches(big[0][off:], big[1][off:])
    for name, t, got, ref in (("K", big[0], gk, kp), ("V", big[1], gv, vp)):
        low = t[:off].view(torch.int16)
        assert int(low.min()) == -1 and int(low.max()) == -1, f"{name}: a lower block was written"
        assert np.array_equal(got, ref), f"{name} pool differs at {np.argwhere(got != ref)[:5]}"
    got = ds.out_f64()[tokens]
    assert np.isfinite(got).all()
    assert np.max(np.abs(got - out[tokens])) <= OUT_TOL
    assert np.max(np.abs(ds.lse_f64()[tokens] - lse[tokens])) <= LSE_TOL


@pytest.mark.parametrize("C", [1, 7, 16, 64, 100, 256])
def test_gpu_chunking_invariance(C):
    """One 256-token prompt prefilled in chunks of C, each chunk appended
    first then attended; every chunking lands within tolerance of the one-shot
    causal prefill computed by the oracle."""
    import torch
    L, Hq, Hkv, D = 256, 16, 4, 128
    w = workloads.random_workload(81, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  decode_ctx=[], chunks=[(0, L)], token_budget=L)
    # one-shot oracle
    bt = w.block_table
    kp, vp = oracle.append(w.k_pool, w.v_pool, w.k_new[:L], w.v_new[:L], [0, L], [0], bt)
    ref, _ = oracle.attention(w.q[:L], kp, vp, [0, L], [0], bt, Hkv, w.scale)
    gk, gv = w.k_pool, w.v_pool
    outs = []
    for a in range(0, L, C):
        b = min(L, a + C)
        wc = workloads.Workload(name="inv", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                token_budget=b - a, long_prefill_cap=0,
                                requests=[workloads.Req(0, a, L, False)], block_table=bt,
                                k_pool=gk, v_pool=gv, q=w.q[a:b], k_new=w.k_new[a:b],
                                v_new=w.v_new[a:b], scale=w.scale)
        ds = DeviceStep(wc)
        ds.run()
        torch.cuda.synchronize()
        outs.append(ds.out_f64())
        gk, gv = ds.pools_bits()
    got = np.concatenate(outs)
    assert np.array_equal(gk, kp) and np.array_equal(gv, vp)
    assert np.max(np.abs(got - ref)) <= OUT_TOL


def test_workspace_too_small_is_rejected():
    import torch
    w = workloads.random_workload(82, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                  decode_ctx=[300], chunks=[])
    ds = DeviceStep(w, decode_split_tokens=16)
    assert ds.counts.num_decode_partials > 0
    ds.workspace = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cpa.CpaError) as e:
        ds.attention()
    assert e.value.status == cpa.CPA_ERR_CAPACITY


def oracle_step_parallel(w, meta, workers=None):
    """oracle_step over every packed token, run in threads over interleaved
    64-token blocks (numpy's array kernels release the GIL, BLAS runs one
    thread per worker); the results of the threads cover disjoint tokens."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    T = meta["num_tokens"]
    bt = w.block_table[meta["order"]]
    kp, vp = oracle.append(w.k_pool, w.v_pool, w.k_new[:T], w.v_new[:T], meta["query_start_loc"],
                           meta["context_lens"], bt)
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    blocks = np.arange(T) // 64
    parts = [np.nonzero(blocks % workers == k)[0] for k in range(workers)]

    def run(tok):
        return tok, oracle.attention(w.q[:T], kp, vp, meta["query_start_loc"],
                                     meta["context_lens"], bt, w.num_kv_heads, w.scale,
                                     tokens=tok)

    out = np.full((T, w.num_q_heads, w.head_dim), np.nan)
    lse = np.full((T, w.num_q_heads), np.nan)
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for tok, (o, l) in ex.map(run, [p for p in parts if p.size]):
            out[tok] = o[tok]
            lse[tok] = l[tok]
    return kp, vp, out, lse


@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_config_end_to_end(config):
    """The measured configurations at full size, every instance: the whole pool
    bit-exact, and the outputs and lse of every token of every row against
    the oracle."""
    import torch
    for inst in range(workloads.num_instances(config)):
        w = workloads.make_workload(config, inst)
        ds = DeviceStep(w)
        print(f"config {config} instance {inst}: {w.name}, {ds.num_tokens} tokens", flush=True)
        ds.run()
        torch.cuda.synchronize()
        kp, vp, out, lse = oracle_step_parallel(w, ds.meta)
        gk, gv = ds.pools_bits()
        assert np.array_equal(gk, kp), f"{w.name}: K pool differs at {np.argwhere(gk != kp)[:5]}"
        assert np.array_equal(gv, vp), f"{w.name}: V pool differs at {np.argwhere(gv != vp)[:5]}"
        del gk, gv, kp, vp
        got = ds.out_f64()
        assert np.isfinite(got).all() and np.isfinite(out).all(), w.name
        err = np.max(np.abs(got - out))
        assert err <= OUT_TOL, f"{w.name}: max |err| {err}"
        lerr = np.max(np.abs(ds.lse_f64() - lse))
        assert lerr <= LSE_TOL, f"{w.name}: lse err {lerr}"
        print(f"  max |out err| {err:.3e}, max |lse err| {lerr:.3e}", flush=True)
        del ds


@pytest.mark.parametrize("config,shard", [(4, 8), (5, 8), (5, 4), (5, 2)])
def test_kv_shard_end_to_end(config, shard):
    """One GPU's share of the long-context and heavy-mixed steps split 8, 4 or
    2 ways by KV head (4 query heads on 1, 2 or 4 KV heads: the planner deals
    the pieces over the XCD ranges of a head and cuts uneven tiles into two
    or three rounds of key pieces), every instance: the pool bit-exact and
    every token against the oracle."""
    import torch
    for inst in range(workloads.num_instances(config)):
        w = workloads.make_workload(config, inst, kv_shard=shard)
        ds = DeviceStep(w)
        print(f"config {config} instance {inst}: {w.name}, {ds.num_tokens} tokens", flush=True)
        ds.run()
        torch.cuda.synchronize()
        kp, vp, out, lse = oracle_step_parallel(w, ds.meta)
        gk, gv = ds.pools_bits()
        assert np.array_equal(gk, kp) and np.array_equal(gv, vp), w.name
        del gk, gv, kp, vp
        err = np.max(np.abs(ds.out_f64() - out))
        assert err <= OUT_TOL, f"{w.name}: max |err| {err}"
        lerr = np.max(np.abs(ds.lse_f64() - lse))
        assert lerr <= LSE_TOL, f"{w.name}: lse err {lerr}"
        del ds


# (Hq, Hkv, D, decode contexts, chunks, decode split tokens, chunk split tokens)
STAIRCASES = [
    (32, 8, 128, [3000, 777, 64, 15], [(1000, 1300), (0, 200)], 0, 0),
    (32, 8, 128, [3000, 777], [(1000, 1300)], 64, 192),
    (32, 8, 128, [2000], [(700, 1100)], 16, 64),
    (8, 2, 64, [900, 300, 77], [(500, 700), (0, 160)], 0, 0),
    (8, 2, 64, [900, 300], [(500, 700)], 32, 64),
    (8, 8, 64, [1200], [(300, 420)], 256, 128),
    (64, 8, 128, [500], [(900, 1000)], 0, 0),
    (16, 16, 128, [1500], [(2000, 2100)], 48, 0),
]


@pytest.mark.parametrize("case", range(len(STAIRCASES)))
def test_score_staircase_moves_the_running_max(case):
    """Scores that climb in steps of 9 to 21 log2 units along each row, and
    again inside each chunk, make the kernels move their running max mid-row
    with a finite rescale factor: inside decode pieces and chunk pieces,
    across 64-key tiles, across split pieces (the log-sum-exp merge), and on
    the masked diagonal tiles; head_dim 64 and 128, G = 1 to 8.  Every token
    and the whole pool against the oracle."""
    Hq, Hkv, D, dec, chunks, dsplit, csplit = STAIRCASES[case]
    w = workloads.staircase_workload(900 + case, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                     decode_ctx=dec, chunks=chunks)
    check_step(w, decode_split_tokens=dsplit, chunk_split_tokens=csplit,
               label=f"staircase{case} Hq={Hq} Hkv={Hkv} D={D} splits={dsplit}/{csplit}")


@pytest.mark.parametrize("config", [2, 3])
def test_graph_replay_matches_eager(config):
    """The step captured as one HIP graph: every replay, with eager work and
    synchronisations between replays, gives the eager step's output and cache
    bits (the library records only kernel launches).  The page-1 step runs
    decode and chunk as separate launches, the budget-8192 step as one."""
    import torch
    w = workloads.make_workload(config, 1)
    eager = DeviceStep(w, with_lse=False)
    eager.run()
    torch.cuda.synchronize()
    ref_out = eager.out.clone()
    ref_k, ref_v = eager.k_cache.clone(), eager.v_cache.clone()
    if config == 2:
        assert eager.counts.num_decode_merges > 0 and eager.counts.num_chunk_merges > 0

    ds = DeviceStep(w, with_lse=False)
    g = ds.capture()
    torch.cuda.synchronize()
    for rep in range(3):
        ds.out.fill_(0)                        # eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(ds.out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert torch.equal(ds.k_cache.view(torch.int16), ref_k.view(torch.int16)), rep
        assert torch.equal(ds.v_cache.view(torch.int16), ref_v.view(torch.int16)), rep


def _random_case(seed):
    """A small random mixed step: supported head shapes, decode contexts from
    0 to 3000, chunks of 1 to 300 tokens at prefixes from 0 to 2000, and
    random split settings."""
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8])) if G < 8 else int(rng.choice([1, 2, 4]))
    D = int(rng.choice([64, 128]))
    dec = rng.integers(0, 3001, size=int(rng.integers(0, 7))).tolist()
    chunks = []
    for _ in range(int(rng.integers(0 if dec else 1, 4))):
        c = int(rng.integers(0, 2001))
        chunks.append((c, c + int(rng.integers(1, 301))))
    dsplit = int(rng.choice([0, 0, 16, 64, 256]))
    csplit = int(rng.choice([0, 0, 64, 192]))
    return G * Hkv, Hkv, D, dec, chunks, dsplit, csplit


@pytest.mark.parametrize("seed", range(24))
def test_random_mixed_steps(seed):
    Hq, Hkv, D, dec, chunks, dsplit, csplit = _random_case(7000 + seed)
    w = workloads.random_workload(7000 + seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  decode_ctx=dec, chunks=chunks)
    check_step(w, decode_split_tokens=dsplit, chunk_split_tokens=csplit,
               label=f"random{seed} Hq={Hq} Hkv={Hkv} D={D} dec={dec} chunks={chunks} "
                     f"splits={dsplit}/{csplit}")
