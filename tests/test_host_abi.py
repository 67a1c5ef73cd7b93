"""Host-side tests of libcpa.so (no GPU needed): the library loads and exports
every symbol include/cpa.h declares; cpa_build_metadata agrees with the
oracle's scheduler element for element, reproduces the pages' worked
numbers, reports every error path, and emits a work plan that covers each
row exactly once."""

import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from chunked_prefill_mixed_amd import cpa, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "cpa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert set(syms) == set(cpa.EXPORTED)
    for s in syms:
        assert hasattr(lib, s), s
    import subprocess
    nm = subprocess.run(["nm", "-D", "--defined-only", cpa.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (cpa_\w+)", nm))
    assert set(syms) <= exported


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5):
        assert cpa.cpa_status_string(st).startswith("CPA_")
    assert "unknown" in cpa.cpa_status_string(7)


def build(reqs, budget, cap=0, Hq=32, Hkv=8, D=128, **kw):
    return cpa.cpa_build_metadata(reqs, token_budget=budget, long_prefill_cap=cap,
                                  num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, **kw)


def same_as_oracle(reqs, budget, cap=0, **kw):
    got = build(reqs, budget, cap, **kw)
    pol = {k: kw[k] for k in ("policy", "max_prefill_tokens", "adaptive", "block_aligned")
           if k in kw}
    ref = oracle.schedule([oracle.Request(r.id, r.num_computed, r.target_len, bool(r.is_decode))
                           for r in reqs], budget, cap, **pol)
    for k in ("order", "num_scheduled", "query_start_loc", "seq_lens", "context_lens", "new_blocks"):
        assert list(got[k]) == list(ref[k]), k
    for k in ("num_seqs", "num_decodes", "num_tokens"):
        assert got[k] == ref[k], k
    return got


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_builder_matches_oracle_on_configs(lib, config):
    for inst in range(workloads.num_instances(config)):
        w = workloads.make_workload(config, inst)
        got = same_as_oracle(w.requests, w.token_budget, w.long_prefill_cap,
                             Hq=w.num_q_heads, Hkv=w.num_kv_heads, D=w.head_dim,
                             host_block_table=w.block_table, num_blocks=w.num_blocks)
        check_plan(got, w.num_q_heads // w.num_kv_heads, w.head_dim, w.num_kv_heads)
        # slot mapping: page * 16 + slot of every scheduled token (checked here
        # with the test's own indexing)
        sm = got["slot_mapping"]
        for s in range(got["num_seqs"]):
            r = w.requests[got["order"][s]]
            for i in range(got["num_scheduled"][s]):
                p = r.num_computed + i
                t = got["query_start_loc"][s] + i
                assert sm[t] == w.block_table[got["order"][s], p // 16] * 16 + p % 16
        if config >= 4:
            break


def chunk_rows(head_dim):
    """(token, head) rows of a chunk tile, as include/cpa.h states them."""
    return 256 if head_dim == 128 else 128


def check_plan(m, group, head_dim, num_kv_heads=8):
    """Every decode row's keys are covered exactly once by page-aligned splits;
    merges list exactly the rows with several splits.  Every chunk row's
    tokens are covered by tiles of R/G tokens (R rows per tile); each tile's keys
    [0, context + q_end) are covered exactly once by pieces whose inner
    boundaries are 64-key aligned and lie in the fully visible prefix
    (<= context + q_begin); split tiles have a merge entry; pieces come
    longest first."""
    sec = cpa.plan_sections(m["plan"], m["counts"])
    nd = m["num_decodes"]
    cover = {s: [] for s in range(nd)}
    slots = []
    for row, b, e, slot in sec["decode_splits"]:
        assert 0 <= row < nd and b % 16 == 0 and b < e
        cover[row].append((b, e, slot))
        if slot >= 0:
            slots.append(slot)
    merged = {row: (first, n) for row, first, n, _ in sec["decode_merges"]}
    assert len(merged) == m["counts"].num_decode_merges
    for s in range(nd):
        pieces = sorted(cover[s])
        assert pieces[0][0] == 0 and pieces[-1][1] == m["seq_lens"][s]
        for (b0, e0, _), (b1, _, _) in zip(pieces, pieces[1:]):
            assert e0 == b1
        if len(pieces) == 1:
            assert pieces[0][2] == -1 and s not in merged
        else:
            first, n = merged[s]
            assert n == len(pieces)
            assert sorted(p[2] for p in pieces) == list(range(first, first + n))
    assert sorted(slots) == list(range(m["counts"].num_decode_partials))

    tt = chunk_rows(head_dim) // group
    tiles = {}
    cslots = []
    for row, qb, qe, kb, ke, slot, z0, z1 in sec["chunk_tiles"]:
        assert nd <= row < m["num_seqs"] and 0 <= qb < qe <= m["num_scheduled"][row]
        assert qe - qb <= tt and qb % tt == 0 and z0 == 0 and z1 == 0
        tiles.setdefault((row, qb, qe), []).append((kb, ke, slot))
        if slot >= 0:
            cslots.append(slot)
    cmerged = {(row, qb, qe): (first, n) for row, qb, qe, first, n, *_ in sec["chunk_merges"]}
    assert len(cmerged) == m["counts"].num_chunk_merges
    for s in range(nd, m["num_seqs"]):
        spans = sorted((qb, qe) for (row, qb, qe) in tiles if row == s)
        assert spans[0][0] == 0 and spans[-1][1] == m["num_scheduled"][s]
        for (a0, b0), (a1, _) in zip(spans, spans[1:]):
            assert b0 == a1
    for (row, qb, qe), pcs in tiles.items():
        c = m["context_lens"][row]
        pcs.sort()
        assert pcs[0][0] == 0 and pcs[-1][1] == c + qe
        for (b0, e0, _), (b1, _, _) in zip(pcs, pcs[1:]):
            assert e0 == b1 and e0 % 64 == 0 and e0 <= c + qb
        if len(pcs) == 1:
            assert pcs[0][2] == -1 and (row, qb, qe) not in cmerged
        else:
            first, n = cmerged[(row, qb, qe)]
            assert n == len(pcs)
            assert sorted(p[2] for p in pcs) == list(range(first, first + n))
    assert sorted(cslots) == list(range(m["counts"].num_chunk_partials))
    # longest first; with fewer than 8 KV heads the list is dealt round-robin
    # into 8 / Hkv consecutive runs (one per XCD range of a head), each
    # longest first: interleaving the runs back gives the sorted list
    lens = [ke - kb for _, _, _, kb, ke, *_ in sec["chunk_tiles"]]
    f = 8 // num_kv_heads if num_kv_heads < 8 and 8 % num_kv_heads == 0 else 1
    P = len(lens)
    runs, at = [], 0
    for r in range(f):
        n = (P - r + f - 1) // f
        runs.append(lens[at:at + n])
        at += n
    assert [runs[j % f][j // f] for j in range(P)] == sorted(lens, reverse=True)


def users_and_prompt(running, prompt):
    reqs = [oracle.Request(i, 100 + i, 101 + i, True) for i in range(running)]
    reqs.append(oracle.Request(running, 0, prompt, False))
    return reqs


def test_builder_reproduces_page_pins(lib):
    # chunk = budget - running users ("Chunked Prefill", "Why a chunk can be nearly free")
    for budget, chunk in [(256, 224), (512, 480), (4096, 4064)]:
        m = build(users_and_prompt(32, 8192), budget)
        assert m["num_scheduled"][-1] == chunk
    # passes for an 8192-token prompt beside 32 users ("The budget points in two directions")
    for budget, passes in [(16384, 1), (2048, 5), (512, 18), (256, 37)]:
        reqs, n = users_and_prompt(32, 8192), 0
        while not reqs[-1].is_decode:
            m = build(reqs, budget)
            reqs = oracle.advance(reqs, {"order": list(m["order"]),
                                         "num_scheduled": list(m["num_scheduled"])})
            n += 1
        assert n == passes
    # budget floor
    with pytest.raises(cpa.CpaError) as e:
        build(users_and_prompt(32, 8192), 16)
    assert e.value.status == cpa.CPA_ERR_BUDGET
    # "05. Chunked Prefill" sections 2 and 4: {A:1, B:1, C:2048} = 2050
    reqs = [oracle.Request(0, 500, 501, True), oracle.Request(1, 900, 901, True),
            oracle.Request(2, 0, 8192, False)]
    m = build(reqs, 8192, 2048)
    assert list(m["num_scheduled"]) == [1, 1, 2048] and m["num_tokens"] == 2050
    # tbr8.org 4.2: 2500 tokens need 157 pages
    m = build([oracle.Request(0, 0, 2500, False)], 4096)
    assert list(m["new_blocks"]) == [157]


def test_builder_random_mixes_match_oracle(lib):
    rng = np.random.default_rng(2024)
    for _ in range(300):
        n = int(rng.integers(0, 40))
        reqs = []
        for i in range(n):
            if rng.random() < 0.6:
                c = int(rng.integers(0, 5000))
                reqs.append(oracle.Request(i, c, c + 1, True))
            else:
                L = int(rng.integers(1, 9000))
                c = int(rng.integers(0, L + 1))
                reqs.append(oracle.Request(i, c, L, False))
        ndec = sum(r.is_decode for r in reqs)
        budget = int(rng.integers(max(1, ndec), ndec + 9000))
        cap = int(rng.choice([0, 0, 16, 100, 2048]))
        G = int(rng.choice([1, 2, 4, 8]))
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 8]))
        split = int(rng.choice([0, 0, 16, 128, 512]))
        csplit = int(rng.choice([0, 0, 64, 256, 1024]))
        m = same_as_oracle(reqs, budget, cap, Hq=G * Hkv, Hkv=Hkv, D=D, decode_split_tokens=split,
                           chunk_split_tokens=csplit)
        check_plan(m, G, D, Hkv)


@pytest.mark.parametrize("G,D", [(3, 128), (5, 64), (7, 128), (12, 64), (16, 128), (17, 128),
                                 (29, 64), (48, 128), (128, 64), (256, 128)])
def test_builder_plans_any_group(lib, G, D):
    """Groups outside 1, 2, 4, 8, up to one tile's rows: the schedule is the
    oracle's and the plan covers every key and query once, with tiles of
    floor(R / G) tokens."""
    rng = np.random.default_rng(9100 + G + D)
    for _ in range(20):
        reqs = []
        for i in range(int(rng.integers(1, 30))):
            if rng.random() < 0.5:
                c = int(rng.integers(0, 6000))
                reqs.append(oracle.Request(i, c, c + 1, True))
            else:
                L = int(rng.integers(1, 3000))
                c = int(rng.integers(0, L + 1))
                reqs.append(oracle.Request(i, c, L, False))
        ndec = sum(r.is_decode for r in reqs)
        budget = int(rng.integers(max(1, ndec), ndec + 4000))
        Hkv = int(rng.choice([1, 2]))
        m = same_as_oracle(reqs, budget, 0, Hq=G * Hkv, Hkv=Hkv, D=D)
        check_plan(m, G, D, Hkv)


def test_decode_pieces_count_the_waves_of_wide_groups(lib):
    """A group of more than 32 heads takes one decode wave per 32 heads (two
    blocks of 16 columns per wave), so the planner cuts the rows into fewer
    pieces for the same wave budget; up to 32 heads take one wave."""
    reqs = [oracle.Request(i, 3000 + 37 * i, 3001 + 37 * i, True) for i in range(40)]
    pieces = {}
    for G in (16, 32, 64, 128):
        m = cpa.cpa_build_metadata(reqs, token_budget=64, long_prefill_cap=0, num_q_heads=G,
                                   num_kv_heads=1, head_dim=128)
        pieces[G] = m["counts"].num_decode_splits
    assert pieces[16] == pieces[32] > pieces[64] > pieces[128] >= len(reqs)


@pytest.mark.parametrize("policy", ["truncate", "defer", "quota"])
@pytest.mark.parametrize("adaptive", [False, True])
@pytest.mark.parametrize("block_aligned", [False, True])
def test_builder_policies_match_oracle(lib, policy, adaptive, block_aligned):
    """The library's budget policies (tbr8.org deep dive 3.1, 3.2, 7.1) give
    the oracle's schedule on random mixes, including decode counts on both
    sides of the quota's 70% line and of the adaptive cap's 10 / 50 steps."""
    rng = np.random.default_rng(7000 + 4 * ["truncate", "defer", "quota"].index(policy)
                                + 2 * adaptive + block_aligned)
    for _ in range(150):
        n = int(rng.integers(0, 80))
        pdec = float(rng.choice([0.0, 0.3, 0.7, 0.95]))
        reqs = []
        for i in range(n):
            if rng.random() < pdec:
                c = int(rng.integers(0, 3000))
                reqs.append(oracle.Request(i, c, c + 1, True))
            else:
                L = int(rng.integers(1, 3000))
                c = int(rng.integers(0, L + 1))
                reqs.append(oracle.Request(i, c, L, False))
        ndec = sum(r.is_decode for r in reqs)
        budget = int(rng.integers(max(1, ndec), max(2, ndec + int(rng.choice([8, 200, 4000])))))
        cap = int(rng.choice([16, 100, 512])) if adaptive else int(rng.choice([0, 0, 16, 512]))
        kw = dict(policy=policy, adaptive=adaptive, block_aligned=block_aligned)
        if policy == "quota":
            kw["max_prefill_tokens"] = int(rng.choice([1, 64, 1000, 6000]))
        G = int(rng.choice([1, 4, 8]))
        m = same_as_oracle(reqs, budget, cap, Hq=G * 2, Hkv=2, D=128, **kw)
        check_plan(m, G, 128, 2)
        if policy != "quota":
            assert m["num_tokens"] <= budget
        else:
            assert m["num_tokens"] <= max(budget, ndec + kw["max_prefill_tokens"])


def test_builder_quota_step_may_exceed_budget(lib):
    """3.2's quota is its own prefill budget: with 10 decodes in a 64-token
    budget (under 70%), a 200-token quota schedules 200 prefill tokens; at 50
    decodes (over 70%) the quota falls back to the 14 the budget leaves."""
    R = oracle.Request
    reqs = [R(i, 30, 31, True) for i in range(10)] + [R(10, 0, 500, False)]
    m = same_as_oracle(reqs, 64, policy="quota", max_prefill_tokens=200)
    assert m["num_tokens"] == 210 and m["num_scheduled"][-1] == 200
    reqs = [R(i, 30, 31, True) for i in range(50)] + [R(50, 0, 500, False)]
    m = same_as_oracle(reqs, 64, policy="quota", max_prefill_tokens=200)
    assert m["num_tokens"] == 64 and m["num_scheduled"][-1] == 14


def test_builder_defer_stops_at_first_misfit(lib):
    """3.1: a chunk that does not fit the remaining budget is not cut down;
    the scan ends there even if a later, smaller prompt would fit."""
    R = oracle.Request
    reqs = [R(0, 10, 11, True), R(1, 0, 40, False), R(2, 0, 100, False), R(3, 0, 5, False)]
    m = same_as_oracle(reqs, 64, policy="defer")
    assert list(m["order"]) == [0, 1] and list(m["num_scheduled"]) == [1, 40]
    m = same_as_oracle(reqs, 64, policy="truncate")
    assert list(m["order"]) == [0, 1, 2] and list(m["num_scheduled"]) == [1, 40, 23]


def test_builder_block_aligned_case(lib):
    """The page-boundary rule on the oracle's hand-worked case: 32 streams,
    budget 512, a prompt at 100 gets 476 tokens (ends at page boundary 576)
    and the 4 left go to the next prompt."""
    R = oracle.Request
    reqs = [R(i, 30, 31, True) for i in range(32)] + [R(32, 100, 8192, False), R(33, 0, 100, False)]
    m = same_as_oracle(reqs, 512, block_aligned=True)
    assert list(m["num_scheduled"][32:]) == [476, 4] and m["seq_lens"][32] == 576


def test_builder_rejects_unknown_policy_value(lib):
    """The C entry point itself rejects policy values it does not define."""
    reqs = (cpa.cpa_req_t * 1)(cpa.cpa_req_t(0, 0, 10, 0))
    bufs = [np.zeros(2, dtype=np.int32) for _ in range(6)]
    for pol, quota, cap, ok in [(3, 0, 0, False), (0x800, 0, 0, False), (-1, 0, 0, False),
                                (2, 0, 0, False), (2, 2**31 - 64, 0, False), (2, 8, 0, True),
                                (0x100, 0, 0, False), (0x101, 0, 16, True), (0, 0, 0, True),
                                (0x200, 0, 0, True), (0x302, 8, 16, True), (0x400, 0, 0, False)]:
        params = cpa.cpa_build_params_t(64, cap, 16, 8, 2, 128, 0, 0, pol, quota)
        meta = cpa.cpa_meta_t()
        meta.max_seqs = 1
        meta.order, meta.num_scheduled, meta.query_start_loc, meta.seq_lens, meta.context_lens, \
            meta.new_blocks = [b.ctypes.data_as(cpa.i32p) for b in bufs]
        st = lib.cpa_build_metadata(reqs, 1, params, None, 0, 0, meta)
        assert (st == cpa.CPA_OK) == ok, (pol, quota, cap, st)
        if not ok:
            assert st == cpa.CPA_ERR_INVALID


@pytest.mark.parametrize("case,status", [
    ("budget_zero", cpa.CPA_ERR_INVALID),
    ("negative_computed", cpa.CPA_ERR_INVALID),
    ("target_below_computed", cpa.CPA_ERR_INVALID),
    ("decodes_over_budget", cpa.CPA_ERR_BUDGET),
    ("head_dim_96", cpa.CPA_ERR_UNSUPPORTED),
    ("group_over_tile_rows", cpa.CPA_ERR_UNSUPPORTED),
    ("group_over_tile_rows_d64", cpa.CPA_ERR_UNSUPPORTED),
    ("heads_not_multiple", cpa.CPA_ERR_UNSUPPORTED),
    ("block_size_32", cpa.CPA_ERR_UNSUPPORTED),
    ("kv_heads_over_256", cpa.CPA_ERR_UNSUPPORTED),
    ("split_not_page_multiple", cpa.CPA_ERR_INVALID),
    ("split_over_64_pages", cpa.CPA_ERR_INVALID),
    ("chunk_split_not_tile_multiple", cpa.CPA_ERR_INVALID),
    ("block_table_too_short", cpa.CPA_ERR_INVALID),
    ("block_id_out_of_range", cpa.CPA_ERR_INVALID),
    ("duplicate_slot", cpa.CPA_ERR_INVALID),
    ("fresh_slot_is_cached_elsewhere", cpa.CPA_ERR_INVALID),
    ("quota_without_max_prefill", cpa.CPA_ERR_INVALID),
    ("adaptive_without_cap", cpa.CPA_ERR_INVALID),
])
def test_builder_error_paths(lib, case, status):
    R = oracle.Request
    reqs = [R(0, 20, 21, True), R(1, 0, 40, False)]
    kw = dict(budget=64)
    bt = np.array([[0, 1, 9], [2, 3, 4]], dtype=np.int32)
    args = dict(Hq=8, Hkv=2, D=128)
    if case == "budget_zero":
        kw["budget"] = 0
    elif case == "negative_computed":
        reqs[0] = R(0, -1, 0, True)
    elif case == "target_below_computed":
        reqs[1] = R(1, 50, 40, False)
    elif case == "decodes_over_budget":
        reqs = [R(i, 5, 6, True) for i in range(10)]
        kw["budget"] = 9
    elif case == "head_dim_96":
        args["D"] = 96
    elif case == "group_over_tile_rows":  # a tile of 256 rows holds no token of 257 heads
        args.update(Hq=257, Hkv=1)
    elif case == "group_over_tile_rows_d64":
        args.update(Hq=129, Hkv=1, D=64)
    elif case == "heads_not_multiple":
        args.update(Hq=7, Hkv=2)
    elif case == "block_size_32":
        kw["block_size"] = 32
    elif case == "kv_heads_over_256":
        args.update(Hq=257, Hkv=257)
    elif case == "split_not_page_multiple":
        kw["decode_split_tokens"] = 24
    elif case == "split_over_64_pages":
        kw["decode_split_tokens"] = 1040
    elif case == "chunk_split_not_tile_multiple":
        kw["chunk_split_tokens"] = 80
    elif case == "block_table_too_short":
        kw.update(host_block_table=bt[:, :2], num_blocks=10)
    elif case == "block_id_out_of_range":
        kw.update(host_block_table=bt, num_blocks=4)  # row 1 uses page id 4
    elif case == "duplicate_slot":
        bt2 = bt.copy()
        bt2[1, 0] = 1  # row 1's first page is row 0's second page; both get written
        reqs[0] = R(0, 16, 17, True)
        kw.update(host_block_table=bt2, num_blocks=10)
    elif case == "fresh_slot_is_cached_elsewhere":
        bt2 = bt.copy()
        bt2[1, 0] = 0  # row 1 would overwrite positions row 0 reads as context
        kw.update(host_block_table=bt2, num_blocks=10)
    elif case == "quota_without_max_prefill":
        kw["policy"] = "quota"
    elif case == "adaptive_without_cap":
        kw["adaptive"] = True
    budget = kw.pop("budget")
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_build_metadata(reqs, token_budget=budget, long_prefill_cap=0,
                               num_q_heads=args["Hq"], num_kv_heads=args["Hkv"],
                               head_dim=args["D"], **kw)
    assert e.value.status == status


def test_builder_valid_block_table_accepted(lib):
    R = oracle.Request
    reqs = [R(0, 20, 21, True), R(1, 0, 40, False)]
    bt = np.array([[0, 1, 9], [2, 3, 4]], dtype=np.int32)
    m = cpa.cpa_build_metadata(reqs, token_budget=64, long_prefill_cap=0, num_q_heads=8,
                               num_kv_heads=2, head_dim=128, host_block_table=bt, num_blocks=10)
    assert m["slot_mapping"][0] == 1 * 16 + 4
    assert list(m["slot_mapping"][1:4]) == [32, 33, 34]


def test_workspace_size(lib):
    up = lambda b: math.ceil(b / 256) * 256
    c = cpa.cpa_plan_counts_t(5, 2, 3, 1, 7, 3)
    # decode slots: fp32 acc, m, l per query head; chunk slots: 8 KV heads x R
    # rows (256 at head_dim 128, 128 at 64), bf16 outputs and fp32 m, l
    want = (up(7 * 32 * 128 * 4) + 2 * up(7 * 32 * 4)
            + up(3 * 8 * 256 * 128 * 2) + 2 * up(3 * 8 * 256 * 4))
    assert cpa.cpa_workspace_size(c, 32, 8, 128) == want
    want64 = (up(7 * 32 * 64 * 4) + 2 * up(7 * 32 * 4)
              + up(3 * 8 * 128 * 64 * 2) + 2 * up(3 * 8 * 128 * 4))
    assert cpa.cpa_workspace_size(c, 32, 8, 64) == want64
    c0 = cpa.cpa_plan_counts_t(5, 0, 3, 0, 0, 0)
    assert cpa.cpa_workspace_size(c0, 32, 8, 128) == 0


def test_chunk_split_sizes(lib):
    """A small chunk beside a long prefix is cut into pieces (enough work for
    the GPU); a large chunk is not."""
    R = oracle.Request
    # Hq=32, Hkv=8, D=128: 256-row tiles of 64 tokens
    m = build([R(0, 7680, 8192, False)], 480)
    assert m["counts"].num_chunk_merges == 8 and m["counts"].num_chunk_tiles > 8
    m = build([R(0, 0, 8192, False)], 8192)
    assert m["counts"].num_chunk_merges == 0 and m["counts"].num_chunk_tiles == 128
    # D=64: 128-row tiles of 32 tokens
    m = build([R(0, 7680, 8192, False)], 480, D=64)
    assert m["counts"].num_chunk_merges == 15 and m["counts"].num_chunk_tiles > 15
    m = build([R(0, 7680, 8192, False)], 480, chunk_split_tokens=1 << 30)
    assert m["counts"].num_chunk_merges == 0


def test_empty_step(lib):
    m = build([], 16)
    assert m["num_seqs"] == 0 and m["num_tokens"] == 0
    assert m["counts"].num_decode_splits == 0 and m["counts"].num_chunk_tiles == 0


def test_budget_sweep_schedule(lib):
    """The budget sweep's steps follow the decode-first split: 32 streams plus
    an 8192-token prompt give chunks of B - 32 tokens and ceil(8192 / (B - 32))
    passes ("Chunked Prefill" (deepconcepts.dev): 224/480/4064-token chunks,
    37/18/5/1 passes at budgets 256/512/2048/8224), the last chunk taking the
    rest; the streams' contexts grow by one token per step."""
    from chunked_prefill_mixed_amd import sweep
    ctx = sweep.stream_contexts()
    assert len(ctx) == 32 and ctx.min() >= 512 and ctx.max() <= 4096
    for budget, chunk, passes in ((256, 224, 37), (512, 480, 18), (2048, 2016, 5),
                                  (4096, 4064, 3), (8224, 8192, 1)):
        steps = sweep.schedule(budget, ctx)
        assert len(steps) == passes, budget
        sizes = [int(m["num_scheduled"][32]) for _, m in steps]
        assert sizes[:-1] == [chunk] * (passes - 1) and sum(sizes) == 8192, budget
        for k, (reqs, m) in enumerate(steps):
            assert m["num_decodes"] == 32 and list(m["context_lens"][:32]) == list(ctx + k)
            assert m["context_lens"][32] == k * chunk
    with pytest.raises(ValueError):
        sweep.schedule(32, ctx)


def test_replay_chunk_scenario_schedule(lib):
    """The chunk-size replay: three streams and an 8000-token prompt with
    budget 3 + C give chunks of C tokens and ceil(8000 / C) passes (32/16/8/4
    at C = 256/512/1024/2048, one pass unchunked), the streams one token a
    step."""
    from chunked_prefill_mixed_amd import sweep
    scn = sweep.SCENARIOS["chunk"]
    ctx = sweep.stream_contexts(scn.seed, scn.streams, scn.ctx_lo, scn.ctx_hi)
    assert len(ctx) == 3 and ctx.min() >= 128 and ctx.max() <= 1024
    for C, passes in ((256, 32), (512, 16), (1024, 8), (2048, 4), (8000, 1)):
        steps = sweep.schedule(scn.budget(C), ctx, scn.prompt)
        assert len(steps) == passes, C
        sizes = [int(m["num_scheduled"][3]) for _, m in steps]
        assert sizes[:-1] == [C] * (passes - 1) and sum(sizes) == 8000, C
        for k, (_, m) in enumerate(steps):
            assert m["num_decodes"] == 3 and list(m["context_lens"][:3]) == list(ctx + k)


def test_replay_figures_arithmetic():
    """Replay figures from given step times: time to first token is the sum
    of the prompt's steps, the worst gap the longest step, the stall that
    minus the decode-only step, the streams' tokens streams x steps."""
    from chunked_prefill_mixed_amd import sweep
    f = sweep.replay_figures([100e-6, 250e-6, 150e-6], 80e-6, 32, ttft_unchunked=400e-6)
    assert f["steps"] == 3 and f["stream_tokens_during_prefill"] == 96
    assert math.isclose(f["ttft_ms"], 0.5) and math.isclose(f["worst_gap_us"], 250.0)
    assert math.isclose(f["stall_us"], 170.0) and math.isclose(f["mean_step_us"], 500 / 3)
    assert math.isclose(f["ttft_vs_unchunked"], 1.25)


def test_c_program_uses_the_abi(lib, tmp_path):
    """tests/c_abi/abi_check.c, compiled as C11 with -Wall -Werror against
    include/cpa.h and linked to libcpa.so, runs the host calls (page 1's
    512-token budget with 32 users; the budget floor) and prints ok."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    libdir = os.path.dirname(cpa.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(root, "include"),
                    os.path.join(here, "c_abi", "abi_check.c"), "-o", exe, "-L", libdir, "-lcpa",
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


@pytest.mark.parametrize("config", [2, 3])
def test_kv_shard_workload_is_one_gpus_share(config):
    """One GPU's share of a step split 8 ways by KV head: the same requests,
    pages and token count, with 4 query heads on 1 KV head."""
    full = workloads.make_workload(config, 1)
    part = workloads.make_workload(config, 1, kv_shard=8)
    assert (part.num_q_heads, part.num_kv_heads) == (4, 1)
    assert part.requests == full.requests and part.token_budget == full.token_budget
    assert np.array_equal(part.block_table, full.block_table)
    assert part.q.shape[1:] == (4, 128) and part.k_pool.shape[1] == 1
    with pytest.raises(ValueError):
        workloads.make_workload(config, 1, kv_shard=3)


def test_chunk_split_balances_uneven_tiles(lib):
    """Tiles of very different lengths that fill about one round of
    workgroups (one GPU's share of the heavy-mixed step at 2 KV heads) are
    cut into two or three rounds of pieces, so the round no longer waits for
    its longest tile; the causal tiles of a 2048-token chunk at prefix 0 at 8
    KV heads (one round, up to twice the mean) stay unsplit."""
    uneven = workloads.make_workload(5, 0, kv_shard=4)
    m = cpa.cpa_build_metadata(uneven.requests, token_budget=uneven.token_budget,
                               long_prefill_cap=0, num_q_heads=8, num_kv_heads=2, head_dim=128)
    wgs = m["counts"].num_chunk_tiles * 2
    assert 256 < wgs <= 3 * 256 and m["counts"].num_chunk_merges > 0
    check_plan(m, 4, 128, 2)
    causal = workloads.make_workload(3, 0)
    m = cpa.cpa_build_metadata(causal.requests, token_budget=causal.token_budget,
                               long_prefill_cap=causal.long_prefill_cap, num_q_heads=32,
                               num_kv_heads=8, head_dim=128)
    assert m["counts"].num_chunk_tiles * 8 == 256 and m["counts"].num_chunk_merges == 0
