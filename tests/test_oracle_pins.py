"""Pins for the fp64 oracle: every check here compares the oracle with something
it does not compute itself (pure-Python brute force on a dense, unpaged
layout; closed forms; torch's own attention routine; worked numbers printed on
the pages).  A second group plants plausible mistakes in the oracle and checks
that at least one pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import step as ostep

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BS = 16


# ---------------------------------------------------------------------------
# helpers written here, independently of the oracle
# ---------------------------------------------------------------------------

def bits(x):
    """float array -> bf16 bits by round-to-nearest-even (test-side copy)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def as_float(b):
    return [float(np.array([int(v) << 16], dtype=np.uint32).view(np.float32)[0]) for v in np.ravel(b)]


def page_dense(K, V, block_ids, num_blocks):
    """Place dense per-position K/V [L, Hkv, D] (bits) into fresh logical
    pools [num_blocks, Hkv, 16, D]: position p goes to page block_ids[p // 16],
    slot p % 16."""
    L, Hkv, D = K.shape
    kp = np.full((num_blocks, Hkv, BS, D), 0xFFFF, dtype=np.uint16)
    vp = np.full((num_blocks, Hkv, BS, D), 0xFFFF, dtype=np.uint16)
    for p in range(L):
        b = block_ids[p // BS]
        for g in range(Hkv):
            for d in range(D):
                kp[b, g, p % BS, d] = K[p, g, d]
                vp[b, g, p % BS, d] = V[p, g, d]
    return kp, vp


def brute_force(q_bits, K_bits, V_bits, c, scale, Hkv, with_lse=False):
    """Pure-Python loops over a dense layout: out[j][h][d] for a chunk of n
    queries at context c, explicit [n, c+n] visibility matrix (and lse[j][h]
    = log of the sum of exp(score) when asked)."""
    n, Hq, D = q_bits.shape
    G = Hq // Hkv
    L = c + n
    qf = np.array(as_float(q_bits)).reshape(n, Hq, D)
    Kf = np.array(as_float(K_bits)).reshape(L, Hkv, D)
    Vf = np.array(as_float(V_bits)).reshape(L, Hkv, D)
    mask = [[k <= c + j for k in range(L)] for j in range(n)]
    out = np.zeros((n, Hq, D))
    lse = np.zeros((n, Hq))
    for j in range(n):
        for h in range(Hq):
            g = h // G
            sc = []
            for k in range(L):
                if mask[j][k]:
                    dot = 0.0
                    for d in range(D):
                        dot += qf[j, h, d] * Kf[k, g, d]
                    sc.append((k, scale * dot))
            mx = max(v for _, v in sc)
            ws = [(k, math.exp(v - mx)) for k, v in sc]
            tot = sum(w for _, w in ws)
            lse[j, h] = mx + math.log(tot)
            for d in range(D):
                out[j, h, d] = sum(w * Vf[k, g, d] for k, w in ws) / tot
    return (out, lse) if with_lse else out


def random_case(rng, Hq, Hkv, D, c, n, num_blocks=None):
    L = c + n
    K = bits(rng.standard_normal((L, Hkv, D)))
    V = bits(rng.standard_normal((L, Hkv, D)))
    q = bits(rng.standard_normal((n, Hq, D)))
    npages = math.ceil(L / BS)
    nb = num_blocks or npages + 3
    ids = rng.permutation(nb)[:npages]
    return q, K, V, ids, nb


def run_oracle_chunk(q, K, V, ids, nb, c, Hkv, scale):
    """Oracle on paged inputs: prefix [0,c) placed by the test, chunk appended
    by oracle.append, then oracle.attention on one row."""
    n = q.shape[0]
    kp, vp = page_dense(K[:c], V[:c], ids, nb)
    bt = np.zeros((1, len(ids)), dtype=np.int32)
    bt[0, :] = ids
    kp, vp = oracle.append(kp, vp, K[c:], V[c:], [0, n], [c], bt)
    out, lse = oracle.attention(q, kp, vp, [0, n], [c], bt, Hkv, scale)
    return out, lse, kp, vp, bt


# ---------------------------------------------------------------------------
# C3 attention pins
# ---------------------------------------------------------------------------

BRUTE_CASES = [
    (Hq, G, D, c, n)
    for (Hq, G) in [(1, 1), (4, 1), (4, 2), (6, 3), (14, 7)]
    for D in (8, 16)
    for c in (0, 1, 15, 16, 17)
    for n in (1, 2, 5, 16)
]


@pytest.mark.parametrize("Hq,G,D,c,n", BRUTE_CASES)
def test_brute_force_dense(Hq, G, D, c, n):
    rng = np.random.default_rng(hash((Hq, G, D, c, n)) % 2**32)
    Hkv = Hq // G
    scale = 1.0 / math.sqrt(D)
    q, K, V, ids, nb = random_case(rng, Hq, Hkv, D, c, n)
    out, _, _, _, _ = run_oracle_chunk(q, K, V, ids, nb, c, Hkv, scale)
    ref = brute_force(q, K, V, c, scale, Hkv)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_softmax_rows_sum_to_one_and_reproduce_output():
    rng = np.random.default_rng(7)
    Hq, Hkv, D, c, n = 4, 2, 8, 21, 9
    scale = 0.3
    q, K, V, ids, nb = random_case(rng, Hq, Hkv, D, c, n)
    out, _, kp, vp, bt = run_oracle_chunk(q, K, V, ids, nb, c, Hkv, scale)
    Vf = np.array(as_float(V)).reshape(c + n, Hkv, D)
    for j in range(n):
        for h in range(Hq):
            w = oracle.softmax_weights(q, kp, bt[0], c, 0, j, h, Hkv, scale)
            assert w.shape == (c + j + 1,)
            assert abs(w.sum() - 1.0) < 1e-12
            assert np.all(w > 0)
            recon = w @ Vf[: c + j + 1, h // (Hq // Hkv)]
            assert np.max(np.abs(recon - out[j, h])) < 1e-12


@pytest.mark.parametrize("L", [256, 201])
def test_chunking_invariance(L):
    """Any chunk size gives the one-shot causal prefill's outputs (P2 section 3;
    P5 'The payoff'; P4 7.2 asks that chunked and unchunked prefill agree)."""
    rng = np.random.default_rng(L)
    Hq, Hkv, D = 4, 2, 16
    scale = 1.0 / math.sqrt(D)
    K = bits(rng.standard_normal((L, Hkv, D)))
    V = bits(rng.standard_normal((L, Hkv, D)))
    q = bits(rng.standard_normal((L, Hq, D)))
    npages = math.ceil(L / BS)
    nb = npages + 5
    ids = rng.permutation(nb)[:npages]
    bt = ids[None, :].astype(np.int32)
    results = {}
    for C in (1, 3, 16, 64, 100, L):
        kp = np.full((nb, Hkv, BS, D), 0xFFFF, dtype=np.uint16)
        vp = np.full((nb, Hkv, BS, D), 0xFFFF, dtype=np.uint16)
        outs = []
        for a in range(0, L, C):
            b = min(L, a + C)
            kp, vp = oracle.append(kp, vp, K[a:b], V[a:b], [0, b - a], [a], bt)
            o, _ = oracle.attention(q[a:b], kp, vp, [0, b - a], [a], bt, Hkv, scale)
            outs.append(o)
        results[C] = np.concatenate(outs)
    one_shot = results[L]
    for C, o in results.items():
        assert np.max(np.abs(o - one_shot)) < 1e-12, C


def test_decode_row_equals_last_prefill_row():
    rng = np.random.default_rng(11)
    Hq, Hkv, D, n = 8, 2, 32, 77
    scale = 1.0 / math.sqrt(D)
    q, K, V, ids, nb = random_case(rng, Hq, Hkv, D, 0, n)
    full, full_lse, _, _, _ = run_oracle_chunk(q, K, V, ids, nb, 0, Hkv, scale)
    dec, dec_lse, _, _, _ = run_oracle_chunk(q[n - 1:], K, V, ids, nb, n - 1, Hkv, scale)
    assert np.max(np.abs(dec[0] - full[n - 1])) < 1e-12
    assert np.max(np.abs(dec_lse[0] - full_lse[n - 1])) < 1e-12


def test_closed_form_single_key():
    """Context 0 and one query: the only visible key is the token itself, so the
    output is its V exactly and lse is its scaled score."""
    rng = np.random.default_rng(3)
    Hq, Hkv, D = 4, 4, 8
    q, K, V, ids, nb = random_case(rng, Hq, Hkv, D, 0, 1)
    out, lse, _, _, _ = run_oracle_chunk(q, K, V, ids, nb, 0, Hkv, 0.5)
    Vf = np.array(as_float(V)).reshape(1, Hkv, D)
    assert np.array_equal(out[0], Vf[0])
    qf = np.array(as_float(q)).reshape(1, Hq, D)
    Kf = np.array(as_float(K)).reshape(1, Hkv, D)
    assert np.allclose(lse[0], 0.5 * (qf[0] * Kf[0]).sum(-1), atol=1e-12)


@pytest.mark.parametrize("c", [0, 5, 16, 33])
def test_closed_form_zero_query_cumulative_mean(c):
    """q = 0 makes every visible key weigh the same, so row j is the mean of V
    over keys 0..c+j; consecutive rows show exactly which key became visible."""
    rng = np.random.default_rng(c + 100)
    Hq, Hkv, D, n = 4, 2, 8, 19
    _, K, V, ids, nb = random_case(rng, Hq, Hkv, D, c, n)
    q = np.zeros((n, Hq, D), dtype=np.uint16)
    out, lse, _, _, _ = run_oracle_chunk(q, K, V, ids, nb, c, Hkv, 0.125)
    Vf = np.array(as_float(V)).reshape(c + n, Hkv, D)
    G = Hq // Hkv
    for j in range(n):
        for h in range(Hq):
            mean = Vf[: c + j + 1, h // G].mean(axis=0)
            assert np.max(np.abs(out[j, h] - mean)) < 1e-12
            assert abs(lse[j, h] - math.log(c + j + 1)) < 1e-12


@pytest.mark.parametrize("c,n", [(0, 40), (37, 23), (64, 1)])
def test_matches_torch_sdpa_float64(c, n):
    """Library special case: torch's scaled_dot_product_attention in float64 on
    the CPU with an explicit boolean mask (c = 0 also with is_causal)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(c * 1000 + n)
    Hq, Hkv, D = 8, 2, 16
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    q, K, V, ids, nb = random_case(rng, Hq, Hkv, D, c, n)
    out, _, _, _, _ = run_oracle_chunk(q, K, V, ids, nb, c, Hkv, scale)
    qt = torch.tensor(as_float(q), dtype=torch.float64).reshape(n, Hq, D).permute(1, 0, 2)
    Kt = torch.tensor(as_float(K), dtype=torch.float64).reshape(c + n, Hkv, D).permute(1, 0, 2)
    Vt = torch.tensor(as_float(V), dtype=torch.float64).reshape(c + n, Hkv, D).permute(1, 0, 2)
    Kt = Kt.repeat_interleave(G, dim=0)
    Vt = Vt.repeat_interleave(G, dim=0)
    mask = torch.tensor([[k <= c + j for k in range(c + n)] for j in range(n)])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=scale)
    assert np.max(np.abs(ref.permute(1, 0, 2).numpy() - out)) < 1e-10
    if c == 0:
        ref2 = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True, scale=scale)
        assert np.max(np.abs(ref2.permute(1, 0, 2).numpy() - out)) < 1e-10


def test_token_subset_matches_full():
    rng = np.random.default_rng(5)
    Hq, Hkv, D, c, n = 4, 2, 8, 10, 30
    q, K, V, ids, nb = random_case(rng, Hq, Hkv, D, c, n)
    kp, vp = page_dense(K[:c], V[:c], ids, nb)
    bt = ids[None, :].astype(np.int32)
    kp, vp = oracle.append(kp, vp, K[c:], V[c:], [0, n], [c], bt)
    full, _ = oracle.attention(q, kp, vp, [0, n], [c], bt, Hkv, 0.3, row_chunk=7)
    sub, _ = oracle.attention(q, kp, vp, [0, n], [c], bt, Hkv, 0.3, tokens=np.array([0, 13, 29]))
    for t in (0, 13, 29):
        assert np.array_equal(sub[t], full[t])
    assert np.isnan(sub[1]).all()


# rows of a packed batch: (context, tokens this step); decodes (one token) first
PACKED_ROWS = [(0, 1), (17, 1), (33, 1), (13, 7), (0, 9), (31, 2)]


def packed_case(seed=2024, Hq=4, Hkv=2, D=8):
    """Dense per-row keys/values/queries of a packed batch, and a shared pool
    in which every row owns its own randomly placed pages."""
    rng = np.random.default_rng(seed)
    rows = []
    all_pages = sum(math.ceil((c + n) / BS) for c, n in PACKED_ROWS)
    nb = all_pages + 5
    ids = rng.permutation(nb)
    at = 0
    width = max(math.ceil((c + n) / BS) for c, n in PACKED_ROWS)
    bt = np.full((len(PACKED_ROWS), width), -1, dtype=np.int32)
    for s, (c, n) in enumerate(PACKED_ROWS):
        npg = math.ceil((c + n) / BS)
        bt[s, :npg] = ids[at:at + npg]
        at += npg
        rows.append(dict(c=c, n=n, K=bits(rng.standard_normal((c + n, Hkv, D))),
                         V=bits(rng.standard_normal((c + n, Hkv, D))),
                         q=bits(rng.standard_normal((n, Hq, D)))))
    return rows, bt, nb


def test_packed_rows_match_per_row_brute_force():
    """One packed batch of six rows -- three decode rows and three chunks with
    distinct contexts, each with its own pages of one shared pool -- through
    oracle.append and oracle.attention equals brute force on each row's own
    dense keys, for outputs and lse (P2 section 4: rows of one 1-D batch told
    apart by query_start_loc; P4 4.2: each request owns its page list)."""
    Hq, Hkv, D = 4, 2, 8
    scale = 0.35
    rows, bt, nb = packed_case(Hq=Hq, Hkv=Hkv, D=D)
    # prefixes placed by the test, row by row, into the shared pool
    kp = np.full((nb, Hkv, BS, D), 0xFFFF, dtype=np.uint16)
    vp = kp.copy()
    want_k, want_v = kp.copy(), vp.copy()
    for s, r in enumerate(rows):
        for p in range(r["c"] + r["n"]):
            b, o = bt[s, p // BS], p % BS
            want_k[b, :, o, :] = r["K"][p]
            want_v[b, :, o, :] = r["V"][p]
            if p < r["c"]:
                kp[b, :, o, :] = r["K"][p]
                vp[b, :, o, :] = r["V"][p]
    qsl = [0]
    for r in rows:
        qsl.append(qsl[-1] + r["n"])
    ctx = [r["c"] for r in rows]
    k_new = np.concatenate([r["K"][r["c"]:] for r in rows])
    v_new = np.concatenate([r["V"][r["c"]:] for r in rows])
    q = np.concatenate([r["q"] for r in rows])
    kp2, vp2 = oracle.append(kp, vp, k_new, v_new, qsl, ctx, bt)
    assert np.array_equal(kp2, want_k) and np.array_equal(vp2, want_v)
    out, lse = oracle.attention(q, kp2, vp2, qsl, ctx, bt, Hkv, scale)
    for s, r in enumerate(rows):
        ref, ref_lse = brute_force(r["q"], r["K"], r["V"], r["c"], scale, Hkv, with_lse=True)
        got = out[qsl[s]:qsl[s + 1]]
        assert np.max(np.abs(got - ref)) < 1e-12, s
        assert np.max(np.abs(lse[qsl[s]:qsl[s + 1]] - ref_lse)) < 1e-12, s


# ---------------------------------------------------------------------------
# C2 append pins
# ---------------------------------------------------------------------------

def test_append_touches_exactly_the_new_slots_and_is_idempotent():
    rng = np.random.default_rng(9)
    Hkv, D = 2, 8
    ctx = [0, 5, 16, 31]
    nq = [3, 1, 20, 16]
    nb = 40
    bt = rng.permutation(nb)[: 4 * 4].reshape(4, 4).astype(np.int32)
    T = sum(nq)
    qsl = np.concatenate([[0], np.cumsum(nq)]).tolist()
    kp0 = bits(rng.standard_normal((nb, Hkv, BS, D)))
    vp0 = bits(rng.standard_normal((nb, Hkv, BS, D)))
    kn = bits(rng.standard_normal((T, Hkv, D)))
    vn = bits(rng.standard_normal((T, Hkv, D)))
    kp, vp = oracle.append(kp0, vp0, kn, vn, qsl, ctx, bt)
    # slots each token must land in, listed here independently
    slots = set()
    for s in range(4):
        for i in range(nq[s]):
            p = ctx[s] + i
            slots.add((int(bt[s, p // BS]), p % BS))
            t = qsl[s] + i
            b, o = int(bt[s, p // BS]), p % BS
            # element (g, d) of slot o of page b, at its flat offset
            for g in range(Hkv):
                for d in range(D):
                    flat = ((b * Hkv + g) * BS + o) * D + d
                    assert kp.ravel()[flat] == kn[t, g, d]
                    assert vp.ravel()[flat] == vn[t, g, d]
    assert len(slots) == T  # injective
    kdiff = np.any(kp != kp0, axis=(1, 3))  # [nb, slot]
    vdiff = np.any(vp != vp0, axis=(1, 3))
    changed = {(b, o) for b, o in zip(*np.nonzero(kdiff | vdiff))}
    assert changed <= slots
    kp2, vp2 = oracle.append(kp, vp, kn, vn, qsl, ctx, bt)
    assert np.array_equal(kp2, kp) and np.array_equal(vp2, vp)
    # input pools are not modified
    assert not np.shares_memory(kp, kp0)


# ---------------------------------------------------------------------------
# C1 scheduler pins (worked numbers printed on the pages)
# ---------------------------------------------------------------------------

def load_pins():
    with open(os.path.join(GOLDEN, "scheduler_pins.json")) as f:
        return json.load(f)


def users_and_prompt(running, prompt):
    reqs = [oracle.Request(i, 100 + i, 101 + i, True) for i in range(running)]
    reqs.append(oracle.Request(running, 0, prompt, False))
    return reqs


def run_prompt(running, prompt, budget, cap=0):
    """Steps until the prompt is fully prefilled; returns (passes, tokens the
    running users received meanwhile, per-pass chunk sizes)."""
    reqs = users_and_prompt(running, prompt)
    passes, delivered, chunks = 0, 0, []
    while not reqs[-1].is_decode:
        sch = oracle.schedule(reqs, budget, cap)
        got = dict(zip(sch["order"], sch["num_scheduled"]))
        chunks.append(got.get(running, 0))
        delivered += sum(got.get(i, 0) for i in range(running))
        passes += 1
        reqs = oracle.advance(reqs, sch)
        assert passes < 10000
    return passes, delivered, chunks


def test_pin_chunk_size_vs_budget():
    pins = load_pins()["chunk_vs_budget"]
    for budget, chunk in pins["cases"]:
        sch = oracle.schedule(users_and_prompt(pins["running"], pins["prompt"]), budget)
        assert sch["num_scheduled"][-1] == chunk
        assert sch["num_tokens"] == budget


def test_pin_passes_and_delivered_tokens():
    pins = load_pins()["passes_for_prompt"]
    for case in pins["cases"]:
        passes, delivered, _ = run_prompt(pins["running"], pins["prompt"], case["budget"])
        assert passes == case["passes"]
        if "tokens_to_users" in case:
            assert delivered == case["tokens_to_users"]
    one = load_pins()["one_user"]
    passes, delivered, _ = run_prompt(one["running"], one["prompt"], one["budget"])
    assert passes == one["passes"] and delivered == one["tokens_to_users"]


def test_pin_budget_floor():
    pins = load_pins()["budget_floor"]
    with pytest.raises(oracle.BudgetError):
        oracle.schedule(users_and_prompt(pins["running"], 8192), pins["budget"])
    # exactly enough budget for the decodes is allowed; the prompt gets nothing
    sch = oracle.schedule(users_and_prompt(pins["running"], 8192), pins["running"])
    assert sch["num_seqs"] == pins["running"]


def test_pin_page2_step_table():
    pins = load_pins()["page2_step_table"]
    reqs = [oracle.Request(0, 500, 501, True), oracle.Request(1, 900, 901, True),
            oracle.Request(2, 0, pins["prompt"], False)]
    bounds = []
    for step in range(len(pins["chunk_bounds"])):
        sch = oracle.schedule(reqs, pins["budget"], pins["long_prefill_cap"])
        if step == 0:
            assert sch["num_scheduled"] == pins["scheduled_first_step"]
            assert sch["num_tokens"] == pins["total"]
            assert sch["query_start_loc"] == [0, 1, 2, 2050]
        c = sch["context_lens"][-1]
        bounds.append([c, c + sch["num_scheduled"][-1]])
        reqs = oracle.advance(reqs, sch)
    assert bounds == pins["chunk_bounds"]
    assert reqs[2].is_decode  # the prompt decodes from the next step on
    sch = oracle.schedule(reqs, pins["budget"], pins["long_prefill_cap"])
    assert sch["num_scheduled"] == [1, 1, 1] and sch["num_decodes"] == 3


def test_pin_page4_block_count():
    pins = load_pins()["page4_blocks"]
    sch = oracle.schedule([oracle.Request(0, 0, pins["tokens"], False)], 4096)
    assert sch["new_blocks"] == [pins["blocks"]]
    # a chunk that starts mid-page only needs the pages it newly reaches
    sch = oracle.schedule([oracle.Request(0, 20, 100, False)], 30)
    assert sch["new_blocks"] == [math.ceil(50 / 16) - math.ceil(20 / 16)]


def test_schedule_several_prefills_fcfs_and_skip():
    reqs = [oracle.Request(0, 0, 100, False), oracle.Request(1, 50, 50, False),
            oracle.Request(2, 10, 30, True), oracle.Request(3, 0, 500, False),
            oracle.Request(4, 0, 10, False)]
    sch = oracle.schedule(reqs, 160, 0)
    assert sch["order"] == [2, 0, 3]
    assert sch["num_scheduled"] == [1, 100, 59]
    assert sch["num_decodes"] == 1
    sch = oracle.schedule(reqs, 160, 40)
    assert sch["order"] == [2, 0, 3, 4]
    assert sch["num_scheduled"] == [1, 40, 40, 10]


# ---------------------------------------------------------------------------
# scheduler policy variants of the tbr8.org deep dive (3.1, 3.2, 7.1): outcomes
# worked out by hand from the printed rules, and invariants that tie each
# variant to the default (truncate) split pinned above
# ---------------------------------------------------------------------------

def _streams(n, ctx=100):
    return [oracle.Request(i, ctx, ctx + 1, True) for i in range(n)]


def test_policy_defer_follows_printed_rule():
    """3.1 as printed: chunk = min(remaining prompt, chunk_size); taken only
    if the remaining budget holds all of it, else the scan stops."""
    reqs = _streams(32) + [oracle.Request(32, 0, 1000, False), oracle.Request(33, 0, 100, False)]
    # no chunk size: the 1000-token prompt does not fit 512 - 32 = 480, and it
    # blocks the 100-token one behind it (truncate gives it 480 instead)
    d = oracle.schedule(reqs, 512, 0, policy="defer")
    assert d["num_tokens"] == 32 and d["num_seqs"] == 32
    assert oracle.schedule(reqs, 512, 0)["num_scheduled"][32:] == [480]
    # chunk size 256: 256 fits (224 left), then 100 fits (124 left)
    d = oracle.schedule(reqs, 512, 256, policy="defer")
    assert d["order"][32:] == [32, 33] and d["num_scheduled"][32:] == [256, 100]
    # chunk size 300 with budget 600: 300 fits (268 left), 100 fits
    d = oracle.schedule(reqs, 600, 300, policy="defer")
    assert d["num_scheduled"][32:] == [300, 100]
    # the scan stops at the first misfit even if a later one would fit
    reqs2 = _streams(2) + [oracle.Request(2, 0, 50, False), oracle.Request(3, 0, 400, False),
                           oracle.Request(4, 0, 10, False)]
    d = oracle.schedule(reqs2, 100, 0, policy="defer")
    assert d["order"] == [0, 1, 2] and d["num_scheduled"] == [1, 1, 50]


def test_policy_defer_equals_truncate_when_every_chunk_fits():
    rng = np.random.default_rng(7)
    for _ in range(50):
        ndec = int(rng.integers(0, 20))
        pre = [oracle.Request(ndec + i, int(c), int(c) + int(rng.integers(1, 300)), False)
               for i, c in enumerate(rng.integers(0, 1000, size=int(rng.integers(1, 5))))]
        cap = 64
        budget = ndec + cap * len(pre) + int(rng.integers(0, 50))  # every chunk fits
        reqs = _streams(ndec) + pre
        assert (oracle.schedule(reqs, budget, cap, policy="defer")
                == oracle.schedule(reqs, budget, cap))


def test_policy_quota_follows_printed_rule():
    """3.2: prefills get max_prefill_tokens of their own; once decodes take
    more than 70% of the total budget it drops to total - decodes."""
    prompt = oracle.Request(1000, 0, 8192, False)
    q = oracle.schedule(_streams(100) + [prompt], 1000, 0, policy="quota",
                        max_prefill_tokens=4096)
    assert q["num_scheduled"][100:] == [4096] and q["num_tokens"] == 4196
    q = oracle.schedule(_streams(700) + [prompt], 1000, 0, policy="quota",
                        max_prefill_tokens=4096)  # exactly 70%: quota unchanged
    assert q["num_scheduled"][700:] == [4096]
    q = oracle.schedule(_streams(701) + [prompt], 1000, 0, policy="quota",
                        max_prefill_tokens=4096)  # above 70%: 1000 - 701 left
    assert q["num_scheduled"][701:] == [299] and q["num_tokens"] == 1000
    # several prompts share the quota in queue order, each capped
    reqs = _streams(10) + [oracle.Request(10 + i, 0, 3000, False) for i in range(3)]
    q = oracle.schedule(reqs, 1000, 2048, policy="quota", max_prefill_tokens=4096)
    assert q["num_scheduled"][10:] == [2048, 2048]
    with pytest.raises(ValueError):
        oracle.schedule(reqs, 1000, 0, policy="quota")


def test_policy_quota_equals_truncate_with_matching_quota():
    rng = np.random.default_rng(11)
    for _ in range(50):
        budget = int(rng.integers(100, 5000))
        ndec = int(rng.integers(0, budget * 7 // 10))  # below 70%, so budget - ndec > 0
        pre = [oracle.Request(ndec + i, 0, int(rng.integers(1, 4000)), False)
               for i in range(int(rng.integers(1, 4)))]
        reqs = _streams(ndec) + pre
        assert (oracle.schedule(reqs, budget, 0, policy="quota", max_prefill_tokens=budget - ndec)
                == oracle.schedule(reqs, budget, 0))


def test_policy_adaptive_chunk_follows_queue_depth():
    """7.1: base chunk x4 with no decode, x2 under 10, x1 under 50, /2 beyond."""
    for ndec, want in ((0, 2048), (1, 1024), (9, 1024), (10, 512), (49, 512), (50, 256),
                       (300, 256)):
        reqs = _streams(ndec) + [oracle.Request(ndec, 0, 8192, False)]
        s = oracle.schedule(reqs, 9000, 512, adaptive=True)
        assert s["num_scheduled"][ndec:] == [want], ndec
        assert oracle.adaptive_chunk(512, ndec) == want
    assert oracle.adaptive_chunk(1, 60) == 1
    with pytest.raises(ValueError):
        oracle.schedule(_streams(3), 100, 0, adaptive=True)


def test_block_aligned_chunks_follow_the_rule():
    """A chunk cut short ends on a page boundary when that leaves it a token;
    the tokens it gives back go to the next prompt; a prompt's last chunk and
    a cut that would leave nothing are unchanged (hand-worked cases)."""
    R = oracle.Request
    reqs = _streams(32) + [R(32, 100, 8192, False), R(33, 0, 100, False)]
    assert oracle.schedule(reqs, 512)["num_scheduled"][32:] == [480]
    s = oracle.schedule(reqs, 512, block_aligned=True)
    assert s["num_scheduled"][32:] == [476, 4] and s["seq_lens"][32] == 576
    # the prompt's last chunk is not cut
    reqs = _streams(32) + [R(32, 100, 300, False)]
    assert oracle.schedule(reqs, 512, block_aligned=True)["num_scheduled"][32:] == [200]
    # 10 + 3 tokens cannot reach page boundary 16: the chunk keeps its 3
    reqs = _streams(32) + [R(32, 10, 500, False)]
    assert oracle.schedule(reqs, 35, block_aligned=True)["num_scheduled"][32:] == [3]
    # the page-2 step table (budget 8192, cap 2048) is already aligned
    reqs = _streams(2) + [R(2, 2048, 8192, False)]
    assert oracle.schedule(reqs, 8192, 2048, block_aligned=True)["num_scheduled"] == [1, 1, 2048]


def test_block_aligned_invariants_on_random_mixes():
    """Random mixes: every chunk that stops short of its prompt's end and
    could reach a page boundary ends on one; the step stays within the
    budget; with the flag off the split is the default one."""
    rng = np.random.default_rng(31)
    R = oracle.Request
    for _ in range(300):
        n = int(rng.integers(1, 30))
        reqs = []
        for i in range(n):
            if rng.random() < 0.5:
                c = int(rng.integers(0, 3000))
                reqs.append(R(i, c, c + 1, True))
            else:
                L = int(rng.integers(1, 3000))
                reqs.append(R(i, int(rng.integers(0, L + 1)), L, False))
        ndec = sum(r.is_decode for r in reqs)
        budget = int(rng.integers(max(1, ndec), ndec + 2000))
        cap = int(rng.choice([0, 0, 100, 512]))
        s = oracle.schedule(reqs, budget, cap, block_aligned=True)
        assert sum(s["num_scheduled"]) <= budget
        for i, nn, c in zip(s["order"], s["num_scheduled"], s["context_lens"]):
            r = reqs[i]
            if r.is_decode or nn == r.target_len - r.num_computed:
                continue
            if (c + nn) // oracle.BLOCK_SIZE * oracle.BLOCK_SIZE > c:
                assert (c + nn) % oracle.BLOCK_SIZE == 0, (c, nn)
        assert oracle.schedule(reqs, budget, cap, block_aligned=False) == oracle.schedule(
            reqs, budget, cap)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin above
# ---------------------------------------------------------------------------

def _pins_pass():
    try:
        for args in [(4, 2, 8, 17, 5), (4, 1, 8, 0, 16), (1, 1, 8, 16, 2)]:
            test_brute_force_dense(*args)
        test_closed_form_zero_query_cumulative_mean(5)
        test_decode_row_equals_last_prefill_row()
        test_packed_rows_match_per_row_brute_force()
    except AssertionError:
        return False
    return True


def test_pins_pass_unmutated():
    assert _pins_pass()


MUTATIONS = ["mask_off_by_one", "mask_strict", "head_map_modulo", "v_rows_reversed",
             "slot_reversed", "drop_scale", "rows_share_first_table", "rows_share_first_context",
             "append_drops_context"]


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_planted_mistake_is_caught(monkeypatch, mutation):
    if mutation == "mask_off_by_one":
        monkeypatch.setattr(ostep, "_visible", lambda pos, c, js: pos[None, :] <= (c + js + 1)[:, None])
    elif mutation == "mask_strict":
        monkeypatch.setattr(ostep, "_visible",
                            lambda pos, c, js: (pos[None, :] < (c + js)[:, None]) | (pos[None, :] == 0))
    elif mutation == "head_map_modulo":
        monkeypatch.setattr(ostep, "_kv_head", lambda h, G: h % 2 if G > 1 else h)
    elif mutation == "v_rows_reversed":
        orig = ostep._row_keys

        def bad(k_pool, v_pool, pages, g, length):
            Ks, Vs = orig(k_pool, v_pool, pages, g, length)
            return Ks, Vs[::-1].copy()
        monkeypatch.setattr(ostep, "_row_keys", bad)
    elif mutation == "slot_reversed":
        # key p read from slot 15 - p % 16 of its page instead of slot p % 16
        def bad(k_pool, v_pool, pages, g, length):
            pos = np.arange(length)
            blocks = np.asarray(pages)[pos // BS]
            offs = BS - 1 - pos % BS
            return (ostep.bf16_bits_to_f64(k_pool[blocks, g, offs, :]),
                    ostep.bf16_bits_to_f64(v_pool[blocks, g, offs, :]))
        monkeypatch.setattr(ostep, "_row_keys", bad)
    elif mutation == "drop_scale":
        orig_att = ostep.attention

        def no_scale(*a, **k):
            a = list(a)
            a[7] = 1.0
            return orig_att(*a, **k)
        monkeypatch.setattr(oracle, "attention", no_scale)
    elif mutation == "rows_share_first_table":
        # every packed row reads (and writes) the pages of row 0
        monkeypatch.setattr(ostep, "_pages", lambda block_table, s: np.asarray(block_table[0]))
    elif mutation == "rows_share_first_context":
        monkeypatch.setattr(ostep, "_context", lambda context_lens, s: int(context_lens[0]))
    elif mutation == "append_drops_context":
        # the append writes token t of a row at position t - qsl[s], as if the
        # row had no cached prefix; attention still reads the true context
        orig_ctx = ostep._context
        orig_append = ostep.append

        def append_no_ctx(*a, **k):
            monkeypatch.setattr(ostep, "_context", lambda context_lens, s: 0)
            try:
                return orig_append(*a, **k)
            finally:
                monkeypatch.setattr(ostep, "_context", orig_ctx)
        monkeypatch.setattr(oracle, "append", append_no_ctx)
    assert not _pins_pass()
