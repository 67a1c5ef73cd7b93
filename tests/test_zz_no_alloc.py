"""cpa_attention_noalloc against cpa_attention, through the C ABI.

The no-allocation entry point runs the same kernels with the split pieces'
partial results in the library's own device array instead of a caller's
workspace.  Two calls in a row, the second on a smaller step (the array keeps
the first call's contents), must each give the same bits as cpa_attention on
the same inputs, and the oracle's outputs within the usual tolerance; a plan
whose partials do not fit the array is rejected before any launch.
"""

import ctypes

import numpy as np
import pytest

import oracle
from chunked_prefill_mixed_amd import cpa, workloads
from chunked_prefill_mixed_amd.step import DeviceStep

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2

# decode rows and chunks with long enough prefixes that both decode and chunk
# pieces are split (split sizes below), the second step smaller than the first
STEPS = [
    dict(seed=2101, Hq=32, Hkv=8, D=128, dec=[3000, 1800, 77, 700], chunks=[(2500, 2660), (0, 90)],
         dsplit=128, csplit=256),
    dict(seed=2102, Hq=16, Hkv=4, D=64, dec=[900, 33], chunks=[(640, 700)], dsplit=64,
         csplit=128),
]


def _noalloc_call(ds, out, lse):
    import torch
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    w = ds.w
    return cpa.load().cpa_attention_noalloc(
        P(ds.q), P(ds.k_cache), P(ds.v_cache), P(ds.block_table), int(ds.block_table.shape[1]),
        P(ds.query_start_loc), P(ds.seq_lens), P(ds.context_lens), P(ds.plan),
        ctypes.byref(ds.counts), ds.num_seqs, ds.num_decodes, ds.num_tokens, w.num_q_heads,
        w.num_kv_heads, w.head_dim, 16, ctypes.c_float(w.scale), P(out), P(lse), stream)


def test_noalloc_matches_workspace_entry_point():
    import torch
    assert torch.cuda.is_available()
    for k, st in enumerate(STEPS):
        w = workloads.random_workload(st["seed"], num_q_heads=st["Hq"], num_kv_heads=st["Hkv"],
                                      head_dim=st["D"], decode_ctx=st["dec"], chunks=st["chunks"])
        ds = DeviceStep(w, decode_split_tokens=st["dsplit"], chunk_split_tokens=st["csplit"])
        c = ds.counts
        assert c.num_decode_merges > 0 and c.num_chunk_merges > 0, k
        need = cpa.cpa_workspace_size(c, w.num_q_heads, w.num_kv_heads, w.head_dim)
        assert 0 < need <= cpa.NOALLOC_SCRATCH_BYTES
        ds.run()  # append, then cpa_attention with a caller's workspace
        torch.cuda.synchronize()
        out = torch.full_like(ds.out, float("nan"))
        lse = torch.full_like(ds.lse, float("nan"))
        assert _noalloc_call(ds, out, lse) == cpa.CPA_OK
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ds.out.view(torch.int16)), k
        assert torch.equal(lse, ds.lse), k
        # and the oracle, to the parity bar
        T = ds.num_tokens
        bt = w.block_table[ds.meta["order"]]
        kp, vp = oracle.append(w.k_pool, w.v_pool, w.k_new[:T], w.v_new[:T],
                               ds.meta["query_start_loc"], ds.meta["context_lens"], bt)
        ref, _ = oracle.attention(w.q[:T], kp, vp, ds.meta["query_start_loc"],
                                  ds.meta["context_lens"], bt, w.num_kv_heads, w.scale)
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        assert np.max(np.abs(got - ref)) <= OUT_TOL, k


def test_noalloc_rejects_partials_beyond_its_array():
    """Counts whose partials exceed the array: CPA_ERR_CAPACITY, nothing
    launched (the output keeps its bits)."""
    import torch
    w = workloads.random_workload(2103, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                  decode_ctx=[300], chunks=[])
    ds = DeviceStep(w, decode_split_tokens=64)
    ds.append()
    big = ds.counts.copy(num_decode_partials=1 << 20)  # 1M slots x 8 heads x 130 x 4 B
    assert cpa.cpa_workspace_size(big, 8, 2, 128) > cpa.NOALLOC_SCRATCH_BYTES
    ds.counts = big
    out = torch.full_like(ds.out, 3.0)
    before = out.clone()
    assert _noalloc_call(ds, out, None) == cpa.CPA_ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.equal(out, before)
