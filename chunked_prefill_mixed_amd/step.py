"""Device buffers for one mixed step and the two launches that run it.

Holds a workload's tensors in HBM (torch allocations), the step metadata
from ``cpa_build_metadata`` and the work plan, and calls ``cpa_append_kv``
then ``cpa_attention`` on the current stream.  No arithmetic of the step is
done here.
"""

from __future__ import annotations

import numpy as np

from . import cpa


def _bits_to_bf16(a, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bf16_to_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# The library's cache layout (include/cpa.h) made from logical pages
# [num_blocks, Hkv, 16, D] and back.  Pure data movement on the device.
def k_pages_to_cache(t):
    """[nb, Hkv, 16, D] -> K cache [nb, Hkv, D/8, 16, 8] (8-value pieces)."""
    nb, h, b, d = t.shape
    return t.reshape(nb, h, b, d // 8, 8).permute(0, 1, 3, 2, 4).contiguous()


def v_pages_to_cache(t):
    """[nb, Hkv, 16, D] -> V cache [nb, Hkv, D, 16] (transposed in a page)."""
    return t.permute(0, 1, 3, 2).contiguous()


def k_cache_to_pages(t):
    """K cache [nb, Hkv, D/8, 16, 8] -> [nb, Hkv, 16, D]."""
    nb, h, p, b, e = t.shape
    return t.permute(0, 1, 3, 2, 4).reshape(nb, h, b, p * e)


def v_cache_to_pages(t):
    """V cache [nb, Hkv, D, 16] -> [nb, Hkv, 16, D]."""
    return t.permute(0, 1, 3, 2)


def caches_from_pools(k_pool, v_pool, device):
    """Device K and V caches in the library's layout from logical uint16 pools."""
    return (k_pages_to_cache(_bits_to_bf16(k_pool, device)),
            v_pages_to_cache(_bits_to_bf16(v_pool, device)))


def pools_from_caches(k_cache, v_cache):
    """Logical uint16 pools [nb, Hkv, 16, D] of device caches."""
    return (bf16_to_bits(k_cache_to_pages(k_cache).contiguous()),
            bf16_to_bits(v_cache_to_pages(v_cache).contiguous()))


class DeviceStep:
    """One step of a workload, resident on the GPU."""

    def __init__(self, w, device="cuda", decode_split_tokens=0, chunk_split_tokens=0,
                 validate=True, with_lse=True):
        import torch
        self.w = w
        self.device = device
        self.meta = cpa.cpa_build_metadata(
            w.requests, token_budget=w.token_budget, long_prefill_cap=w.long_prefill_cap,
            num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
            decode_split_tokens=decode_split_tokens, chunk_split_tokens=chunk_split_tokens,
            host_block_table=w.block_table if validate else None, num_blocks=w.num_blocks)
        m = self.meta
        self.num_tokens = T = m["num_tokens"]
        self.num_seqs = m["num_seqs"]
        self.num_decodes = m["num_decodes"]
        self.counts = m["counts"]
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        bt_rows = w.block_table[m["order"]] if self.num_seqs else w.block_table[:1]
        self.block_table = i32(bt_rows)
        self.query_start_loc = i32(m["query_start_loc"])
        self.seq_lens = i32(m["seq_lens"])
        self.context_lens = i32(m["context_lens"])
        plan = m["plan"] if m["plan"].size else np.zeros(1, dtype=np.int32)
        self.plan = i32(plan)
        self.k_cache, self.v_cache = caches_from_pools(w.k_pool, w.v_pool, device)
        self.q = _bits_to_bf16(w.q[:T], device)
        self.k_new = _bits_to_bf16(w.k_new[:T], device)
        self.v_new = _bits_to_bf16(w.v_new[:T], device)
        self.out = torch.empty((T, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=device)
        self.lse = (torch.empty((T, w.num_q_heads), dtype=torch.float32, device=device)
                    if with_lse else None)
        ws = cpa.cpa_workspace_size(self.counts, w.num_q_heads, w.num_kv_heads, w.head_dim)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device) if ws else None
        self.scale = w.scale

    def append(self, stream=None):
        cpa.cpa_append_kv(self.k_new, self.v_new, self.query_start_loc, self.context_lens,
                          self.block_table, self.k_cache, self.v_cache, num_seqs=self.num_seqs,
                          num_tokens=self.num_tokens, stream=stream)

    def attention(self, stream=None):
        cpa.cpa_attention(self.q, self.k_cache, self.v_cache, self.block_table,
                          self.query_start_loc, self.seq_lens, self.context_lens, self.plan,
                          self.counts, num_seqs=self.num_seqs, num_decodes=self.num_decodes,
                          num_tokens=self.num_tokens, softmax_scale=self.scale, out=self.out,
                          lse=self.lse, workspace=self.workspace, stream=stream)

    def run(self, stream=None):
        self.append(stream)
        self.attention(stream)

    def capture(self):
        """The step (append, then attention) captured as one HIP graph (torch's
        CUDAGraph) on a capture stream.  Replaying it re-runs both calls on
        the same buffers; the library issues only kernel launches, so the
        graph holds no memset or copy nodes."""
        import torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()  # default priority
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            self.run(torch.cuda.current_stream())
        torch.cuda.current_stream().wait_stream(s)
        return g

    def _section_call(self, section, stream):
        """cpa_attention over one plan section only."""
        import ctypes
        import torch
        c = self.counts
        zero = dict(num_decode_splits=0, num_decode_merges=0, num_chunk_tiles=0,
                    num_chunk_merges=0)
        field = {"decode_splits": "num_decode_splits", "decode_merges": "num_decode_merges",
                 "chunk_tiles": "num_chunk_tiles", "chunk_merges": "num_chunk_merges"}[section]
        counts = c.copy(**{**zero, field: getattr(c, field)})
        off = cpa.section_offsets(c)[section]
        plan_view = self.plan[off:] if off < self.plan.numel() else self.plan
        cpa.cpa_attention(self.q, self.k_cache, self.v_cache, self.block_table,
                          self.query_start_loc, self.seq_lens, self.context_lens, plan_view,
                          counts, num_seqs=self.num_seqs, num_decodes=self.num_decodes,
                          num_tokens=self.num_tokens, softmax_scale=self.scale, out=self.out,
                          lse=self.lse, workspace=self.workspace, stream=stream)

    def run_two_streams(self, aux):
        """Append on the current stream, then the chunk sections on ``aux``
        concurrently with the decode sections; the current stream waits for
        both."""
        import torch
        main = torch.cuda.current_stream()
        self.append(main)
        appended = torch.cuda.Event()
        appended.record(main)
        aux.wait_event(appended)
        self._section_call("chunk_tiles", aux)
        self._section_call("chunk_merges", aux)
        self._section_call("decode_splits", main)
        self._section_call("decode_merges", main)
        done = torch.cuda.Event()
        done.record(aux)
        main.wait_event(done)

    # host copies for checking
    def pools_bits(self):
        """Both caches as logical pools [nb, Hkv, 16, D] of bf16 bits."""
        return pools_from_caches(self.k_cache, self.v_cache)

    def out_f64(self):
        import torch
        return self.out.detach().float().cpu().numpy().astype(np.float64)

    def lse_f64(self):
        return None if self.lse is None else self.lse.detach().cpu().numpy().astype(np.float64)
