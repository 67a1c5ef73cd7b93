"""Thin ctypes binding of libcpa.so: same call names as include/cpa.h.

Argument marshalling only.  Every step of the attention path runs inside the
library; torch is used for device memory (``data_ptr()``) and the current
HIP stream.  The library must be built (``__graft_entry__.build()``); a
missing library raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpa.so")

CPA_OK = 0
CPA_ERR_INVALID = -1
CPA_ERR_BUDGET = -2
CPA_ERR_CAPACITY = -3
CPA_ERR_UNSUPPORTED = -4
CPA_ERR_DEVICE = -5
BLOCK_SIZE = 16
DECODE_SPLIT_WORDS = 4
DECODE_MERGE_WORDS = 4
CHUNK_TILE_WORDS = 8
CHUNK_MERGE_WORDS = 8

EXPORTED = ("cpa_build_metadata", "cpa_append_kv", "cpa_workspace_size", "cpa_attention",
            "cpa_attention_noalloc", "cpa_status_string")
NOALLOC_SCRATCH_BYTES = 64 << 20  # CPA_NOALLOC_SCRATCH_BYTES

i32p = ctypes.POINTER(ctypes.c_int32)
i64p = ctypes.POINTER(ctypes.c_int64)


class CpaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {cpa_status_string(status)} ({status})")


class cpa_req_t(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("num_computed", ctypes.c_int32),
                ("target_len", ctypes.c_int32), ("is_decode", ctypes.c_int32)]


class cpa_build_params_t(ctypes.Structure):
    _fields_ = [("token_budget", ctypes.c_int32), ("long_prefill_cap", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("decode_split_tokens", ctypes.c_int32), ("chunk_split_tokens", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("max_prefill_tokens", ctypes.c_int32)]


# budget policies of cpa_build_metadata (values of include/cpa.h)
CPA_POLICY_TRUNCATE, CPA_POLICY_DEFER, CPA_POLICY_QUOTA = 0, 1, 2
CPA_POLICY_ADAPTIVE_CHUNK = 0x100
CPA_POLICY_BLOCK_ALIGNED = 0x200
POLICY_NAMES = {"truncate": CPA_POLICY_TRUNCATE, "defer": CPA_POLICY_DEFER,
                "quota": CPA_POLICY_QUOTA}


class cpa_plan_counts_t(ctypes.Structure):
    _fields_ = [("num_decode_splits", ctypes.c_int32), ("num_decode_merges", ctypes.c_int32),
                ("num_chunk_tiles", ctypes.c_int32), ("num_chunk_merges", ctypes.c_int32),
                ("num_decode_partials", ctypes.c_int32), ("num_chunk_partials", ctypes.c_int32)]

    def copy(self, **changes):
        vals = {f: getattr(self, f) for f, _ in self._fields_}
        vals.update(changes)
        return cpa_plan_counts_t(**vals)


class cpa_meta_t(ctypes.Structure):
    _fields_ = [("max_seqs", ctypes.c_int32), ("order", i32p), ("num_scheduled", i32p),
                ("query_start_loc", i32p), ("seq_lens", i32p), ("context_lens", i32p),
                ("new_blocks", i32p), ("max_tokens", ctypes.c_int32), ("slot_mapping", i64p),
                ("plan_capacity", ctypes.c_int32), ("plan", i32p), ("num_seqs", ctypes.c_int32),
                ("num_decodes", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("plan_words", ctypes.c_int32), ("counts", cpa_plan_counts_t)]


_lib = None


def _hip_runtimes_mapped() -> set:
    """Distinct libamdhip64 files mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1] if line.strip() else ""
                if "libamdhip64.so" in path:
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def load():
    """Load libcpa.so (once).  Raises if it has not been built.

    torch is imported first when it is installed: libcpa.so then binds to
    the HIP runtime torch already loaded (same soname) instead of mapping a
    second runtime next to it, which would give two device contexts in one
    process.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    vp = ctypes.c_void_p
    lib.cpa_build_metadata.argtypes = [ctypes.POINTER(cpa_req_t), ctypes.c_int,
                                       ctypes.POINTER(cpa_build_params_t), i32p, ctypes.c_int,
                                       ctypes.c_int, ctypes.POINTER(cpa_meta_t)]
    lib.cpa_build_metadata.restype = ctypes.c_int
    lib.cpa_append_kv.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.cpa_append_kv.restype = ctypes.c_int
    lib.cpa_workspace_size.argtypes = [ctypes.POINTER(cpa_plan_counts_t), ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int]
    lib.cpa_workspace_size.restype = ctypes.c_size_t
    lib.cpa_attention.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                  ctypes.POINTER(cpa_plan_counts_t), ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp]
    lib.cpa_attention.restype = ctypes.c_int
    lib.cpa_attention_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                          ctypes.POINTER(cpa_plan_counts_t), ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, vp]
    lib.cpa_attention_noalloc.restype = ctypes.c_int
    lib.cpa_status_string.argtypes = [ctypes.c_int]
    lib.cpa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def cpa_status_string(status: int) -> str:
    return load().cpa_status_string(int(status)).decode()


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(i32p)


def cpa_build_metadata(requests, *, token_budget, long_prefill_cap, num_q_heads, num_kv_heads,
                       head_dim, decode_split_tokens=0, chunk_split_tokens=0,
                       host_block_table=None, num_blocks=0, block_size=BLOCK_SIZE,
                       policy="truncate", max_prefill_tokens=0, adaptive=False,
                       block_aligned=False) -> dict:
    """Decode-first budget split + work plan (host only, no GPU needed).

    ``requests``: sequence of objects with id, num_computed, target_len,
    is_decode (queue order).  ``policy`` is "truncate", "defer" or "quota"
    (``max_prefill_tokens`` is the quota); ``adaptive`` scales
    ``long_prefill_cap`` with the decode count; ``block_aligned`` ends chunks
    cut short on page boundaries.  Returns numpy arrays and
    counts; raises CpaError on a non-OK status.
    """
    if policy not in POLICY_NAMES:
        raise ValueError(f"unknown policy {policy!r}")
    pol = (POLICY_NAMES[policy] | (CPA_POLICY_ADAPTIVE_CHUNK if adaptive else 0)
           | (CPA_POLICY_BLOCK_ALIGNED if block_aligned else 0))
    lib = load()
    n = len(requests)
    reqs = (cpa_req_t * max(1, n))()
    for i, r in enumerate(requests):
        reqs[i] = cpa_req_t(int(r.id), int(r.num_computed), int(r.target_len), int(bool(r.is_decode)))
    params = cpa_build_params_t(int(token_budget), int(long_prefill_cap), int(block_size),
                                int(num_q_heads), int(num_kv_heads), int(head_dim),
                                int(decode_split_tokens), int(chunk_split_tokens), pol,
                                int(max_prefill_tokens))
    max_seqs = max(1, n)
    bufs = {k: np.zeros(max_seqs + (1 if k == "query_start_loc" else 0), dtype=np.int32)
            for k in ("order", "num_scheduled", "query_start_loc", "seq_lens", "context_lens",
                      "new_blocks")}
    max_tokens = max(1, int(token_budget) + (int(max_prefill_tokens) if policy == "quota" else 0))
    slots = np.zeros(max_tokens, dtype=np.int64)
    bt_ptr, bt_stride = None, 0
    if host_block_table is not None:
        bt_arr, bt_ptr = _i32(host_block_table)
        bt_stride = bt_arr.shape[1]
    meta = cpa_meta_t()
    meta.max_seqs = max_seqs
    for k, a in bufs.items():
        setattr(meta, k, a.ctypes.data_as(i32p))
    meta.max_tokens = max_tokens
    meta.slot_mapping = slots.ctypes.data_as(i64p) if host_block_table is not None else None
    # first pass sizes the plan
    meta.plan_capacity = 0
    meta.plan = None
    st = lib.cpa_build_metadata(reqs, n, ctypes.byref(params), bt_ptr, bt_stride,
                                int(num_blocks), ctypes.byref(meta))
    if st != CPA_OK:
        raise CpaError(st, "cpa_build_metadata")
    plan = np.zeros(max(1, meta.plan_words), dtype=np.int32)
    meta.plan_capacity = plan.size
    meta.plan = plan.ctypes.data_as(i32p)
    st = lib.cpa_build_metadata(reqs, n, ctypes.byref(params), bt_ptr, bt_stride,
                                int(num_blocks), ctypes.byref(meta))
    if st != CPA_OK:
        raise CpaError(st, "cpa_build_metadata")
    ns = meta.num_seqs
    out = {k: (a[: ns + 1] if k == "query_start_loc" else a[:ns]).copy() for k, a in bufs.items()}
    out.update(
        num_seqs=ns, num_decodes=meta.num_decodes, num_tokens=meta.num_tokens,
        plan=plan[: meta.plan_words].copy(),
        counts=meta.counts.copy(),
    )
    if host_block_table is not None:
        out["slot_mapping"] = slots[: meta.num_tokens].copy()
    return out


SECTIONS = (("decode_splits", "num_decode_splits", DECODE_SPLIT_WORDS),
            ("chunk_tiles", "num_chunk_tiles", CHUNK_TILE_WORDS),
            ("decode_merges", "num_decode_merges", DECODE_MERGE_WORDS),
            ("chunk_merges", "num_chunk_merges", CHUNK_MERGE_WORDS))


def section_offsets(counts) -> dict:
    """Word offset of each plan section."""
    out, at = {}, 0
    for name, field, words in SECTIONS:
        out[name] = at
        at += getattr(counts, field) * words
    out["end"] = at
    return out


def plan_sections(plan: np.ndarray, counts) -> dict:
    """Split a plan array into its four entry tables (for inspection)."""
    off = section_offsets(counts)
    res = {}
    for name, field, words in SECTIONS:
        a = off[name]
        res[name] = plan[a:a + getattr(counts, field) * words].reshape(-1, words)
    return res


def cpa_workspace_size(counts, num_q_heads: int, num_kv_heads: int, head_dim: int) -> int:
    return int(load().cpa_workspace_size(ctypes.byref(counts), int(num_q_heads),
                                         int(num_kv_heads), int(head_dim)))


# ---------------------------------------------------------------------------
# device calls (torch tensors in, launches on torch's current stream)
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_dev(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("device call needs GPU tensors")


def _check_cache(k_cache, v_cache, Hkv, D):
    """K pages [num_blocks][Hkv][D/8][16][8] (16-token pages in 8-value pieces),
    V pages [num_blocks][Hkv][D][16]."""
    nb = k_cache.shape[0]
    if tuple(k_cache.shape) != (nb, Hkv, D // 8, BLOCK_SIZE, 8) or \
            tuple(v_cache.shape) != (nb, Hkv, D, BLOCK_SIZE):
        raise ValueError(f"cache shapes {tuple(k_cache.shape)} / {tuple(v_cache.shape)} do not match "
                         f"K [nb, {Hkv}, {D // 8}, 16, 8] and V [nb, {Hkv}, {D}, 16]")


def cpa_append_kv(k_new, v_new, query_start_loc, context_lens, block_table, k_cache, v_cache, *,
                  num_seqs, num_tokens, stream=None):
    _check_dev(k_new, v_new, query_start_loc, context_lens, block_table, k_cache, v_cache)
    Hkv, D = k_new.shape[1], k_new.shape[2]
    _check_cache(k_cache, v_cache, Hkv, D)
    st = load().cpa_append_kv(_ptr(k_new), _ptr(v_new), _ptr(query_start_loc), _ptr(context_lens),
                              _ptr(block_table), int(block_table.shape[1]), int(num_seqs),
                              int(num_tokens), int(Hkv), int(D), BLOCK_SIZE, _ptr(k_cache),
                              _ptr(v_cache), _stream(stream))
    if st != CPA_OK:
        raise CpaError(st, "cpa_append_kv")


def cpa_attention(q, k_cache, v_cache, block_table, query_start_loc, seq_lens, context_lens, plan,
                  counts, *, num_seqs, num_decodes, num_tokens, softmax_scale, out, lse=None,
                  workspace=None, stream=None):
    _check_dev(q, k_cache, v_cache, block_table, query_start_loc, context_lens, plan, out, lse,
               workspace)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_cache.shape[1]
    _check_cache(k_cache, v_cache, Hkv, D)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().cpa_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                              int(block_table.shape[1]), _ptr(query_start_loc), _ptr(seq_lens),
                              _ptr(context_lens), _ptr(plan), ctypes.byref(counts), int(num_seqs),
                              int(num_decodes), int(num_tokens), int(Hq), int(Hkv), int(D),
                              BLOCK_SIZE, float(softmax_scale), _ptr(out), _ptr(lse),
                              _ptr(workspace), int(ws_bytes), _stream(stream))
    if st != CPA_OK:
        raise CpaError(st, "cpa_attention")


def cpa_attention_noalloc(q, k_cache, v_cache, block_table, query_start_loc, seq_lens,
                          context_lens, plan, counts, *, num_seqs, num_decodes, num_tokens,
                          softmax_scale, out, lse=None, stream=None):
    """cpa_attention with the library's own scratch array for split pieces."""
    _check_dev(q, k_cache, v_cache, block_table, query_start_loc, context_lens, plan, out, lse)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_cache.shape[1]
    _check_cache(k_cache, v_cache, Hkv, D)
    st = load().cpa_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                      int(block_table.shape[1]), _ptr(query_start_loc),
                                      _ptr(seq_lens), _ptr(context_lens), _ptr(plan),
                                      ctypes.byref(counts), int(num_seqs), int(num_decodes),
                                      int(num_tokens), int(Hq), int(Hkv), int(D), BLOCK_SIZE,
                                      float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream))
    if st != CPA_OK:
        raise CpaError(st, "cpa_attention_noalloc")
