"""Host-side figures of the knee / free-ride sweep (no GPU).

The chunk's flops are checked against a count of visible (query, key) pairs
made by brute force over the causal mask of a chunk after a cached prefix
("Chunked Prefill", "Why a chunk can be nearly free": a chunk attends to
everything prefilled before it; "05. Chunked Prefill" section 3: causal inside
the chunk), and the fit is checked on step times built from a known fixed
cost and rate.
"""

import numpy as np
import pytest

from chunked_prefill_mixed_amd import sweep


@pytest.mark.parametrize("c,prefix", [(1, 0), (5, 0), (7, 3), (16, 40), (33, 17)])
def test_chunk_flops_counts_visible_pairs(c, prefix):
    pairs = 0
    for j in range(c):          # query at position prefix + j
        for k in range(prefix + c):
            if k <= prefix + j:
                pairs += 1
    # QK^T and PV: 2 d flops each per (query head, key) pair
    assert sweep.chunk_flops(c, prefix, hq=3, d=8) == 4 * 8 * 3 * pairs


@pytest.mark.parametrize("prefix", [0, 1024, 4096])
def test_tokens_for_flops_inverts_chunk_flops(prefix):
    for c in (1, 16, 480, 2048):
        assert sweep.tokens_for_flops(sweep.chunk_flops(c, prefix), prefix) == pytest.approx(c)


def test_decode_kv_bytes():
    # 2 rows of context 15 and 0: 16 + 1 keys and values, Hkv 8 x D 128 x 2 bytes
    assert sweep.decode_kv_bytes([15, 0]) == (16 + 1) * 8 * 128 * 2 * 2


def test_knee_figures_recover_fixed_cost_and_rate():
    sizes = sweep.KNEE_SIZES
    prefix, dec, fixed, rate = 1024, 85e-6, 20e-6, 1.0e15
    steps = [dec + fixed + sweep.chunk_flops(c, prefix) / rate for c in sizes]
    f = sweep.knee_figures(sizes, steps, dec, prefix, decode_bytes=300e6)
    assert f["fixed_us"] == pytest.approx(20.0)
    assert f["rate_tflops"] == pytest.approx(1000.0)
    # the knee: compute time equals the fixed cost
    assert sweep.chunk_flops(f["knee_tokens"], prefix) / rate == pytest.approx(fixed)
    # free ride at peak: the flops that fit in 300 MB / 8 TB/s at 2.5 PFLOP/s
    assert sweep.chunk_flops(f["free_ride_peak_tokens"], prefix) == pytest.approx(
        300e6 / 8e12 * 2.5e15)
    # as run, every step is above decode + 10% once the fixed 20 us is added
    assert f["free_ride_as_run_tokens"] == 0
    # small chunks within 5% of the decode-only step, larger ones on the line
    steps2 = [dec * 1.05 if c <= 256 else dec + fixed + sweep.chunk_flops(c, prefix) / rate
              for c in sizes]
    assert sweep.knee_figures(sizes, steps2, dec, prefix, 300e6)["free_ride_as_run_tokens"] == 256
