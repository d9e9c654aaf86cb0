"""GPU: paged_attention_decode_noalloc, the decode whose workspace is the library's static per-GPU scratch.

It runs the same kernel as paged_attention_decode, so on the same inputs it must give the same bits; it is
also held to the oracle at the decode's tolerances.  Each case makes two calls in a row, the second with a
smaller batch, so the second call runs on the scratch the first one left behind (its counters must be back at
zero, its slots hold stale states).  Sizes whose states do not fit the scratch are refused before any launch.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_369_amd as pkv
from paged_kv_cache_369_amd import workloads as W
from tests import _gpu

pytestmark = pytest.mark.gpu


def _noalloc(w, kp, vp, partition_size):
    q = _gpu.to_dev(w.q, w.q_dtype)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode_noalloc(out, q, kp, vp, _gpu.to_dev(w.layout.block_table, "i32"),
                                       _gpu.to_dev(w.context_lens, "i32"), w.scale, w.k_scale, w.v_scale,
                                       partition_size=partition_size)
    torch.cuda.synchronize()
    return _gpu.widen(_gpu.to_host(out, w.q_dtype), w.q_dtype)


# (workload law, sequences of the first call, of the second, length cap, partition size)
CASES = [
    ("gqa8b", 48, 13, None, 0),       # runs cut over many waves: the merge tree lives in the scratch
    ("gqa8b", 40, 7, None, 64),       # partitions of 64 tokens
    ("longfp8", 5, 2, 12000, 512),    # fp8 pools, 8 query heads per run
    ("13b", 24, 5, None, 0),          # one head per run
    ("tiny", 4, 2, None, 32),         # fp32 pools
]


@pytest.mark.parametrize("name,n1,n2,cap,part", CASES)
def test_noalloc_matches_decode_on_two_calls(gpu, name, n1, n2, cap, part):
    for n in (n1, n2):
        w = W.make_scaled(name, n, cap)
        _gpu.note(f"noalloc decode {name} seqs={n} part={part}")
        kp, vp = _gpu.gpu_pools(w, w.layout)
        got = _noalloc(w, kp, vp, part)
        ref = _gpu.gpu_decode(w, w.layout, kp, vp, partition_size=part)
        assert np.array_equal(got, ref), "no-allocation decode differs from paged_attention_decode"
        ok, ov = _gpu.oracle_pools(w, w.layout)
        want = _gpu.oracle_decode(w, w.layout, ok, ov)
        err, where = _gpu.max_err(got, want)
        assert err <= _gpu.TOL[w.cache_dtype], (err, where)


def test_noalloc_sixteen_heads_per_run_at_head_dim_64(gpu):
    """16 query heads per KV head at head_dim 64: states of 32 + 16 * 64 floats per wave still fit."""
    for n in (30, 9):
        w = W.make_custom("noalloc16", 500 + n, np.random.default_rng(n).integers(1, 3000, n), 32, 2, 64,
                          "bf16", "bf16")
        _gpu.note(f"noalloc decode 32/2 heads d=64 seqs={n}")
        kp, vp = _gpu.gpu_pools(w, w.layout)
        got = _noalloc(w, kp, vp, 0)
        ref = _gpu.gpu_decode(w, w.layout, kp, vp, partition_size=0)
        assert np.array_equal(got, ref)


def test_noalloc_refuses_states_beyond_the_scratch(gpu):
    """16 query heads per KV head at head_dim 128 need 34 MB of states: refused, nothing launched or written."""
    w = W.make_custom("noalloc_big", 77, [100, 40], 16, 1, 128, "bf16", "bf16")
    kp, vp = _gpu.gpu_pools(w, w.layout)
    q = _gpu.to_dev(w.q, "bf16")
    out = torch.full_like(q, float("nan"))
    _gpu.note("noalloc decode refusal (16 heads per run, d=128)")
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_noalloc(out, q, kp, vp, _gpu.to_dev(w.layout.block_table, "i32"),
                                           _gpu.to_dev(w.context_lens, "i32"), w.scale)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert bool(torch.isnan(out.float()).all())
