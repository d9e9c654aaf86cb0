"""Seeded input generator: determinism and the structure each workload promises."""
import numpy as np
import pytest

from paged_kv_cache_369_amd import workloads as W


def _all_slots(layout):
    return np.concatenate([b.slots for b in layout.history] + [layout.new_slots[layout.new_slots >= 0]])


def _check_layout(w, layout, aliased=False):
    bt, lens = layout.block_table, w.context_lens
    used = []
    for s, L in enumerate(lens):
        nb = W.blocks_for(L)
        row = bt[s]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < layout.num_blocks)
        assert np.all(row[nb:] == -1)
        used.extend(row[:nb].tolist())
    if not aliased:
        assert len(used) == len(set(used))
    slots = _all_slots(layout)
    assert len(slots) == len(set(slots.tolist()))  # every cached token has its own slot
    if not aliased:
        assert len(slots) == int(lens.sum())


def test_tiny_matches_the_stated_case():
    w = W.make("tiny")
    assert w.context_lens.tolist() == [7, 16, 33, 100]
    assert (w.num_heads, w.num_kv_heads, w.head_dim) == (4, 4, 64)
    assert w.layout.num_blocks == 64 and w.max_blocks_per_seq == 7
    assert w.scale == 0.125 and w.cache_dtype == "f32"
    _check_layout(w, w.layout)
    # 1 + 1 + 3 + 7 blocks, the pages' 100-token example needing 7
    assert int((w.layout.block_table >= 0).sum()) == 12


def test_determinism_and_thread_independence():
    a = W.make("tiny")
    b = W.make("tiny")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.layout.history[0].k, b.layout.history[0].k)
    x1 = W._normal_f32(5, 1, 3 * W.CHUNK + 17, threads=1)
    x2 = W._normal_f32(5, 1, 3 * W.CHUNK + 17, threads=7)
    assert np.array_equal(x1, x2)
    c = W.make("tiny", seed=1)
    assert not np.array_equal(a.q, c.q)


@pytest.mark.parametrize("name", ["13b", "gqa8b", "longfp8"])
def test_scaled_workloads_structure(name):
    w = W.make_scaled(name, 6, len_cap=700)
    _check_layout(w, w.layout)
    assert w.q.shape == (6, w.num_heads, w.head_dim)


def test_length_laws():
    rng = lambda: np.random.Generator(np.random.PCG64(np.random.SeedSequence(W.SEEDS["gqa8b"], spawn_key=(9,))))
    L = W._lens_for("gqa8b", rng())
    assert L.min() >= 256 and L.max() <= 8192 and len(L) == 256
    # log-uniform: the median sits near sqrt(256 * 8192) = 1448
    assert 1000 < np.median(L) < 2100
    L = W._lens_for("13b", rng())
    assert L.min() >= 128 and L.max() <= 2048 and len(L) == 64
    L = W._lens_for("longfp8", rng())
    assert L.min() >= 16384 and L.max() <= 32768 and len(L) == 16


def test_prefix_aliasing_structure():
    w = W.make_scaled("prefix", 16)
    bt = w.layout.block_table
    pb = 256 // 16
    for p in range(2):
        rows = bt[p * 8:(p + 1) * 8, :pb]
        assert np.all(rows == rows[0])  # 8 samples share the prefix blocks
    tw = w.twin.block_table
    assert len(set(tw[:, :pb].reshape(-1).tolist())) == 16 * pb  # the twin copies them
    _check_layout(w, w.twin)
    # new tokens never land in a shared block
    shared = set(bt[:, :pb].reshape(-1).tolist())
    assert not any(int(s) // 16 in shared for s in w.layout.new_slots)


def test_fp8_scales_are_amax_over_448():
    w = W.make_scaled("longfp8", 2, len_cap=300)
    ks = np.float32(w.k_scale) * np.float32(448)
    allk = np.concatenate([W.bf16_bits_to_f32(w.layout.history[0].k).ravel(), W.bf16_bits_to_f32(w.new_k).ravel()])
    assert abs(float(ks) - float(np.abs(allk).max())) <= 1e-6 * float(ks)
