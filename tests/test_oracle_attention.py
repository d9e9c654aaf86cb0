"""Pins for the oracle's paged attention (CPU only).

The oracle is held to things other than itself: dense attention by numpy and
by torch's scaled_dot_product_attention (float64), closed forms, a bit-exact
selector sweep over every logical position, invariance under physical block
permutation and prefix aliasing, GQA against replicated MHA, poisoned tails,
split-and-merge against one pass, and the pages' block arithmetic.
"""
import os

import numpy as np
import pytest

import oracle
from tests import _refs

BS = 16
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_perm_blocks(rng, lens, pool):
    perm = rng.permutation(pool)
    out, k = [], 0
    for L in lens:
        n = (L + BS - 1) // BS
        out.append([int(b) for b in perm[k:k + n]])
        k += n
    return out


def _case(rng, lens, hq, hkv, d, pool_extra=5, fill=np.nan):
    dense_k = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    dense_v = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    need = sum((L + BS - 1) // BS for L in lens)
    pool = need + pool_extra
    pb = _rand_perm_blocks(rng, lens, pool)
    kp, vp, bt = _refs.place_dense(dense_k, dense_v, lens, pb, pool, hkv, d, fill=fill, dtype=np.float32)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    return q, dense_k, dense_v, kp, vp, bt


def _run(q, kp, vp, bt, lens, scale, **kw):
    return oracle.paged_attention(q, "f32", kp, vp, "f32", bt, np.asarray(lens, np.int32), scale, **kw)


@pytest.mark.parametrize("lens,hq,hkv,d", [
    ([7, 16, 33, 100], 4, 4, 64),        # the tiny workload's lengths
    ([1, 17, 200, 64], 8, 2, 128),       # GQA group 4, ragged tails
    ([300, 5], 8, 1, 64),                # MQA-like group 8
])
def test_matches_dense_numpy_and_torch_sdpa(lens, hq, hkv, d):
    rng = np.random.default_rng(sum(lens) + hq)
    q, dk, dv, kp, vp, bt = _case(rng, lens, hq, hkv, d)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    got = _run(q, kp, vp, bt, lens, scale)
    q64 = q.astype(np.float64)
    dk64 = [x.astype(np.float64) for x in dk]
    dv64 = [x.astype(np.float64) for x in dv]
    ref_np = _refs.dense_attention_numpy(q64, dk64, dv64, scale, hq // hkv)
    ref_t = _refs.dense_attention_torch(q64, dk64, dv64, scale, hq // hkv)
    assert np.max(np.abs(got - ref_np)) <= 1e-12
    assert np.max(np.abs(got - ref_t)) <= 1e-12


def test_fp8_pool_matches_dense_on_dequantised_values():
    rng = np.random.default_rng(3)
    lens, hq, hkv, d = [40, 9, 130], 8, 2, 64
    codes_k = [rng.integers(0, 256, (L, hkv, d)).astype(np.uint8) for L in lens]
    codes_v = [rng.integers(0, 256, (L, hkv, d)).astype(np.uint8) for L in lens]
    for c in codes_k + codes_v:  # no NaN codes in a real cache
        c[(c & 0x7F) == 0x7F] = 0x38
    import torch
    deq = lambda c, s: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
    ks, vs = 0.01, 0.02
    ks32, vs32 = float(np.float32(ks)), float(np.float32(vs))
    pool = sum((L + BS - 1) // BS for L in lens) + 2
    pb = _rand_perm_blocks(rng, lens, pool)
    kp, vp, bt = _refs.place_dense(codes_k, codes_v, lens, pb, pool, hkv, d, fill=0x7F, dtype=np.uint8)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    scale = float(np.float32(0.125))
    got = oracle.paged_attention(q, "f32", kp, vp, "fp8", bt, np.array(lens, np.int32), scale, ks, vs)
    ref = _refs.dense_attention_numpy(q.astype(np.float64), [deq(c, ks32) for c in codes_k],
                                      [deq(c, vs32) for c in codes_v], scale, hq // hkv)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_closed_forms():
    rng = np.random.default_rng(4)
    hq = hkv = 2
    d = 64
    scale = 0.125
    # L = 1: the output is the single value row, exactly
    q, dk, dv, kp, vp, bt = _case(rng, [1, 1], hq, hkv, d)
    got = _run(q, kp, vp, bt, [1, 1], scale)
    for s in range(2):
        for h in range(hq):
            assert np.array_equal(got[s, h], dv[s][0, h].astype(np.float64))
    # q = 0: uniform weights, the output is the mean of V
    lens = [50, 3]
    q, dk, dv, kp, vp, bt = _case(rng, lens, hq, hkv, d)
    got = _run(np.zeros_like(q), kp, vp, bt, lens, scale)
    for s, L in enumerate(lens):
        assert np.max(np.abs(got[s] - dv[s].astype(np.float64).mean(axis=0))) <= 1e-14
    # all keys equal: uniform weights again
    dk2 = [np.broadcast_to(x[:1], x.shape).copy() for x in dk]
    kp2, vp2, bt2 = _refs.place_dense(dk2, dv, lens, [list(r[r >= 0]) for r in bt], kp.shape[0], hkv, d,
                                      dtype=np.float32)
    got = _run(q, kp2, vp2, bt2, lens, scale)
    for s, L in enumerate(lens):
        assert np.max(np.abs(got[s] - dv[s].astype(np.float64).mean(axis=0))) <= 1e-14
    # V == c: every output is c (rows of the softmax sum to one)
    dv3 = [np.full_like(x, 0.75) for x in dv]
    kp3, vp3, bt3 = _refs.place_dense(dk, dv3, lens, [list(r[r >= 0]) for r in bt], kp.shape[0], hkv, d,
                                      dtype=np.float32)
    got = _run(q, kp3, vp3, bt3, lens, scale)
    assert np.max(np.abs(got - 0.75)) <= 1e-15
    # V[t] = e_t (D >= L): the output is the softmax row itself
    L = 60
    dk4 = [rng.standard_normal((L, hkv, d)).astype(np.float32)]
    dv4 = [np.zeros((L, hkv, d), np.float32)]
    for t in range(L):
        dv4[0][t, :, t] = 1.0
    kp4, vp4, bt4 = _refs.place_dense(dk4, dv4, [L], [[3, 0, 2, 1]], 5, hkv, d, dtype=np.float32)
    q4 = rng.standard_normal((1, hq, d)).astype(np.float32)
    got = _run(q4, kp4, vp4, bt4, [L], scale)
    for h in range(hq):
        row = got[0, h]
        assert abs(row[:L].sum() - 1.0) <= 1e-14 and np.all(row[L:] == 0)
        sc = dk4[0][:, h, :].astype(np.float64) @ q4[0, h].astype(np.float64) * scale
        p = np.exp(sc - sc.max()); p /= p.sum()
        assert np.max(np.abs(row[:L] - p)) <= 1e-15


def _selector_case(lens, hkv, d, js, c=2.0 ** 14):
    """K = 0 except K[j] = e_(j mod D) per (seq, head); q = c e_(j mod D): out must be V[j] exactly."""
    rng = np.random.default_rng(sum(js[0]))
    dk = [np.zeros((L, hkv, d), np.float32) for L in lens]
    dv = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    q = np.zeros((len(lens), hkv, d), np.float32)
    for s in range(len(lens)):
        for h in range(hkv):
            j = js[s][h]
            dk[s][j, h, j % d] = 1.0
            q[s, h, j % d] = c
    return q, dk, dv


def test_selector_sweep_every_position_bit_exact():
    """Every logical position of every sequence is selected once through a permuted table."""
    lens, hkv, d = [7, 16, 33, 100], 4, 64
    rng = np.random.default_rng(9)
    pool = 64
    pb = _rand_perm_blocks(rng, lens, pool)
    scale = 0.125  # c * scale = 2048: every other weight underflows to exactly 0
    maxL = max(lens)
    for step in range(0, maxL, hkv):
        js = [[min(step + h, L - 1) for h in range(hkv)] for L in lens]
        q, dk, dv = _selector_case(lens, hkv, d, js)
        kp, vp, bt = _refs.place_dense(dk, dv, lens, pb, pool, hkv, d, dtype=np.float32)
        got = _run(q, kp, vp, bt, lens, scale)
        for s in range(len(lens)):
            for h in range(hkv):
                assert np.array_equal(got[s, h], dv[s][js[s][h], h].astype(np.float64)), (s, h, js[s][h])


def test_block_permutation_and_poison_invariance_bit_exact():
    rng = np.random.default_rng(10)
    lens, hq, hkv, d = [7, 16, 33, 100, 1], 8, 2, 64
    dk = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    dv = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    pool = 40
    outs = []
    for trial in range(3):
        pb = _rand_perm_blocks(np.random.default_rng(100 + trial), lens, pool)
        fill = np.nan if trial else 0.0
        kp, vp, bt = _refs.place_dense(dk, dv, lens, pb, pool, hkv, d, fill=fill, dtype=np.float32)
        if trial == 2:  # padding entries may hold anything
            bt[bt < 0] = 123456
        outs.append(_run(q, kp, vp, bt, lens, 0.125))
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_prefix_aliasing_equals_private_copies():
    rng = np.random.default_rng(12)
    hq, hkv, d = 4, 2, 64
    prefix = 48  # three full blocks
    priv = [5, 1, 20]
    lens = [prefix + n for n in priv]
    pk = rng.standard_normal((prefix, hkv, d)).astype(np.float32)
    pv = rng.standard_normal((prefix, hkv, d)).astype(np.float32)
    dk = [np.concatenate([pk, rng.standard_normal((n, hkv, d)).astype(np.float32)]) for n in priv]
    dv = [np.concatenate([pv, rng.standard_normal((n, hkv, d)).astype(np.float32)]) for n in priv]
    q = rng.standard_normal((3, hq, d)).astype(np.float32)
    # private copies
    pb_priv = _rand_perm_blocks(rng, lens, 20)
    kp1, vp1, bt1 = _refs.place_dense(dk, dv, lens, pb_priv, 20, hkv, d, dtype=np.float32)
    # aliased: all three sequences point at blocks 0..2 for the prefix
    pb_al = [[0, 1, 2] + [3 + 2 * s + i for i in range((n + BS - 1) // BS)] for s, n in enumerate(priv)]
    kp2, vp2, bt2 = _refs.place_dense(dk, dv, lens, pb_al, 10, hkv, d, dtype=np.float32)
    assert np.array_equal(bt2[:, :3], np.tile([0, 1, 2], (3, 1)))
    assert np.array_equal(_run(q, kp1, vp1, bt1, lens, 0.125), _run(q, kp2, vp2, bt2, lens, 0.125))


def test_gqa_equals_replicated_mha_bit_exact():
    rng = np.random.default_rng(13)
    lens, hq, hkv, d = [70, 3, 33], 8, 2, 64
    q, dk, dv, kp, vp, bt = _case(rng, lens, hq, hkv, d)
    got = _run(q, kp, vp, bt, lens, 0.125)
    G = hq // hkv
    kp_r = np.ascontiguousarray(np.repeat(kp, G, axis=1))
    vp_r = np.ascontiguousarray(np.repeat(vp, G, axis=1))
    got_r = _run(q, kp_r, vp_r, bt, lens, 0.125)
    assert np.array_equal(got, got_r)


@pytest.mark.parametrize("part", [16, 48, 512])
def test_split_merge_equals_one_pass(part):
    rng = np.random.default_rng(14)
    lens, hq, hkv, d = [7, 16, 33, 100, 700], 4, 2, 64
    q, dk, dv, kp, vp, bt = _case(rng, lens, hq, hkv, d)
    one = _run(q, kp, vp, bt, lens, 0.125)
    split = _run(q, kp, vp, bt, lens, 0.125, partition_size=part)
    assert np.max(np.abs(one - split)) <= 1e-13


def test_zero_length_gives_zeros():
    rng = np.random.default_rng(15)
    q, dk, dv, kp, vp, bt = _case(rng, [5, 0, 9], 2, 2, 64)
    got = _run(q, kp, vp, bt, [5, 0, 9], 0.125)
    assert np.all(got[1] == 0)


def test_block_arithmetic_fixture():
    """The pages' example: 100 tokens under a 2048-token reservation, with 16-token blocks."""
    rows = []
    with open(os.path.join(GOLDEN, "block_arithmetic.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    rng = np.random.default_rng(16)
    for tokens, blocks, slots, reserved in rows:
        assert slots == BS * blocks
        if tokens == 0:
            continue
        # exactly `blocks` table entries are needed: capacity blocks*16 accepts, one token more rejects
        q, dk, dv, kp, vp, bt = _case(rng, [tokens], 2, 2, 64)
        assert bt.shape[1] == blocks
        _run(q, kp, vp, bt, [tokens], 0.125)
        _run(q, kp, vp, bt, [slots], 0.125) if slots <= kp.shape[0] * BS else None
        with pytest.raises(oracle.OracleError):
            _run(q, kp, vp, bt, [slots + 1], 0.125)
    # utilisation of the pages' example: 100 of 112 paged slots vs 100 of 2048 reserved
    t, b, s, r = rows[0]
    assert (t, b, s, r) == (100, 7, 112, 2048)
    assert round(100 * t / s, 1) == 89.3 and round(100 * t / r, 1) == 4.9


def test_error_paths():
    rng = np.random.default_rng(17)
    q, dk, dv, kp, vp, bt = _case(rng, [20, 5], 4, 2, 64)
    with pytest.raises(oracle.OracleError):  # a used table entry out of range
        bad = bt.copy(); bad[0, 1] = kp.shape[0]
        _run(q, kp, vp, bad, [20, 5], 0.125)
    with pytest.raises(oracle.OracleError):  # negative entry in the used range
        bad = bt.copy(); bad[1, 0] = -1
        _run(q, kp, vp, bad, [20, 5], 0.125)
    with pytest.raises(oracle.OracleError):  # negative length
        _run(q, kp, vp, bt, [20, -1], 0.125)
    with pytest.raises(oracle.OracleError):  # heads not a multiple of KV heads
        q3 = rng.standard_normal((2, 3, 64)).astype(np.float32)
        _run(q3, kp, vp, bt, [20, 5], 0.125)
