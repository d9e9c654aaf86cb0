"""Pins for the oracle's multi-token-query (varlen) attention.

Each case builds a paged cache with the oracle's write (pinned on its own)
from contiguous K/V drawn here, and checks oracle_paged_attention_varlen
against things it is not: dense causal softmax attention computed with numpy
on the contiguous K/V (which fixes the causal mask, the position of a chunk
of new tokens at the end of the context, and the GQA head mapping), the
decode oracle for the last new token (which sees every cached token), and the
closed form of a token at position 0 (its output is its own V row).
"""
import numpy as np
import pytest

import oracle


def _cache(lens, hkv, d, dtype, seed, perm=True, k_scale=1.0, v_scale=1.0):
    """Contiguous K/V per sequence (float64 values exactly representable in dtype), and a paged cache of them."""
    rng = np.random.default_rng(seed)
    nb = [-(-L // 16) for L in lens]
    pool = sum(nb) + 2
    ids = rng.permutation(pool) if perm else np.arange(pool)
    mb = max(nb + [1])
    bt = np.full((len(lens), mb), -1, dtype=np.int32)
    k = 0
    for s, n in enumerate(nb):
        bt[s, :n] = ids[k:k + n]
        k += n
    npdt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]
    kp = np.zeros(oracle.k_pool_shape(pool, hkv, d, dtype), dtype=npdt)
    vp = np.zeros(oracle.v_pool_shape(pool, hkv, d, dtype), dtype=npdt)
    Ks, Vs = [], []
    for s, L in enumerate(lens):
        kk = rng.standard_normal((L, hkv, d)).astype(np.float32)
        vv = rng.standard_normal((L, hkv, d)).astype(np.float32)
        slots = np.array([bt[s, t // 16] * 16 + t % 16 for t in range(L)], dtype=np.int32)
        if dtype == "fp8":
            oracle.kv_write(kk, vv, "f32", kp, vp, "fp8", slots, k_scale=k_scale, v_scale=v_scale)
            # the pool scales are fp32 values, widened exactly
            Ks.append(oracle.fp8_decode(oracle.fp8_quantise(kk, k_scale)) * np.float64(np.float32(k_scale)))
            Vs.append(oracle.fp8_decode(oracle.fp8_quantise(vv, v_scale)) * np.float64(np.float32(v_scale)))
        else:
            oracle.kv_write(kk, vv, "f32", kp, vp, "f32", slots)
            Ks.append(kk.astype(np.float64))
            Vs.append(vv.astype(np.float64))
    return kp, vp, bt, Ks, Vs


def _dense_causal(Q, K, V, scale, n_new):
    """numpy: rows of the last n_new positions of causal attention over contiguous K/V [L, Hkv, D]."""
    L, hkv, d = K.shape
    h = Q.shape[1]
    G = h // hkv
    out = np.zeros((n_new, h, d))
    for r in range(n_new):
        pos = L - n_new + r
        for hh in range(h):
            kh = K[: pos + 1, hh // G, :]
            s = scale * (kh @ Q[r, hh])
            w = np.exp(s - s.max())
            out[r, hh] = (w / w.sum()) @ V[: pos + 1, hh // G, :]
    return out


@pytest.mark.parametrize("lens,nnew", [([1, 17, 40], None), ([30, 50, 16], [7, 16, 1]), ([65, 3], [65, 0])])
def test_matches_dense_causal_attention(lens, nnew):
    hq, hkv, d = 8, 2, 64
    nnew = lens if nnew is None else nnew
    kp, vp, bt, Ks, Vs = _cache(lens, hkv, d, "f32", 5)
    rng = np.random.default_rng(6)
    cu = np.concatenate([[0], np.cumsum(nnew)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), hq, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    got = oracle.paged_attention_varlen(q, "f32", cu, kp, vp, "f32", bt, np.array(lens), scale)
    for s in range(len(lens)):
        want = _dense_causal(q[cu[s]:cu[s + 1]].astype(np.float64), Ks[s], Vs[s], np.float64(np.float32(scale)), nnew[s])
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], want, rtol=0, atol=1e-12)


def test_last_new_token_equals_decode():
    lens, nnew = [40, 23, 100], [5, 23, 9]
    hq, hkv, d = 16, 4, 64
    kp, vp, bt, _, _ = _cache(lens, hkv, d, "f32", 11)
    cu = np.concatenate([[0], np.cumsum(nnew)]).astype(np.int32)
    q = np.random.default_rng(12).standard_normal((int(cu[-1]), hq, d)).astype(np.float32)
    got = oracle.paged_attention_varlen(q, "f32", cu, kp, vp, "f32", bt, np.array(lens), 0.125)
    last = np.ascontiguousarray(q[cu[1:] - 1])
    dec = oracle.paged_attention(last, "f32", kp, vp, "f32", bt, np.array(lens), 0.125)
    np.testing.assert_array_equal(got[cu[1:] - 1], dec)


def test_position_zero_returns_its_value_row():
    lens = [16, 3]
    kp, vp, bt, _, Vs = _cache(lens, 2, 64, "f32", 21)
    q = np.random.default_rng(22).standard_normal((19, 4, 64)).astype(np.float32)
    cu = np.array([0, 16, 19], dtype=np.int32)
    got = oracle.paged_attention_varlen(q, "f32", cu, kp, vp, "f32", bt, np.array(lens), 0.3)
    for s, r in ((0, 0), (1, 16)):
        for h in range(4):
            np.testing.assert_array_equal(got[r, h], Vs[s][0, h // 2])


def test_fp8_pool_and_bf16_queries():
    lens, nnew = [33, 18], [8, 18]
    hq, hkv, d = 8, 8, 128
    ks, vs = 0.011, 0.009
    kp, vp, bt, Ks, Vs = _cache(lens, hkv, d, "fp8", 31, k_scale=ks, v_scale=vs)
    rng = np.random.default_rng(32)
    cu = np.array([0, 8, 26], dtype=np.int32)
    qf = rng.standard_normal((26, hq, d)).astype(np.float32)
    import torch
    qb = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    qd = oracle.bf16_to_double(qb).reshape(qf.shape)
    scale = float(np.float32(1 / np.sqrt(d)))
    got = oracle.paged_attention_varlen(qb, "bf16", cu, kp, vp, "fp8", bt, np.array(lens), scale, k_scale=ks,
                                        v_scale=vs)
    for s in range(2):
        want = _dense_causal(qd[cu[s]:cu[s + 1]], Ks[s], Vs[s], np.float64(np.float32(scale)), nnew[s])
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], want, rtol=0, atol=1e-12)


def test_rejects_bad_arguments():
    lens = [10, 4]
    kp, vp, bt, _, _ = _cache(lens, 2, 64, "f32", 41)
    q = np.zeros((6, 4, 64), dtype=np.float32)
    with pytest.raises(oracle.OracleError):     # more new tokens than cached tokens
        oracle.paged_attention_varlen(q, "f32", np.array([0, 1, 6]), kp, vp, "f32", bt, np.array(lens), 1.0)
    with pytest.raises(oracle.OracleError):     # cu_seqlens_q decreasing
        oracle.paged_attention_varlen(q, "f32", np.array([0, 7, 6]), kp, vp, "f32", bt, np.array(lens), 1.0)
    empty = oracle.paged_attention_varlen(np.zeros((0, 4, 64), dtype=np.float32), "f32", np.array([0, 0, 0]), kp, vp,
                                          "f32", bt, np.array(lens), 1.0)
    assert empty.shape == (0, 4, 64)
