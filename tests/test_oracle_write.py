"""Pins for the oracle's KV write through slot_mapping (CPU only)."""
import os

import numpy as np
import pytest
import torch

import oracle
from tests import _refs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BS = 16


def test_hand_worked_layout_fixture():
    H, D = 2, 8
    k_new = np.zeros((4, H, D), np.float32)
    for h in range(H):
        for d in range(D):
            k_new[0, h, d] = 10 * h + d + 1
            k_new[1, h, d] = 99
            k_new[2, h, d] = 20 + 10 * h + d + 1
            k_new[3, h, d] = 40 + 10 * h + d + 1
    v_new = k_new + 100
    slots = np.array([5, -1, 17, 31], np.int32)
    kc, vc = _refs.empty_pools(2, H, D, -7.0, np.float32)
    oracle.kv_write(k_new, v_new, "f32", kc, vc, "f32", slots)
    want = {"K": np.full(512, -7.0, np.float32), "V": np.full(512, -7.0, np.float32)}
    with open(os.path.join(GOLDEN, "kv_write_layout.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                pool, i, val = line.split()
                want[pool][int(i)] = float(val)
    assert np.array_equal(kc.reshape(-1), want["K"])
    assert np.array_equal(vc.reshape(-1), want["V"])


def test_write_builds_the_same_pool_as_dense_placement():
    """Writing every token through slot_mapping == placing dense blocks by numpy transposes."""
    rng = np.random.default_rng(20)
    lens, hkv, d = [7, 16, 33, 100], 3, 64
    pool = 20
    perm = rng.permutation(pool)
    pb, k = [], 0
    for L in lens:
        n = (L + BS - 1) // BS
        pb.append([int(b) for b in perm[k:k + n]]); k += n
    dk = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    dv = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    kp_ref, vp_ref, bt = _refs.place_dense(dk, dv, lens, pb, pool, hkv, d, fill=-1.0, dtype=np.float32)
    # token list in a shuffled order, slots from the table
    toks = [(s, t) for s, L in enumerate(lens) for t in range(L)]
    order = rng.permutation(len(toks))
    kn = np.stack([dk[toks[i][0]][toks[i][1]] for i in order])
    vn = np.stack([dv[toks[i][0]][toks[i][1]] for i in order])
    slots = np.array([bt[toks[i][0], toks[i][1] // BS] * BS + toks[i][1] % BS for i in order], np.int32)
    kp = np.full_like(kp_ref, -1.0); vp = np.full_like(vp_ref, -1.0)
    oracle.kv_write(kn, vn, "f32", kp, vp, "f32", slots)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)


def test_bf16_copy_keeps_bits_and_fp8_write_quantises_each_element():
    rng = np.random.default_rng(21)
    T, H, D, NB = 9, 2, 128, 4
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots = rng.permutation(NB * BS)[:T].astype(np.int32)
    slots[3] = -1
    kc, vc = _refs.empty_pools(NB, H, D, 0xFFFF, np.uint16)
    oracle.kv_write(xb, xb, "bf16", kc, vc, "bf16", slots)
    for i, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(_refs.k_rows(kc, sl // BS, [sl % BS])[:, 0], xb[i])
            assert np.array_equal(_refs.v_rows(vc, sl // BS, [sl % BS])[:, 0], xb[i])
    assert np.count_nonzero(kc != 0xFFFF) <= (T - 1) * H * D
    assert np.count_nonzero(vc != 0xFFFF) <= (T - 1) * H * D
    # fp8: quantised element by element with the pool's scale
    k8, v8 = _refs.empty_pools(NB, H, D, 0x7F, np.uint8)
    ks, vs = 0.01, 0.003
    oracle.kv_write(xb, xb, "bf16", k8, v8, "fp8", slots, k_scale=ks, v_scale=vs)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    for i, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(_refs.k_rows(k8, sl // BS, [sl % BS])[:, 0], oracle.fp8_quantise(xf[i], ks))
            assert np.array_equal(_refs.v_rows(v8, sl // BS, [sl % BS])[:, 0], oracle.fp8_quantise(xf[i], vs))
    untouched = np.ones(NB * BS, bool); untouched[slots[slots >= 0]] = False
    for sl in np.nonzero(untouched)[0]:
        assert np.all(_refs.k_rows(k8, sl // BS, [sl % BS]) == 0x7F)
        assert np.all(_refs.v_rows(v8, sl // BS, [sl % BS]) == 0x7F)


def test_write_then_single_token_attention_returns_the_value():
    rng = np.random.default_rng(22)
    H, D, NB = 2, 64, 8
    kn = rng.standard_normal((1, H, D)).astype(np.float32)
    vn = rng.standard_normal((1, H, D)).astype(np.float32)
    for slot in (0, 15, 16, 77, NB * BS - 1):
        kc, vc = _refs.empty_pools(NB, H, D, np.nan, np.float32)
        oracle.kv_write(kn, vn, "f32", kc, vc, "f32", np.array([slot], np.int32))
        bt = np.array([[slot // BS]], np.int32)
        # a one-token context whose token sits at offset slot % 16 of its block:
        # position slot % 16 of a length (slot % 16 + 1) sequence; earlier rows are NaN,
        # so read it back as the only token by building a table whose first block is it
        if slot % BS == 0:
            out = oracle.paged_attention(rng.standard_normal((1, H, D)).astype(np.float32), "f32", kc, vc, "f32",
                                         bt, np.array([1], np.int32), 0.125)
            assert np.array_equal(out[0], vn[0].astype(np.float64))
        else:
            assert np.array_equal(_refs.v_rows(vc, slot // BS, [slot % BS])[:, 0], vn[0])
            assert np.array_equal(_refs.k_rows(kc, slot // BS, [slot % BS])[:, 0], kn[0])


def test_write_error_paths():
    k = np.zeros((2, 1, 16), np.float32)
    kc, vc = _refs.empty_pools(2, 1, 16, 0.0, np.float32)
    for bad in ([3, 3], [0, 32], [-2, 0]):  # duplicate, past the pool, below -1
        with pytest.raises(oracle.OracleError):
            oracle.kv_write(k, k, "f32", kc.copy(), vc.copy(), "f32", np.array(bad, np.int32))
    with pytest.raises(oracle.OracleError):  # f32 -> bf16 is not a supported pair
        kb, vb = _refs.empty_pools(2, 1, 16, 0, np.uint16)
        oracle.kv_write(k, k, "f32", kb, vb, "bf16", np.array([0, 1], np.int32))
    with pytest.raises(oracle.OracleError):  # fp8 needs a positive finite scale
        k8, v8 = _refs.empty_pools(2, 1, 16, 0, np.uint8)
        oracle.kv_write(k, k, "f32", k8, v8, "fp8", np.array([0, 1], np.int32), k_scale=0.0)
    with pytest.raises(oracle.OracleError):  # head_dim must be a multiple of the 16-byte chunk (16 fp8 codes)
        k6 = np.zeros((2, 1, 8), np.float32)
        oracle.kv_write(k6, k6, "f32", np.zeros((2, 1, 0, 16, 16), np.uint8), np.zeros((2, 1, 8, 16), np.uint8),
                        "fp8", np.array([0, 1], np.int32))
    oracle.kv_write(k, k, "f32", kc.copy(), vc.copy(), "f32", np.array([-1, -1], np.int32))
