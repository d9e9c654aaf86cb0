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
    k_new = np.array([[[1, 2], [3, 4]], [[5, 6], [7, 8]], [[9, 9], [9, 9]], [[10, 11], [12, 13]]], np.float32)
    v_new = k_new + 100
    slots = np.array([5, 17, -1, 47], np.int32)
    kc = np.full((3, 2, BS, 2), -7.0, np.float32)
    vc = np.full((3, 2, BS, 2), -7.0, np.float32)
    oracle.kv_write(k_new, v_new, "f32", kc, vc, "f32", slots)
    want_k = np.full(192, -7.0, np.float32)
    want_v = np.full(192, -7.0, np.float32)
    with open(os.path.join(GOLDEN, "kv_write_layout.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                i, val = line.split()
                want_k[int(i)] = float(val)
                want_v[int(i)] = float(val) + 100
    assert np.array_equal(kc.reshape(-1), want_k)
    assert np.array_equal(vc.reshape(-1), want_v)


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
    kc = np.full((NB, H, BS, D), 0xFFFF, np.uint16); vc = kc.copy()
    oracle.kv_write(xb, xb, "bf16", kc, vc, "bf16", slots)
    for i, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(kc[sl // BS, :, sl % BS, :], xb[i])
    assert np.count_nonzero(kc != 0xFFFF) <= (T - 1) * H * D
    # fp8: quantised element by element with the pool's scale
    k8 = np.full((NB, H, BS, D), 0x7F, np.uint8); v8 = k8.copy()
    ks, vs = 0.01, 0.003
    oracle.kv_write(xb, xb, "bf16", k8, v8, "fp8", slots, k_scale=ks, v_scale=vs)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    for i, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(k8[sl // BS, :, sl % BS, :], oracle.fp8_quantise(xf[i], ks))
            assert np.array_equal(v8[sl // BS, :, sl % BS, :], oracle.fp8_quantise(xf[i], vs))
    untouched = np.ones(NB * BS, bool); untouched[slots[slots >= 0]] = False
    assert np.all(k8.transpose(0, 2, 1, 3).reshape(NB * BS, H, D)[untouched] == 0x7F)


def test_write_then_single_token_attention_returns_the_value():
    rng = np.random.default_rng(22)
    H, D, NB = 2, 64, 8
    kn = rng.standard_normal((1, H, D)).astype(np.float32)
    vn = rng.standard_normal((1, H, D)).astype(np.float32)
    for slot in (0, 15, 16, 77, NB * BS - 1):
        kc = np.full((NB, H, BS, D), np.nan, np.float32); vc = kc.copy()
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
            got = vc[slot // BS, :, slot % BS, :]
            assert np.array_equal(got, vn[0])


def test_write_error_paths():
    k = np.zeros((2, 1, 16), np.float32)
    kc = np.zeros((2, 1, BS, 16), np.float32)
    for bad in ([3, 3], [0, 32], [-2, 0]):  # duplicate, past the pool, below -1
        with pytest.raises(oracle.OracleError):
            oracle.kv_write(k, k, "f32", kc.copy(), kc.copy(), "f32", np.array(bad, np.int32))
    with pytest.raises(oracle.OracleError):  # f32 -> bf16 is not a supported pair
        oracle.kv_write(k, k, "f32", np.zeros((2, 1, BS, 16), np.uint16), np.zeros((2, 1, BS, 16), np.uint16),
                        "bf16", np.array([0, 1], np.int32))
    with pytest.raises(oracle.OracleError):  # fp8 needs a positive finite scale
        oracle.kv_write(k, k, "f32", np.zeros((2, 1, BS, 16), np.uint8), np.zeros((2, 1, BS, 16), np.uint8),
                        "fp8", np.array([0, 1], np.int32), k_scale=0.0)
    oracle.kv_write(k, k, "f32", kc.copy(), kc.copy(), "f32", np.array([-1, -1], np.int32))
