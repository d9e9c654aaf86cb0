"""GPU: block copies of a copy-on-write, and a fork / copy-on-write / write /
decode round trip through the library's block manager, against the oracle's
write and attention on the same slots and copies."""
import random

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_369_amd as pkv
from paged_kv_cache_369_amd import workloads as W
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("fp8", 128), ("f32", 64)])
def test_copy_blocks_byte_exact(gpu, dt, d):
    rng = np.random.default_rng(7)
    nb, h = 50, 4
    kshape, vshape = pkv.k_cache_shape(nb, h, d, dt), pkv.v_cache_shape(nb, h, d)
    npdt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dt]
    k0 = rng.integers(0, 255, int(np.prod(kshape)) * np.dtype(npdt).itemsize, dtype=np.uint8).view(npdt).reshape(kshape)
    v0 = rng.integers(0, 255, int(np.prod(vshape)) * np.dtype(npdt).itemsize, dtype=np.uint8).view(npdt).reshape(vshape)
    perm = rng.permutation(nb)
    src, dst = perm[:12].astype(np.int32), perm[12:24].astype(np.int32)   # distinct, no chains
    src = np.append(src, [7, 60]).astype(np.int32)       # an out-of-range pair is skipped
    dst = np.append(dst, [-1, 3]).astype(np.int32)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dt]
    kt = torch.from_numpy(k0.view(np.int16) if dt == "bf16" else k0).cuda().view(tdt)
    vt = torch.from_numpy(v0.view(np.int16) if dt == "bf16" else v0).cuda().view(tdt)
    _gpu.note(f"copy_blocks {dt} d={d}")
    pkv.paged_kv_copy_blocks(kt, vt, _gpu.to_dev(src, "i32"), _gpu.to_dev(dst, "i32"))
    torch.cuda.synchronize()
    kw, vw = k0.copy(), v0.copy()
    for s, t in zip(src[:12], dst[:12]):
        kw[t] = k0[s]
        vw[t] = v0[s]
    kg = kt.view(torch.int16 if dt == "bf16" else tdt).cpu().numpy().view(npdt)
    vg = vt.view(torch.int16 if dt == "bf16" else tdt).cpu().numpy().view(npdt)
    assert np.array_equal(kg.view(np.uint8), kw.view(np.uint8))
    assert np.array_equal(vg.view(np.uint8), vw.view(np.uint8))


def test_fork_copy_on_write_decode(gpu):
    rnd = random.Random(3)
    rng = np.random.default_rng(3)
    nb, mbs, hq, hkv, d = 96, 16, 8, 2, 128
    bm = pkv.BlockManager(nb, mbs)
    kshape, vshape = pkv.k_cache_shape(nb, hkv, d, "bf16"), pkv.v_cache_shape(nb, hkv, d)
    kg = torch.zeros(kshape, dtype=torch.bfloat16, device="cuda")
    vg = torch.zeros(vshape, dtype=torch.bfloat16, device="cuda")
    ko = np.zeros(oracle.k_pool_shape(nb, hkv, d, "bf16"), dtype=np.uint16)
    vo = np.zeros(oracle.v_pool_shape(nb, hkv, d, "bf16"), dtype=np.uint16)

    def tokens(n):
        return W.to_bf16_bits(rng.standard_normal((n, hkv, d), dtype=np.float32))

    def run_copies():
        while True:
            src, dst = bm.take_copies(8)
            if len(src) == 0:
                return
            pkv.paged_kv_copy_blocks(kg, vg, _gpu.to_dev(src, "i32"), _gpu.to_dev(dst, "i32"))
            for s, t in zip(src, dst):
                ko[t] = ko[s]
                vo[t] = vo[s]

    def write(seq, n):
        slots = bm.append(seq, n)
        run_copies()  # copies before the write of the new tokens, on the same stream
        k, v = tokens(n), tokens(n)
        pkv.paged_kv_write(_gpu.to_dev(k, "bf16"), _gpu.to_dev(v, "bf16"), kg, vg, _gpu.to_dev(slots, "i32"))
        oracle.kv_write(k, v, "bf16", ko, vo, "bf16", slots)

    bm.add(0)
    write(0, 37)                         # prompt: two full blocks and a partial one
    for c in (1, 2, 3):
        bm.fork(0, c)                    # parallel samples share the prompt's blocks
    live = [0, 1, 2, 3]
    for step in range(12):
        for s in live:
            write(s, rnd.choice([1, 1, 2, 7]))
        if step == 5:
            bm.free(2)                   # a sample ends; its private blocks return to the pool
            live.remove(2)
            bm.add(4)
            live.append(4)
            write(4, 20)
    seqs = [0, 1, 3, 4]
    table, lens = bm.table(seqs, mbs)
    assert bm.stats()[4] == 0            # every copy ran
    q = W.to_bf16_bits(rng.standard_normal((len(seqs), hq, d), dtype=np.float32))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    out = torch.empty((len(seqs), hq, d), dtype=torch.bfloat16, device="cuda")
    _gpu.note(f"fork/cow decode lens={lens.tolist()}")
    pkv.paged_attention_decode(out, _gpu.to_dev(q, "bf16"), kg, vg, _gpu.to_dev(table, "i32"),
                               _gpu.to_dev(lens, "i32"), scale)
    torch.cuda.synchronize()
    got = _gpu.widen(_gpu.to_host(out, "bf16"), "bf16")
    want = oracle.paged_attention(q, "bf16", ko, vo, "bf16", table, lens, scale)
    assert np.max(np.abs(got - want)) <= _gpu.TOL["bf16"]
    # the pools agree byte for byte too
    assert np.array_equal(kg.view(torch.int16).cpu().numpy().view(np.uint16), ko)
    assert np.array_equal(vg.view(torch.int16).cpu().numpy().view(np.uint16), vo)


def _kv_of_prefix(tokens, hkv, d):
    """K and V rows (float32) of the last token of `tokens`: a function of the whole prefix, as a model's are."""
    seed = hash(tuple(int(t) for t in tokens)) & 0x7fffffff
    rng = np.random.default_rng(seed)
    return rng.standard_normal((hkv, d)).astype(np.float32), rng.standard_normal((hkv, d)).astype(np.float32)


def test_prefix_cache_reuse_decodes_like_private_copies(gpu):
    """Prompts sharing system prefixes go through the manager with prefix caching; only the tokens it does not
    reuse are written.  Decoding each sequence over its table equals attention over a private copy of its own
    tokens' K/V (oracle)."""
    rnd = random.Random(5)
    hq, hkv, d, nb = 8, 2, 64, 120
    systems = [[rnd.randint(0, 20) for _ in range(n)] for n in (48, 33, 80)]
    bm = pkv.BlockManager(nb, 16)
    bm.enable_prefix_caching()
    kc = torch.zeros(pkv.k_cache_shape(nb, hkv, d, "f32"), dtype=torch.float32, device="cuda")
    vc = torch.zeros(pkv.v_cache_shape(nb, hkv, d), dtype=torch.float32, device="cuda")
    prompts = {}
    reused = 0
    for s in range(12):
        toks = list(rnd.choice(systems)) + [rnd.randint(0, 20) for _ in range(rnd.randint(1, 30))]
        slots, cached = bm.add_prompt(s, toks)
        reused += cached
        prompts[s] = toks
        kn = np.stack([_kv_of_prefix(toks[:p + 1], hkv, d)[0] for p in range(cached, len(toks))])
        vn = np.stack([_kv_of_prefix(toks[:p + 1], hkv, d)[1] for p in range(cached, len(toks))])
        pkv.paged_kv_write(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), kc, vc,
                           torch.from_numpy(slots.astype(np.int32)).cuda())
        if s in (3, 7):
            bm.free(s - 1)             # released blocks stay registered and may be reused or evicted
            del prompts[s - 1]
    assert reused > 0
    seqs = sorted(prompts)
    tab, lens = bm.table(seqs, 16)
    q = np.random.default_rng(9).standard_normal((len(seqs), hq, d)).astype(np.float32)
    out = torch.empty((len(seqs), hq, d), dtype=torch.float32, device="cuda")
    _gpu.note("prefix cache reuse decode")
    pkv.paged_attention_decode(out, torch.from_numpy(q).cuda(), kc, vc, torch.from_numpy(tab).cuda(),
                               torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(), 0.125)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # oracle: each sequence's own tokens in a private pool
    priv_tab = np.full((len(seqs), 16), -1, dtype=np.int32)
    kp = np.zeros(oracle.k_pool_shape(len(seqs) * 16, hkv, d, "f32"), dtype=np.float32)
    vp = np.zeros(oracle.v_pool_shape(len(seqs) * 16, hkv, d, "f32"), dtype=np.float32)
    for r, s in enumerate(seqs):
        toks = prompts[s]
        nblk = -(-len(toks) // 16)
        priv_tab[r, :nblk] = np.arange(r * 16, r * 16 + nblk)
        kk = np.stack([_kv_of_prefix(toks[:p + 1], hkv, d)[0] for p in range(len(toks))])
        vv = np.stack([_kv_of_prefix(toks[:p + 1], hkv, d)[1] for p in range(len(toks))])
        sl = np.array([priv_tab[r, p // 16] * 16 + p % 16 for p in range(len(toks))], dtype=np.int32)
        oracle.kv_write(kk, vv, "f32", kp, vp, "f32", sl)
    want = oracle.paged_attention(q, "f32", kp, vp, "f32", priv_tab, np.asarray(lens, dtype=np.int32), 0.125)
    assert np.max(np.abs(got - want)) <= _gpu.TOL["f32"]
