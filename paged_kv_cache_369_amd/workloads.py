"""Seeded synthetic inputs for paged-KV decode (host side, numpy).

This module draws inputs only.  It holds none of the attention arithmetic:
it picks sequence lengths, places logical blocks on physical blocks, derives
the slot of every cached token from that placement (the caller's job in a
serving engine), and draws Q/K/V values.  Both the GPU path and the CPU oracle
are fed from here; neither is imported by this module.

Workloads (shapes and distributions of the decode batches the pages discuss;
block size 16 from the ipipp.com vLLM article, section 二):

  tiny     4 seqs, lengths {7, 16, 33, 100}, 4/4 heads, D=64, fp32 cache,
           a 64-block pool placed by a seeded permutation, table padded -1.
  13b      LLaMA-2-13B-shaped: B=64, 40/40 heads, D=128, bf16,
           lengths uniform in [128, 2048], pool 1.2x the need, shuffled.
  gqa8b    Llama-3-8B-shaped GQA: B=256, 32 query / 8 KV heads, D=128, bf16,
           lengths log-uniform in [256, 8192], pool exactly the need, shuffled.
  prefix   shared-prefix sampling: 32 prompts x 8 samples, 32/8 heads, D=128,
           bf16; a 1024-token prefix per prompt whose blocks are aliased by
           its 8 samples, then 1..512 private tokens per sample; an unshared
           twin layout holds a private copy of every prefix.
  longfp8  B=16, 64 query / 8 KV heads, D=128, fp8-e4m3 cache with one fp32
           scale per pool, bf16 Q and new K/V, lengths uniform in
           [16384, 32768], 512-token partitions.
  spec4    the gqa8b batch verifying speculated tokens: 4 new query tokens
           per sequence (3 guesses and the token before them), lengths as
           gqa8b counting the new tokens.
  chunk512 chunked prefill: 16 sequences, 32/8 heads, D=128, bf16, each
           taking a 512-token chunk of its prompt, contexts (chunk included)
           uniform in [2048, 8192].

Values: N(0, 1) drawn as float32 from PCG64 sub-streams of fixed size (so
the bytes do not depend on the thread count), then cast to bf16 with torch's
CPU round-to-nearest-even cast where the workload is bf16.  The fp8 scales
are amax(|x|) / 448 over each pool's tokens, in float32.

Every sequence of length L caches tokens 0..L-1: tokens 0..L-2 are the
"history" (written once when the workload is set up) and token L-1 is the
"new" token written in every decode step before attention reads it.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16
CHUNK = 1 << 22  # values per PCG64 sub-stream

WORKLOADS = ("tiny", "13b", "gqa8b", "prefix", "longfp8", "spec4", "chunk512")
SEEDS = {name: 20260000 + i for i, name in enumerate(WORKLOADS)}


@dataclasses.dataclass
class WriteBatch:
    """Tokens to write: k, v are [T, H_kv, D] in ``in_dtype``; slots [T] int32."""
    k: np.ndarray
    v: np.ndarray
    slots: np.ndarray


@dataclasses.dataclass
class Layout:
    """One physical placement of the sequences' blocks."""
    num_blocks: int
    block_table: np.ndarray          # [B, MB] int32, -1 padded
    history: List[WriteBatch]        # writes that build tokens 0..L-2
    new_slots: np.ndarray            # [B] int32 slot of token L-1 (-1 if L == 0)


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str                     # "f32" | "bf16"
    in_dtype: str                    # dtype of the K/V tokens handed to the write
    cache_dtype: str                 # "f32" | "bf16" | "fp8"
    context_lens: np.ndarray         # [B] int32
    q: np.ndarray                    # [B, H_q, D]
    new_k: np.ndarray                # [B, H_kv, D] token L-1 of each sequence
    new_v: np.ndarray
    layout: Layout
    twin: Optional[Layout] = None    # unshared copy of an aliased layout
    scale: float = 1.0               # softmax scale, float32 value
    k_scale: float = 1.0
    v_scale: float = 1.0
    partition_size: int = 0          # 0 = library default
    block_size: int = BLOCK_SIZE
    prefix_leader: Optional[np.ndarray] = None  # [B] int32 first sequence of each sharing group
    prefix_blocks: Optional[np.ndarray] = None  # [B] int32 leading blocks the group shares
    cu_q: Optional[np.ndarray] = None           # [B + 1] int32 query rows per sequence (several new tokens)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.layout.block_table.shape[1])

    def kv_elt_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.cache_dtype]

    def kv_bytes(self) -> int:
        """Bytes of K and V that attention must read: sum_s L_s * H_kv * D * 2 * elt."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * self.kv_elt_bytes()

    def kv_unique_bytes(self) -> int:
        """Bytes of the distinct cached tokens attention reads: a physical block shared by several sequences
        (an aliased prefix) counts once, with the most tokens any of them uses."""
        used = {}
        for s, L in enumerate(self.context_lens.tolist()):
            for j in range((L + 15) // 16):
                b = int(self.layout.block_table[s, j])
                used[b] = max(used.get(b, 0), min(16, L - 16 * j))
        return sum(used.values()) * self.num_kv_heads * self.head_dim * 2 * self.kv_elt_bytes()


# ---------------------------------------------------------------------------
# value draws
# ---------------------------------------------------------------------------

def _normal_f32(seed: int, stream: int, n: int, threads: int = 0) -> np.ndarray:
    """n float32 N(0,1) values; chunk c comes from PCG64(SeedSequence(seed, spawn_key=(stream, c)))."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        workers = threads or min(16, os.cpu_count() or 1)
        with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16) with torch's CPU round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _values(seed: int, stream: int, shape: Tuple[int, ...], dtype: str) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    x = _normal_f32(seed, stream, n)
    if dtype == "f32":
        return x.reshape(shape)
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        step = 1 << 26
        for lo in range(0, n, step):
            out[lo:lo + step] = to_bf16_bits(x[lo:lo + step])
        return out.reshape(shape)
    raise ValueError(dtype)


def _amax(arrs: List[np.ndarray], dtype: str) -> float:
    m = 0.0
    for a in arrs:
        if a.size == 0:
            continue
        f = bf16_bits_to_f32(a) if dtype == "bf16" else a
        m = max(m, float(np.max(np.abs(f))))
    return m


# ---------------------------------------------------------------------------
# placement
# ---------------------------------------------------------------------------

def blocks_for(length: int, block_size: int = BLOCK_SIZE) -> int:
    return (int(length) + block_size - 1) // block_size


def _table_from_lists(lists: List[List[int]], mb: int) -> np.ndarray:
    bt = np.full((len(lists), max(mb, 1)), -1, dtype=np.int32)
    for s, blocks in enumerate(lists):
        bt[s, :len(blocks)] = blocks
    return bt


def _slots_for(bt_row: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Physical slot of each logical position of one sequence under its table row."""
    return (bt_row[positions // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + positions % BLOCK_SIZE).astype(np.int32)


def _private_layout(rng: np.random.Generator, lens: np.ndarray, pool: int, mb: int):
    need = [blocks_for(L) for L in lens]
    perm = rng.permutation(pool).astype(np.int64)
    lists, k = [], 0
    for n in need:
        lists.append([int(b) for b in perm[k:k + n]])
        k += n
    return _table_from_lists(lists, mb)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def _history_batch(seed, bt, lens, hkv, d, dtype, stream_k, stream_v) -> Tuple[WriteBatch, np.ndarray, np.ndarray]:
    """Draw tokens 0..L-1 of each sequence; return the history batch (0..L-2) and the new tokens (L-1)."""
    total = int(np.sum(lens))
    k_all = _values(seed, stream_k, (total, hkv, d), dtype)
    v_all = _values(seed, stream_v, (total, hkv, d), dtype)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    hist_idx, hist_slots, new_idx = [], [], []
    B = len(lens)
    new_k = np.zeros((B, hkv, d), dtype=k_all.dtype)
    new_v = np.zeros((B, hkv, d), dtype=v_all.dtype)
    for s, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        pos = np.arange(L - 1, dtype=np.int64)
        hist_idx.append(starts[s] + pos)
        hist_slots.append(_slots_for(bt[s], pos))
        new_k[s] = k_all[starts[s] + L - 1]
        new_v[s] = v_all[starts[s] + L - 1]
    hi = np.concatenate(hist_idx) if hist_idx else np.zeros(0, dtype=np.int64)
    hs = np.concatenate(hist_slots) if hist_slots else np.zeros(0, dtype=np.int32)
    batch = WriteBatch(np.ascontiguousarray(k_all[hi]), np.ascontiguousarray(v_all[hi]), hs.astype(np.int32))
    return batch, new_k, new_v


def _new_slots(bt: np.ndarray, lens: np.ndarray) -> np.ndarray:
    out = np.full(len(lens), -1, dtype=np.int32)
    for s, L in enumerate(lens):
        if L > 0:
            out[s] = _slots_for(bt[s], np.array([L - 1]))[0]
    return out


def make_custom(name: str, seed: int, lens, num_heads: int, num_kv_heads: int, head_dim: int,
                q_dtype: str, cache_dtype: str, pool_factor: float = 1.0, pool_blocks: int = 0,
                max_blocks_per_seq: int = 0, partition_size: int = 0,
                in_dtype: Optional[str] = None) -> Workload:
    """A private-block workload with given lengths (used by the named workloads and by tests)."""
    lens = np.asarray(lens, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(0,))))
    need = int(sum(blocks_for(L) for L in lens))
    pool = pool_blocks or int(math.ceil(need * pool_factor))
    pool = max(pool, need)
    mb = max_blocks_per_seq or max([blocks_for(L) for L in lens] + [1])
    bt = _private_layout(rng, lens, pool, mb)
    if in_dtype is None:
        in_dtype = q_dtype if cache_dtype == "fp8" else cache_dtype
    hist, new_k, new_v = _history_batch(seed, bt, lens, num_kv_heads, head_dim, in_dtype, 2, 3)
    q = _values(seed, 1, (len(lens), num_heads, head_dim), q_dtype)
    w = Workload(name=name, num_seqs=len(lens), num_heads=num_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, q_dtype=q_dtype, in_dtype=in_dtype, cache_dtype=cache_dtype,
                 context_lens=lens, q=q, new_k=new_k, new_v=new_v,
                 layout=Layout(pool, bt, [hist], _new_slots(bt, lens)),
                 scale=float(np.float32(1.0) / np.sqrt(np.float32(head_dim))),
                 partition_size=partition_size)
    if cache_dtype == "fp8":
        w.k_scale = float(np.float32(_amax([hist.k, new_k], in_dtype)) / np.float32(448.0))
        w.v_scale = float(np.float32(_amax([hist.v, new_v], in_dtype)) / np.float32(448.0))
    return w


def _lens_for(name: str, rng: np.random.Generator) -> np.ndarray:
    if name == "tiny":
        return np.array([7, 16, 33, 100], dtype=np.int32)
    if name == "13b":
        return rng.integers(128, 2048, size=64, endpoint=True).astype(np.int32)
    if name == "gqa8b":
        u = rng.uniform(np.log(256.0), np.log(8192.0), size=256)
        return np.clip(np.floor(np.exp(u)), 256, 8192).astype(np.int32)
    if name == "longfp8":
        return rng.integers(16384, 32768, size=16, endpoint=True).astype(np.int32)
    if name == "spec4":
        u = rng.uniform(np.log(256.0), np.log(8192.0), size=256)
        return np.clip(np.floor(np.exp(u)), 256, 8192).astype(np.int32)
    if name == "chunk512":
        return rng.integers(2048, 8192, size=16, endpoint=True).astype(np.int32)
    raise ValueError(name)


def _prefix_private_lens(rng: np.random.Generator, n: int, priv_max: int) -> np.ndarray:
    return rng.integers(1, priv_max, size=n, endpoint=True).astype(np.int32)


def _make_prefix(seed: int, prompts: int = 32, samples: int = 8, prefix: int = 1024,
                 priv_max: int = 512, hq: int = 32, hkv: int = 8, d: int = 128) -> Workload:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(0,))))
    B = prompts * samples
    priv = _prefix_private_lens(rng, B, priv_max)
    lens = (prefix + priv).astype(np.int32)
    pb = prefix // BLOCK_SIZE
    priv_blocks = [blocks_for(n) for n in priv]
    mb = pb + max(priv_blocks)

    # values: prefix tokens per prompt, private tokens per sample
    pre_k = _values(seed, 2, (prompts, prefix, hkv, d), "bf16")
    pre_v = _values(seed, 3, (prompts, prefix, hkv, d), "bf16")
    ptot = int(priv.sum())
    prv_k = _values(seed, 4, (ptot, hkv, d), "bf16")
    prv_v = _values(seed, 5, (ptot, hkv, d), "bf16")
    pstart = np.concatenate([[0], np.cumsum(priv)[:-1]]).astype(np.int64)
    q = _values(seed, 1, (B, hq, d), "bf16")

    def build(shared: bool) -> Layout:
        n_prefix = prompts * pb if shared else B * pb
        pool = n_prefix + int(sum(priv_blocks))
        perm = rng.permutation(pool).astype(np.int64)
        k = 0
        prefix_ids = []
        if shared:
            for p in range(prompts):
                prefix_ids.append([int(b) for b in perm[k:k + pb]]); k += pb
        lists = []
        for s in range(B):
            if shared:
                ids = list(prefix_ids[s // samples])
            else:
                ids = [int(b) for b in perm[k:k + pb]]; k += pb
            ids += [int(b) for b in perm[k:k + priv_blocks[s]]]; k += priv_blocks[s]
            lists.append(ids)
        bt = _table_from_lists(lists, mb)
        # prefix writes: once per prompt (shared) or once per sample (twin)
        pk, pv, ps = [], [], []
        writers = range(prompts) if shared else range(B)
        for w in writers:
            s = w * samples if shared else w
            p = w if shared else w // samples
            pk.append(pre_k[p]); pv.append(pre_v[p])
            ps.append(_slots_for(bt[s], np.arange(prefix, dtype=np.int64)))
        prefix_batch = WriteBatch(np.ascontiguousarray(np.concatenate(pk)), np.ascontiguousarray(np.concatenate(pv)),
                                  np.concatenate(ps).astype(np.int32))
        # private history: positions prefix .. L-2 of each sample
        hk, hv, hs = [], [], []
        for s in range(B):
            n = int(priv[s]) - 1
            if n <= 0:
                continue
            hk.append(prv_k[pstart[s]:pstart[s] + n]); hv.append(prv_v[pstart[s]:pstart[s] + n])
            hs.append(_slots_for(bt[s], np.arange(prefix, prefix + n, dtype=np.int64)))
        priv_batch = WriteBatch(np.ascontiguousarray(np.concatenate(hk)), np.ascontiguousarray(np.concatenate(hv)),
                                np.concatenate(hs).astype(np.int32))
        return Layout(pool, bt, [prefix_batch, priv_batch], _new_slots(bt, lens))

    shared = build(True)
    twin = build(False)
    new_k = np.stack([prv_k[pstart[s] + priv[s] - 1] for s in range(B)])
    new_v = np.stack([prv_v[pstart[s] + priv[s] - 1] for s in range(B)])
    return Workload(name="prefix", num_seqs=B, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                    q_dtype="bf16", in_dtype="bf16", cache_dtype="bf16", context_lens=lens, q=q,
                    new_k=new_k, new_v=new_v, layout=shared, twin=twin,
                    scale=float(np.float32(1.0) / np.sqrt(np.float32(d))),
                    prefix_leader=(np.arange(B, dtype=np.int32) // samples * samples).astype(np.int32),
                    prefix_blocks=np.full(B, pb, dtype=np.int32))


def make_shared(name: str, seed: int, groups, num_heads: int, num_kv_heads: int, head_dim: int,
                q_dtype: str, cache_dtype: str, in_dtype: Optional[str] = None, partition_size: int = 0,
                spare_blocks: int = 3) -> Workload:
    """Consecutive groups of sequences that share a prompt prefix (parallel samples of one prompt).

    groups: list of (prefix_tokens, [length of each member]), every length >= prefix_tokens.  The
    prefix_tokens // 16 whole blocks of a group's prefix are one set of physical blocks in every member's
    table; a partly filled last prefix block is a private copy per member (what a copy-on-write leaves),
    followed by the member's private tokens.  Each token value is drawn once: the prefix per group, the rest
    per member.  The new token of a member is its last one; when that lies in a shared block (the member has
    no private token), it is written with the prefix and the member's new slot is -1."""
    if in_dtype is None:
        in_dtype = q_dtype if cache_dtype == "fp8" else cache_dtype
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(0,))))
    lens, leader, pblocks, gid, pre_len = [], [], [], [], []
    for g, (pre, members) in enumerate(groups):
        first = len(lens)
        for L in members:
            if L < pre:
                raise ValueError("a member is shorter than its group's prefix")
            lens.append(int(L)); leader.append(first); pblocks.append(pre // BLOCK_SIZE)
            gid.append(g); pre_len.append(pre)
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    shared_n = [pre // BLOCK_SIZE for pre, _ in groups]
    own_n = [blocks_for(L) - pblocks[s] for s, L in enumerate(lens.tolist())]
    pool = sum(shared_n) + sum(own_n) + spare_blocks
    perm = rng.permutation(pool).astype(np.int64)
    k = 0
    gblocks = []
    for n in shared_n:
        gblocks.append([int(b) for b in perm[k:k + n]]); k += n
    lists = []
    for s in range(B):
        ids = list(gblocks[gid[s]]) + [int(b) for b in perm[k:k + own_n[s]]]
        k += own_n[s]
        lists.append(ids)
    mb = max([len(x) for x in lists] + [1])
    bt = _table_from_lists(lists, mb)

    pre_tot = sum(pre for pre, _ in groups)
    own_tot = int(sum(int(L) - pre_len[s] for s, L in enumerate(lens.tolist())))
    pk = _values(seed, 2, (pre_tot, num_kv_heads, head_dim), in_dtype)
    pv = _values(seed, 3, (pre_tot, num_kv_heads, head_dim), in_dtype)
    ok_ = _values(seed, 4, (own_tot, num_kv_heads, head_dim), in_dtype)
    ov_ = _values(seed, 5, (own_tot, num_kv_heads, head_dim), in_dtype)
    pstart = np.concatenate([[0], np.cumsum([pre for pre, _ in groups])[:-1]]).astype(np.int64)
    ostart = np.concatenate([[0], np.cumsum([int(L) - pre_len[s] for s, L in enumerate(lens.tolist())])[:-1]]
                            ).astype(np.int64) if B else np.zeros(0, dtype=np.int64)

    def token(s: int, t: int):
        """K and V rows of position t of sequence s."""
        if t < pre_len[s]:
            i = pstart[gid[s]] + t
            return pk[i], pv[i]
        i = ostart[s] + t - pre_len[s]
        return ok_[i], ov_[i]

    hk, hv, hs = [], [], []
    new_k = np.zeros((B, num_kv_heads, head_dim), dtype=pk.dtype)
    new_v = np.zeros((B, num_kv_heads, head_dim), dtype=pv.dtype)
    new_slots = np.full(B, -1, dtype=np.int32)
    for s in range(B):
        L = int(lens[s])
        sh = pblocks[s] * BLOCK_SIZE
        first_of_group = leader[s] == s
        for t in range(L):
            kt, vt = token(s, t)
            slot = int(_slots_for(bt[s], np.array([t]))[0])
            if t < sh:
                if first_of_group:
                    hk.append(kt); hv.append(vt); hs.append(slot)
            elif t == L - 1:
                new_k[s], new_v[s], new_slots[s] = kt, vt, slot
            else:
                hk.append(kt); hv.append(vt); hs.append(slot)
        if L > 0 and L - 1 < sh:  # last token inside the shared prefix: written with the prefix
            new_k[s], new_v[s] = token(s, L - 1)
    shp = (0, num_kv_heads, head_dim)
    hist = WriteBatch(np.ascontiguousarray(np.stack(hk)) if hk else np.zeros(shp, dtype=pk.dtype),
                      np.ascontiguousarray(np.stack(hv)) if hv else np.zeros(shp, dtype=pv.dtype),
                      np.asarray(hs, dtype=np.int32))
    q = _values(seed, 1, (B, num_heads, head_dim), q_dtype)
    w = Workload(name=name, num_seqs=B, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                 q_dtype=q_dtype, in_dtype=in_dtype, cache_dtype=cache_dtype, context_lens=lens, q=q,
                 new_k=new_k, new_v=new_v, layout=Layout(pool, bt, [hist], new_slots),
                 scale=float(np.float32(1.0) / np.sqrt(np.float32(head_dim))), partition_size=partition_size,
                 prefix_leader=np.asarray(leader, dtype=np.int32), prefix_blocks=np.asarray(pblocks, dtype=np.int32))
    if cache_dtype == "fp8":
        w.k_scale = float(np.float32(_amax([pk, ok_], in_dtype)) / np.float32(448.0))
        w.v_scale = float(np.float32(_amax([pv, ov_], in_dtype)) / np.float32(448.0))
    return w


def make_multi(name: str, seed: int, lens, new_tokens, num_heads: int, num_kv_heads: int, head_dim: int,
               q_dtype: str, cache_dtype: str, in_dtype: Optional[str] = None, partition_size: int = 0,
               pool_factor: float = 1.0) -> Workload:
    """Several new tokens per sequence (a chunk of a prompt, or speculated tokens to verify).

    Sequence s caches lens[s] tokens; its last new_tokens[s] are this step's new tokens (written through
    slot_mapping in the step, ``layout.new_slots`` / ``new_k`` / ``new_v``, one row per new token), the rest
    are history.  q holds one row per new token, sequence by sequence; cu_q [B + 1] gives the rows."""
    lens = np.asarray(lens, dtype=np.int32)
    nnew = np.asarray(new_tokens, dtype=np.int32)
    if np.any(nnew < 0) or np.any(nnew > lens):
        raise ValueError("each sequence needs 0 <= new tokens <= cached tokens")
    if in_dtype is None:
        in_dtype = q_dtype if cache_dtype == "fp8" else cache_dtype
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(0,))))
    need = int(sum(blocks_for(L) for L in lens))
    pool = max(int(math.ceil(need * pool_factor)), need, 1)
    mb = max([blocks_for(L) for L in lens] + [1])
    bt = _private_layout(rng, lens, pool, mb)
    total = int(lens.sum())
    k_all = _values(seed, 2, (total, num_kv_heads, head_dim), in_dtype)
    v_all = _values(seed, 3, (total, num_kv_heads, head_dim), in_dtype)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    hist_idx, hist_slots, new_idx, new_slots = [], [], [], []
    for s_, L in enumerate(lens.tolist()):
        n = int(nnew[s_])
        pos_h = np.arange(L - n, dtype=np.int64)
        pos_n = np.arange(L - n, L, dtype=np.int64)
        hist_idx.append(starts[s_] + pos_h)
        hist_slots.append(_slots_for(bt[s_], pos_h))
        new_idx.append(starts[s_] + pos_n)
        new_slots.append(_slots_for(bt[s_], pos_n))
    hi = np.concatenate(hist_idx).astype(np.int64)
    ni = np.concatenate(new_idx).astype(np.int64)
    hist = WriteBatch(np.ascontiguousarray(k_all[hi]), np.ascontiguousarray(v_all[hi]),
                      np.concatenate(hist_slots).astype(np.int32))
    cu = np.concatenate([[0], np.cumsum(nnew)]).astype(np.int32)
    q = _values(seed, 1, (int(cu[-1]), num_heads, head_dim), q_dtype)
    w = Workload(name=name, num_seqs=len(lens), num_heads=num_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, q_dtype=q_dtype, in_dtype=in_dtype, cache_dtype=cache_dtype, context_lens=lens,
                 q=q, new_k=np.ascontiguousarray(k_all[ni]), new_v=np.ascontiguousarray(v_all[ni]),
                 layout=Layout(pool, bt, [hist], np.concatenate(new_slots).astype(np.int32)),
                 scale=float(np.float32(1.0) / np.sqrt(np.float32(head_dim))), partition_size=partition_size,
                 cu_q=cu)
    if cache_dtype == "fp8":
        w.k_scale = float(np.float32(_amax([k_all], in_dtype)) / np.float32(448.0))
        w.v_scale = float(np.float32(_amax([v_all], in_dtype)) / np.float32(448.0))
    return w


def context_lengths(name: str, seed: Optional[int] = None) -> np.ndarray:
    """The context lengths ``make(name, seed)`` gives, without drawing any values (fast at every size).
    For "prefix" the samples of a prompt are consecutive, 8 to a prompt, each 1024 + its private length."""
    seed = SEEDS[name] if seed is None else seed
    if name == "prefix":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(0,))))
        return (1024 + _prefix_private_lens(rng, 32 * 8, 512)).astype(np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(9,))))
    return _lens_for(name, rng)


def make(name: str, seed: Optional[int] = None) -> Workload:
    """Build one of the named workloads (deterministic in ``seed``)."""
    seed = SEEDS[name] if seed is None else seed
    if name == "prefix":
        return _make_prefix(seed)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(9,))))
    lens = _lens_for(name, rng)
    if name == "tiny":
        return make_custom("tiny", seed, lens, 4, 4, 64, "f32", "f32", pool_blocks=64, max_blocks_per_seq=7)
    if name == "13b":
        return make_custom("13b", seed, lens, 40, 40, 128, "bf16", "bf16", pool_factor=1.2, max_blocks_per_seq=128)
    if name == "gqa8b":
        return make_custom("gqa8b", seed, lens, 32, 8, 128, "bf16", "bf16", max_blocks_per_seq=512)
    if name == "longfp8":
        return make_custom("longfp8", seed, lens, 64, 8, 128, "bf16", "fp8", max_blocks_per_seq=2048,
                           partition_size=512, in_dtype="bf16")
    if name == "spec4":
        return make_multi("spec4", seed, lens, [4] * len(lens), 32, 8, 128, "bf16", "bf16")
    if name == "chunk512":
        return make_multi("chunk512", seed, lens, [512] * len(lens), 32, 8, 128, "bf16", "bf16")
    raise ValueError(name)


def make_scaled(name: str, max_seqs: int, len_cap: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    """A reduced workload with the same head shape, dtypes and length law (first ``max_seqs`` draws)."""
    seed = SEEDS[name] if seed is None else seed
    if name == "prefix":
        return _make_prefix(seed, prompts=max(1, max_seqs // 8), prefix=256, priv_max=64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(9,))))
    lens = _lens_for(name, rng)[:max_seqs]
    if len_cap:
        lens = np.minimum(lens, len_cap).astype(np.int32)
    spec = {"tiny": (4, 4, 64, "f32", "f32", 0), "13b": (40, 40, 128, "bf16", "bf16", 0),
            "gqa8b": (32, 8, 128, "bf16", "bf16", 0), "longfp8": (64, 8, 128, "bf16", "fp8", 512)}[name]
    hq, hkv, d, qd, cd, part = spec
    return make_custom(name + "-scaled", seed, lens, hq, hkv, d, qd, cd, pool_factor=1.2,
                       partition_size=part, in_dtype=("bf16" if cd == "fp8" else None))
